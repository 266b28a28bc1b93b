// fp4_api.cpp -- the C ABI declared in include/fp4.h: host-side argument
// validation (no HIP call happens before it passes), the gfx950 device check,
// and dispatch to the kernels.
#include "fp4.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "launch.h"

using namespace fp4impl;

static_assert(FP4_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "the header states the scratch size");

namespace {

constexpr uint32_t kKnownFlags =
    FP4_FOUR_OVER_SIX | FP4_BLOCK2D | FP4_TRANSPOSE | FP4_STOCHASTIC | FP4_HADAMARD | FP4_SCALE_SEARCH | FP4_TENSOR_SCALE;
constexpr int64_t kMaxGridYZ = 65535;
constexpr int64_t kMaxGridX = 2147483647;
// fp4_gemm_grouped: every tile scans the group offsets 64 at a time
constexpr int64_t kMaxGroupsVar = 4096;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Per-device cache of "is gfx950": 0 unknown, 1 yes, 2 no.
std::atomic<int> g_device_ok[64];

fp4_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FP4_ERR_DEVICE;
  }
  if (dev < 64) {
    int c = g_device_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return FP4_OK;
    if (c == 2) return FP4_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return FP4_ERR_DEVICE;
  }
  bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FP4_OK : FP4_ERR_DEVICE;
}

std::atomic<int> g_cu_count[64];

}  // namespace

int fp4impl::device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

namespace {

struct QuantPlan {
  int64_t R = 0, C = 0;
  int blk = 0;
  int nparts = 0;
  size_t ws = 0;
};

// Validation shared by fp4_quantize_workspace and fp4_quantize that only
// depends on sizes and options.
fp4_status plan_quantize(int64_t batch, int64_t rows, int64_t cols, const fp4_quant_opts* o, QuantPlan* p) {
  if (!o || o->size != sizeof(fp4_quant_opts)) return FP4_ERR_INVALID;
  if (o->format != FP4_MXFP4 && o->format != FP4_NVFP4) return FP4_ERR_INVALID;
  if (o->flags & ~kKnownFlags) return FP4_ERR_INVALID;
  if (batch < 0 || rows < 0 || cols < 0) return FP4_ERR_INVALID;
  const bool nv = o->format == FP4_NVFP4;
  if (!nv && (o->flags & (FP4_BLOCK2D | FP4_SCALE_SEARCH | FP4_TENSOR_SCALE))) return FP4_ERR_UNSUPPORTED;
  if ((o->flags & FP4_TENSOR_SCALE) && (o->flags & (FP4_FOUR_OVER_SIX | FP4_SCALE_SEARCH | FP4_BLOCK2D)))
    return FP4_ERR_UNSUPPORTED;
  if ((o->flags & FP4_BLOCK2D) && (o->flags & FP4_HADAMARD) && (o->flags & FP4_TRANSPOSE)) return FP4_ERR_UNSUPPORTED;
  const bool tr = o->flags & FP4_TRANSPOSE;
  p->blk = nv ? 16 : 32;
  p->R = tr ? cols : rows;
  p->C = tr ? rows : cols;
  if (p->C % p->blk != 0) return FP4_ERR_INVALID;
  if (tr && (p->R % 8 != 0)) return FP4_ERR_INVALID;
  if ((o->flags & FP4_BLOCK2D) && (p->R % 16 != 0)) return FP4_ERR_INVALID;
  if (batch > kMaxGridYZ) return FP4_ERR_UNSUPPORTED;
  if (tr) {
    // transposed kernel: one workgroup per 256 source rows x 64 source
    // columns (128 with 16 x 16 tiles), in a one-dimensional grid padded to
    // whole XCD lanes
    const int64_t wcols = (o->flags & FP4_BLOCK2D) ? 128 : 64;
    if (((batch * ((cols + wcols - 1) / wcols) + 7) / 8) * 8 * ((rows + 255) / 256) > kMaxGridX)
      return FP4_ERR_UNSUPPORTED;
  } else if (o->flags & FP4_BLOCK2D) {
    if (p->R / 16 > kMaxGridYZ || ((p->C / 16) + 15) / 16 > kMaxGridX) return FP4_ERR_UNSUPPORTED;
  } else {
    if (p->R > 0 && ((p->R * (p->C / 16)) + 255) / 256 > kMaxGridX) return FP4_ERR_UNSUPPORTED;
  }
  if (nv && !o->amax_in && batch > 0 && rows > 0 && cols > 0) {
    p->nparts = amax_partials(rows, cols, o->flags);
    // the partial maxima of every item, then each item's folded amax
    p->ws = (size_t)batch * (size_t)(p->nparts + 1) * sizeof(float);
  }
  return FP4_OK;
}

}  // namespace

extern "C" {

const char* fp4_status_str(int32_t s) {
  switch (s) {
    case FP4_OK: return "FP4_OK";
    case FP4_ERR_INVALID: return "FP4_ERR_INVALID: invalid argument";
    case FP4_ERR_UNSUPPORTED: return "FP4_ERR_UNSUPPORTED: unsupported option or shape combination";
    case FP4_ERR_ALIGN: return "FP4_ERR_ALIGN: misaligned pointer or stride";
    case FP4_ERR_DEVICE: return "FP4_ERR_DEVICE: current HIP device is not gfx950";
    case FP4_ERR_WORKSPACE: return "FP4_ERR_WORKSPACE: workspace missing or too small";
    case FP4_ERR_HIP: return "FP4_ERR_HIP: HIP runtime error";
    case FP4_ERR_SCRATCH: return "FP4_ERR_SCRATCH: needs more than the built-in scratch, or it could not be located";
    default: return "unknown fp4 status";
  }
}

size_t fp4_quantize_workspace(int64_t batch, int64_t rows, int64_t cols, const fp4_quant_opts* opts) {
  QuantPlan p;
  if (plan_quantize(batch, rows, cols, opts, &p) != FP4_OK) return 0;
  return p.ws;
}

}  // extern "C"

// fp4_quantize and fp4_quantize_noalloc: the amax partials go to the
// caller's workspace, or (noalloc) to the library's per-GPU scratch array.
static fp4_status quantize_impl(const void* x, int32_t x_dtype, int64_t batch, int64_t rows, int64_t cols,
                                int64_t ld_x, int64_t batch_stride_x, const fp4_quant_opts* opts,
                                uint8_t* codes, int64_t ld_codes, int64_t batch_stride_codes,
                                uint8_t* scales, int64_t ld_scales, int64_t batch_stride_scales,
                                float* tensor_scale, void* workspace, size_t workspace_bytes, bool noalloc,
                                void* stream) {
  QuantPlan p;
  fp4_status st = plan_quantize(batch, rows, cols, opts, &p);
  if (st != FP4_OK) return st;
  if (x_dtype != FP4_F32 && x_dtype != FP4_BF16) return FP4_ERR_INVALID;
  if (batch == 0 || rows == 0 || cols == 0) return FP4_OK;
  const bool nv = opts->format == FP4_NVFP4;
  if (!x || !codes || !scales || (nv && !tensor_scale)) return FP4_ERR_INVALID;
  if (ld_x < cols || ld_codes < p.C / 2 || ld_scales < p.C / p.blk) return FP4_ERR_INVALID;
  if (batch > 1) {
    if (batch_stride_x < 0) return FP4_ERR_INVALID;
    if (batch_stride_codes < (p.R - 1) * ld_codes + p.C / 2) return FP4_ERR_INVALID;
    if (batch_stride_scales < (p.R - 1) * ld_scales + p.C / p.blk) return FP4_ERR_INVALID;
  }
  const int64_t esize = x_dtype == FP4_BF16 ? 2 : 4;
  if (!aligned(x, 16) || (ld_x * esize) % 16 != 0 || (batch > 1 && (batch_stride_x * esize) % 16 != 0))
    return FP4_ERR_ALIGN;
  if (!aligned(codes, 8) || ld_codes % 8 != 0 || (batch > 1 && batch_stride_codes % 8 != 0)) return FP4_ERR_ALIGN;
  if (nv && !aligned(tensor_scale, 4)) return FP4_ERR_ALIGN;
  if (nv && opts->amax_in && !aligned(opts->amax_in, 4)) return FP4_ERR_ALIGN;
  if (noalloc) {
    if (p.ws > kNoAllocScratchBytes) return FP4_ERR_SCRATCH;
  } else if (p.ws > 0) {
    if (!workspace || workspace_bytes < p.ws) return FP4_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return FP4_ERR_ALIGN;
  }
  st = check_device();
  if (st != FP4_OK) return st;
  if (noalloc && p.ws > 0) {
    float* sp = nullptr;
    if (noalloc_scratch(&sp) != hipSuccess) {
      (void)hipGetLastError();
      return FP4_ERR_SCRATCH;
    }
    workspace = sp;
  }

  QuantArgs a{};
  a.x = x;
  a.x_bf16 = x_dtype == FP4_BF16;
  a.batch = batch;
  a.src_rows = rows;
  a.src_cols = cols;
  a.ld_x = ld_x;
  a.bs_x = batch > 1 ? batch_stride_x : 0;
  a.R = p.R;
  a.C = p.C;
  a.nvfp4 = nv;
  a.flags = opts->flags;
  a.signs = opts->rht_signs & 0xffffu;
  a.seed = opts->seed;
  a.offset = opts->offset;
  a.amax_in = opts->amax_in;
  a.codes = codes;
  a.ld_c = ld_codes;
  a.bs_c = batch > 1 ? batch_stride_codes : 0;
  a.scales = scales;
  a.ld_s = ld_scales;
  a.bs_s = batch > 1 ? batch_stride_scales : 0;
  a.tensor_scale = tensor_scale;
  a.partials = static_cast<float*>(workspace);
  a.nparts = p.nparts;
  (void)hipGetLastError();
  return launch_quantize(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

extern "C" {

fp4_status fp4_quantize(const void* x, int32_t x_dtype, int64_t batch, int64_t rows, int64_t cols,
                        int64_t ld_x, int64_t batch_stride_x, const fp4_quant_opts* opts,
                        uint8_t* codes, int64_t ld_codes, int64_t batch_stride_codes,
                        uint8_t* scales, int64_t ld_scales, int64_t batch_stride_scales,
                        float* tensor_scale, void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_impl(x, x_dtype, batch, rows, cols, ld_x, batch_stride_x, opts, codes, ld_codes,
                       batch_stride_codes, scales, ld_scales, batch_stride_scales, tensor_scale, workspace,
                       workspace_bytes, false, stream);
}

fp4_status fp4_quantize_noalloc(const void* x, int32_t x_dtype, int64_t batch, int64_t rows, int64_t cols,
                                int64_t ld_x, int64_t batch_stride_x, const fp4_quant_opts* opts,
                                uint8_t* codes, int64_t ld_codes, int64_t batch_stride_codes,
                                uint8_t* scales, int64_t ld_scales, int64_t batch_stride_scales,
                                float* tensor_scale, void* stream) {
  return quantize_impl(x, x_dtype, batch, rows, cols, ld_x, batch_stride_x, opts, codes, ld_codes,
                       batch_stride_codes, scales, ld_scales, batch_stride_scales, tensor_scale, nullptr, 0,
                       true, stream);
}

fp4_status fp4_dequantize(int32_t format, int64_t batch, int64_t rows, int64_t cols,
                          const uint8_t* codes, int64_t ld_codes, int64_t batch_stride_codes,
                          const uint8_t* scales, int64_t ld_scales, int64_t batch_stride_scales,
                          const float* tensor_scale, void* y, int32_t y_dtype, int64_t ld_y,
                          int64_t batch_stride_y, void* stream) {
  if (format != FP4_MXFP4 && format != FP4_NVFP4) return FP4_ERR_INVALID;
  if (y_dtype != FP4_F32 && y_dtype != FP4_BF16) return FP4_ERR_INVALID;
  if (batch < 0 || rows < 0 || cols < 0) return FP4_ERR_INVALID;
  const bool nv = format == FP4_NVFP4;
  const int64_t blk = nv ? 16 : 32;
  if (cols % blk != 0) return FP4_ERR_INVALID;
  if (batch > kMaxGridYZ) return FP4_ERR_UNSUPPORTED;
  if (rows > 0 && ((rows * (cols / 16)) + 255) / 256 > kMaxGridX) return FP4_ERR_UNSUPPORTED;
  if (batch == 0 || rows == 0 || cols == 0) return FP4_OK;
  if (!codes || !scales || !y || (nv && !tensor_scale)) return FP4_ERR_INVALID;
  if (ld_codes < cols / 2 || ld_scales < cols / blk || ld_y < cols) return FP4_ERR_INVALID;
  if (batch > 1 && (batch_stride_codes < 0 || batch_stride_scales < 0 ||
                    batch_stride_y < (rows - 1) * ld_y + cols))
    return FP4_ERR_INVALID;
  const int64_t esize = y_dtype == FP4_BF16 ? 2 : 4;
  if (!aligned(codes, 8) || ld_codes % 8 != 0 || (batch > 1 && batch_stride_codes % 8 != 0)) return FP4_ERR_ALIGN;
  if (!aligned(y, 16) || (ld_y * esize) % 16 != 0 || (batch > 1 && (batch_stride_y * esize) % 16 != 0))
    return FP4_ERR_ALIGN;
  if (nv && !aligned(tensor_scale, 4)) return FP4_ERR_ALIGN;
  fp4_status st = check_device();
  if (st != FP4_OK) return st;
  DequantArgs a;
  a.nvfp4 = nv;
  a.batch = batch;
  a.rows = rows;
  a.cols = cols;
  a.codes = codes;
  a.ld_c = ld_codes;
  a.bs_c = batch > 1 ? batch_stride_codes : 0;
  a.scales = scales;
  a.ld_s = ld_scales;
  a.bs_s = batch > 1 ? batch_stride_scales : 0;
  a.tensor_scale = tensor_scale;
  a.y = y;
  a.y_bf16 = y_dtype == FP4_BF16;
  a.ld_y = ld_y;
  a.bs_y = batch > 1 ? batch_stride_y : 0;
  (void)hipGetLastError();
  return launch_dequantize(a, static_cast<hipStream_t>(stream)) == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

// Checks shared by the dense GEMM entry points (everything but the output)
// and the operand half of GemmArgs.
static fp4_status plan_gemm_operands(int32_t format, int64_t groups, int64_t M, int64_t N, int64_t K,
                                     const uint8_t* a_codes, int64_t lda, int64_t a_group_stride,
                                     const uint8_t* a_scales, int64_t lda_scales, int64_t a_scales_group_stride,
                                     const float* a_tensor_scale,
                                     const uint8_t* b_codes, int64_t ldb, int64_t b_group_stride,
                                     const uint8_t* b_scales, int64_t ldb_scales, int64_t b_scales_group_stride,
                                     const float* b_tensor_scale, GemmArgs* g) {
  if (format != FP4_MXFP4 && format != FP4_NVFP4) return FP4_ERR_INVALID;
  if (groups < 0 || M < 0 || N < 0 || K < 0) return FP4_ERR_INVALID;
  if (K % 64 != 0) return FP4_ERR_INVALID;
  if (groups > kMaxGridYZ || (M + 127) / 128 > kMaxGridYZ || (N + 127) / 128 > kMaxGridX) return FP4_ERR_UNSUPPORTED;
  const bool nv = format == FP4_NVFP4;
  const int64_t blk = nv ? 16 : 32;
  if (!a_codes || !a_scales || !b_codes || !b_scales) return FP4_ERR_INVALID;
  if (nv && (!a_tensor_scale || !b_tensor_scale)) return FP4_ERR_INVALID;
  if (lda < K / 2 || ldb < K / 2 || lda_scales < K / blk || ldb_scales < K / blk) return FP4_ERR_INVALID;
  if (groups > 1 && (a_group_stride < 0 || b_group_stride < 0 || a_scales_group_stride < 0 ||
                     b_scales_group_stride < 0))
    return FP4_ERR_INVALID;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || lda % 16 != 0 || ldb % 16 != 0) return FP4_ERR_ALIGN;
  // per-group operand panels are addressed with 32-bit offsets, and a
  // 256-row tile's offsets stay below 2^31 (row pitches below 8 MiB)
  if (M * lda >= (int64_t(1) << 31) || N * ldb >= (int64_t(1) << 31) || M * lda_scales >= (int64_t(1) << 31) ||
      N * ldb_scales >= (int64_t(1) << 31))
    return FP4_ERR_UNSUPPORTED;
  if (lda >= (int64_t(1) << 23) || ldb >= (int64_t(1) << 23) || lda_scales >= (int64_t(1) << 23) ||
      ldb_scales >= (int64_t(1) << 23))
    return FP4_ERR_UNSUPPORTED;
  if (groups > 1 && (a_group_stride % 16 != 0 || b_group_stride % 16 != 0)) return FP4_ERR_ALIGN;
  // scale rows are read 16 bytes at a time, up to the next multiple of 16
  if (!aligned(a_scales, 16) || !aligned(b_scales, 16) || lda_scales % 16 != 0 || ldb_scales % 16 != 0 ||
      (groups > 1 && (a_scales_group_stride % 16 != 0 || b_scales_group_stride % 16 != 0)))
    return FP4_ERR_ALIGN;
  if (nv && (!aligned(a_tensor_scale, 4) || !aligned(b_tensor_scale, 4))) return FP4_ERR_ALIGN;
  *g = GemmArgs{};
  g->nvfp4 = nv;
  g->groups = groups;
  g->M = M;
  g->N = N;
  g->K = K;
  g->a = a_codes;
  g->lda = lda;
  g->a_gs = groups > 1 ? a_group_stride : 0;
  g->as = a_scales;
  g->lda_s = lda_scales;
  g->as_gs = groups > 1 ? a_scales_group_stride : 0;
  g->a_ts = a_tensor_scale;
  g->a_ts_gs = 1;
  g->b = b_codes;
  g->ldb = ldb;
  g->b_gs = groups > 1 ? b_group_stride : 0;
  g->bs = b_scales;
  g->ldb_s = ldb_scales;
  g->bs_gs = groups > 1 ? b_scales_group_stride : 0;
  g->b_ts = b_tensor_scale;
  return FP4_OK;
}

fp4_status fp4_gemm(int32_t format, int64_t groups, int64_t M, int64_t N, int64_t K,
                    const uint8_t* a_codes, int64_t lda, int64_t a_group_stride,
                    const uint8_t* a_scales, int64_t lda_scales, int64_t a_scales_group_stride,
                    const float* a_tensor_scale,
                    const uint8_t* b_codes, int64_t ldb, int64_t b_group_stride,
                    const uint8_t* b_scales, int64_t ldb_scales, int64_t b_scales_group_stride,
                    const float* b_tensor_scale,
                    void* c, int32_t c_dtype, int64_t ldc, int64_t c_group_stride, void* stream) {
  if (format != FP4_MXFP4 && format != FP4_NVFP4) return FP4_ERR_INVALID;
  if (c_dtype != FP4_F32 && c_dtype != FP4_BF16) return FP4_ERR_INVALID;
  if (groups < 0 || M < 0 || N < 0 || K < 0) return FP4_ERR_INVALID;
  if (K % 64 != 0) return FP4_ERR_INVALID;
  if (groups > kMaxGridYZ || (M + 127) / 128 > kMaxGridYZ || (N + 127) / 128 > kMaxGridX) return FP4_ERR_UNSUPPORTED;
  if (groups == 0 || M == 0 || N == 0) return FP4_OK;
  GemmArgs g;
  fp4_status st = plan_gemm_operands(format, groups, M, N, K, a_codes, lda, a_group_stride, a_scales, lda_scales,
                                     a_scales_group_stride, a_tensor_scale, b_codes, ldb, b_group_stride, b_scales,
                                     ldb_scales, b_scales_group_stride, b_tensor_scale, &g);
  if (st != FP4_OK) return st;
  if (!c || ldc < N) return FP4_ERR_INVALID;
  if (groups > 1 && c_group_stride < (M - 1) * ldc + N) return FP4_ERR_INVALID;
  if (!aligned(c, c_dtype == FP4_BF16 ? 2 : 4)) return FP4_ERR_ALIGN;
  st = check_device();
  if (st != FP4_OK) return st;
  g.c = c;
  g.c_bf16 = c_dtype == FP4_BF16;
  g.ldc = ldc;
  g.c_gs = groups > 1 ? c_group_stride : 0;
  {
    const int64_t es = c_dtype == FP4_BF16 ? 2 : 4;
    g.c_vec_ok = aligned(c, 16) && (ldc * es) % 16 == 0 && (groups == 1 || (c_group_stride * es) % 16 == 0);
  }
  (void)hipGetLastError();
  return launch_gemm(g, static_cast<hipStream_t>(stream)) == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status fp4_gemm_quantize_output(int32_t format, int64_t groups, int64_t M, int64_t N, int64_t K,
                                    const uint8_t* a_codes, int64_t lda, int64_t a_group_stride,
                                    const uint8_t* a_scales, int64_t lda_scales, int64_t a_scales_group_stride,
                                    const float* a_tensor_scale,
                                    const uint8_t* b_codes, int64_t ldb, int64_t b_group_stride,
                                    const uint8_t* b_scales, int64_t ldb_scales, int64_t b_scales_group_stride,
                                    const float* b_tensor_scale, const fp4_quant_opts* out_opts,
                                    uint8_t* out_codes, int64_t ld_out_codes, int64_t out_codes_group_stride,
                                    uint8_t* out_scales, int64_t ld_out_scales, int64_t out_scales_group_stride,
                                    float* out_tensor_scale, void* stream) {
  if (format != FP4_MXFP4 && format != FP4_NVFP4) return FP4_ERR_INVALID;
  if (!out_opts || out_opts->size != sizeof(fp4_quant_opts)) return FP4_ERR_INVALID;
  if (out_opts->format != FP4_MXFP4 && out_opts->format != FP4_NVFP4) return FP4_ERR_INVALID;
  if (out_opts->flags & ~kKnownFlags) return FP4_ERR_INVALID;
  const bool qnv = out_opts->format == FP4_NVFP4;
  if (out_opts->flags & (FP4_BLOCK2D | FP4_TRANSPOSE | FP4_TENSOR_SCALE)) return FP4_ERR_UNSUPPORTED;
  if (!qnv && (out_opts->flags & FP4_SCALE_SEARCH)) return FP4_ERR_UNSUPPORTED;
  if (groups < 0 || M < 0 || N < 0 || K < 0) return FP4_ERR_INVALID;
  const int64_t qblk = qnv ? 16 : 32;
  if (K % 64 != 0 || N % qblk != 0) return FP4_ERR_INVALID;
  if (groups > kMaxGridYZ || (M + 127) / 128 > kMaxGridYZ || (N + 127) / 128 > kMaxGridX) return FP4_ERR_UNSUPPORTED;
  if (groups == 0 || M == 0 || N == 0) return FP4_OK;
  GemmArgs g;
  fp4_status st = plan_gemm_operands(format, groups, M, N, K, a_codes, lda, a_group_stride, a_scales, lda_scales,
                                     a_scales_group_stride, a_tensor_scale, b_codes, ldb, b_group_stride, b_scales,
                                     ldb_scales, b_scales_group_stride, b_tensor_scale, &g);
  if (st != FP4_OK) return st;
  if (!out_codes || !out_scales || ld_out_codes < N / 2 || ld_out_scales < N / qblk) return FP4_ERR_INVALID;
  if (qnv && (!out_tensor_scale || !out_opts->amax_in)) return FP4_ERR_INVALID;
  if (groups > 1 && (out_codes_group_stride < (M - 1) * ld_out_codes + N / 2 ||
                     out_scales_group_stride < (M - 1) * ld_out_scales + N / qblk))
    return FP4_ERR_INVALID;
  if (!aligned(out_codes, 8) || ld_out_codes % 8 != 0 || (groups > 1 && out_codes_group_stride % 8 != 0))
    return FP4_ERR_ALIGN;
  if (qnv && (!aligned(out_tensor_scale, 4) || !aligned(out_opts->amax_in, 4))) return FP4_ERR_ALIGN;
  st = check_device();
  if (st != FP4_OK) return st;
  g.qc = out_codes;
  g.ldqc = ld_out_codes;
  g.qc_gs = groups > 1 ? out_codes_group_stride : 0;
  g.qs = out_scales;
  g.ldqs = ld_out_scales;
  g.qs_gs = groups > 1 ? out_scales_group_stride : 0;
  g.q_ts = out_tensor_scale;
  g.q_amax = out_opts->amax_in;
  g.q_nv = qnv;
  g.q_sel = (out_opts->flags & FP4_SCALE_SEARCH) ? 2 : (out_opts->flags & FP4_FOUR_OVER_SIX) ? 1 : 0;
  g.q_sr = (out_opts->flags & FP4_STOCHASTIC) != 0;
  g.q_rht = (out_opts->flags & FP4_HADAMARD) != 0;
  g.q_signs = out_opts->rht_signs;
  g.q_seed = out_opts->seed;
  g.q_offset = out_opts->offset;
  (void)hipGetLastError();
  return launch_gemm(g, static_cast<hipStream_t>(stream)) == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status fp4_gemm_grouped(int32_t format, int64_t groups, const int32_t* group_offsets, int64_t M, int64_t N,
                            int64_t K, const uint8_t* a_codes, int64_t lda, const uint8_t* a_scales,
                            int64_t lda_scales, const float* a_tensor_scale,
                            const uint8_t* b_codes, int64_t ldb, int64_t b_group_stride,
                            const uint8_t* b_scales, int64_t ldb_scales, int64_t b_scales_group_stride,
                            const float* b_tensor_scale, void* c, int32_t c_dtype, int64_t ldc, void* stream) {
  if (format != FP4_MXFP4 && format != FP4_NVFP4) return FP4_ERR_INVALID;
  if (c_dtype != FP4_F32 && c_dtype != FP4_BF16) return FP4_ERR_INVALID;
  if (groups < 0 || M < 0 || N < 0 || K < 0) return FP4_ERR_INVALID;
  if (K % 64 != 0) return FP4_ERR_INVALID;
  if (groups > kMaxGroupsVar || (N + 127) / 128 > kMaxGridX) return FP4_ERR_UNSUPPORTED;
  if (groups == 0 || M == 0 || N == 0) return FP4_OK;
  const bool nv = format == FP4_NVFP4;
  const int64_t blk = nv ? 16 : 32;
  if (!group_offsets || !a_codes || !a_scales || !b_codes || !b_scales || !c) return FP4_ERR_INVALID;
  if (nv && (!a_tensor_scale || !b_tensor_scale)) return FP4_ERR_INVALID;
  if (lda < K / 2 || ldb < K / 2 || lda_scales < K / blk || ldb_scales < K / blk || ldc < N) return FP4_ERR_INVALID;
  if (groups > 1 && (b_group_stride < 0 || b_scales_group_stride < 0)) return FP4_ERR_INVALID;
  if (!aligned(group_offsets, 4)) return FP4_ERR_ALIGN;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || lda % 16 != 0 || ldb % 16 != 0) return FP4_ERR_ALIGN;
  if (M * lda >= (int64_t(1) << 31) || N * ldb >= (int64_t(1) << 31) || M * lda_scales >= (int64_t(1) << 31) ||
      N * ldb_scales >= (int64_t(1) << 31))
    return FP4_ERR_UNSUPPORTED;
  if (lda >= (int64_t(1) << 23) || ldb >= (int64_t(1) << 23) || lda_scales >= (int64_t(1) << 23) ||
      ldb_scales >= (int64_t(1) << 23))
    return FP4_ERR_UNSUPPORTED;
  if (groups > 1 && b_group_stride % 16 != 0) return FP4_ERR_ALIGN;
  if (!aligned(c, c_dtype == FP4_BF16 ? 2 : 4)) return FP4_ERR_ALIGN;
  if (!aligned(a_scales, 16) || !aligned(b_scales, 16) || lda_scales % 16 != 0 || ldb_scales % 16 != 0 ||
      (groups > 1 && b_scales_group_stride % 16 != 0))
    return FP4_ERR_ALIGN;
  if (nv && (!aligned(a_tensor_scale, 4) || !aligned(b_tensor_scale, 4))) return FP4_ERR_ALIGN;
  fp4_status st = check_device();
  if (st != FP4_OK) return st;
  GemmArgs g{};
  g.nvfp4 = nv;
  g.groups = groups;
  g.M = M;
  g.N = N;
  g.K = K;
  g.a = a_codes;
  g.lda = lda;
  g.a_gs = 0;
  g.as = a_scales;
  g.lda_s = lda_scales;
  g.as_gs = 0;
  g.a_ts = a_tensor_scale;
  g.a_ts_gs = 0;
  g.b = b_codes;
  g.ldb = ldb;
  g.b_gs = groups > 1 ? b_group_stride : 0;
  g.bs = b_scales;
  g.ldb_s = ldb_scales;
  g.bs_gs = groups > 1 ? b_scales_group_stride : 0;
  g.b_ts = b_tensor_scale;
  g.c = c;
  g.c_bf16 = c_dtype == FP4_BF16;
  g.ldc = ldc;
  g.c_gs = 0;
  g.c_vec_ok = aligned(c, 16) && (ldc * (c_dtype == FP4_BF16 ? 2 : 4)) % 16 == 0;
  g.offs = group_offsets;
  (void)hipGetLastError();
  return launch_gemm(g, static_cast<hipStream_t>(stream)) == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

}  // extern "C"
