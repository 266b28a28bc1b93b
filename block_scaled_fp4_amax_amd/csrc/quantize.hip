// quantize.hip -- block-scaled FP4 quantization kernels for gfx950.
//
//   amax_kernel        NVFP4 tensor-amax pre-pass (after the Hadamard
//                      transform when on): per-workgroup partial maxima.
//   quant_rows_kernel  blocks along contiguous rows. One lane owns one
//                      16-value slice (two 16-byte loads of bf16): an NVFP4
//                      block, half an MXFP4 block (lane pair), or one row of a
//                      16x16 tile (16 lanes).
//   quant_cols_kernel  transposed input: blocks run down the columns of X.
//                      One lane owns a 16-row x 4-column patch (sixteen
//                      8-byte row loads of bf16), or 16 x 8 for 16x16
//                      tiles: one block per source column; an MXFP4 block
//                      is a vertical lane pair, a 16x16 tile a horizontal
//                      one. Output goes through LDS so each output row is
//                      written as whole lines.
//
// The method is stated in quant_common.h.
#include <mutex>

#include "quant_common.h"

namespace fp4impl {

// ------------------------------------------------------------------------
// Scratch of fp4_quantize_noalloc: the NVFP4 amax partials of a call, in an
// array every GPU holds a copy of until the process ends, so the call needs
// no workspace and allocates nothing. In host code `scratch` names a host
// stand-in, not device memory: kernels get the device address that
// hipGetSymbolAddress reports for the current device, never the name.
// ------------------------------------------------------------------------
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(float** ptr) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static float* per_dev[kMaxDev] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (dev < kMaxDev && per_dev[dev]) {
    *ptr = per_dev[dev];
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  if (dev < kMaxDev) per_dev[dev] = static_cast<float*>(p);
  *ptr = static_cast<float*>(p);
  return hipSuccess;
}

// ------------------------------------------------------------------------
// amax pre-pass
// ------------------------------------------------------------------------
enum AmaxMode { kAmaxPlain = 0, kAmaxRhtRows = 1, kAmaxRhtCols = 2 };

int amax_partials(int64_t src_rows, int64_t src_cols, uint32_t flags) {
  int64_t units;
  if (!(flags & kHadamard)) units = src_rows * (src_cols / 8);
  else if (flags & kTranspose) units = (src_rows / 16) * (src_cols / 8);
  else units = src_rows * (src_cols / 16);
  int64_t p = (units + 4 * 256 - 1) / (4 * 256);
  if (p < 1) p = 1;
  if (p > 1024) p = 1024;
  return (int)p;
}

// Position (r, c) of a unit in a grid of per_row units per row, advanced by
// a fixed number of units with an add and a compare instead of a division.
struct UnitPos {
  int64_t r, c;
  __device__ __forceinline__ void init(int64_t u, int64_t per_row) {
    r = u / per_row;
    c = u - r * per_row;
  }
  __device__ __forceinline__ void advance(int64_t dq, int64_t dr, int64_t per_row) {
    r += dq;
    c += dr;
    if (c >= per_row) {
      c -= per_row;
      r++;
    }
  }
};

// Grid-stride over the units of one batch item, NU units per lane per step
// (units u, u + stride, ..., u + (NU - 1) stride), so that every lane has
// NU units' loads in flight before it reduces any of them.
template <typename TIn, int MODE>
__global__ __launch_bounds__(256) void amax_kernel(QuantArgs a) {
  const int64_t b = blockIdx.y;
  const TIn* x = reinterpret_cast<const TIn*>(a.x) + b * a.bs_x;
  const int64_t rows = a.src_rows, cols = a.src_cols;
  // plain: 8 values of a row; RHT rows: one 16-value slice of a row; RHT
  // columns: 16 rows x 8 columns (eight slices down the columns)
  const int64_t per_row = MODE == kAmaxRhtRows ? cols / 16 : cols / 8;
  const int64_t unit_rows = MODE == kAmaxRhtCols ? rows / 16 : rows;
  // (for bf16, 4 units per lane measured faster than 8 and much faster than 16)
  constexpr int NU = MODE == kAmaxRhtCols ? 1 : 4;
  const int64_t stride = (int64_t)gridDim.x * 256;
  UnitPos pos[NU];
  pos[0].init((int64_t)blockIdx.x * 256 + threadIdx.x, per_row);
  const int64_t sq = stride / per_row, sr = stride - sq * per_row;
#pragma unroll
  for (int k = 1; k < NU; k++) {
    pos[k] = pos[k - 1];
    pos[k].advance(sq, sr, per_row);
  }
  const int64_t step = (int64_t)NU * stride;
  const int64_t dq = step / per_row, dr = step - dq * per_row;
  float m = 0.0f;
  // units run in order, so every unit of a step lies past pos[0]
  while (pos[0].r < unit_rows) {
    if constexpr (MODE == kAmaxPlain) {
      float v[NU][8];
#pragma unroll
      for (int k = 0; k < NU; k++) {
        if (pos[k].r < unit_rows) {
          load8<TIn>(x + pos[k].r * a.ld_x + pos[k].c * 8, v[k]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; i++) v[k][i] = 0.0f;
        }
      }
#pragma unroll
      for (int k = 0; k < NU; k++)
#pragma unroll
        for (int i = 0; i < 8; i++) m = __builtin_fmaxf(m, __builtin_fabsf(v[k][i]));
    } else if constexpr (MODE == kAmaxRhtRows) {
      float v[NU][16];
#pragma unroll
      for (int k = 0; k < NU; k++) {
        if (pos[k].r < unit_rows) {
          load8<TIn>(x + pos[k].r * a.ld_x + pos[k].c * 16, v[k]);
          load8<TIn>(x + pos[k].r * a.ld_x + pos[k].c * 16 + 8, v[k] + 8);
        } else {
#pragma unroll
          for (int i = 0; i < 16; i++) v[k][i] = 0.0f;
        }
      }
#pragma unroll
      for (int k = 0; k < NU; k++) {
        rht16(v[k], a.signs);
        m = __builtin_fmaxf(m, max_abs16(v[k]));
      }
    } else {
      float t[16][8];
#pragma unroll
      for (int i = 0; i < 16; i++) load8<TIn>(x + (pos[0].r * 16 + i) * a.ld_x + pos[0].c * 8, t[i]);
#pragma unroll
      for (int j = 0; j < 8; j++) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = t[i][j];
        rht16(v, a.signs);
        m = __builtin_fmaxf(m, max_abs16(v));
      }
    }
#pragma unroll
    for (int k = 0; k < NU; k++) pos[k].advance(dq, dr, per_row);
  }
  m = __builtin_fmaxf(m, xor_shfl<32>(m));
  m = __builtin_fmaxf(m, xor_shfl<16>(m));
  m = __builtin_fmaxf(m, xor_shfl<8>(m));
  m = __builtin_fmaxf(m, xor_shfl<4>(m));
  m = __builtin_fmaxf(m, xor_shfl<2>(m));
  m = __builtin_fmaxf(m, xor_shfl<1>(m));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    a.partials[b * a.nparts + blockIdx.x] =
        __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
}

// Folds batch item b's nparts partial maxima into T, written after all the
// items' partials (workspace word batch * nparts + b), so that the quantizer
// reads one word instead of every workgroup folding the partials again.
constexpr int64_t kFoldOnceElems = int64_t(1) << 25;
__global__ __launch_bounds__(256) void amax_finalize_kernel(QuantArgs a) {
  const int64_t b = blockIdx.x;
  const float* p = a.partials + b * a.nparts;
  float m = 0.0f;
  if ((a.nparts & 3) == 0) {
    // 16-byte loads (the workspace is 16-byte aligned): up to 1024 partials
    // in one load per lane instead of a chain of dependent ones
    for (int i = 4 * threadIdx.x; i < a.nparts; i += 4 * 256) {
      const float4 q = *reinterpret_cast<const float4*>(p + i);
      m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(q.x, q.y), __builtin_fmaxf(q.z, q.w)));
    }
  } else {
    for (int i = threadIdx.x; i < a.nparts; i += 256) m = __builtin_fmaxf(m, p[i]);
  }
  m = __builtin_fmaxf(m, xor_shfl<32>(m));
  m = __builtin_fmaxf(m, xor_shfl<16>(m));
  m = __builtin_fmaxf(m, xor_shfl<8>(m));
  m = __builtin_fmaxf(m, xor_shfl<4>(m));
  m = __builtin_fmaxf(m, xor_shfl<2>(m));
  m = __builtin_fmaxf(m, xor_shfl<1>(m));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    a.partials[a.batch * a.nparts + b] =
        __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
}

// ------------------------------------------------------------------------
// Row-major quantization
// ------------------------------------------------------------------------
// 16 consecutive input values as loaded (two 16-byte loads of bf16, four of
// fp32), so that the loads can be in flight during the tensor-scale prologue.
template <typename TIn>
struct Raw16;
template <>
struct Raw16<uint16_t> {
  uint4 w0, w1;
  __device__ __forceinline__ void load(const uint16_t* p) {
    w0 = reinterpret_cast<const uint4*>(p)[0];
    w1 = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ __forceinline__ void unpack(float (&v)[16]) const {
    const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
  }
};
template <>
struct Raw16<float> {
  float4 f[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; i++) f[i] = reinterpret_cast<const float4*>(p)[i];
  }
  __device__ __forceinline__ void unpack(float (&v)[16]) const {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[4 * i] = f[i].x;
      v[4 * i + 1] = f[i].y;
      v[4 * i + 2] = f[i].z;
      v[4 * i + 3] = f[i].w;
    }
  }
};

template <typename TIn, bool NV, int SEL, bool B2D, bool SR, bool RHT>
__global__ __launch_bounds__(256) void quant_rows_kernel(QuantArgs a) {
  const int64_t b = blockIdx.z;
  const int64_t upr = a.C >> 4;  // 16-value units per row
  int64_t row, cu;
  if constexpr (B2D) {
    row = (int64_t)blockIdx.y * 16 + (threadIdx.x & 15);
    cu = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  } else {
    int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    row = u / upr;
    cu = u - row * upr;
  }
  // validity is uniform across every group of lanes that exchanges data
  const bool valid = row < a.R && cu < upr;
  Raw16<TIn> raw;
  if (valid) raw.load(reinterpret_cast<const TIn*>(a.x) + b * a.bs_x + row * a.ld_x + cu * 16);

  NvConsts nc{};
  if constexpr (NV) nc = nv_prologue<SEL>(a, b, blockIdx.x == 0 && blockIdx.y == 0);  // every lane takes part
  if (!valid) return;

  float v[16];
  raw.unpack(v);
  if constexpr (RHT) rht16(v, a.signs);

  uint32_t w0, w1, sbyte;
  const uint64_t L0 = ((uint64_t)b * (uint64_t)a.R + (uint64_t)row) * (uint64_t)a.C + (uint64_t)cu * 16;
  quantize_unit<NV, SEL, B2D, SR>(v, nc, L0, a.seed, a.offset, w0, w1, sbyte);

  uint8_t* cp = a.codes + b * a.bs_c + row * a.ld_c + cu * 8;
  *reinterpret_cast<uint2*>(cp) = make_uint2(w0, w1);
  if constexpr (NV) {
    a.scales[b * a.bs_s + row * a.ld_s + cu] = (uint8_t)sbyte;
  } else {
    if ((cu & 1) == 0) a.scales[b * a.bs_s + row * a.ld_s + (cu >> 1)] = (uint8_t)sbyte;
  }
}

// ------------------------------------------------------------------------
// Transposed quantization (output = Q(X^T))
// ------------------------------------------------------------------------
// A workgroup takes 256 source rows (k) x 16 PW source columns (n). Lane
// (wave w, g = lane / 2, h = lane % 2) owns the 16 x PW patch at
// k = 64 w + 32 (g / 16) + 16 h, n = PW (g % 16): sixteen row loads of PW
// values. Its PW 16-value blocks (one per source column) land in an LDS
// image of the workgroup's output, 16 PW rows of 128 code bytes plus their
// scale bytes, which the workgroup then stores with consecutive lanes along
// each output row, so every output row gets one whole 128-byte line per
// workgroup. PW = 8 for 16 x 16 tiles, whose tile error adds a lane's 8
// columns to its horizontal partner's; else PW = 4, which halves the
// registers a lane holds its patch in and doubles the workgroups.
constexpr int kColsK = 256;
constexpr int kColsPitch = kColsK / 2 + 8;  // staged code row, padded (bytes)
constexpr int kColsScales = kColsK / 16;    // staged scale bytes per row (NVFP4; MXFP4 uses half)
constexpr int cols_pw(bool b2d) { return b2d ? 8 : 4; }
constexpr int cols_n(int pw) { return 16 * pw; }  // source columns per workgroup

// The patch rows are read once and the staged code lines written once, so
// both go through the caches non-temporally: the streamed input then does
// not displace the lines that the workgroups of one XCD are still filling.
__device__ __forceinline__ float4 nt_load_f4(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
template <typename TIn, int PW>
struct Patch16;
template <>
struct Patch16<uint16_t, 8> {
  uint4 r[16];
  __device__ __forceinline__ void load(const uint16_t* p, int64_t ld) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + i * ld));
      r[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  }
  // Hides the loaded words from the compiler's view, so that a pass over
  // the patch converts them anew instead of keeping an earlier pass's fp32
  // values live (128 registers) across the passes.
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      u32x4 v = {r[i].x, r[i].y, r[i].z, r[i].w};
      asm volatile("" : "+v"(v));
      r[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  }
  __device__ __forceinline__ float get(int i, int j) const {
    const uint32_t w = (j >> 1) == 0 ? r[i].x : (j >> 1) == 1 ? r[i].y : (j >> 1) == 2 ? r[i].z : r[i].w;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <>
struct Patch16<uint16_t, 4> {
  uint2 r[16];
  __device__ __forceinline__ void load(const uint16_t* p, int64_t ld) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p + i * ld));
      r[i] = make_uint2(v.x, v.y);
    }
  }
  __device__ __forceinline__ float get(int i, int j) const {
    const uint32_t w = (j >> 1) == 0 ? r[i].x : r[i].y;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <>
struct Patch16<float, 8> {
  float4 r[16][2];
  __device__ __forceinline__ void load(const float* p, int64_t ld) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      r[i][0] = nt_load_f4(p + i * ld);
      r[i][1] = nt_load_f4(p + i * ld + 4);
    }
  }
  __device__ __forceinline__ float get(int i, int j) const {
    const float4& f = r[i][j >> 2];
    return (j & 3) == 0 ? f.x : (j & 3) == 1 ? f.y : (j & 3) == 2 ? f.z : f.w;
  }
  __device__ __forceinline__ void opaque() {}  // fp32 values are used as loaded
};
template <>
struct Patch16<float, 4> {
  float4 r[16];
  __device__ __forceinline__ void load(const float* p, int64_t ld) {
#pragma unroll
    for (int i = 0; i < 16; i++) r[i] = nt_load_f4(p + i * ld);
  }
  __device__ __forceinline__ float get(int i, int j) const {
    const float4& f = r[i];
    return (j & 3) == 0 ? f.x : (j & 3) == 1 ? f.y : (j & 3) == 2 ? f.z : f.w;
  }
};

template <typename TIn, bool NV, int SEL, bool B2D, bool SR, bool RHT>
__global__ __launch_bounds__(256) void quant_cols_kernel(QuantArgs a) {
  constexpr int PW = cols_pw(B2D), kColsN = cols_n(PW);
  __shared__ __attribute__((aligned(16))) uint8_t cst[kColsN * kColsPitch];
  __shared__ __attribute__((aligned(16))) uint8_t sst[kColsN * kColsScales];
  // Workgroup order: a column strip (batch item, kColsN source columns) is
  // walked down K by consecutive workgroups of one XCD (workgroup ids go
  // round-robin to the 8 XCDs, each with its own L2). An output row's 128-byte
  // segments straddle cache lines whenever its pitch is not a multiple of 128;
  // the two halves of such a line then come from neighbouring K blocks in the
  // same L2, which merges them before they reach HBM.
  const int64_t ncb = (a.src_cols + kColsN - 1) / kColsN, nkb = (a.src_rows + kColsK - 1) / kColsK;
  const int64_t wid = blockIdx.x, i_x = wid >> 3;
  const int64_t strip = (i_x / nkb) * 8 + (wid & 7);
  if (strip >= a.batch * ncb) return;
  const int64_t b = strip / ncb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane & 1, g = lane >> 1;
  const int nl = (g & 15) * PW;                        // patch columns, workgroup-relative
  const int kl = wave * 64 + (g >> 4) * 32 + h * 16;   // patch rows, workgroup-relative
  const int64_t nb = (strip - b * ncb) * kColsN, kb = (i_x % nkb) * kColsK;
  const int64_t n0 = nb + nl, k0 = kb + kl;
  // A vertical lane pair (an MXFP4 block) and a horizontal one (a 16 x 16
  // tile) are valid together: rows come in whole blocks, columns in whole
  // tiles.
  const bool valid = n0 < a.src_cols && k0 < a.src_rows;
  Patch16<TIn, PW> t;
  if (valid) t.load(reinterpret_cast<const TIn*>(a.x) + b * a.bs_x + k0 * a.ld_x + n0, a.ld_x);
  NvConsts nc{};
  if constexpr (NV) nc = nv_prologue<SEL>(a, b, nb == 0 && kb == 0);  // while the loads are in flight
  if (valid) {
    const uint64_t Lrow = (uint64_t)b * (uint64_t)a.R;
    uint8_t* crow = cst + nl * kColsPitch + (kl >> 1);
    uint8_t* srow = sst + nl * kColsScales;

    if constexpr (NV && B2D) {
      // one 16x16 tile per horizontal lane pair (lanes g and g^1)
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; i++)
#pragma unroll
        for (int j = 0; j < PW; j++) amax = __builtin_fmaxf(amax, __builtin_fabsf(t.get(i, j)));
      amax = __builtin_fmaxf(amax, xor_shfl<2>(amax));
      NvCand c = nv_candidate(amax, nc.k6, nc);
      // a candidate's error sum: per source row, the FMA chain over this
      // lane's 8 columns plus the partner's over the other 8, then a
      // pairwise tree over the 16 source rows
      // (the tree is formed as the row sums arrive: level[d] holds the
      // pending left operand of depth d, so few sums are live at once)
      auto tile_sum = [&](const NvCand& cc) {
        float level[4];
#pragma unroll
        for (int i = 0; i < 16; i++) {
          float qq[8];
#pragma unroll
          for (int j = 0; j < PW; j++) qq[j] = t.get(i, j) * cc.r;
          uint32_t ww = e2m1_pack2<0>(0u, qq[0], qq[1]);
          ww = e2m1_pack2<1>(ww, qq[2], qq[3]);
          ww = e2m1_pack2<2>(ww, qq[4], qq[5]);
          ww = e2m1_pack2<3>(ww, qq[6], qq[7]);
          float x = sq_chain8(qq, ww);
          x = x + xor_shfl<2>(x);
          // While bit d of i is set, x completes the right half of a subtree
          // whose left half's sum waits in level[d]: add it on the left and
          // go up a level. At the first clear bit, x waits there itself. At
          // i = 15 every bit is set and x is the whole tile's sum.
#pragma unroll
          for (int d = 0; d < 4; d++) {
            if (!((i >> d) & 1)) {
              level[d] = x;
              break;
            }
            x = level[d] + x;
          }
          if (i == 15) level[0] = x;
        }
        return level[0];
      };
      if constexpr (SEL == 1) {
        NvCand c4 = nv_candidate(amax, nc.k4, nc);
        t.opaque();
        const float s6 = tile_sum(c);
        t.opaque();
        const float s4 = tile_sum(c4);
        if (cand_error(c4, s4) < cand_error(c, s6)) c = c4;
      } else if constexpr (SEL == 2) {
        // the lane pair shares amax, hence the loop bounds
        t.opaque();
        float best = cand_error(c, tile_sum(c));
        const uint32_t hi = nv_candidate(amax, nc.k4, nc).code;
        for (uint32_t code = c.code + 1; code <= hi; code++) {
          const NvCand cc = nv_code_candidate(code, nc);
          t.opaque();
          const float err = cand_error(cc, tile_sum(cc));
          if (err < best) {
            best = err;
            c = cc;
          }
        }
      }
      t.opaque();
#pragma unroll
      for (int j = 0; j < PW; j++) {
        float q[16];
#pragma unroll
        for (int i = 0; i < 16; i++) q[i] = t.get(i, j) * c.r;
        uint32_t w0, w1;
        if constexpr (SR)
          sr16(q, (Lrow + (uint64_t)(n0 + j)) * (uint64_t)a.C + (uint64_t)k0, a.seed, a.offset, w0, w1);
        else
          pack16(q, w0, w1);
        *reinterpret_cast<uint2*>(crow + j * kColsPitch) = make_uint2(w0, w1);
        srow[j * kColsScales + (kl >> 4)] = (uint8_t)c.code;
      }
    } else {
#pragma unroll
      for (int j = 0; j < PW; j++) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; i++) v[i] = t.get(i, j);
        if constexpr (RHT) rht16(v, a.signs);
        const uint64_t L0 = (Lrow + (uint64_t)(n0 + j)) * (uint64_t)a.C + (uint64_t)k0;
        uint32_t w0, w1, sbyte;
        // an MXFP4 block is the vertical lane pair (lanes xor 1, 32 rows)
        quantize_unit<NV, SEL, false, SR>(v, nc, L0, a.seed, a.offset, w0, w1, sbyte);
        if constexpr (NV) srow[j * kColsScales + (kl >> 4)] = (uint8_t)sbyte;
        else if (h == 0) srow[j * kColsScales + (kl >> 5)] = (uint8_t)sbyte;
        *reinterpret_cast<uint2*>(crow + j * kColsPitch) = make_uint2(w0, w1);
      }
    }
  }
  __syncthreads();

  // Store the staged image: 8-byte chunks, 16 lanes per 128-byte output row.
  const int nrows = (int)(a.src_cols - nb < kColsN ? a.src_cols - nb : kColsN);
  const int kbytes = (int)(a.src_rows - kb < kColsK ? a.src_rows - kb : kColsK) / 2;
  uint8_t* cout = a.codes + b * a.bs_c + nb * a.ld_c + (kb >> 1);
#pragma unroll
  for (int i = 0; i < (kColsN * kColsK / 2) / (8 * 256); i++) {
    const int c = threadIdx.x + 256 * i, r = c >> 4, cb = (c & 15) * 8;
    if (r < nrows && cb < kbytes)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x2*>(cst + r * kColsPitch + cb),
                                  reinterpret_cast<u32x2*>(cout + r * a.ld_c + cb));
  }
  constexpr int kSPer = NV ? kColsScales : kColsScales / 2;  // scale bytes per row per workgroup
  const int svalid = NV ? kbytes / 8 : kbytes / 16;
  uint8_t* sout = a.scales + b * a.bs_s + nb * a.ld_s + kb / (NV ? 16 : 32);
#pragma unroll
  for (int i = 0; i < kColsN * kSPer / 256; i++) {
    const int c = threadIdx.x + 256 * i, r = c / kSPer, sc = c % kSPer;
    if (r < nrows && sc < svalid) sout[r * a.ld_s + sc] = sst[r * kColsScales + sc];
  }
}

// ------------------------------------------------------------------------
// dispatch
// ------------------------------------------------------------------------
template <typename TIn, bool NV, int SEL, bool B2D, bool SR, bool RHT>
static void launch_one(const QuantArgs& a, hipStream_t s) {
  if (a.flags & kTranspose) {
    if constexpr (B2D && RHT) {
      return;  // rejected by the API
    } else {
      // 8 XCD lanes of ceil(strips / 8) column strips, each strip nkb workgroups
      constexpr int kColsN = cols_n(cols_pw(B2D));
      const int64_t strips = a.batch * ((a.src_cols + kColsN - 1) / kColsN);
      const int64_t nkb = (a.src_rows + kColsK - 1) / kColsK;
      dim3 grid((unsigned)(8 * ((strips + 7) / 8) * nkb));
      hipLaunchKernelGGL((quant_cols_kernel<TIn, NV, SEL, B2D, SR, RHT>), grid, dim3(256), 0, s, a);
    }
  } else if (B2D) {
    dim3 grid((unsigned)(((a.C >> 4) + 15) / 16), (unsigned)(a.R / 16), (unsigned)a.batch);
    hipLaunchKernelGGL((quant_rows_kernel<TIn, NV, SEL, B2D, SR, RHT>), grid, dim3(256), 0, s, a);
  } else {
    int64_t units = a.R * (a.C >> 4);
    dim3 grid((unsigned)((units + 255) / 256), 1, (unsigned)a.batch);
    hipLaunchKernelGGL((quant_rows_kernel<TIn, NV, SEL, B2D, SR, RHT>), grid, dim3(256), 0, s, a);
  }
}

template <typename TIn, bool NV, int SEL, bool B2D>
static void launch_sr_rht(const QuantArgs& a, hipStream_t s) {
  const bool sr = a.flags & kStochastic, rht = a.flags & kHadamard;
  if (sr) {
    if (rht) launch_one<TIn, NV, SEL, B2D, true, true>(a, s);
    else launch_one<TIn, NV, SEL, B2D, true, false>(a, s);
  } else {
    if (rht) launch_one<TIn, NV, SEL, B2D, false, true>(a, s);
    else launch_one<TIn, NV, SEL, B2D, false, false>(a, s);
  }
}

template <typename TIn, int SEL>
static void launch_nv_sel(const QuantArgs& a, hipStream_t s) {
  if (a.flags & kBlock2D) launch_sr_rht<TIn, true, SEL, true>(a, s);
  else launch_sr_rht<TIn, true, SEL, false>(a, s);
}

template <typename TIn>
static void launch_typed(const QuantArgs& a, hipStream_t s) {
  if (!a.nvfp4) {
    if (a.flags & kFourOverSix) launch_sr_rht<TIn, false, 1, false>(a, s);
    else launch_sr_rht<TIn, false, 0, false>(a, s);
    return;
  }
  if (!a.amax_in) {
    int mode = !(a.flags & kHadamard) ? kAmaxPlain : ((a.flags & kTranspose) ? kAmaxRhtCols : kAmaxRhtRows);
    dim3 grid((unsigned)a.nparts, (unsigned)a.batch);
    if (mode == kAmaxPlain) hipLaunchKernelGGL((amax_kernel<TIn, kAmaxPlain>), grid, dim3(256), 0, s, a);
    else if (mode == kAmaxRhtRows) hipLaunchKernelGGL((amax_kernel<TIn, kAmaxRhtRows>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((amax_kernel<TIn, kAmaxRhtCols>), grid, dim3(256), 0, s, a);
  }
  QuantArgs q = a;
  // Large items: fold the partials once (one more small launch) rather than
  // in every one of the quantizer's many workgroups; small ones keep the
  // fold in the quantizer's prologue, where it costs less than a launch.
  if (!a.amax_in && a.src_rows * a.src_cols >= kFoldOnceElems) {
    hipLaunchKernelGGL(amax_finalize_kernel, dim3((unsigned)a.batch), dim3(256), 0, s, a);
    q.amax_in = q.partials + q.batch * q.nparts;
  }
  if (q.flags & kTensorScale) launch_sr_rht<TIn, true, 3, false>(q, s);  // one scale: no 2D
  else if (q.flags & kScaleSearch) launch_nv_sel<TIn, 2>(q, s);
  else if (q.flags & kFourOverSix) launch_nv_sel<TIn, 1>(q, s);
  else launch_nv_sel<TIn, 0>(q, s);
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  if (a.x_bf16) launch_typed<uint16_t>(a, s);
  else launch_typed<float>(a, s);
  return hipGetLastError();
}

}  // namespace fp4impl
