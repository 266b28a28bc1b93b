// launch.h -- internal launch interface between the C ABI (fp4_api.cpp) and
// the HIP kernels. Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4impl {

enum Flags : uint32_t {
  kFourOverSix = 1u,
  kBlock2D = 2u,
  kTranspose = 4u,
  kStochastic = 8u,
  kHadamard = 16u,
  kScaleSearch = 32u,
  kTensorScale = 64u,
};

struct QuantArgs {
  const void* x;
  bool x_bf16;
  int64_t batch, src_rows, src_cols;  // source matrix per batch item
  int64_t ld_x, bs_x;                 // elements
  int64_t R, C;                       // output matrix (C is the block direction)
  bool nvfp4;
  uint32_t flags;
  uint32_t signs;
  uint64_t seed, offset;
  const float* amax_in;   // [batch] or null
  uint8_t* codes;
  int64_t ld_c, bs_c;
  uint8_t* scales;
  int64_t ld_s, bs_s;
  float* tensor_scale;    // [batch] (NVFP4)
  float* partials;        // workspace [batch][nparts] (NVFP4 without amax_in)
  int nparts;
};

// Number of per-workgroup partial maxima the NVFP4 amax pre-pass writes for
// one batch item (also fixes its grid).
int amax_partials(int64_t src_rows, int64_t src_cols, uint32_t flags);

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);

// Bytes of the library's own scratch array (one copy per GPU) that
// fp4_quantize_noalloc puts the NVFP4 amax partials in.
constexpr size_t kNoAllocScratchBytes = 262144;

// The current device's address of that array, looked up on the first call
// per device and cached; hipSuccess or the runtime's error.
hipError_t noalloc_scratch(float** ptr);

struct DequantArgs {
  bool nvfp4;
  int64_t batch, rows, cols;
  const uint8_t* codes;
  int64_t ld_c, bs_c;
  const uint8_t* scales;
  int64_t ld_s, bs_s;
  const float* tensor_scale;
  void* y;
  bool y_bf16;
  int64_t ld_y, bs_y;
};

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t stream);

struct GemmArgs {
  bool nvfp4;
  int64_t groups, M, N, K;
  const uint8_t* a;
  int64_t lda, a_gs;
  const uint8_t* as;
  int64_t lda_s, as_gs;
  const float* a_ts;
  int64_t a_ts_gs;  // a_ts step per group: 1, or 0 when one scale covers all of A
  const uint8_t* b;
  int64_t ldb, b_gs;
  const uint8_t* bs;
  int64_t ldb_s, bs_gs;
  const float* b_ts;
  void* c;
  bool c_bf16;
  int64_t ldc, c_gs;
  bool c_vec_ok;  // C and its row / group pitches are 16-byte aligned
  // NULL: `groups` equal groups of M rows at the group strides. Else device
  // int32[groups + 1]: group g is rows [offs[g], offs[g + 1]) of one A and
  // one C of M rows (group strides of A and C zero).
  const int32_t* offs;
  // Quantized output instead of C (qc non-NULL; equal groups only): C_g
  // quantized along its rows into codes qc [M, N/2] and scales qs
  // [M, N/blk] per group; NVFP4 (q_nv) takes S_t from q_amax[g] and writes
  // it to q_ts[g].
  uint8_t* qc;
  int64_t ldqc, qc_gs;
  uint8_t* qs;
  int64_t ldqs, qs_gs;
  float* q_ts;
  const float* q_amax;
  bool q_nv, q_sr, q_rht;
  int q_sel;  // scale selection: 0 plain, 1 4/6, 2 search (NVFP4)
  uint32_t q_signs;
  uint64_t q_seed, q_offset;
};

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace fp4impl
