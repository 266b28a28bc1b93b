// gemm.hip -- W4A4 block-scaled GEMM C_g = deq(A_g) * deq(B_g)^T for gfx950
// (Ultralytics glossary "FP4", section "Inferencia e Treinamento FP4": matrix
// products in FP4, accumulated at higher precision).
//
//   MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands; each lane
//          feeds 32 consecutive K values of one row (16 bytes) and that run's
//          E8M0 byte as its scale operand, so the block scales are applied by
//          the matrix core itself.
//   NVFP4: the MFMA scale operand is a power of two per 32 values, which
//          cannot carry an E4M3 scale per 16, so each lane dequantizes its
//          codes exactly to bf16 (val * E4M3 has at most 6 significant bits
//          and lies in [2^-10, 2688]) and feeds v_mfma_f32_32x32x16_bf16; the
//          two tensor scales multiply the fp32 accumulator in the epilogue.
//          A lane loads 32 consecutive K values (16 bytes) and spends them on
//          four K=16 MFMAs: the K order inside the product is permuted the
//          same way for A and B, which leaves the sum unchanged.
//
// Tiling: 256 threads = 4 waves in a 2x2 grid; each wave owns 64x64 of C as
// 2x2 MFMA tiles of 32x32; a workgroup owns 128x128; grid (N/128, M/128,
// groups). Accumulator layout of a 32x32 MFMA: lane l, register q holds
// C[(q/4)*8 + (l/32)*4 + q%4][l%32].
#include "fp4_device.h"
#include "launch.h"

namespace fp4impl {
using namespace fp4dev;

__device__ __forceinline__ bf16x8 deq8_bf16(uint32_t w, float dec) {
  f32x2 p0 = e2m1_unpack2<0>(w), p1 = e2m1_unpack2<1>(w), p2 = e2m1_unpack2<2>(w), p3 = e2m1_unpack2<3>(w);
  bf16x8 o = {(__bf16)(p0.x * dec), (__bf16)(p0.y * dec), (__bf16)(p1.x * dec), (__bf16)(p1.y * dec),
              (__bf16)(p2.x * dec), (__bf16)(p2.y * dec), (__bf16)(p3.x * dec), (__bf16)(p3.y * dec)};
  return o;
}

template <bool NV, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  const int64_t grp = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r = lane & 31, hh = lane >> 5;
  const int64_t m_base = (int64_t)blockIdx.y * 128 + wm * 64;
  const int64_t n_base = (int64_t)blockIdx.x * 128 + wn * 64;
  const uint8_t* A = g.a + grp * g.a_gs;
  const uint8_t* As = g.as + grp * g.as_gs;
  const uint8_t* B = g.b + grp * g.b_gs;
  const uint8_t* Bs = g.bs + grp * g.bs_gs;

  int64_t arow[2] = {m_base + r, m_base + 32 + r};
  int64_t brow[2] = {n_base + r, n_base + 32 + r};
  bool aval[2] = {arow[0] < g.M, arow[1] < g.M};
  bool bval[2] = {brow[0] < g.N, brow[1] < g.N};

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int q = 0; q < 16; q++) acc[i][j][q] = 0.0f;

  for (int64_t k = 0; k < g.K; k += 64) {
    uint4 aw[2], bw[2];
    uint32_t as_[2], bs_[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      aw[i] = aval[i] ? *reinterpret_cast<const uint4*>(A + arow[i] * g.lda + (k >> 1) + hh * 16) : make_uint4(0, 0, 0, 0);
      bw[i] = bval[i] ? *reinterpret_cast<const uint4*>(B + brow[i] * g.ldb + (k >> 1) + hh * 16) : make_uint4(0, 0, 0, 0);
      if constexpr (NV) {
        const uint8_t* pa = As + arow[i] * g.lda_s + (k >> 4) + hh * 2;
        const uint8_t* pb = Bs + brow[i] * g.ldb_s + (k >> 4) + hh * 2;
        as_[i] = aval[i] ? (uint32_t)pa[0] | ((uint32_t)pa[1] << 8) : 0u;
        bs_[i] = bval[i] ? (uint32_t)pb[0] | ((uint32_t)pb[1] << 8) : 0u;
      } else {
        as_[i] = aval[i] ? (uint32_t)As[arow[i] * g.lda_s + (k >> 5) + hh] : 127u;
        bs_[i] = bval[i] ? (uint32_t)Bs[brow[i] * g.ldb_s + (k >> 5) + hh] : 127u;
      }
    }
    if constexpr (!NV) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        i32x8 af = {(int)aw[i].x, (int)aw[i].y, (int)aw[i].z, (int)aw[i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 2; j++) {
          i32x8 bf = {(int)bw[j].x, (int)bw[j].y, (int)bw[j].z, (int)bw[j].w, 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bf, acc[i][j], 4, 4, 0, (int)as_[i], 0,
                                                                      (int)bs_[j]);
        }
      }
    } else {
      float da[2][2], db[2][2];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        da[i][0] = e4m3_decode(as_[i] & 0xffu);
        da[i][1] = e4m3_decode(as_[i] >> 8);
        db[i][0] = e4m3_decode(bs_[i] & 0xffu);
        db[i][1] = e4m3_decode(bs_[i] >> 8);
      }
#pragma unroll
      for (int s = 0; s < 4; s++) {
        bf16x8 af[2], bf[2];
#pragma unroll
        for (int i = 0; i < 2; i++) {
          uint32_t wa = s == 0 ? aw[i].x : s == 1 ? aw[i].y : s == 2 ? aw[i].z : aw[i].w;
          uint32_t wb = s == 0 ? bw[i].x : s == 1 ? bw[i].y : s == 2 ? bw[i].z : bw[i].w;
          af[i] = deq8_bf16(wa, da[i][s >> 1]);
          bf[i] = deq8_bf16(wb, db[i][s >> 1]);
        }
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
          for (int j = 0; j < 2; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  float alpha = 1.0f;
  if constexpr (NV) alpha = g.a_ts[grp] * g.b_ts[grp];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int64_t col = n_base + j * 32 + r;
      if (col >= g.N) continue;
#pragma unroll
      for (int q = 0; q < 16; q++) {
        const int64_t row = m_base + i * 32 + (q >> 2) * 8 + hh * 4 + (q & 3);
        if (row >= g.M) continue;
        float v = acc[i][j][q];
        if constexpr (NV) v = v * alpha;
        if constexpr (OUT_BF16)
          reinterpret_cast<__bf16*>(g.c)[grp * g.c_gs + row * g.ldc + col] = (__bf16)v;
        else
          reinterpret_cast<float*>(g.c)[grp * g.c_gs + row * g.ldc + col] = v;
      }
    }
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  dim3 grid((unsigned)((g.N + 127) / 128), (unsigned)((g.M + 127) / 128), (unsigned)g.groups);
  if (g.nvfp4) {
    if (g.c_bf16) hipLaunchKernelGGL((gemm_kernel<true, true>), grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL((gemm_kernel<true, false>), grid, dim3(256), 0, s, g);
  } else {
    if (g.c_bf16) hipLaunchKernelGGL((gemm_kernel<false, true>), grid, dim3(256), 0, s, g);
    else hipLaunchKernelGGL((gemm_kernel<false, false>), grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace fp4impl
