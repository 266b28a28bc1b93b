// quant_common.h -- per-block quantization steps shared by the row-major and
// the transposed quantize kernels.
//
// Method (Ultralytics glossary "FP4", section "Como funciona FP4"; Hugging
// Face transformers "Four Over Six", introduction):
//   MXFP4  block of 32 along the row, scale 2^e with e = floor(log2 amax) - 2
//          (E8M0), element code = nearest E2M1 of x / 2^e.
//   NVFP4  block of 16, E4M3 scale of amax / (M * S_t) with M = 6, element
//          code = nearest E2M1 of x * (1 / (E4M3 * S_t)).
//   4/6    also try M = 4 and keep the candidate with the smaller squared
//          error; the error of a 16-slice is eff^2 * (FMA chain over elements
//          0..7 of (val - q)^2 + FMA chain over elements 8..15).
// Scale selection modes (template parameter SEL):
//   0  the plain scale;
//   1  4/6: NVFP4 M = 6 or 4; MXFP4 exponent e or e + 1 (block max in
//      [4, 8) or in [2, 4)), by the same squared error with the 4^e factor
//      cancelled (e + 1 wins iff 4 S_{e+1} < S_e);
//   2  NVFP4 scale search: every E4M3 code from the M = 6 candidate's to the
//      M = 4 candidate's, smallest error wins, ties keep the smaller code;
//   3  NVFP4 whole-tensor scale: every block scale is E4M3 1.0 (code 0x38)
//      and S_t = T / 6, so the tensor max maps to 6.
#pragma once

#include "fp4_device.h"
#include "launch.h"

namespace fp4impl {
using namespace fp4dev;

constexpr float kInf = __builtin_huge_valf();
constexpr uint32_t kUnitScaleCode = 0x38u;  // E4M3 1.0

// One NVFP4 scale candidate: effective block scale eff = E4M3(code) * S_t and
// its correctly rounded reciprocal. eff below the smallest normal makes the
// block a zero block (r = 0, so every code keeps only its sign).
struct NvCand {
  float eff, r;
  uint32_t code;
  bool zero;
};

// The per-workgroup NVFP4 constants: S_t, the candidate multipliers
// 1 / (6 S_t) and 1 / (4 S_t), and rtab[code] = the reciprocal above for every
// non-negative E4M3 code (0 for a zero block), filled once per workgroup in
// LDS so that a block looks its reciprocal up instead of dividing.
struct NvConsts {
  float St, k6, k4;
  const float* rtab;
};

// TAB false: no table; the reciprocal is divided out (the same correctly
// rounded value the table holds).
template <bool TAB = true>
__device__ __forceinline__ NvCand nv_candidate(float amax, float k, const NvConsts& nc) {
  NvCand c;
  float s = amax * k;
  s = s > kE4M3Max ? kE4M3Max : s;
  c.code = e4m3_encode(s);
  c.eff = e4m3_decode(c.code) * nc.St;
  c.zero = !(c.eff >= kFltMin);
  if constexpr (TAB) c.r = nc.rtab[c.code & 127u];
  else c.r = c.zero ? 0.0f : 1.0f / c.eff;
  return c;
}

// Nearest-even E2M1 codes of 16 scaled values, packed 2 per byte.
__device__ __forceinline__ void pack16(const float q[16], uint32_t& w0, uint32_t& w1) {
  w0 = e2m1_pack2<0>(0u, q[0], q[1]);
  w0 = e2m1_pack2<1>(w0, q[2], q[3]);
  w0 = e2m1_pack2<2>(w0, q[4], q[5]);
  w0 = e2m1_pack2<3>(w0, q[6], q[7]);
  w1 = e2m1_pack2<0>(0u, q[8], q[9]);
  w1 = e2m1_pack2<1>(w1, q[10], q[11]);
  w1 = e2m1_pack2<2>(w1, q[12], q[13]);
  w1 = e2m1_pack2<3>(w1, q[14], q[15]);
}

// FMA chain of (val(code) - q)^2 over 8 elements whose codes are packed in w.
__device__ __forceinline__ float sq_chain8(const float q[8], uint32_t w) {
  f32x2 d0 = e2m1_unpack2<0>(w), d1 = e2m1_unpack2<1>(w), d2 = e2m1_unpack2<2>(w), d3 = e2m1_unpack2<3>(w);
  float acc = 0.0f, e;
  e = d0.x - q[0]; acc = __builtin_fmaf(e, e, acc);
  e = d0.y - q[1]; acc = __builtin_fmaf(e, e, acc);
  e = d1.x - q[2]; acc = __builtin_fmaf(e, e, acc);
  e = d1.y - q[3]; acc = __builtin_fmaf(e, e, acc);
  e = d2.x - q[4]; acc = __builtin_fmaf(e, e, acc);
  e = d2.y - q[5]; acc = __builtin_fmaf(e, e, acc);
  e = d3.x - q[6]; acc = __builtin_fmaf(e, e, acc);
  e = d3.y - q[7]; acc = __builtin_fmaf(e, e, acc);
  return acc;
}

__device__ __forceinline__ float sq_sum16(const float q[16], uint32_t w0, uint32_t w1) {
  return sq_chain8(q, w0) + sq_chain8(q + 8, w1);
}

// The NVFP4 candidate with E4M3 code `code`.
template <bool TAB = true>
__device__ __forceinline__ NvCand nv_code_candidate(uint32_t code, const NvConsts& nc) {
  NvCand c;
  c.code = code;
  c.eff = e4m3_decode(code) * nc.St;
  c.zero = !(c.eff >= kFltMin);
  if constexpr (TAB) c.r = nc.rtab[code & 127u];
  else c.r = c.zero ? 0.0f : 1.0f / c.eff;
  return c;
}

// MXFP4 under 4/6: the exponent e (scale byte sbyte, shared by the lane pair
// xor 1 that holds the 32-value block) or e + 1, by the squared error of the
// nearest-even codes; returns the chosen byte and that exponent's codes of
// this lane's 16 values. Both lanes of the pair call it together.
__device__ __forceinline__ uint32_t mx_pair_choice(const float v[16], uint32_t sbyte, uint32_t& w0, uint32_t& w1) {
  const int e = (int)sbyte - 127;
  float q0[16];
#pragma unroll
  for (int i = 0; i < 16; i++) q0[i] = __builtin_ldexpf(v[i], -e);
  pack16(q0, w0, w1);
  if (e >= 127) return sbyte;  // e + 1 has no E8M0 byte
  float q1[16];
#pragma unroll
  for (int i = 0; i < 16; i++) q1[i] = __builtin_ldexpf(v[i], -e - 1);
  uint32_t x0, x1;
  pack16(q1, x0, x1);
  float s0 = sq_sum16(q0, w0, w1), s1 = sq_sum16(q1, x0, x1);
  s0 = s0 + xor_shfl<1>(s0);
  s1 = s1 + xor_shfl<1>(s1);
  if (4.0f * s1 < s0) {
    w0 = x0;
    w1 = x1;
    return sbyte + 1;
  }
  return sbyte;
}

// Candidate error eff^2 * partial sum; a zero block never wins.
__device__ __forceinline__ float cand_error(const NvCand& c, float sum) {
  return c.zero ? kInf : (c.eff * c.eff) * sum;
}

// Stochastic rounding of 16 scaled values whose first element has linear
// output index L0 (a multiple of 16): Philox4x32-10 with counter
// (L/8, offset) and key seed gives 128 bits per 8 elements, 16 bits each
// (element L uses word (L/2) % 4, low half when L is even).
__device__ __forceinline__ void sr16(const float q[16], uint64_t L0, uint64_t seed, uint64_t offset,
                                     uint32_t& w0, uint32_t& w1) {
  uint64_t n = L0 >> 3;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  uint32_t o0 = (uint32_t)offset, o1 = (uint32_t)(offset >> 32);
  u32x4 ra = philox4x32_10(u32x4{(uint32_t)n, (uint32_t)(n >> 32), o0, o1}, k0, k1);
  n += 1;
  u32x4 rb = philox4x32_10(u32x4{(uint32_t)n, (uint32_t)(n >> 32), o0, o1}, k0, k1);
  w0 = 0u;
  w1 = 0u;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    uint32_t wa = ra[(i >> 1) & 3], wb = rb[(i >> 1) & 3];
    uint32_t r16a = (i & 1) ? (wa >> 16) : (wa & 0xffffu);
    uint32_t r16b = (i & 1) ? (wb >> 16) : (wb & 0xffffu);
    w0 |= e2m1_sr(q[i], r16a) << (4 * i);
    w1 |= e2m1_sr(q[8 + i], r16b) << (4 * i);
  }
}

// Quantize the 16 consecutive values v of one lane (a 16-value unit of an
// output row, after the Hadamard transform if any) whose first element has
// linear output index L0: packed codes w0 (elements 0..7), w1 (8..15) and
// the scale byte. Lanes exchange data, so every lane of a wave calls this
// together: MXFP4 units pair with the xor-1 lane into one 32-value block;
// under B2D the 16 lanes xor 1..8 hold the 16 rows of one 16 x 16 tile.
template <bool NV, int SEL, bool B2D, bool SR, bool TAB = true>
__device__ __forceinline__ void quantize_unit(const float v[16], const NvConsts& nc, uint64_t L0, uint64_t seed,
                                              uint64_t offset, uint32_t& w0, uint32_t& w1, uint32_t& sbyte) {
  float amax = max_abs16(v);
  if constexpr (!NV) {
    amax = __builtin_fmaxf(amax, xor_shfl<1>(amax));
    sbyte = e8m0_from_amax(amax);
    if constexpr (SEL == 1) sbyte = mx_pair_choice(v, sbyte, w0, w1);
    if constexpr (SR) {
      float q[16];
#pragma unroll
      for (int i = 0; i < 16; i++) q[i] = __builtin_ldexpf(v[i], 127 - (int)sbyte);
      sr16(q, L0, seed, offset, w0, w1);
    } else if constexpr (SEL == 0) {
      float sc = e8m0_scale_operand(sbyte);
      w0 = e2m1_pack2_scaled<0>(0u, v[0], v[1], sc);
      w0 = e2m1_pack2_scaled<1>(w0, v[2], v[3], sc);
      w0 = e2m1_pack2_scaled<2>(w0, v[4], v[5], sc);
      w0 = e2m1_pack2_scaled<3>(w0, v[6], v[7], sc);
      w1 = e2m1_pack2_scaled<0>(0u, v[8], v[9], sc);
      w1 = e2m1_pack2_scaled<1>(w1, v[10], v[11], sc);
      w1 = e2m1_pack2_scaled<2>(w1, v[12], v[13], sc);
      w1 = e2m1_pack2_scaled<3>(w1, v[14], v[15], sc);
    }
  } else {
    if constexpr (SEL == 3) {
      const NvCand c = nv_code_candidate<TAB>(kUnitScaleCode, nc);
      float q[16];
#pragma unroll
      for (int i = 0; i < 16; i++) q[i] = v[i] * c.r;
      if constexpr (SR) sr16(q, L0, seed, offset, w0, w1);
      else pack16(q, w0, w1);
      sbyte = c.code;
      return;
    }
    if constexpr (B2D) {
      amax = __builtin_fmaxf(amax, xor_shfl<1>(amax));
      amax = __builtin_fmaxf(amax, xor_shfl<2>(amax));
      amax = __builtin_fmaxf(amax, xor_shfl<4>(amax));
      amax = __builtin_fmaxf(amax, xor_shfl<8>(amax));
    }
    NvCand c = nv_candidate<TAB>(amax, nc.k6, nc);
    float q[16];
#pragma unroll
    for (int i = 0; i < 16; i++) q[i] = v[i] * c.r;
    pack16(q, w0, w1);
    if constexpr (SEL == 1) {
      NvCand c4 = nv_candidate<TAB>(amax, nc.k4, nc);
      float q4[16];
#pragma unroll
      for (int i = 0; i < 16; i++) q4[i] = v[i] * c4.r;
      uint32_t x0, x1;
      pack16(q4, x0, x1);
      float s6 = sq_sum16(q, w0, w1), s4 = sq_sum16(q4, x0, x1);
      if constexpr (B2D) {
        // pairwise tree over the tile's 16 rows (lanes), adjacent rows first
        s6 = s6 + xor_shfl<1>(s6); s4 = s4 + xor_shfl<1>(s4);
        s6 = s6 + xor_shfl<2>(s6); s4 = s4 + xor_shfl<2>(s4);
        s6 = s6 + xor_shfl<4>(s6); s4 = s4 + xor_shfl<4>(s4);
        s6 = s6 + xor_shfl<8>(s6); s4 = s4 + xor_shfl<8>(s4);
      }
      if (cand_error(c4, s4) < cand_error(c, s6)) {
        c = c4;
        w0 = x0;
        w1 = x1;
#pragma unroll
        for (int i = 0; i < 16; i++) q[i] = q4[i];
      }
    } else if constexpr (SEL == 2) {
      float s6 = sq_sum16(q, w0, w1);
      if constexpr (B2D) {
        s6 = s6 + xor_shfl<1>(s6);
        s6 = s6 + xor_shfl<2>(s6);
        s6 = s6 + xor_shfl<4>(s6);
        s6 = s6 + xor_shfl<8>(s6);
      }
      float best = cand_error(c, s6);
      // under B2D the 16 lanes of a tile share amax, hence the loop bounds
      const uint32_t hi = nv_candidate<TAB>(amax, nc.k4, nc).code;
      for (uint32_t code = c.code + 1; code <= hi; code++) {
        const NvCand cc = nv_code_candidate<TAB>(code, nc);
        float qq[16];
#pragma unroll
        for (int i = 0; i < 16; i++) qq[i] = v[i] * cc.r;
        uint32_t x0, x1;
        pack16(qq, x0, x1);
        float sc = sq_sum16(qq, x0, x1);
        if constexpr (B2D) {
          sc = sc + xor_shfl<1>(sc);
          sc = sc + xor_shfl<2>(sc);
          sc = sc + xor_shfl<4>(sc);
          sc = sc + xor_shfl<8>(sc);
        }
        const float err = cand_error(cc, sc);
        if (err < best) {
          best = err;
          c = cc;
          w0 = x0;
          w1 = x1;
#pragma unroll
          for (int i = 0; i < 16; i++) q[i] = qq[i];
        }
      }
    }
    if constexpr (SR) sr16(q, L0, seed, offset, w0, w1);
    sbyte = c.code;
  }
}

// Divisor D of the tensor scale S_t = T / D for scale selection mode SEL:
// 6 * 448 (plain), 4 * 448 (4/6 and the scale search: the M = 4 candidate of
// the block holding T does not saturate E4M3), 6 (whole-tensor scale).
template <int SEL>
constexpr float tensor_divisor() {
  return SEL == 0 ? 2688.0f : SEL == 3 ? 6.0f : 1792.0f;
}

// NVFP4 tensor scale for batch item b, computed identically by every
// workgroup: T from amax_in or the max of the pre-pass partials; S_t = T / D
// (tensor_divisor), replaced by 1 when zero, denormal or not finite. The
// item's first workgroup (first) stores S_t.
template <int SEL>
__device__ __forceinline__ float tensor_scale_prologue(const QuantArgs& a, int64_t b, bool first) {
  __shared__ float red[4];
  float T;
  if (a.amax_in) {
    T = a.amax_in[b];
  } else {
    float m = 0.0f;
    const float* p = a.partials + b * a.nparts;
    if ((a.nparts & 3) == 0) {
      // 16-byte loads (the workspace is 16-byte aligned)
      for (int i = 4 * threadIdx.x; i < a.nparts; i += 4 * blockDim.x) {
        const float4 q = *reinterpret_cast<const float4*>(p + i);
        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(q.x, q.y), __builtin_fmaxf(q.z, q.w)));
      }
    } else {
      for (int i = threadIdx.x; i < a.nparts; i += blockDim.x) m = __builtin_fmaxf(m, p[i]);
    }
    m = __builtin_fmaxf(m, xor_shfl<32>(m));
    m = __builtin_fmaxf(m, xor_shfl<16>(m));
    m = __builtin_fmaxf(m, xor_shfl<8>(m));
    m = __builtin_fmaxf(m, xor_shfl<4>(m));
    m = __builtin_fmaxf(m, xor_shfl<2>(m));
    m = __builtin_fmaxf(m, xor_shfl<1>(m));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    T = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  }
  float St = T / tensor_divisor<SEL>();
  if (!(St >= kFltMin && St <= 3.40282347e38f)) St = 1.0f;
  if (first && threadIdx.x == 0) a.tensor_scale[b] = St;
  return St;
}

// S_t (tensor_scale_prologue) and the workgroup's NvConsts; every thread of
// the (256-thread) workgroup takes part.
template <int SEL>
__device__ __forceinline__ NvConsts nv_prologue(const QuantArgs& a, int64_t b, bool first) {
  __shared__ float rtab[128];
  __shared__ float kk[2];
  NvConsts nc;
  nc.St = tensor_scale_prologue<SEL>(a, b, first);
  const int t = threadIdx.x;
  if (t < 128) {
    const float eff = e4m3_decode((uint32_t)t) * nc.St;
    rtab[t] = eff >= kFltMin ? 1.0f / eff : 0.0f;
  } else if (t == 128) {
    kk[0] = 1.0f / (6.0f * nc.St);
  } else if (t == 129) {
    kk[1] = 1.0f / (4.0f * nc.St);
  }
  __syncthreads();
  nc.k6 = kk[0];
  nc.k4 = kk[1];
  nc.rtab = rtab;
  return nc;
}

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float v[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float v[8]) {
  uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float v[8]) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

}  // namespace fp4impl
