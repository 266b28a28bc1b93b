// dequantize.hip -- FP4 codes + block scales -> fp32 / bf16 (Ultralytics
// glossary "FP4", section "Como funciona FP4": dequantized value = grid
// value * sign * block scale).
//   MXFP4: val * 2^e, exact, on the scaled conversion unit.
//   NVFP4: val * (E4M3 * S_t), one fp32 rounding, then bf16 (nearest even) if
//          asked.
// One lane per 16 codes (8 bytes); a wave covers 1024 consecutive elements.
#include "fp4_device.h"
#include "launch.h"

namespace fp4impl {
using namespace fp4dev;

template <bool NV, bool OUT_BF16>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const int64_t b = blockIdx.z;
  const int64_t upr = a.cols >> 4;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = u / upr, cu = u - row * upr;
  if (row >= a.rows) return;
  const uint2 w = *reinterpret_cast<const uint2*>(a.codes + b * a.bs_c + row * a.ld_c + cu * 8);
  const uint8_t* srow = a.scales + b * a.bs_s + row * a.ld_s;
  float v[16];
  if constexpr (!NV) {
    float sc = e8m0_scale_operand(srow[cu >> 1]);
    if constexpr (OUT_BF16) {
      uint4 o0 = make_uint4(e2m1_unpack2_bf16<0>(w.x, sc), e2m1_unpack2_bf16<1>(w.x, sc),
                            e2m1_unpack2_bf16<2>(w.x, sc), e2m1_unpack2_bf16<3>(w.x, sc));
      uint4 o1 = make_uint4(e2m1_unpack2_bf16<0>(w.y, sc), e2m1_unpack2_bf16<1>(w.y, sc),
                            e2m1_unpack2_bf16<2>(w.y, sc), e2m1_unpack2_bf16<3>(w.y, sc));
      uint4* yp = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.y) + b * a.bs_y + row * a.ld_y + cu * 16);
      yp[0] = o0;
      yp[1] = o1;
      return;
    } else {
      f32x2 p[8] = {e2m1_unpack2<0>(w.x, sc), e2m1_unpack2<1>(w.x, sc), e2m1_unpack2<2>(w.x, sc),
                    e2m1_unpack2<3>(w.x, sc), e2m1_unpack2<0>(w.y, sc), e2m1_unpack2<1>(w.y, sc),
                    e2m1_unpack2<2>(w.y, sc), e2m1_unpack2<3>(w.y, sc)};
#pragma unroll
      for (int i = 0; i < 8; i++) { v[2 * i] = p[i].x; v[2 * i + 1] = p[i].y; }
    }
  } else {
    const float eff = e4m3_decode(srow[cu]) * a.tensor_scale[b];
    f32x2 p[8] = {e2m1_unpack2<0>(w.x), e2m1_unpack2<1>(w.x), e2m1_unpack2<2>(w.x), e2m1_unpack2<3>(w.x),
                  e2m1_unpack2<0>(w.y), e2m1_unpack2<1>(w.y), e2m1_unpack2<2>(w.y), e2m1_unpack2<3>(w.y)};
#pragma unroll
    for (int i = 0; i < 8; i++) { v[2 * i] = p[i].x * eff; v[2 * i + 1] = p[i].y * eff; }
  }
  if constexpr (OUT_BF16) {
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      bf16x2 pr = {(__bf16)v[2 * i], (__bf16)v[2 * i + 1]};
      o[i] = __builtin_bit_cast(uint32_t, pr);
    }
    uint4* yp = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.y) + b * a.bs_y + row * a.ld_y + cu * 16);
    yp[0] = make_uint4(o[0], o[1], o[2], o[3]);
    yp[1] = make_uint4(o[4], o[5], o[6], o[7]);
  } else {
    float4* yp = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + b * a.bs_y + row * a.ld_y + cu * 16);
    yp[0] = make_float4(v[0], v[1], v[2], v[3]);
    yp[1] = make_float4(v[4], v[5], v[6], v[7]);
    yp[2] = make_float4(v[8], v[9], v[10], v[11]);
    yp[3] = make_float4(v[12], v[13], v[14], v[15]);
  }
}

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t s) {
  int64_t units = a.rows * (a.cols >> 4);
  dim3 grid((unsigned)((units + 255) / 256), 1, (unsigned)a.batch);
  if (a.nvfp4) {
    if (a.y_bf16) hipLaunchKernelGGL((dequant_kernel<true, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dequant_kernel<true, false>), grid, dim3(256), 0, s, a);
  } else {
    if (a.y_bf16) hipLaunchKernelGGL((dequant_kernel<false, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((dequant_kernel<false, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace fp4impl
