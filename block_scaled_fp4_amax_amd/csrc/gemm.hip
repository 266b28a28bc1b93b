// gemm.hip -- W4A4 block-scaled GEMM for gfx950:
//   C_g = deq(A_g) deq(B_g)^T, fp32 accumulation, fp32 or bf16 output,
// A_g [M, K] and B_g [N, K] as fp4_quantize writes them (Ultralytics glossary
// "FP4", section "Inferencia e Treinamento FP4": matrix products in FP4 with
// higher-precision accumulation; section "Como funciona FP4": MXFP4 and NVFP4
// block formats).
//
// MXFP4 runs on v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands: every
// lane feeds 32 consecutive K values of one row (16 bytes of codes) and that
// run's E8M0 byte as its scale operand, so the matrix core applies the block
// scales itself.
//
// NVFP4: the MFMA scale operand is a power of two per 32 values, which cannot
// carry an E4M3 scale per 16. Each lane therefore dequantizes its codes
// exactly to fp16: the converter v_cvt_scalef32_pk_f16_fp4 gives
// val * 2^E for the power-of-two part 2^E of the block scale, and one packed
// fp16 multiply applies its mantissa factor 1 + m/8 (the product has at most
// 6 significant bits and lies in [2^-10, 2688], so fp16 holds it exactly);
// v_mfma_f32_32x32x16_f16 multiplies, and the two tensor scales multiply the
// accumulator in the epilogue. A lane's 32 K values feed four K=16 MFMAs
// (8 values each); the K order inside the product is permuted identically
// for A and B, which leaves the sum unchanged.
//
// Tiling: a workgroup (4 waves, 2 x 2) owns a 256 x BN tile of C (BN = 256
// for MXFP4 unless fewer tiles than compute units would result, else 128;
// NVFP4 always 128); each wave owns
// 128 x BN/2 as 32 x 32 MFMA tiles. The grid is persistent (one workgroup per
// CU) and walks tiles in an order that keeps operand panels within one XCD's
// L2. K advances 64 values per stage; each stage's codes (32 bytes per row)
// and scale bytes are copied global -> LDS with the direct-to-LDS loads, six
// stages in flight in a ring of distinct LDS arrays. Within a row the two
// 16-byte halves are stored swapped on rows whose bit 3 is set, so each
// 16-lane group of a ds_read_b128 hits 16 distinct bank groups. A wave reads
// the next stage's fragments while its MFMAs on the current stage run. The B matrix feeds the MFMA's first
// operand and A the second, so lane l holds C[m = l % 32][n = 8 (q / 4) +
// 4 (l / 32) + q % 4]. The output goes through a per-wave LDS buffer so that
// global stores write whole row segments (16 or 32 bytes per lane).
#include "fp4_device.h"
#include "launch.h"

namespace fp4impl {
using namespace fp4dev;

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBM = 256;
constexpr int kRowBytes = 32;  // codes per row per stage (64 values)
constexpr int kStages = 6;

template <int BN>
struct Tile {
  static constexpr int kABytes = kBM * kRowBytes;
  static constexpr int kBBytes = BN * kRowBytes;
  static constexpr int kASBytes = kBM * 4;  // one LDS dword of scale bytes per row per stage
  static constexpr int kBSBytes = 256 * 4;  // (rows of a 128-wide B tile are loaded twice)
  static constexpr int kStage = kABytes + kBBytes + kASBytes + kBSBytes;
  static constexpr int kWN = BN / 2;        // wave tile width
  static constexpr int kNJ = kWN / 32;      // MFMA tiles across a wave
  static constexpr int kLoads = BN == 256 ? 6 : 5;  // copies per thread per stage
};

__device__ __forceinline__ void g2l16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)l, 16, 0, 0);
}
// Sub-dword and dword direct-to-LDS loads fill one LDS dword per lane.
__device__ __forceinline__ void g2l4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)l, 4, 0, 0);
}
__device__ __forceinline__ void g2l2(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)l, 2, 0, 0);
}

// s_waitcnt vmcnt(n) (gfx9 encoding), leaving expcnt / lgkmcnt unconstrained
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0), leaving vmcnt / expcnt unconstrained
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Wait until every copy of stage `need` has landed, given that the copies
// issued so far cover stages up to `last` (L loads per stage per thread,
// completing in order); the copies of the later stages may stay in flight.
template <int L>
__device__ __forceinline__ void wait_stage_landed(int need, int last) {
  switch (last - need) {
    case 4: wait_vmcnt<4 * L>(); break;
    case 3: wait_vmcnt<3 * L>(); break;
    case 2: wait_vmcnt<2 * L>(); break;
    case 1: wait_vmcnt<1 * L>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// Workgroup barrier without the release/acquire fences of __syncthreads()
// (those would force vmcnt(0) and drain the copies in flight). The empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Persistent tile order. The grid has one workgroup per CU (a multiple of 8)
// and consecutive workgroup ids go round-robin to the 8 XCDs, each with its
// own L2. Tiles are ordered group-major, then by N tile, then by M tile; XCD
// x owns the contiguous range [x * per, (x + 1) * per) and its workgroups
// walk it interleaved, so tiles sharing an operand panel run on one XCD at
// about the same time.
struct TileWalk {
  int64_t tiles_m, tiles_n, T, per, wpx, x, i;
  __device__ TileWalk(int64_t tm, int64_t tn, int64_t groups) {
    tiles_m = tm;
    tiles_n = tn;
    T = tm * tn * groups;
    per = (T + 7) / 8;
    wpx = gridDim.x / 8;
    x = blockIdx.x % 8;
    i = blockIdx.x / 8;
  }
  __device__ bool get(int64_t j, int64_t* grp, int64_t* tm, int64_t* tn) const {
    const int64_t k = i + j * wpx;
    if (k >= per) return false;
    const int64_t tile = x * per + k;
    if (tile >= T) return false;
    *tm = tile % tiles_m;
    *tn = (tile / tiles_m) % tiles_n;
    *grp = tile / (tiles_m * tiles_n);
    return true;
  }
};

// NVFP4 block scale split for the fp16 dequant: the converter's scale operand
// (only its exponent is used, so the decoded scale itself serves) and the
// mantissa factor 1 + m/8 as an fp16 pair.
struct NvScale {
  float pow2;
  f16x2 mant;
};
__device__ __forceinline__ NvScale nv_scale(uint32_t byte) {
  const float dec = e4m3_decode(byte);
  const float m = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, dec) & 0x007fffffu) | 0x3f800000u);
  const _Float16 mh = (_Float16)m;
  return NvScale{dec, f16x2{mh, mh}};
}
// 8 codes (one dword) -> 8 exact fp16 values of val * scale
__device__ __forceinline__ f16x8 nv_dequant8(uint32_t w, const NvScale& s) {
  f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 0) * s.mant;
  f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 1) * s.mant;
  f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 2) * s.mant;
  f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.pow2, 3) * s.mant;
  return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

}  // namespace

// Store a wave's 128 x WN block of C through its LDS buffer, 16 rows at a
// time. Lane (r32, h) holds row 32 i + r32 of the block and, in register
// group a of MFMA tile j, the four columns 32 j + 8 a + 4 h + 0..3. The lanes
// owning the slab's rows write their column groups (fp32) into padded LDS
// rows; the whole wave then reads back 8 consecutive values per lane,
// converts them to the output type and stores whole row segments.
template <int WN, bool OUT_BF16>
__device__ __forceinline__ void store_wave_tile(const GemmArgs& g, const f32x16 (&acc)[4][WN / 32], float alpha,
                                                uint8_t* stage, int64_t grp, int64_t mw, int64_t nw, int lane) {
  constexpr int kPitch = WN * 4 + 16;       // padded LDS row pitch (bytes)
  constexpr int kPerRow = WN / 8;           // 8-value chunks per row
  constexpr int kChunks = 16 * kPerRow;     // per 16-row slab
  constexpr int kES = OUT_BF16 ? 2 : 4;
  const int r32 = lane & 31, h = lane >> 5;
  const bool vec = g.c_vec_ok;
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int half = 0; half < 2; half++) {
      if ((r32 >> 4) == half) {
        uint8_t* rowp = stage + (r32 & 15) * kPitch;
#pragma unroll
        for (int j = 0; j < WN / 32; j++)
#pragma unroll
          for (int a = 0; a < 4; a++)
            *reinterpret_cast<float4*>(rowp + (j * 32 + 8 * a + 4 * h) * 4) =
                make_float4(acc[i][j][4 * a] * alpha, acc[i][j][4 * a + 1] * alpha, acc[i][j][4 * a + 2] * alpha,
                            acc[i][j][4 * a + 3] * alpha);
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int c0 = 0; c0 < kChunks; c0 += 64) {
        const int c = c0 + lane;
        const int row = c / kPerRow, col = (c % kPerRow) * 8;
        const float4 v0 = *reinterpret_cast<const float4*>(stage + row * kPitch + col * 4);
        const float4 v1 = *reinterpret_cast<const float4*>(stage + row * kPitch + col * 4 + 16);
        const int64_t m = mw + i * 32 + 16 * half + row;
        const int64_t n = nw + col;
        if (m < g.M && n < g.N) {
          uint8_t* dst = reinterpret_cast<uint8_t*>(g.c) + (grp * g.c_gs + m * g.ldc + n) * kES;
          const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          if (vec && n + 8 <= g.N) {
            if constexpr (OUT_BF16) {
              uint32_t o[4];
#pragma unroll
              for (int e = 0; e < 4; e++)
                o[e] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)vv[2 * e], (__bf16)vv[2 * e + 1]});
              *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
            } else {
              reinterpret_cast<float4*>(dst)[0] = v0;
              reinterpret_cast<float4*>(dst)[1] = v1;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; e++) {
              if (n + e < g.N) {
                if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(dst)[e] = (__bf16)vv[e];
                else reinterpret_cast<float*>(dst)[e] = vv[e];
              }
            }
          }
        }
      }
      asm volatile("" ::: "memory");
    }
  }
}

template <bool NV, int BN, bool OUT_BF16>
__global__ __launch_bounds__(256, 1) void gemm_fp4_kernel(GemmArgs g) {
  using T = Tile<BN>;
  constexpr int NJ = T::kNJ;
  constexpr int L = T::kLoads;
  __shared__ __attribute__((aligned(16))) uint8_t slot0[T::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t slot1[T::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t slot2[T::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t slot3[T::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t slot4[T::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t slot5[T::kStage];
  constexpr int kOutPitch = T::kWN * 4 + 16;
  __shared__ __attribute__((aligned(16))) uint8_t outbuf[4 * 16 * kOutPitch];

  const TileWalk walk((g.M + kBM - 1) / kBM, (g.N + BN - 1) / BN, g.groups);
  int64_t grp, tm, tn;
  if (!walk.get(0, &grp, &tm, &tn)) return;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int r32 = lane & 31, h = lane >> 5;
  const int S = (int)(g.K / 64);

  // Copy sources of the current tile: a wave-uniform base per matrix (kept in
  // scalar registers and advanced per stage) plus a 32-bit per-lane offset.
  // Codes: LDS chunk q holds row q / 2, half (q & 1) ^ bit 3 of the row. Rows
  // past M / N re-read the last row (their results are never stored).
  const uint8_t* a_base;
  const uint8_t* b_base;
  const uint8_t* as_base;
  const uint8_t* bs_base;
  uint32_t a_off[2], b_off[2], as_off, bs_off;
  auto set_sources = [&](int64_t grp_, int64_t m0_, int64_t n0_) {
    a_base = g.a + grp_ * g.a_gs + m0_ * g.lda;
    b_base = g.b + grp_ * g.b_gs + n0_ * g.ldb;
    as_base = g.as + grp_ * g.as_gs + m0_ * g.lda_s;
    bs_base = g.bs + grp_ * g.bs_gs + n0_ * g.ldb_s;
    const int64_t am = g.M - 1 - m0_, bm = g.N - 1 - n0_;  // last valid row, tile-relative
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int q = t + 256 * j, row = q >> 1, half = (q & 1) ^ ((row >> 3) & 1);
      const int64_t ar = row < am ? row : am;
      const int64_t br = (row % BN) < bm ? (row % BN) : bm;
      a_off[j] = (uint32_t)(ar * g.lda + half * 16);
      b_off[j] = (uint32_t)(br * g.ldb + half * 16);
    }
    as_off = (uint32_t)((t < am ? t : am) * g.lda_s);
    bs_off = (uint32_t)(((t % BN) < bm ? (t % BN) : bm) * g.ldb_s);
  };

#define G_ISSUE(BASE, SS)                                                               \
  do {                                                                                  \
    const uint8_t* ab_ = a_base + (SS) * kRowBytes;                                     \
    const uint8_t* bb_ = b_base + (SS) * kRowBytes;                                     \
    g2l16(ab_ + a_off[0], (BASE) + (w * 64) * 16);                                      \
    g2l16(ab_ + a_off[1], (BASE) + (256 + w * 64) * 16);                                \
    g2l16(bb_ + b_off[0], (BASE) + T::kABytes + (w * 64) * 16);                         \
    if constexpr (BN == 256) g2l16(bb_ + b_off[1], (BASE) + T::kABytes + (256 + w * 64) * 16); \
    if constexpr (NV) {                                                                 \
      g2l4(as_base + 4 * (SS) + as_off, (BASE) + T::kABytes + T::kBBytes + w * 256);    \
      g2l4(bs_base + 4 * (SS) + bs_off, (BASE) + T::kABytes + T::kBBytes + T::kASBytes + w * 256); \
    } else {                                                                            \
      g2l2(as_base + 2 * (SS) + as_off, (BASE) + T::kABytes + T::kBBytes + w * 256);    \
      g2l2(bs_base + 2 * (SS) + bs_off, (BASE) + T::kABytes + T::kBBytes + T::kASBytes + w * 256); \
    }                                                                                   \
  } while (0)

  f32x16 acc[4][NJ];

  // Fragments of one stage, raw (codes + scale bytes), double-buffered in
  // registers. A rows wm*128 + i*32 + r32; B rows wn*kWN + j*32 + r32.
  const int swz = h ^ ((r32 >> 3) & 1);
  const int offa = (wm * 128 + r32) * kRowBytes + swz * 16;
  const int offb = T::kABytes + (wn * T::kWN + r32) * kRowBytes + swz * 16;
  const int offsa = T::kABytes + T::kBBytes + (wm * 128 + r32) * 4 + (NV ? 2 * h : h);
  const int offsb = T::kABytes + T::kBBytes + T::kASBytes + (wn * T::kWN + r32) * 4 + (NV ? 2 * h : h);
  uint4 ca0[4], ca1[4], cb0[NJ], cb1[NJ];
  uint32_t sa0[4], sa1[4], sb0[NJ], sb1[NJ];

#define G_READ(BASE, CA, CB, SA, SB)                                                    \
  do {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < 4; i++) {                                     \
      CA[i] = *reinterpret_cast<const uint4*>((BASE) + offa + i * 32 * kRowBytes);      \
      if constexpr (NV) SA[i] = *reinterpret_cast<const uint16_t*>((BASE) + offsa + i * 128); \
      else SA[i] = (BASE)[offsa + i * 128];                                             \
    }                                                                                   \
    _Pragma("unroll") for (int j = 0; j < NJ; j++) {                                    \
      CB[j] = *reinterpret_cast<const uint4*>((BASE) + offb + j * 32 * kRowBytes);      \
      if constexpr (NV) SB[j] = *reinterpret_cast<const uint16_t*>((BASE) + offsb + j * 128); \
      else SB[j] = (BASE)[offsb + j * 128];                                             \
    }                                                                                   \
  } while (0)

#define G_MFMAS(CA, CB, SA, SB)                                                         \
  do {                                                                                  \
    if constexpr (!NV) {                                                                \
      _Pragma("unroll") for (int i = 0; i < 4; i++) {                                   \
        const i32x8 fa = {(int)CA[i].x, (int)CA[i].y, (int)CA[i].z, (int)CA[i].w, 0, 0, 0, 0}; \
        _Pragma("unroll") for (int j = 0; j < NJ; j++) {                                \
          const i32x8 fb = {(int)CB[j].x, (int)CB[j].y, (int)CB[j].z, (int)CB[j].w, 0, 0, 0, 0}; \
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc[i][j], 4, 4, 0, (int)SB[j], \
                                                                      0, (int)SA[i]);   \
        }                                                                               \
      }                                                                                 \
    } else {                                                                            \
      NvScale na[4], nb[NJ];                                                            \
      _Pragma("unroll") for (int kt = 0; kt < 4; kt++) {                                \
        if ((kt & 1) == 0) {                                                            \
          _Pragma("unroll") for (int i = 0; i < 4; i++)                                 \
            na[i] = nv_scale(kt == 0 ? (SA[i] & 0xffu) : (SA[i] >> 8));                 \
          _Pragma("unroll") for (int j = 0; j < NJ; j++)                                \
            nb[j] = nv_scale(kt == 0 ? (SB[j] & 0xffu) : (SB[j] >> 8));                 \
        }                                                                               \
        f16x8 ha[4], hb[NJ];                                                            \
        _Pragma("unroll") for (int i = 0; i < 4; i++) {                                 \
          const uint32_t wa = kt == 0 ? CA[i].x : kt == 1 ? CA[i].y : kt == 2 ? CA[i].z : CA[i].w; \
          ha[i] = nv_dequant8(wa, na[i]);                                               \
        }                                                                               \
        _Pragma("unroll") for (int j = 0; j < NJ; j++) {                                \
          const uint32_t wb = kt == 0 ? CB[j].x : kt == 1 ? CB[j].y : kt == 2 ? CB[j].z : CB[j].w; \
          hb[j] = nv_dequant8(wb, nb[j]);                                               \
        }                                                                               \
        _Pragma("unroll") for (int i = 0; i < 4; i++)                                   \
        _Pragma("unroll") for (int j = 0; j < NJ; j++)                                  \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hb[j], ha[i], acc[i][j], 0, 0, 0); \
      }                                                                                 \
    }                                                                                   \
  } while (0)

  // Stage SS sits in slot SS % 6 with its fragments already in registers
  // (buffer SS % 2): wait for stage SS+1, barrier, start the copy of stage
  // SS+5 into the slot stage SS-1 used, read stage SS+1's fragments into the
  // other buffer, then run stage SS. The slots are distinct arrays, so
  // fragment reads are not serialised behind the copies in flight.
#define G_STEP(SS, NEXT, REFILL, CA, CB, SA, SB, NCA, NCB, NSA, NSB)                    \
  do {                                                                                  \
    if ((SS) + 1 < S) {                                                                 \
      wait_lgkm0();                                                                     \
      wait_stage_landed<L>((SS) + 1, min((SS) + kStages - 2, S - 1));                   \
      lds_barrier();                                                                    \
      if ((SS) + kStages - 1 < S) G_ISSUE(REFILL, (SS) + kStages - 1);                  \
      G_READ(NEXT, NCA, NCB, NSA, NSB);                                                 \
    }                                                                                   \
    G_MFMAS(CA, CB, SA, SB);                                                            \
  } while (0)

#define G_PROLOGUE()                                                                    \
  do {                                                                                  \
    if (S > 0) G_ISSUE(slot0, 0);                                                       \
    if (S > 1) G_ISSUE(slot1, 1);                                                       \
    if (S > 2) G_ISSUE(slot2, 2);                                                       \
    if (S > 3) G_ISSUE(slot3, 3);                                                       \
    if (S > 4) G_ISSUE(slot4, 4);                                                       \
  } while (0)

  set_sources(grp, tm * kBM, tn * BN);
  G_PROLOGUE();
  for (int64_t jt = 0;; jt++) {
    const int64_t m0 = tm * kBM, n0 = tn * BN, cgrp = grp;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < NJ; j++)
#pragma unroll
        for (int q = 0; q < 16; q++) acc[i][j][q] = 0.0f;
    if (S > 0) {
      // the previous tile's output stores are counted too: wait for all
      wait_vmcnt<0>();
      lds_barrier();
      G_READ(slot0, ca0, cb0, sa0, sb0);
    }
    for (int s = 0; s < S; s += 6) {
      G_STEP(s, slot1, slot5, ca0, cb0, sa0, sb0, ca1, cb1, sa1, sb1);
      if (s + 1 < S) G_STEP(s + 1, slot2, slot0, ca1, cb1, sa1, sb1, ca0, cb0, sa0, sb0);
      if (s + 2 < S) G_STEP(s + 2, slot3, slot1, ca0, cb0, sa0, sb0, ca1, cb1, sa1, sb1);
      if (s + 3 < S) G_STEP(s + 3, slot4, slot2, ca1, cb1, sa1, sb1, ca0, cb0, sa0, sb0);
      if (s + 4 < S) G_STEP(s + 4, slot5, slot3, ca0, cb0, sa0, sb0, ca1, cb1, sa1, sb1);
      if (s + 5 < S) G_STEP(s + 5, slot0, slot4, ca1, cb1, sa1, sb1, ca0, cb0, sa0, sb0);
    }

    // Start the next tile's first copies (every wave is past its last LDS
    // read of this tile), then store this tile while they are in flight.
    const bool more = walk.get(jt + 1, &grp, &tm, &tn);
    if (more) {
      wait_lgkm0();
      lds_barrier();
      set_sources(grp, tm * kBM, tn * BN);
      G_PROLOGUE();
    }
    float alpha = 1.0f;
    if constexpr (NV) alpha = g.a_ts[cgrp] * g.b_ts[cgrp];
    store_wave_tile<T::kWN, OUT_BF16>(g, acc, alpha, outbuf + w * 16 * kOutPitch, cgrp, m0 + wm * 128,
                                     n0 + wn * T::kWN, lane);
    if (!more) break;
  }
#undef G_PROLOGUE
#undef G_STEP
#undef G_MFMAS
#undef G_READ
#undef G_ISSUE
}

template <bool NV, int BN>
static void launch_tiles(const GemmArgs& g, hipStream_t s) {
  const int64_t T = ((g.N + BN - 1) / BN) * ((g.M + kBM - 1) / kBM) * g.groups;
  int64_t wgs = ((T + 7) / 8) * 8;
  const int64_t cus = device_cu_count();
  if (wgs > cus) wgs = cus - cus % 8;
  dim3 grid((unsigned)wgs);
  if (g.c_bf16) hipLaunchKernelGGL((gemm_fp4_kernel<NV, BN, true>), grid, dim3(256), 0, s, g);
  else hipLaunchKernelGGL((gemm_fp4_kernel<NV, BN, false>), grid, dim3(256), 0, s, g);
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  // 256-wide tiles when they still give every compute unit a tile
  const int64_t t256 = ((g.N + 255) / 256) * ((g.M + kBM - 1) / kBM) * g.groups;
  const bool wide = t256 >= device_cu_count();
  if (g.nvfp4) {
    // NVFP4 keeps the 256 x 128 tile: its fp16 dequant temporaries do not
    // fit beside 256 accumulators
    launch_tiles<true, 128>(g, s);
  } else {
    if (wide) launch_tiles<false, 256>(g, s);
    else launch_tiles<false, 128>(g, s);
  }
  return hipGetLastError();
}

}  // namespace fp4impl
