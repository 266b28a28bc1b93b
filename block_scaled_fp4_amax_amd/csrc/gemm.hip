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
// exactly to fp16: v_cvt_scalef32_pk_f16_fp4 gives the E2M1 values, and one
// packed fp16 multiply applies the block scale, itself converted to fp16
// (exact: every E4M3 value is a normal fp16; the product has at most 6
// significant bits and lies in [2^-10, 2688], so fp16 holds it exactly);
// v_mfma_f32_32x32x16_f16 multiplies, and the two tensor scales multiply the
// accumulator in the epilogue. A lane's 32 K values feed four K=16 MFMAs
// (8 values each); the K order inside the product is permuted identically
// for A and B, which leaves the sum unchanged.
//
// Tiling: a workgroup (4 waves, 2 x 2) owns a 256 x BN tile of C (BN = 256
// unless fewer tiles than compute units would result, or, for NVFP4, K is
// short; else 128); each wave owns 128 x BN/2 as 32 x 32 MFMA tiles. The
// grid is persistent (one workgroup per CU) and walks tiles in an order that
// keeps operand panels within one XCD's L2.
//
// Operand staging is shaped by the number of L2 requests, not by bytes: a
// stage covers 128 K values, so each row contributes one 64-byte segment,
// and the scale bytes of a row are copied 16 at a time, covering four stages
// (MXFP4) or two (NVFP4). Stages move global -> LDS with direct-to-LDS
// buffer loads (16 bytes per lane) whose range check against the tile's rows
// turns rows past M or N into zeros. All four waves copy, each a quarter of
// a stage, spread over the MFMAs of a half-stage so that the copies never
// hold a wave's matrix core idle. Four stages are in flight in a ring of LDS
// slots, plus two scale chunks. Within a row the four 16-byte pieces are
// rotated by bits 2-3 of the row so that each 16-lane group of a
// ds_read_b128 hits 16 distinct bank groups. A wave reads the next
// half-stage's fragments while its MFMAs on the current one run. The B
// matrix feeds the MFMA's first operand and A the second, so lane l holds
// C[m = l % 32][n = 8 (q / 4) + 4 (l / 32) + q % 4]. The output goes through
// the (then idle) stage slots so that global stores write whole row segments.
#include <type_traits>

#include "fp4_device.h"
#include "launch.h"
#include "quant_common.h"

namespace fp4impl {
using namespace fp4dev;

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBM = 256;
constexpr int kBK = 128;             // K values per stage
constexpr int kRowBytes = kBK / 2;   // code bytes per row per stage

typedef int i32x4 __attribute__((ext_vector_type(4)));

// voffset addend that puts every lane of a copy out of range (a stage past
// the end of K: its copies land zeros in a slot that is never read)
constexpr uint32_t kPastEnd = 0x80000000u;

template <bool NV, int BN, int WAVES>
struct Tile {
  static constexpr int kABytes = kBM * kRowBytes;
  static constexpr int kBBytes = BN * kRowBytes;
  static constexpr int kSlot = kABytes + kBBytes;
  static constexpr int kCS = NV ? 2 : 4;     // stages per 16-byte scale chunk
  static constexpr int kSABytes = kBM * 16;  // scale chunk: 16 bytes per row
  static constexpr int kSBBytes = 256 * 16;  // (rows of a 128-wide B tile are loaded twice)
  static constexpr int kChunk = kSABytes + kSBBytes;
  static constexpr int kChunk0 = 4 * kSlot;  // LDS offset of scale chunk 0; chunk 1 follows
  static constexpr int kLds = 4 * kSlot + 2 * kChunk;
  // WAVES waves: 2 along M (128 rows each), WAVES / 2 along N
  static constexpr int kWN = BN / (WAVES / 2);  // wave tile width
  static constexpr int kNJ = kWN / 32;          // MFMA tiles across a wave
  // A copy moves 1 KB (64 lanes x 16 bytes). Wave w takes the 1 KB blocks
  // w, w + WAVES, w + 2 WAVES, ... of a stage slot and of a scale chunk.
  static constexpr int kLW = kSlot / 1024 / WAVES;     // per wave per stage
  static constexpr int kLWA = kABytes / 1024 / WAVES;  // of which A rows
  static constexpr int kLCW = kChunk / 1024 / WAVES;   // per wave per scale chunk
  // output staging: WAVES / 4 waves share a slot
  static constexpr int kWPS = WAVES / 4;
};

// Raw buffer resource over [base, base + bytes): loads past its end return
// zeros (gfx9 descriptor: 48-bit base, stride 0, record count in bytes,
// 32-bit untyped data format).
__device__ __forceinline__ i32x4 buffer_rsrc(const uint8_t* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)b, (int)(uint32_t)((b >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// Direct-to-LDS copy of 16 bytes per lane: lane i reads the buffer at byte
// voff (zeros when its 16 bytes lie past the buffer's end) and its bytes land
// at LDS address lds + 16 i (lds wave-uniform, passed in m0). Written as
// inline assembly so that the compiler, which cannot match the copies in
// flight to the stage slots, adds no vmcnt waits of its own before LDS reads:
// every wait on these copies is explicit below. The instruction has no output
// register. It writes m0, which cannot be named as clobbered: the compiler
// reserves m0 (it rejects it on a clobber list) and sets it itself right
// before each instruction of its own that reads it, never holding a value in
// it across other code; in this kernel nothing but these copies reads m0.
__device__ __forceinline__ void b2l16(const i32x4& rsrc, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(lds)
      : "memory");
}
// Scalar (wave-uniform) fp32 load, completed inside the statement. A vector
// load here would make the compiler wait for every copy in flight before
// its first use.
__device__ __forceinline__ float scalar_load_f32(const float* p) {
  float v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}
// LDS byte address of a __shared__ object
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// s_waitcnt vmcnt(n) (gfx9 encoding), leaving expcnt / lgkmcnt unconstrained
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0), leaving vmcnt / expcnt unconstrained
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

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
// own L2. Within a group, tiles are numbered band by band: a band is
// kBandN consecutive N tiles, walked M tile by M tile with its N tiles
// innermost. XCD x owns the contiguous range [x * per, (x + 1) * per) of that
// numbering and its workgroups walk it interleaved, so the tiles in flight
// on one XCD form a block of a few M tiles by kBandN N tiles, whose A and B
// panels its L2 shares.
constexpr int64_t kBandN = 8;
struct TileWalk {
  int64_t tiles_m, tiles_n, T, per, wpx, x, i;
  __device__ __forceinline__ TileWalk(int64_t tm, int64_t tn, int64_t groups) {
    tiles_m = tm;
    tiles_n = tn;
    T = tm * tn * groups;
    per = (T + 7) / 8;
    wpx = gridDim.x / 8;
    x = blockIdx.x % 8;
    i = blockIdx.x / 8;
  }
  __device__ __forceinline__ bool get(int64_t j, int64_t* grp, int64_t* tm, int64_t* tn) const {
    const int64_t k = i + j * wpx;
    if (k >= per) return false;
    const int64_t tile = x * per + k;
    if (tile >= T) return false;
    const int64_t per_grp = tiles_m * tiles_n;
    *grp = tile / per_grp;
    const int64_t r = tile - *grp * per_grp;
    const int64_t band = kBandN * tiles_m;
    const int64_t nb = r / band, rr = r - nb * band;
    const int64_t rem = tiles_n - nb * kBandN;
    const int64_t width = rem < kBandN ? rem : kBandN;  // the last band may be narrower
    *tm = rr / width;
    *tn = nb * kBandN + (rr - *tm * width);
    return true;
  }
};

// Where a tile sits: its group, its first A (and C) row m0 and the end of
// the group's rows mend (rows in [m0, min(m0 + kBM, mend)) are valid), and
// its first column n0.
struct TilePos {
  int64_t grp, m0, mend, n0;
};

// Groups of equal size: group g's A, C panels start at g times their group
// strides, so row indices are group-local.
struct DenseWalk {
  TileWalk w;
  int64_t M;
  int bn;
  __device__ __forceinline__ DenseWalk(const GemmArgs& g, int BN)
      : w((g.M + kBM - 1) / kBM, (g.N + BN - 1) / BN, g.groups), M(g.M), bn(BN) {}
  __device__ __forceinline__ bool get(int64_t j, TilePos* p) const {
    int64_t tm, tn;
    if (!w.get(j, &p->grp, &tm, &tn)) return false;
    p->m0 = tm * kBM;
    p->mend = M;
    p->n0 = tn * bn;
    return true;
  }
};

// Group g's rows are [offs[g], offs[g + 1]) of one A and one C; the offsets
// live in device memory (a router writes them), so every workgroup counts
// the M tiles itself: group g has ceil(rows_g / kBM) of them, and the M
// tiles of all groups, concatenated in group order, take the place of one
// group's M tiles in the banded walk. Each offset is clamped into [0, M] and
// each group's end to at least its start, so any offsets keep every access
// inside A and C. A wave scans the groups 64 at a time (lane l holds group
// c + l), with a prefix sum of the tile counts.
__device__ __forceinline__ void group_rows(const int32_t* offs, int64_t G, int64_t M, int64_t g, int64_t* s,
                                           int64_t* e) {
  int64_t a = 0, b = 0;
  if (g < G) {
    a = offs[g];
    b = offs[g + 1];
    a = a < 0 ? 0 : (a > M ? M : a);
    b = b < a ? a : (b > M ? M : b);
  }
  *s = a;
  *e = b;
}
__device__ __forceinline__ int wave_inclusive_sum(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}
struct VarWalk {
  TileWalk w;
  const int32_t* offs;
  int64_t G, M;
  int bn;
  __device__ __forceinline__ static int64_t count_tiles(const GemmArgs& g) {
    const int lane = threadIdx.x & 63;
    int64_t total = 0;
    for (int64_t c = 0; c < g.groups; c += 64) {
      int64_t s, e;
      group_rows(g.offs, g.groups, g.M, c + lane, &s, &e);
      const int n = (int)((e - s + kBM - 1) / kBM);
      total += __builtin_amdgcn_readlane(wave_inclusive_sum(n, lane), 63);
    }
    return total;
  }
  __device__ __forceinline__ VarWalk(const GemmArgs& g, int BN)
      : w(count_tiles(g), (g.N + BN - 1) / BN, 1), offs(g.offs), G(g.groups), M(g.M), bn(BN) {}
  __device__ __forceinline__ bool get(int64_t j, TilePos* p) const {
    int64_t grp0, tmg, tn;
    if (!w.get(j, &grp0, &tmg, &tn)) return false;
    const int lane = threadIdx.x & 63;
    int64_t before = 0;
    for (int64_t c = 0; c < G; c += 64) {
      int64_t s, e;
      group_rows(offs, G, M, c + lane, &s, &e);
      const int n = (int)((e - s + kBM - 1) / kBM);
      const int incl = wave_inclusive_sum(n, lane);
      const uint64_t hit = __ballot(before + incl > tmg);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        const int64_t first = before + __builtin_amdgcn_readlane(incl - n, l);
        p->grp = c + l;
        p->m0 = (int64_t)__builtin_amdgcn_readlane((int)s, l) + (tmg - first) * kBM;
        p->mend = __builtin_amdgcn_readlane((int)e, l);
        p->n0 = tn * bn;
        return true;
      }
      before += __builtin_amdgcn_readlane(incl, 63);
    }
    return false;  // not reached: the tile count came from the same offsets
  }
};

// An FP4 MFMA operand: the instruction reads the low four of its eight
// registers (32 E2M1 codes); the high four are left undefined so the
// compiler need not copy the fragment into a zero-padded tuple.
__device__ __forceinline__ i32x8 fp4_operand(const uint4& v) {
  typedef int i32x4v __attribute__((ext_vector_type(4)));
  const i32x4v q = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
  return __builtin_shufflevector(q, q, 0, 1, 2, 3, -1, -1, -1, -1);
}

// The E4M3 scales of a lane's two blocks of one half-stage (bytes 0 and 1 of
// `pair`) as an fp16 pair, block 0's in the low half, in one conversion:
// every E4M3 value is a normal fp16, so the conversion is exact.
__device__ __forceinline__ f16x2 nv_scale_pair(uint32_t pair) {
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pair, 1.0f, false));
}
// block B's scale (B compile-time) in both halves
template <int B>
__device__ __forceinline__ f16x2 nv_block(f16x2 s) {
  return B ? f16x2{s.y, s.y} : f16x2{s.x, s.x};
}
// Codes 2 pr and 2 pr + 1 of w (pr 0..3, compile-time after unrolling) ->
// their exact fp16 values of val * scale: the converter gives the E2M1
// values, one packed fp16 multiply applies the block scale s (the product
// has at most 6 significant bits and lies in [2^-10, 2688], so fp16 holds
// it exactly).
__device__ __forceinline__ f16x2 nv_dequant2(uint32_t w, int pr, f16x2 s) {
  const f16x2 p = pr == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)
                : pr == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)
                : pr == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)
                          : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return p * s;
}
// four fp16 pairs, in order, as one 8-value MFMA operand
__device__ __forceinline__ f16x8 join4(const f16x2 (&q)[4]) {
  return f16x8{q[0].x, q[0].y, q[1].x, q[1].y, q[2].x, q[2].y, q[3].x, q[3].y};
}
// all 8 codes of w
__device__ __forceinline__ f16x8 nv_dequant8(uint32_t w, f16x2 s) {
  const f16x2 q[4] = {nv_dequant2(w, 0, s), nv_dequant2(w, 1, s), nv_dequant2(w, 2, s), nv_dequant2(w, 3, s)};
  return join4(q);
}
// The dword of a lane's 16-byte fragment that sub-step kt (0..3) reads.
__device__ __forceinline__ uint32_t nv_word(const uint4& c, int kt) {
  return kt == 0 ? c.x : kt == 1 ? c.y : kt == 2 ? c.z : c.w;
}

}  // namespace

// Output staging. A wave's 128 x WN block of C goes, in fp32, to its own
// stage slot, RR rows at a time (RR = 128, or 64 when 128 rows do not fit a
// slot), as rows of 16-byte chunks whose position is XORed with the low row
// bits so that the lanes' writes and the store waves' reads spread over the
// banks. Lane (r32, h) holds, in register group a of MFMA tile (i, j), the
// four columns 32 j + 8 a + 4 h + 0..3 of row 32 i + r32: one chunk.
template <int WN>
struct Epi {
  static constexpr int kRowB = WN * 4;             // staged row bytes (fp32)
  static constexpr int kCPR = kRowB / 16;          // 16-byte chunks per row
  static constexpr int kSwz = (kCPR < 16 ? kCPR : 16) - 1;
};

template <int WN, int RR>
__device__ __forceinline__ void stage_wave_rows(const f32x16 (&acc)[4][WN / 32], float alpha, uint8_t* region,
                                                int round, int lane) {
  using E = Epi<WN>;
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ii = 0; ii < RR / 32; ii++) {
    const int i = round * (RR / 32) + ii;
    const int row = ii * 32 + r32;
    uint8_t* rowp = region + row * E::kRowB;
#pragma unroll
    for (int j = 0; j < WN / 32; j++)
#pragma unroll
      for (int a = 0; a < 4; a++) {
        const int chunk = (8 * j + 2 * a + h) ^ (row & E::kSwz);
        *reinterpret_cast<float4*>(rowp + chunk * 16) =
            make_float4(acc[i][j][4 * a] * alpha, acc[i][j][4 * a + 1] * alpha, acc[i][j][4 * a + 2] * alpha,
                        acc[i][j][4 * a + 3] * alpha);
      }
  }
}

// A wave writes rows row0 + [0, NR) of a round's staged blocks: each row
// joins the NWN staged blocks of the waves with one wm (block wn at
// reg0 + wn * reg_stride, columns [wn WN, (wn + 1) WN)) and goes to output row
// m_base + row; a lane converts 8 consecutive values and writes them in one
// piece, consecutive lanes along the row.
// What the epilogue writes: C in fp32 or bf16, or C quantized along its rows
// (MXFP4 or NVFP4 codes and scales).
enum OutKind { kOutF32 = 0, kOutBF16 = 1, kOutMX = 2, kOutNV = 3 };

// C is written once and never read back by the kernel: non-temporal stores
// keep its lines from displacing in L2 the operand panels that the tiles in
// flight still read.
__device__ __forceinline__ void store_c16(uint8_t* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

template <int WN, int NWN, int NR, bool OUT_BF16>
__device__ __forceinline__ void store_staged_rows(const GemmArgs& g, const uint8_t* reg0, int reg_stride, int row0,
                                                  int64_t grp, int64_t m_base, int64_t m_end, int64_t n0, int lane) {
  using E = Epi<WN>;
  constexpr int kGPR = WN / 8;  // 8-value groups per row per block
  constexpr int kES = OUT_BF16 ? 2 : 4;
  const bool vec = g.c_vec_ok;
#pragma unroll 2
  for (int c0 = 0; c0 < NR * NWN * kGPR; c0 += 64) {
    const int c = c0 + lane;
    const int row = row0 + c / (NWN * kGPR), k = c % (NWN * kGPR);
    const int wn = k / kGPR, p = k % kGPR;
    const uint8_t* rp = reg0 + wn * reg_stride + row * E::kRowB;
    const float4 v0 = *reinterpret_cast<const float4*>(rp + (((2 * p) ^ (row & E::kSwz)) * 16));
    const float4 v1 = *reinterpret_cast<const float4*>(rp + (((2 * p + 1) ^ (row & E::kSwz)) * 16));
    const int64_t m = m_base + row;
    const int64_t n = n0 + wn * WN + p * 8;
    if (m < m_end && n < g.N) {
      uint8_t* dst = reinterpret_cast<uint8_t*>(g.c) + (grp * g.c_gs + m * g.ldc + n) * kES;
      const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      if (vec && n + 8 <= g.N) {
        if constexpr (OUT_BF16) {
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; e++) o[e] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)vv[2 * e], (__bf16)vv[2 * e + 1]});
          store_c16(dst, u32x4{o[0], o[1], o[2], o[3]});
        } else {
          store_c16(dst, __builtin_bit_cast(u32x4, f32x4{v0.x, v0.y, v0.z, v0.w}));
          store_c16(dst + 16, __builtin_bit_cast(u32x4, f32x4{v1.x, v1.y, v1.z, v1.w}));
        }
      } else {
        // row end or unaligned C: element by element
#pragma unroll 1
        for (int e = 0; e < 8 && n + e < g.N; e++) {
          if constexpr (OUT_BF16) reinterpret_cast<__bf16*>(dst)[e] = (__bf16)vv[e];
          else reinterpret_cast<float*>(dst)[e] = vv[e];
        }
      }
    }
  }
}

// NVFP4 constants of the quantized output of group grp: S_t from the
// caller's amax of C exactly as fp4_quantize forms it, the candidate
// multipliers, and no reciprocal table (a block divides instead).
__device__ __forceinline__ float out_tensor_scale(const GemmArgs& g, int64_t grp) {
  float St = g.q_amax[grp] / (g.q_sel ? 1792.0f : 2688.0f);
  if (!(St >= kFltMin && St <= 3.40282347e38f)) St = 1.0f;
  return St;
}

// Quantized output: a wave quantizes rows row0 + [0, NR) of a round's staged
// blocks (as store_staged_rows joins them), one 16-value unit per lane with
// consecutive lanes along the row, so an MXFP4 block is a lane pair (xor 1).
// The unit is quantized as fp4_quantize quantizes a row-major matrix holding
// C (with the Hadamard transform, 4/6 and stochastic rounding as set; the
// stochastic-rounding index of element (m, n) of group grp is
// (grp M + m) N + n); every lane takes part, stores only for valid units.
template <int WN, int NWN, int NR, bool QNV>
__device__ __forceinline__ void store_staged_rows_q(const GemmArgs& g, const uint8_t* reg0, int reg_stride, int row0,
                                                    int64_t grp, int64_t m_base, int64_t m_end, int64_t n0,
                                                    int lane, const NvConsts& nc) {
  using E = Epi<WN>;
  constexpr int kUPR = WN / 16;  // units per row per block
#pragma unroll 1
  for (int c0 = 0; c0 < NR * NWN * kUPR; c0 += 64) {
    const int c = c0 + lane;
    const int row = row0 + c / (NWN * kUPR), k = c % (NWN * kUPR);
    const int wn = k / kUPR, u = k % kUPR;
    const uint8_t* rp = reg0 + wn * reg_stride + row * E::kRowB;
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const float4 f = *reinterpret_cast<const float4*>(rp + (((4 * u + q) ^ (row & E::kSwz)) * 16));
      v[4 * q] = f.x;
      v[4 * q + 1] = f.y;
      v[4 * q + 2] = f.z;
      v[4 * q + 3] = f.w;
    }
    const int64_t m = m_base + row;
    const int64_t n = n0 + wn * WN + u * 16;
    if (g.q_rht) rht16(v, g.q_signs);
    const uint64_t L0 = (uint64_t)((grp * g.M + m) * g.N + n);
    uint32_t w0, w1, sbyte;
#define G_QUNIT(SEL, SR) quantize_unit<QNV, SEL, false, SR, false>(v, nc, L0, g.q_seed, g.q_offset, w0, w1, sbyte)
    if (g.q_sel == 0) {
      if (g.q_sr) G_QUNIT(0, true);
      else G_QUNIT(0, false);
    } else if (g.q_sel == 1 || !QNV) {
      if (g.q_sr) G_QUNIT(1, true);
      else G_QUNIT(1, false);
    } else {
      if constexpr (QNV) {
        if (g.q_sr) G_QUNIT(2, true);
        else G_QUNIT(2, false);
      }
    }
#undef G_QUNIT
    if (m < m_end && n < g.N) {
      __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(g.qc + grp * g.qc_gs + m * g.ldqc + n / 2));
      if constexpr (QNV) g.qs[grp * g.qs_gs + m * g.ldqs + n / 16] = (uint8_t)sbyte;
      else if ((u & 1) == 0) g.qs[grp * g.qs_gs + m * g.ldqs + n / 32] = (uint8_t)sbyte;
    }
  }
}

template <bool NV, int BN, int WAVES, int OUT, bool VAR>
__global__ __launch_bounds__(WAVES * 64, 1) void gemm_fp4_kernel(GemmArgs g) {
  using T = Tile<NV, BN, WAVES>;
  constexpr int NJ = T::kNJ;
  // Only the 256-wide NVFP4 tile runs short of registers around its K loop;
  // it alone forms its per-tile addresses anew each tile (below) instead of
  // keeping them live, which costs VALU work the other forms do not need.
  constexpr bool kOpaqueTile = NV && BN == 256;
  constexpr int CS = T::kCS;
  __shared__ __attribute__((aligned(16))) uint8_t lds[T::kLds];

  using Walk = typename std::conditional<VAR, VarWalk, DenseWalk>::type;
  const Walk walk(g, BN);
  if constexpr (OUT == kOutNV) {
    // the output tensor scales, written once for every group
    if (blockIdx.x == 0)
      for (int64_t i = threadIdx.x; i < g.groups; i += blockDim.x) g.q_ts[i] = out_tensor_scale(g, i);
  }
  TilePos pos;
  if (!walk.get(0, &pos)) return;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int r32 = lane & 31, h = lane >> 5;
  const uint32_t wl = __builtin_amdgcn_readfirstlane(w);  // the wave index, in a scalar register
  const uint32_t L = lds_u32(lds);      // LDS address of the slot ring
  const int S64 = (int)(g.K / 64);      // 64-K half-stages
  const int S = (S64 + 1) / 2;          // stages; the last one is half when S64 is odd

  // Copy sources. Lane l of a 1 KB block fills LDS piece l % 4 of the
  // block's row l / 4 with the row's 16-byte K piece (l % 4) ^ (bits 2-3 of
  // the row) = (l % 4) ^ (bits 4-5 of l), blocks starting at multiples of
  // 16 rows. Code block q < 16 holds A rows 16 q + [0, 16), block q >= 16 B
  // rows 16 (q - 16) + [0, 16); scale-chunk blocks hold 64 rows of 16 bytes,
  // four of A, then four of B (a 128-row B tile's rows twice). The lane
  // offsets are fixed for the kernel; a tile sets four buffer resources whose
  // size ends at its last valid row, and a stage adds its K offset.
  const uint32_t lda = (uint32_t)g.lda, ldb = (uint32_t)g.ldb;
  // The lane offsets of lane ln (scale-chunk block q = w + WAVES j, j <
  // kLCW: A rows 64 q + lane for q < 4, else B rows (64 (q - 4) + lane)
  // mod BN). Under kOpaqueTile each tile forms them anew from an opaque
  // copy of the lane index, so that none is kept (spilled) across the
  // epilogue; elsewhere the compiler keeps one set for the kernel.
  auto lane_offsets = [&](int ln, uint32_t (&vo)[T::kLW], uint32_t (&vs)[T::kLCW]) {
    const uint32_t piece = (uint32_t)(((ln & 3) ^ ((ln >> 4) & 3)) * 16);
#pragma unroll
    for (int j = 0; j < T::kLW; j++) {
      const int q = w + WAVES * j;
      vo[j] = j < T::kLWA ? (uint32_t)(16 * q + (ln >> 2)) * lda + piece
                          : (uint32_t)(16 * (q - 16) + (ln >> 2)) * ldb + piece;
    }
#pragma unroll
    for (int j = 0; j < T::kLCW; j++) {
      const int q = w + WAVES * j;
      vs[j] = q < 4 ? (uint32_t)(64 * q + ln) * (uint32_t)g.lda_s
                    : (uint32_t)((64 * (q - 4) + ln) & (BN - 1)) * (uint32_t)g.ldb_s;
    }
  };
  auto tile_lane = [&]() {
    int ln = lane;
    if constexpr (kOpaqueTile) asm volatile("" : "+v"(ln));
    return ln;
  };
  i32x4 ra, rb, rsa, rsb;
  auto set_sources = [&](int64_t grp_, int64_t m0_, int64_t mend_, int64_t n0_) {
    const int64_t rows_a = mend_ - m0_ < kBM ? mend_ - m0_ : kBM;
    const int64_t rows_b = g.N - n0_ < BN ? g.N - n0_ : BN;
    ra = buffer_rsrc(g.a + grp_ * g.a_gs + m0_ * g.lda, (uint32_t)(rows_a * g.lda));
    rb = buffer_rsrc(g.b + grp_ * g.b_gs + n0_ * g.ldb, (uint32_t)(rows_b * g.ldb));
    rsa = buffer_rsrc(g.as + grp_ * g.as_gs + m0_ * g.lda_s, (uint32_t)(rows_a * g.lda_s));
    rsb = buffer_rsrc(g.bs + grp_ * g.bs_gs + n0_ * g.ldb_s, (uint32_t)(rows_b * g.ldb_s));
  };

  // Copy k of a stage whose K offsets are YO (codes) and YOS (scale chunk),
  // into slot LSLOT and, with WITH_CHUNK, scale chunk LCHUNK (LDS
  // addresses): the chunk's copies first, then A's, then B's. k and
  // WITH_CHUNK are compile-time after unrolling.
#define G_COPY(LSLOT, LCHUNK, YO, YOS, WITH_CHUNK, K)                                   \
  do {                                                                                  \
    const int k_ = (K);                                                                 \
    const int q_ = k_ - ((WITH_CHUNK) ? T::kLCW : 0);                                   \
    if (q_ < 0) {                                                                       \
      b2l16(wl + WAVES * k_ < 4 ? rsa : rsb, voffs[k_] + (YOS), (LCHUNK) + (wl + WAVES * k_) * 1024); \
    } else {                                                                            \
      b2l16(q_ < T::kLWA ? ra : rb, voff[q_] + (YO), (LSLOT) + (wl + WAVES * q_) * 1024); \
    }                                                                                   \
  } while (0)
  // K offsets of stage Y; a stage at or past S reads nothing (every lane out
  // of range), so that every stage issues the same number of copies and every
  // wait below is a compile-time count.
#define G_YO(Y) ((Y) < S ? (uint32_t)(Y) * kRowBytes : kPastEnd)
#define G_YOS(Y) ((Y) < S ? (uint32_t)((Y) / CS) * 16 : kPastEnd)
  // every copy of stage Y at once
#define G_ISSUE(LSLOT, LCHUNK, Y, WITH_CHUNK)                                            \
  do {                                                                                  \
    const int yi_ = (Y);                                                                \
    const uint32_t yo_ = G_YO(yi_), yos_ = G_YOS(yi_);                                  \
    _Pragma("unroll") for (int k = 0; k < T::kLW + ((WITH_CHUNK) ? T::kLCW : 0); k++)   \
      G_COPY(LSLOT, LCHUNK, yo_, yos_, WITH_CHUNK, k);                                  \
  } while (0)

  f32x16 acc[4][NJ];

  // LDS read bases of lane ln. Fragments: A rows wm*128 + i*32 + r32, B
  // rows wn*kWN + j*32 + r32; the lane's 16-byte K piece of half-stage kb is
  // 2 kb + h, rotated. The bases are held opaque to the compiler, so that
  // every read is a base plus an immediate under 64 KB (ds_read's offset
  // field) instead of one register per (slot, row block, stage) address past
  // 64 KB: the scale words' base in chunk 0, and per operand and half-stage
  // a low fragment base (slot 0) and a high one (64 KB above it); frag_at
  // picks, at compile time, the one that leaves the immediate under 64 KB.
  // Under kOpaqueTile each tile forms them anew (from tile_lane()).
  struct LdsBases {
    uint32_t sa, sb, a0_lo, a1_lo, b0_lo, b1_lo, a0_hi, a1_hi, b0_hi, b1_hi;
  };
  auto lds_bases = [&](int ln) {
    const int r = ln & 31, hh = ln >> 5, rot = (r >> 2) & 3;
    LdsBases o;
    o.a0_lo = (uint32_t)((wm * 128 + r) * kRowBytes + ((0 + hh) ^ rot) * 16);
    o.a1_lo = (uint32_t)((wm * 128 + r) * kRowBytes + ((2 + hh) ^ rot) * 16);
    o.b0_lo = (uint32_t)(T::kABytes + (wn * T::kWN + r) * kRowBytes + ((0 + hh) ^ rot) * 16);
    o.b1_lo = (uint32_t)(T::kABytes + (wn * T::kWN + r) * kRowBytes + ((2 + hh) ^ rot) * 16);
    o.sa = (uint32_t)(T::kChunk0 + (wm * 128 + r) * 16);
    o.sb = (uint32_t)(T::kChunk0 + T::kSABytes + (wn * T::kWN + r) * 16);
    o.a0_hi = o.a0_lo + 65536u;
    o.a1_hi = o.a1_lo + 65536u;
    o.b0_hi = o.b0_lo + 65536u;
    o.b1_hi = o.b1_lo + 65536u;
    asm volatile("" : "+v"(o.sa), "+v"(o.sb));
    asm volatile("" : "+v"(o.a0_lo), "+v"(o.a1_lo), "+v"(o.b0_lo), "+v"(o.b1_lo));
    asm volatile("" : "+v"(o.a0_hi), "+v"(o.a1_hi), "+v"(o.b0_hi), "+v"(o.b1_hi));
    return o;
  };
  const LdsBases bases_k = lds_bases(lane);
  auto frag_at = [&](uint32_t lo, uint32_t hi, int imm) -> const uint4* {
    return reinterpret_cast<const uint4*>(imm < 65536 ? lds + lo + imm : lds + hi + (imm - 65536));
  };
  uint4 ca0[4], ca1[4], cb0[NJ], cb1[NJ];
  // scale words of a stage, double-buffered by stage parity. MXFP4: one
  // dword per row = the E8M0 bytes of (kb, h) at byte 2 kb + h. NVFP4: two
  // dwords per row, dword kb holding the four E4M3 bytes of half-stage kb.
  uint32_t sa0[4][NV ? 2 : 1], sa1[4][NV ? 2 : 1], sb0[NJ][NV ? 2 : 1], sb1[NJ][NV ? 2 : 1];

#define G_READ(SLOT, KB, CA, CB)                                                        \
  do {                                                                                  \
    const int so_ = (int)((SLOT) - lds);                                                \
    _Pragma("unroll") for (int i = 0; i < 4; i++)                                       \
      CA[i] = *frag_at((KB) ? lb.a1_lo : lb.a0_lo, (KB) ? lb.a1_hi : lb.a0_hi, so_ + i * 32 * kRowBytes); \
    _Pragma("unroll") for (int j = 0; j < NJ; j++)                                      \
      CB[j] = *frag_at((KB) ? lb.b1_lo : lb.b0_lo, (KB) ? lb.b1_hi : lb.b0_hi, so_ + j * 32 * kRowBytes); \
  } while (0)

#define G_READ_SCALES(CHUNK, U, SA, SB)                                                 \
  do {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < 4; i++) {                                     \
      if constexpr (NV) {                                                               \
        const uint2 v_ = *reinterpret_cast<const uint2*>(lds + lb.sa + ((CHUNK) - lds - T::kChunk0) + i * 512 + ((U) % CS) * 8); \
        SA[i][0] = v_.x;                                                                \
        SA[i][NV ? 1 : 0] = v_.y;                                                       \
      } else {                                                                          \
        SA[i][0] = *reinterpret_cast<const uint32_t*>(lds + lb.sa + ((CHUNK) - lds - T::kChunk0) + i * 512 + ((U) % CS) * 4); \
      }                                                                                 \
    }                                                                                   \
    _Pragma("unroll") for (int j = 0; j < NJ; j++) {                                    \
      if constexpr (NV) {                                                               \
        const uint2 v_ = *reinterpret_cast<const uint2*>(lds + lb.sb + ((CHUNK) - lds - T::kChunk0) + j * 512 + ((U) % CS) * 8); \
        SB[j][0] = v_.x;                                                                \
        SB[j][NV ? 1 : 0] = v_.y;                                                       \
      } else {                                                                          \
        SB[j][0] = *reinterpret_cast<const uint32_t*>(lds + lb.sb + ((CHUNK) - lds - T::kChunk0) + j * 512 + ((U) % CS) * 4); \
      }                                                                                 \
    }                                                                                   \
  } while (0)

  // MFMAs of one half-stage, part [P0, P1) of it: MFMA rows i (MXFP4) or
  // K sub-steps kt (NVFP4), each 0..3. With CP (compile-time) the whole
  // half-stage runs with the copies of stage Y (into slot LSLOT, and scale
  // chunk LCHUNK when WC) spread over it, after the MFMAs they follow: a
  // copy holds the wave's issue while the texture unit takes its addresses,
  // and the MFMA in flight covers that time.
#define G_MFMAS_X(CA, CB, SA, SB, KB, P0, P1, CP, LSLOT, LCHUNK, Y, WC)                 \
  do {                                                                                  \
    constexpr int nc_ = T::kLW + ((WC) ? T::kLCW : 0);                                  \
    const uint32_t yo_ = (CP) ? G_YO(Y) : 0u, yos_ = (CP) ? G_YOS(Y) : 0u;              \
    (void)yo_;                                                                          \
    (void)yos_;                                                                         \
    if constexpr (!NV) {                                                                \
      constexpr int nm_ = 4 * NJ;                                                       \
      uint32_t sa_[4], sb_[NJ];                                                         \
      _Pragma("unroll") for (int i = (P0); i < (P1); i++) sa_[i] = (SA[i][0] >> (16 * (KB) + 8 * h)) & 0xffu; \
      _Pragma("unroll") for (int j = 0; j < NJ; j++) sb_[j] = (SB[j][0] >> (16 * (KB) + 8 * h)) & 0xffu; \
      _Pragma("unroll") for (int i = (P0); i < (P1); i++) {                             \
        const i32x8 fa = fp4_operand(CA[i]);                                            \
        _Pragma("unroll") for (int j = 0; j < NJ; j++) {                                \
          const i32x8 fb = fp4_operand(CB[j]);                                          \
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb, fa, acc[i][j], 4, 4, 0, (int)sb_[j], \
                                                                      0, (int)sa_[i]);  \
          if constexpr (CP) {                                                           \
            _Pragma("unroll") for (int c = 0; c < nc_; c++)                             \
              if ((c * nm_) / nc_ == i * NJ + j) G_COPY(LSLOT, LCHUNK, yo_, yos_, (WC), c); \
            __builtin_amdgcn_sched_barrier(0);                                          \
          }                                                                             \
        }                                                                               \
      }                                                                                 \
    } else {                                                                            \
      /* software-pipelined: sub-step kt's MFMAs run while the fp16 fragments \
         of kt + 1 are dequantized, in equal shares after each MFMA: every \
         MFMA is followed by (4 + NJ) / NJ converter + multiply pairs, so \
         that no burst of VALU work outlasts the MFMA it hides behind */     \
      constexpr int nm_ = 16 * NJ;                                                      \
      uint32_t pa_[4], pb_[NJ];                                                         \
      _Pragma("unroll") for (int i = 0; i < 4; i++) pa_[i] = SA[i][(KB) & (NV ? 1 : 0)] >> (16 * h); \
      _Pragma("unroll") for (int j = 0; j < NJ; j++) pb_[j] = SB[j][(KB) & (NV ? 1 : 0)] >> (16 * h); \
      f16x2 na[4], nb[NJ];                                                               \
      f16x8 ha[4], hb[NJ];                                                              \
      f16x2 qa_[4][4], qb_[NJ][4];                                                      \
      _Pragma("unroll") for (int i = 0; i < 4; i++) {                                   \
        na[i] = nv_scale_pair(pa_[i]);                                                      \
        ha[i] = nv_dequant8(nv_word(CA[i], (P0)), nv_block<((P0) >> 1)>(na[i]));         \
      }                                                                                 \
      _Pragma("unroll") for (int j = 0; j < NJ; j++) {                                  \
        nb[j] = nv_scale_pair(pb_[j]);                                                      \
        hb[j] = nv_dequant8(nv_word(CB[j], (P0)), nv_block<((P0) >> 1)>(nb[j]));         \
      }                                                                                 \
      _Pragma("unroll") for (int kt = (P0); kt < (P1); kt++) {                          \
        const int kn_ = kt + 1;                                                         \
        _Pragma("unroll") for (int i = 0; i < 4; i++)                                   \
        _Pragma("unroll") for (int j = 0; j < NJ; j++) {                                \
          const int m_ = i * NJ + j;                                                    \
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hb[j], ha[i], acc[i][j], 0, 0, 0); \
          if (kn_ < (P1)) {                                                             \
            constexpr int qpm_ = (4 + NJ) / NJ;                                         \
            _Pragma("unroll") for (int qq = 0; qq < qpm_; qq++) {                       \
              const int q_ = m_ * qpm_ + qq, f_ = q_ >> 2, pr_ = q_ & 3;                \
              if (f_ < 4)                                                               \
                qa_[f_][pr_] = nv_dequant2(nv_word(CA[f_], kn_), pr_, kn_ < 2 ? nv_block<0>(na[f_]) : nv_block<1>(na[f_])); \
              else if (f_ - 4 < NJ)                                                     \
                qb_[f_ - 4][pr_] = nv_dequant2(nv_word(CB[f_ - 4], kn_), pr_, kn_ < 2 ? nv_block<0>(nb[f_ - 4]) : nv_block<1>(nb[f_ - 4])); \
            }                                                                           \
          }                                                                             \
          if constexpr (CP) {                                                           \
            _Pragma("unroll") for (int c = 0; c < nc_; c++)                             \
              if ((c * nm_) / nc_ == (kt * 4 + i) * NJ + j) G_COPY(LSLOT, LCHUNK, yo_, yos_, (WC), c); \
          }                                                                             \
          __builtin_amdgcn_sched_barrier(0);                                            \
        }                                                                               \
        if (kn_ < (P1)) {                                                               \
          _Pragma("unroll") for (int i = 0; i < 4; i++) ha[i] = join4(qa_[i]);          \
          _Pragma("unroll") for (int j = 0; j < NJ; j++) hb[j] = join4(qb_[j]);         \
        }                                                                               \
      }                                                                                 \
    }                                                                                   \
  } while (0)
#define G_MFMAS(CA, CB, SA, SB, KB, P0, P1) G_MFMAS_X(CA, CB, SA, SB, KB, P0, P1, false, 0u, 0u, 0, false)

  // Stage x = x0 + U (U compile-time, x0 a multiple of 8) sits in slot U % 4,
  // its scales in chunk (U / CS) % 2 and scale buffer U % 2, and its first
  // half-stage's fragments are in ca0 / cb0. Half-stage 0: read half-stage
  // 1's fragments (and, half-way through, stage x+1's scales when its chunk
  // is already there), run half-stage 0. Half-stage 1: wait for stage x+1
  // (each wave for its own copies: those of stages x+2 and x+3 may still be
  // in flight), barrier (every wave is then done with this slot and sees
  // stage x+1 whole), read stage x+1's first fragments (and its scales if its
  // chunk came with it), run half-stage 1 with the copies of stage x+4 into
  // this slot spread over it. The last stage keeps the barrier: its copies
  // (past K, landing zeros) must not overtake another wave's last reads of
  // this slot or of the scale chunk they refill. The LDS reads are issued on every path, also
  // past the last stage (they then read data that is never used), so that
  // the compiler can count them exactly and waits only for the reads a
  // half-stage consumes. A chunk slot is refilled at stage 4 c - 4 (c the
  // chunk's index, in chunk-sized steps of CS stages): by then the last stage
  // of the chunk two back has had its scales read, in half-stage 0 of the
  // stage before it.
#define G_STAGE(U)                                                                      \
  do {                                                                                  \
    uint8_t* const slot_ = lds + ((U) % 4) * T::kSlot;                                  \
    uint8_t* const nslot_ = lds + (((U) + 1) % 4) * T::kSlot;                           \
    uint8_t* const nchunk_ = lds + T::kChunk0 + ((((U) + 1) / CS) % 2) * T::kChunk;     \
    const uint32_t lslot_ = L + ((U) % 4) * T::kSlot;                                   \
    const uint32_t lrchunk_ = L + T::kChunk0 + ((((U) + 4) / CS) % 2) * T::kChunk;      \
    auto& sa_c = ((U) % 2) ? sa1 : sa0;                                                 \
    auto& sb_c = ((U) % 2) ? sb1 : sb0;                                                 \
    auto& sa_n = ((U) % 2) ? sa0 : sa1;                                                 \
    auto& sb_n = ((U) % 2) ? sb0 : sb1;                                                 \
    const int x_ = x0 + (U);                                                            \
    const bool kb1_ = 2 * x_ + 1 < S64;                                                 \
    const bool next_ = x_ + 1 < S;                                                      \
    G_READ(slot_, 1, ca1, cb1);                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    if constexpr (NV) {                                                                 \
      /* one pipelined run over the half-stage */                                      \
      if (((U) + 1) % CS != 0) G_READ_SCALES(nchunk_, (U) + 1, sa_n, sb_n);             \
      __builtin_amdgcn_sched_barrier(0);                                                \
      G_MFMAS(ca0, cb0, sa_c, sb_c, 0, 0, 4);                                           \
    } else {                                                                            \
      G_MFMAS(ca0, cb0, sa_c, sb_c, 0, 0, 2);                                           \
      if (((U) + 1) % CS != 0) {                                                        \
        __builtin_amdgcn_sched_barrier(0);                                              \
        G_READ_SCALES(nchunk_, (U) + 1, sa_n, sb_n);                                    \
        __builtin_amdgcn_sched_barrier(0);                                              \
      }                                                                                 \
      G_MFMAS(ca0, cb0, sa_c, sb_c, 0, 2, 4);                                           \
    }                                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    wait_lgkm0();                                                                       \
    if (next_)                                                                          \
      wait_vmcnt<2 * T::kLW + (((U) + 2) % CS == 0 ? T::kLCW : 0) + (((U) + 3) % CS == 0 ? T::kLCW : 0)>(); \
    lds_barrier();                                                                      \
    G_READ(nslot_, 0, ca0, cb0);                                                        \
    if (((U) + 1) % CS == 0) G_READ_SCALES(nchunk_, (U) + 1, sa_n, sb_n);               \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    if (kb1_) G_MFMAS_X(ca1, cb1, sa_c, sb_c, 1, 0, 4, true, lslot_, lrchunk_, x_ + 4, ((U) + 4) % CS == 0); \
  } while (0)

  // A tile starts with stages 0-3 in flight and waits for stage 0.
  constexpr int kAfter0 = 3 * T::kLW + (1 % CS == 0 ? T::kLCW : 0) + (2 % CS == 0 ? T::kLCW : 0) +
                          (3 % CS == 0 ? T::kLCW : 0);
  auto issue_first_stages = [&]() {
    uint32_t voff[T::kLW], voffs[T::kLCW];
    lane_offsets(tile_lane(), voff, voffs);
    G_ISSUE(L, L + T::kChunk0, 0, true);
    G_ISSUE(L + T::kSlot, L + T::kChunk0 + ((1 / CS) % 2) * T::kChunk, 1, 1 % CS == 0);
    G_ISSUE(L + 2 * T::kSlot, L + T::kChunk0 + ((2 / CS) % 2) * T::kChunk, 2, 2 % CS == 0);
    G_ISSUE(L + 3 * T::kSlot, L + T::kChunk0 + ((3 / CS) % 2) * T::kChunk, 3, 3 % CS == 0);
  };
  set_sources(pos.grp, pos.m0, pos.mend, pos.n0);
  issue_first_stages();
  for (int64_t jt = 0;; jt++) {
    const int64_t m0 = pos.m0, mend = pos.mend, n0 = pos.n0, cgrp = pos.grp;
    // the K loop's copy offsets (used by G_COPY) and LDS read bases (used by
    // G_READ, G_READ_SCALES)
    uint32_t voff[T::kLW], voffs[T::kLCW];
    lane_offsets(tile_lane(), voff, voffs);
    const LdsBases lb = kOpaqueTile ? lds_bases(tile_lane()) : bases_k;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < NJ; j++)
#pragma unroll
        for (int q = 0; q < 16; q++) acc[i][j][q] = 0.0f;
    if (S > 0) {
      wait_vmcnt<kAfter0>();
      lds_barrier();
      G_READ(lds, 0, ca0, cb0);
      G_READ_SCALES(lds + T::kChunk0, 0, sa0, sb0);
    }
    for (int x0 = 0; x0 < S; x0 += 8) {
      G_STAGE(0);
      if (x0 + 1 < S) G_STAGE(1);
      if (x0 + 2 < S) G_STAGE(2);
      if (x0 + 3 < S) G_STAGE(3);
      if (x0 + 4 < S) G_STAGE(4);
      if (x0 + 5 < S) G_STAGE(5);
      if (x0 + 6 < S) G_STAGE(6);
      if (x0 + 7 < S) G_STAGE(7);
    }

    // Every wave is done with the slots once the copies past the last stage
    // have landed: stage the tile's C there, store it, then start the next
    // tile's first stages.
    const bool more = walk.get(jt + 1, &pos);
    wait_vmcnt<0>();
    wait_lgkm0();
    lds_barrier();
    float alpha = 1.0f;
    if constexpr (NV) alpha = scalar_load_f32(g.a_ts + cgrp * g.a_ts_gs) * scalar_load_f32(g.b_ts + cgrp);
    NvConsts nc_out{};
    if constexpr (OUT == kOutNV) {
      nc_out.St = out_tensor_scale(g, cgrp);
      nc_out.k6 = 1.0f / (6.0f * nc_out.St);
      nc_out.k4 = 1.0f / (4.0f * nc_out.St);
    }
    {
      // wave w = wm + 2 wn stages into region(w): slot w / kWPS, part w % kWPS
      using E = Epi<T::kWN>;
      constexpr int kReg = T::kSlot / T::kWPS;
      constexpr int RR = kReg / E::kRowB >= 128 ? 128 : 64;
      constexpr int kNR = 2 * RR / WAVES;  // rows each wave stores per round
      auto region = [&](int v) { return lds + (v / T::kWPS) * T::kSlot + (v % T::kWPS) * kReg; };
      const int sm = (int)(wl & 1), sh = (int)(wl >> 1);
      // the lane index as a value the compiler cannot see through, so that
      // the epilogue's many LDS and global addresses are formed here, once
      // per tile, rather than before the tile loop and kept (spilled) across
      // the K loop
      int lane_e = lane;
      if constexpr (kOpaqueTile) asm volatile("" : "+v"(lane_e));
#pragma unroll
      for (int round = 0; round < 128 / RR; round++) {
        stage_wave_rows<T::kWN, RR>(acc, alpha, region(w), round, lane_e);
        wait_lgkm0();
        lds_barrier();
        // wave s: rows (s >> 1) * kNR + [0, kNR) of the blocks of the waves with wm = s & 1
        if constexpr (OUT == kOutF32 || OUT == kOutBF16) {
          store_staged_rows<T::kWN, WAVES / 2, kNR, OUT == kOutBF16>(g, region(sm),
                                                                    (int)(region(sm + 2) - region(sm)), sh * kNR,
                                                                    cgrp, m0 + sm * 128 + round * RR, mend, n0, lane_e);
        } else {
          store_staged_rows_q<T::kWN, WAVES / 2, kNR, OUT == kOutNV>(g, region(sm),
                                                                    (int)(region(sm + 2) - region(sm)), sh * kNR,
                                                                    cgrp, m0 + sm * 128 + round * RR, mend, n0, lane_e,
                                                                    nc_out);
        }
        wait_lgkm0();
        lds_barrier();
      }
    }
    if (!more) break;
    set_sources(pos.grp, pos.m0, pos.mend, pos.n0);
    issue_first_stages();
  }
  // no copy into LDS may outlive the workgroup
  wait_vmcnt<0>();
#undef G_STAGE
#undef G_MFMAS
#undef G_MFMAS_X
#undef G_READ_SCALES
#undef G_READ
#undef G_ISSUE
#undef G_YO
#undef G_YOS
#undef G_COPY
}

// M tiles of the launch: exact for equal groups; for groups given by row
// offsets (known only on the device), the most M rows can split into,
// sum ceil(rows_g / kBM) <= floor((M + groups (kBM - 1)) / kBM).
static int64_t m_tiles(const GemmArgs& g) {
  return g.offs ? (g.M + g.groups * (kBM - 1)) / kBM : ((g.M + kBM - 1) / kBM) * g.groups;
}

template <bool NV, int BN, int WAVES, bool VAR>
static void launch_tiles_v(const GemmArgs& g, hipStream_t s) {
  const int64_t T = ((g.N + BN - 1) / BN) * m_tiles(g);
  int64_t wgs = ((T + 7) / 8) * 8;
  const int64_t cus = device_cu_count();
  if (wgs > cus) wgs = cus - cus % 8;
  dim3 grid((unsigned)wgs);
  if constexpr (!VAR && BN == 128) {
    if (g.qc) {
      if (g.q_nv) hipLaunchKernelGGL((gemm_fp4_kernel<NV, BN, WAVES, kOutNV, false>), grid, dim3(WAVES * 64), 0, s, g);
      else hipLaunchKernelGGL((gemm_fp4_kernel<NV, BN, WAVES, kOutMX, false>), grid, dim3(WAVES * 64), 0, s, g);
      return;
    }
  }
  if (g.c_bf16) hipLaunchKernelGGL((gemm_fp4_kernel<NV, BN, WAVES, kOutBF16, VAR>), grid, dim3(WAVES * 64), 0, s, g);
  else hipLaunchKernelGGL((gemm_fp4_kernel<NV, BN, WAVES, kOutF32, VAR>), grid, dim3(WAVES * 64), 0, s, g);
}
template <bool NV, int BN, int WAVES>
static void launch_tiles(const GemmArgs& g, hipStream_t s) {
  if (g.offs) launch_tiles_v<NV, BN, WAVES, true>(g, s);
  else launch_tiles_v<NV, BN, WAVES, false>(g, s);
}

// Waves per workgroup. Eight (two per SIMD, 128 x BN/4 each) double the
// LDS read rate a SIMD can draw, but measured slower end to end on every
// workload shape (fewer MFMAs per fragment read, more dequant per MFMA for
// NVFP4), so one wave per SIMD it is.
constexpr int kWavesMx = 4, kWavesNv = 4;
// shortest K at which the 256-wide NVFP4 tile is the faster one
constexpr int64_t kNvWideMinK = 1024;

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  // 256-wide tiles when they still give every compute unit a tile
  const int64_t t256 = ((g.N + 255) / 256) * (g.offs ? (g.M + kBM - 1) / kBM : m_tiles(g));
  const bool wide = t256 >= device_cu_count();
  if (g.nvfp4) {
    // NVFP4: the 256-wide tile dequantizes 0.5 instead of 0.75 fragments per
    // MFMA, but it spills in the tile epilogue (256 accumulators beside the
    // fp16 dequant state), which long K amortizes
    if (wide && !g.qc && g.K >= kNvWideMinK) launch_tiles<true, 256, kWavesNv>(g, s);
    else launch_tiles<true, 128, kWavesNv>(g, s);
  } else {
    // a quantized output keeps the 128-wide tile: beside 256 accumulators
    // the quantizer's temporaries would spill
    if (wide && !g.qc) launch_tiles<false, 256, kWavesMx>(g, s);
    else launch_tiles<false, 128, kWavesMx>(g, s);
  }
  return hipGetLastError();
}

}  // namespace fp4impl
