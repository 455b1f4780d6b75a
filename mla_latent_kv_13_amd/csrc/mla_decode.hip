// MI355X (gfx950 / CDNA4) kernels for single-token MLA decode and the
// C-ABI entry points that launch them.
//
// Method (kernelindex.com "kernelbot-amd-mixed-mla-668813": the mxfp4 stage-1
// kernel and its log2 stage-2 combine; "...-695854": the fp8 single-pass,
// split and reduce kernels and the torch fallback that states the plain math):
// 16 query heads attend over one latent KV head of width 576; V is the first
// 512 latent dims; the logit scale is 1/sqrt(576).  Stage 1 handles one
// (request, split) per workgroup; stage 2 merges the splits.
//
// Stage-1 design (one workgroup = 4 independent waves, or 2 when the grid has
// more workgroups than the device has CUs, so that two workgroups share a CU):
//   * A split's tokens are cut into 32-token sub-tiles dealt round-robin to the
//     waves.  Each wave streams its sub-tiles HBM -> LDS with direct-to-LDS
//     16-byte loads (global_load_lds_dwordx4) into a private ring of NBUF
//     slots, the page table being gathered by the same asynchronous path one
//     or two sub-tiles ahead, and waits with explicit vmcnt counts so several
//     sub-tiles stay in flight while it computes.
//   * QK^T runs on MFMA with the 16 heads as the N=16 side: s^T = K * Q^T,
//     Q held in registers as the B operand.  bf16 x bf16 and bf16 x fp8 (fp8
//     widened exactly to bf16) use v_mfma_f32_16x16x32_bf16; fp8 x fp8 and
//     mxfp4 x mxfp4 use v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales for
//     fp8, the e8m0 block scales for mxfp4); bf16 Q over mxfp4 K runs as an
//     exact pair of fp8 operands on the same instruction.
//   * Online softmax in the log2 domain.  The QK accumulator layout puts one
//     head per lane, so the running max / sum are per-lane scalars and the
//     P tile is already the B operand of P*V (no LDS round trip).
//   * P*V as O^T = V^T * P^T on v_mfma_f32_16x16x32_bf16, V taken from the
//     SAME staged tile (no second HBM read): transposing LDS reads
//     (ds_read_b64_tr_b16 / _b8) for bf16 / fp8, per-token e2m1->bf16
//     conversion plus register shuffles for mxfp4.
//   * The waves merge their (max, sum, O) through LDS at the end; S == 1
//     writes bf16 out directly, otherwise fp32 partial O / base-2 LSE.
//   * Split cache (page 695854's mxfp4 q=1 routes): K from the mxfp4 cache and
//     V from the first 512 dims of an fp8 cache on the same rows.  Both rows
//     of a token are staged into one slot; QK^T runs as for mxfp4 and P*V as
//     for fp8.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "mla_decode.h"

namespace {

constexpr int kHeads = 16;
constexpr int kDqk = 576;
constexpr int kDv = 512;
// Waves per stage-1 workgroup: four, or two when the grid has more
// workgroups than the chip has CUs -- two such workgroups then share a CU
// (each fits half its LDS) and the grid runs in one round instead of two.
constexpr int kMaxWaves = 4;
constexpr int kSub = 32;  // tokens per wave sub-tile

constexpr int FBF16 = MLA_DTYPE_BF16;
constexpr int FFP8 = MLA_DTYPE_FP8_E4M3FN;
constexpr int FMX = MLA_DTYPE_MXFP4;
constexpr int FMIX = MLA_KV_MXFP4_K_FP8_V;  // mxfp4 K + fp8 V, two caches
constexpr int FQ8S = MLA_Q_BF16_FP8_STATIC;  // bf16 Q, quantised to fp8 in the prologue
constexpr int FQ4 = MLA_Q_BF16_MXFP4;        // bf16 Q, quantised to mxfp4 in the prologue

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(8))) unsigned u32x8_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) short i16x2_t;
typedef __attribute__((address_space(3))) char lds_char;

// ------------------------------------------------------------------ layout
// Per-format cache row geometry and ring depth.
template <int KF> struct Kv;
template <> struct Kv<FBF16> {
  static constexpr int kRow = 2 * kDqk;  // bytes per cache row
  static constexpr int kUnits = kRow / 16;
  static constexpr int kNdmaX4 = kUnits / 2;  // 64 lanes x 16 B = 2 units of 32 tokens
  static constexpr int kNdmaSc = 0;
  static constexpr int kNbuf = 1;
};
template <> struct Kv<FFP8> {
  static constexpr int kRow = kDqk;
  static constexpr int kUnits = kRow / 16;
  static constexpr int kNdmaX4 = kUnits / 2;
  static constexpr int kNdmaSc = 0;
  static constexpr int kNbuf = 2;
};
template <> struct Kv<FMX> {
  static constexpr int kRow = MLA_MXFP4_ROW_BYTES;
  static constexpr int kUnits = kRow / 16;
  static constexpr int kNdmaX4 = kUnits / 2;
  static constexpr int kNdmaSc = 3;  // 32 tokens x 5 aligned dwords = 160 lanes
  static constexpr int kNbuf = 3;
};
// Split cache: a slot holds the 32 tokens' mxfp4 K rows (18 units each, as
// for mxfp4) followed by their fp8 V rows cut to the 512 value dims (32
// units each); one slot per wave fits the LDS.
template <> struct Kv<FMIX> {
  static constexpr int kRow = MLA_MXFP4_ROW_BYTES;  // K cache row; V rows are 576 B
  static constexpr int kUnitsK = kRow / 16;
  static constexpr int kUnitsV = kDv / 16;
  static constexpr int kUnits = kUnitsK + kUnitsV;
  static constexpr int kNdmaK = kUnitsK / 2;
  static constexpr int kNdmaX4 = kUnits / 2;
  static constexpr int kNdmaSc = 3;
  static constexpr int kNbuf = 1;
};

template <int KF, int kWaves = kMaxWaves> struct Lay {
  static constexpr int kNbuf = Kv<KF>::kNbuf;
  static constexpr int kSlot = Kv<KF>::kUnits * 512;           // 32 tokens x row
  static constexpr int kScSlot = Kv<KF>::kNdmaSc ? 768 : 0;     // 3 x 64 dwords
  static constexpr int kParSlot = Kv<KF>::kNdmaSc ? 16 : 0;     // row parity bit per token (one word, padded)
  static constexpr int kD = kNbuf > 1 ? kNbuf - 1 : 1;          // page-id prefetch distance
  // page-id ring: a power of two >= kD + 1, so the ring index is a mask
  static constexpr int kNpid = kD + 1 <= 2 ? 2 : 4;
  static constexpr int kPidSlot = 256;                          // 64 lanes x 4 B
  static constexpr int kScOff = kNbuf * kSlot;
  static constexpr int kParOff = kScOff + kNbuf * kScSlot;
  static constexpr int kPidOff = kParOff + kNbuf * kParSlot;
  static constexpr int kRowOff = kPidOff + kNpid * kPidSlot;       // physical row per token (u32)
  static constexpr int kPtrOff = kRowOff + 4 * kSub;                // row base address per token (u64)
  // split cache: the V rows' base addresses follow the K rows'
  static constexpr int kPtrBytes = (KF == FMIX ? 2 : 1) * 8 * kSub;
  static constexpr int kWaveBytes = kPtrOff + kPtrBytes;
  static constexpr int kCombine = kWaves * 32768 + 2 * kWaves * kHeads * 4;  // per-wave O^T + (m, l)
  static constexpr int kTotal = kWaves * kWaveBytes > kCombine ? kWaves * kWaveBytes : kCombine;
  static constexpr int kNdma = Kv<KF>::kNdmaX4 + Kv<KF>::kNdmaSc;  // VMEM instrs per sub-tile
  // every region starts 16-byte aligned: the DMA writes and the row-pointer
  // table need it
  static_assert(kSlot % 16 == 0 && kScOff % 16 == 0 && kParOff % 16 == 0 && kPidOff % 16 == 0 &&
                    kRowOff % 16 == 0 && kPtrOff % 16 == 0 && kWaveBytes % 16 == 0,
                "per-wave LDS regions must stay 16-byte aligned");
};

// A sub-tile is stored as its row-major byte stream: token t's 16-byte unit k
// sits in LDS chunk t*U + (k ^ tswz(t)).  The swizzle only flips the two low
// bits of the unit index with bits of the token index; U is a multiple of 4
// for bf16/fp8, so the map stays inside each token's row and is an
// involution, and the DMA instruction that fills chunks 64i..64i+63 still
// reads 1 KB of consecutive stream bytes.  The token bits were chosen by an
// exhaustive search over a 64-bank model so that the QK fragment reads
// (8 tokens, one unit), the transposing P*V reads and the mxfp4 block reads
// all hit distinct banks; mxfp4 needs no swizzle (U = 18).
template <int KF>
__device__ __forceinline__ int tswz(int t) {
  if constexpr (KF == FFP8) return (((t >> 2) ^ (t >> 4)) & 1) << 1;
  else if constexpr (KF == FBF16) return ((t >> 2) & 1) | (((t >> 1) & 1) << 1);
  else return 0;
}
// The split cache's V rows are 32 units (512 B) long, so every token's unit k
// falls in the same bank group; flipping the three low unit bits with token
// bits 0, 1 and 4 gives the eight tokens of one transposing-read phase
// (4g..4g+3, 16+4g..16+4g+3) eight different groups.
__device__ __forceinline__ int vswz(int t) { return (t & 3) | (((t >> 4) & 1) << 2); }

// ------------------------------------------------------------- primitives
template <class T>
__device__ __forceinline__ T lds_ld(int off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(static_cast<uintptr_t>(off));
}
template <class T>
__device__ __forceinline__ void lds_st(int off, T v) {
  *reinterpret_cast<__attribute__((address_space(3))) T*>(static_cast<uintptr_t>(off)) = v;
}

// Direct-to-LDS loads.  LDS address = m0 + 16*lane (x4) or m0 + 4*lane (dword).
// Cache rows are read exactly once, so the 16-byte stream loads carry the
// non-temporal policy bit.
__device__ __forceinline__ void dma_x4_nt(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"(__builtin_amdgcn_readfirstlane(m0))
               : "memory");
}
__device__ __forceinline__ void dma_b32(const void* g, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(__builtin_amdgcn_readfirstlane(m0))
               : "memory");
}
// Partial results (fp32 O rows and base-2 LSEs) are read back by the
// combine kernel, on any XCD.  kPol is the store's cache-policy operand:
// kCpolDev (sc1, device scope) writes them through the L2, so that none are
// left dirty in it for the write-back at the end of the launch.
constexpr int kCpolDev = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}
template <int kPol>
__device__ __forceinline__ void st_pol(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, static_cast<int>(off), 0, kPol);
}
template <int kPol>
__device__ __forceinline__ void st_pol(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(off), 0, kPol);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }
// Compiler-only fence: LDS reads issued above it cannot be sunk below it, so
// a batch of fragment reads is in flight together instead of one at a time.
__device__ __forceinline__ void sched_fence() { asm volatile("" : : : "memory"); }
// Pin eight fragments: their loads must have completed here (the compiler
// waits for exactly these), later reads stay below and in flight, and the
// consumers of the values cannot be hoisted above.
template <class T>
__device__ __forceinline__ void pin2(T& a, T& b) {
  asm volatile("" : "+v"(a), "+v"(b) : : "memory");
}
// Keep eight accumulator tiles in AGPRs at this point.  The O accumulator is
// only touched by MFMA except in the rare rescale branch; without this the
// loop-carried value is kept in VGPRs and copied both ways every iteration.
template <class T>
__device__ __forceinline__ void pin_acc8(T* v) {
  asm volatile("" : "+a"(v[0]), "+a"(v[1]), "+a"(v[2]), "+a"(v[3]), "+a"(v[4]), "+a"(v[5]), "+a"(v[6]), "+a"(v[7]));
}
template <class T>
__device__ __forceinline__ void pin8(T* v) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
               :
               : "memory");
}


// 2^(e-127), exact for every code including e = 0 (a denormal): one ldexp
// of the constant 2^-127
__device__ __forceinline__ float e8m0_f32(uint32_t e) {
  return __builtin_amdgcn_ldexpf(0x1p-127f, static_cast<int>(e));
}

__device__ __forceinline__ uint32_t bits(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }

// Exact two-term fp8 form of one lane's 32 bf16 values of a QK MFMA B
// operand: x = hi * 2^(s-127) + lo * 2^(s'-127), s and s' the e8m0 scales of
// x's scale block.  In the 8-bit operand of the 16x16x128 f8f6f4 MFMA, byte
// half h (16 values) of lane group g belongs to scale block 2h + (g >> 1),
// shared with the partner group g ^ 1, and lane group g supplies the scale of
// block g.  hi carries the leading four significant bits of x (RNE to e4m3),
// lo the rest: a bf16 significand has eight bits, so both terms are exact for
// every element within 2^13 of its block maximum (both stay in the e4m3
// normal range); smaller elements keep an absolute resolution of 2^-13 times
// the block maximum.  The hi scale puts the block maximum in [128, 256).
// raw[0..1] hold the 16 values of half 0, raw[2..3] those of half 1.
__device__ __forceinline__ void split_q_fp8(const u32x4_t raw[4], int g, i32x8_t& hi, i32x8_t& lo, uint32_t& sh,
                                            uint32_t& sl) {
  float x[32];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * j + 2 * e] = __uint_as_float(raw[j][e] << 16);
      x[8 * j + 2 * e + 1] = __uint_as_float(raw[j][e] & 0xffff0000u);
    }
  float am[2] = {0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 32; ++i) am[i >> 4] = fmaxf(am[i >> 4], fabsf(x[i]));
  int eh[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float bm = fmaxf(am[h], __shfl_xor(am[h], 16));  // block max over the lane pair
    eh[h] = max(static_cast<int>((__float_as_uint(bm) >> 23) & 0xffu) - 127 - 7, -127);
  }
  u32x8_t hv, lv;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int h = k >> 2;
    const int el = max(eh[h] - 4, -127);
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - eh[h]) << 23);     // 2^-eh
    const float up = __uint_as_float(static_cast<uint32_t>(127 + eh[h] - el) << 23);  // 2^(eh-el)
    const float a0 = x[4 * k] * inv, a1 = x[4 * k + 1] * inv, a2 = x[4 * k + 2] * inv, a3 = x[4 * k + 3] * inv;
    // the scalef32 converters use the OCP e4m3 encoding the f8f6f4 MFMA reads
    i16x2_t ph = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, a0, a1, 1.0f, false);
    ph = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(ph, a2, a3, 1.0f, true);
    const int phi = __builtin_bit_cast(int, ph);
    const f32x2_t d01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(phi, 1.0f, false);
    const f32x2_t d23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(phi, 1.0f, true);
    i16x2_t pl = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, (a0 - d01[0]) * up, (a1 - d01[1]) * up,
                                                          1.0f, false);
    pl = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pl, (a2 - d23[0]) * up, (a3 - d23[1]) * up, 1.0f, true);
    hv[k] = static_cast<uint32_t>(phi);
    lv[k] = __builtin_bit_cast(uint32_t, pl);
  }
  hi = __builtin_bit_cast(i32x8_t, hv);
  lo = __builtin_bit_cast(i32x8_t, lv);
  // lane group g supplies block g = (half g >> 1 of pair g & 1): groups 0 and 3
  // hold it themselves, groups 1 and 2 swap
  const int send = g == 2 ? eh[0] : eh[1];
  const int ln = __lane_id();
  const int got = __shfl(send, g == 1 ? ln + 16 : g == 2 ? ln - 16 : ln);
  const int e_blk = g == 0 ? eh[0] : g == 3 ? eh[1] : got;
  sh = static_cast<uint32_t>(e_blk + 127);
  sl = static_cast<uint32_t>(max(e_blk - 4, -127) + 127);
}

// bf16 pair (lo = low half of x, hi = low half of y) and the same for high
// halves: one byte permute each (v_perm_b32 indexes bytes 0-3 of its second
// operand and 4-7 of its first)
__device__ __forceinline__ uint32_t lo_pair(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }

__device__ __forceinline__ bf16x8_t cvt_fp8x8(i32x2_t v) {
  u32x4_t r;
  r.x = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false));
  r.y = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true));
  r.z = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false));
  r.w = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true));
  return __builtin_bit_cast(bf16x8_t, r);
}
// eight e2m1 codes (one dword) times a block scale -> 8 bf16
__device__ __forceinline__ bf16x8_t cvt_fp4x8(uint32_t v, float sc) {
  u32x4_t r;
  r.x = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 0));
  r.y = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 1));
  r.z = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 2));
  r.w = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 3));
  return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_fp8(i32x8_t a, i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// e2m1 K with its block scales x fp8 Q with its block scales
__device__ __forceinline__ f32x4_t mfma_fp4_fp8(i32x4_t a, uint32_t sa, i32x8_t b, uint32_t sb, f32x4_t c) {
  i32x8_t A = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, b, c, 4, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ f32x4_t mfma_fp4(i32x4_t a, uint32_t sa, i32x4_t b, uint32_t sb, f32x4_t c) {
  i32x8_t A = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  i32x8_t B = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, sa, 0, sb);
}

__device__ __forceinline__ float fmax3(float a, float b) { return a > b ? a : b; }
// bit t of pm (t < 32), kept opaque so that the caller's doubling stays a
// v_lshl_add: the compiler otherwise folds (pm >> t) & 1 feeding a shifted
// add into three instructions in place of v_bfe_u32 + v_lshl_add_u32
__device__ __forceinline__ uint32_t bit_of(uint32_t pm, int t) {
  uint32_t b = (pm >> t) & 1u;
  asm("" : "+v"(b));
  return b;
}
// three- and two-input maxima of values that are never NaN (logits and
// -inf), as one instruction each: written out because fmaxf would first quiet
// each input and a select compiles to a compare, a hazard wait and a cndmask
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Reductions over the four 16-lane groups (lanes l, l^16, l^32, l^48) with
// gfx950's cross-row swaps: VALU-only, no LDS round trip.
__device__ __forceinline__ float group_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = vmax2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax2(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// The softmax reference max is moved only when a logit exceeds it by more
// than this many binades (base-2 log domain), bounding every weight by 2^8.
constexpr float kLazy = 8.0f;

// ------------------------------------------------------------- arguments
struct Stage1Args {
  const void* q;
  const void* q_scale;
  const char* kv;
  const void* kv_scale;
  const char* kv2;        // split cache: fp8 V rows (576 B, dims 0..511 read), else NULL
  const float* kv2_scale;  // split cache: the V cache's per-tensor scale
  const int32_t* kv_indptr;
  const int32_t* page_table;
  const int32_t* page_indptr;
  float* part_o;
  float* part_lse;
  uint16_t* out;
  const int32_t* items;  // work-list plan (int32[num_items][4]), or NULL: split grid
  int32_t batch;
  int32_t groups;        // 16-row query groups per request (q_seq_len x heads / 16)
  int32_t units;         // (request, split) pairs or work items
  int32_t page_size;
  int32_t num_splits;
  uint32_t max_row;      // last physical cache row: gathered rows are clamped to it
  float sm_scale_log2e;
};

// Number of QK MFMA "B operands" (Q fragments) a lane holds, per format pair.
// The static-scale fp8 quantiser of bf16 Q, on one lane's 32 values of a QK
// B operand (raw[0..3], eight bf16 each, in dimension order) into their 32
// e4m3fn codes: each code is the nearest e4m3fn value (ties to even) to the
// fp32 quotient x / s clamped to +-448, the per-element rule of the fp8
// quantiser of page 668813 that mla_quantize_fp8 implements.  With
// r = 1/s correctly rounded, q0 = x r, e = x - q0 s (exact, one fma) and
// q0 + e r (one fma) is the correctly rounded quotient (Markstein's
// reciprocal-based division) when nothing overflows or underflows; x is
// clamped first to +-896 s, beyond which the clamped result is 448 anyway,
// and the sign is copied from x so that -0 stays -0.  On MI355X the codes
// matched those of x / s and the software encoder of mla_quantize_fp8 for
// every finite bf16 x under 4,000 scales spread over [2^-60, 2^60], and the
// hardware e4m3 encoder matched the software one for every fp32 of
// magnitude <= 448.  Scales outside that range take the division itself
// (kExact).
template <bool kExact>
__device__ __forceinline__ i32x8_t quant_q_fp8(const u32x4_t raw[4], float s, float r) {
  const float bnd = 896.0f * s;
  u32x8_t out;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t u = raw[w >> 1][2 * (w & 1) + (k >> 1)];
      const float x = __uint_as_float((k & 1) ? (u & 0xffff0000u) : (u << 16));
      float y;
      if constexpr (kExact) {
        y = x / s;
      } else {
        const float xc = __builtin_amdgcn_fmed3f(x, -bnd, bnd);
        const float q0 = xc * r;
        y = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, xc), r, q0), x);
      }
      q[k] = __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f);
    }
    i16x2_t p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(i16x2_t{0, 0}, q[0], q[1], 1.0f, false);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, q[2], q[3], 1.0f, true);
    out[w] = __builtin_bit_cast(uint32_t, p);
  }
  return __builtin_bit_cast(i32x8_t, out);
}

// The mxfp4 quantiser of bf16 Q on one lane's 32-element block (raw[0..3],
// eight bf16 each, in element order): the rule of mla_quantize_mxfp4 (shared
// exponent X = floor(log2 amax) - 2 clamped to [-127, 127], e8m0 = X + 127,
// an all-zero block X = -127; code = nearest e2m1 value, ties to even,
// saturating at 6, of v * 2^-X; element 2i in the low nibble of byte i).
// v * 2^-X is ldexp(v, -X) exactly: for bf16 amax, X <= 125, so 2^-X is a
// normal float and the product is exact or, when subnormal, rounded as
// ldexp rounds.  On MI355X the hardware e2m1 encoder (scale 1) matched the
// software encoder of mla_quantize_mxfp4 for every non-NaN fp32, and this
// routine matched it on 2^20 random and special blocks.
__device__ __forceinline__ void quant_q_mxfp4(const u32x4_t raw[4], i32x4_t& codes, uint32_t& e8) {
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * i + 2 * k] = __uint_as_float(raw[i][k] << 16);
      v[8 * i + 2 * k + 1] = __uint_as_float(raw[i][k] & 0xffff0000u);
    }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float a = __builtin_fabsf(v[i]);
    amax = a > amax ? a : amax;  // NaN compares false and is skipped
  }
  int X = amax == 0.0f ? -127 : __builtin_amdgcn_frexp_expf(amax) - 3;
  X = X < -127 ? -127 : (X > 126 ? 126 : X);
  e8 = static_cast<uint32_t>(X + 127);
  const float f = __uint_as_float(static_cast<uint32_t>(127 - X) << 23);  // 2^-X
  u32x4_t w;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t d = 0;
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[8 * k + 0] * f, v[8 * k + 1] * f, 1.0f, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[8 * k + 2] * f, v[8 * k + 3] * f, 1.0f, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[8 * k + 4] * f, v[8 * k + 5] * f, 1.0f, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[8 * k + 6] * f, v[8 * k + 7] * f, 1.0f, 3);
    w[k] = d;
  }
  codes = __builtin_bit_cast(i32x4_t, w);
}

template <int QF, int KF> struct QFrag;
template <> struct QFrag<FBF16, FBF16> { static constexpr int kN = 18; };
template <> struct QFrag<FBF16, FFP8> { static constexpr int kN = 18; };
template <> struct QFrag<FBF16, FMX> { static constexpr int kN = 5; };  // hi/lo fp8 pairs
template <> struct QFrag<FFP8, FFP8> { static constexpr int kN = 5; };
template <> struct QFrag<FQ8S, FFP8> { static constexpr int kN = 5; };
template <> struct QFrag<FQ4, FMX> { static constexpr int kN = 5; };
template <> struct QFrag<FMX, FMX> { static constexpr int kN = 5; };
template <> struct QFrag<FBF16, FMIX> { static constexpr int kN = 5; };
template <> struct QFrag<FMX, FMIX> { static constexpr int kN = 5; };

// First latent dim of the 8 bf16 values that QK MFMA m takes from lane group g,
// for bf16 Q (the permutation mirrors how the K operand is read from LDS).
template <int KF>
__device__ __forceinline__ int qdim_bf16(int m, int g) {
  if constexpr (KF == FBF16) return 32 * m + 8 * g;
  else if constexpr (KF == FFP8) return 64 * (m >> 1) + 16 * g + 8 * (m & 1);
  else return m < 16 ? 128 * (m >> 2) + 32 * g + 8 * (m & 3) : 512 + 32 * (m - 16) + 8 * g;
}

// ------------------------------------------------------------------ stage 1
template <int QF, int KF, int kWaves>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void stage1_kernel(Stage1Args a) {
  static_assert(kWaves == 2 || kWaves == 4, "two or four waves");
  using L = Lay<KF, kWaves>;
  // two-wave workgroups must fit two to a CU
  static_assert(kWaves == 4 || 2 * L::kTotal <= 160 * 1024, "LDS of two workgroups exceeds a CU");
  constexpr int NBUF = L::kNbuf;
  constexpr int D = L::kD;
  constexpr int NDMA = L::kNdma;
  constexpr int ROW = Kv<KF>::kRow;
  // bf16 Q quantised in the prologue: each wave quantises some of the five
  // B-operand chunks and they meet in LDS past the rings - fp8 with four
  // waves (10 KB; the 151 KB fp8 layout plus this still fits a CU), mxfp4
  // with either wave count (6.25 KB of codes and scales)
  constexpr bool kShareQ = (QF == FQ8S && kWaves == 4) || QF == FQ4;
  constexpr int kQxBytes = !kShareQ ? 0 : QF == FQ8S ? 5 * 64 * 32 : 5 * 64 * 20;
  __shared__ __attribute__((aligned(1024))) char smem[L::kTotal + kQxBytes];
  static_assert((kWaves == 4 ? 1 : 2) * (L::kTotal + kQxBytes) <= 160 * 1024, "LDS of one CU exceeded");
  const uint32_t smem0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_char*)smem));

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // MFMA lane group
  const int hq = lane & 15;  // head (QK / PV output column of the 16-wide side)
  const int S = a.num_splits;
  // work decomposition: workgroup = (request, split) of a uniform split grid,
  // or one item {request, first token, tokens, slot} of a work-list plan,
  // times the request's G 16-row query groups.  Workgroups are dealt to the
  // eight XCDs round-robin by index, so with G > 1 the G groups of a unit
  // get indices congruent mod 8: they run on one XCD, close together, and
  // re-read the unit's tokens from that XCD's L2.  The grid is padded to a
  // multiple of 8G; padding workgroups leave at once.
  const int G = a.groups;
  int b, s = 0, slot = -1, it_t0 = 0, it_n = 0;
  int unit, r;
  if (G == 1) {
    unit = blockIdx.x;
    r = 0;
  } else {
    const int k = blockIdx.x >> 3;
    unit = 8 * (k / G) + (blockIdx.x & 7);
    r = k - (k / G) * G;
    if (unit >= a.units) return;
  }
  if (a.items) {
    const int32_t* it = a.items + 4 * unit;
    b = min(max(it[0], 0), a.batch - 1);
    it_t0 = it[1];
    it_n = it[2];
    slot = it[3];
  } else {
    b = unit / S;
    s = unit - b * S;
  }
  const int v = b * G + r;  // query group: Q and output rows 16v .. 16v + 15

  // ---- Q fragments (B operands) for this lane's head.  Issued first: they
  // depend on the request index only, so their latency overlaps the
  // kv_indptr load and the page-id gathers that follow.
  constexpr int NQ = QFrag<QF, KF>::kN;
  // bf16 Q over the mxfp4 cache runs QK on the scaled f8f6f4 MFMA with Q as
  // an exact hi + lo pair of fp8 operands (split_q_fp8), so the e2m1 K needs
  // no conversion; raw bf16 blocks are held until the loads have landed.  The
  // split costs a few microseconds per wave (the fp8 encoder is a slow
  // instruction), which only the long, compute-bound mxfp4 splits repay; over
  // the fp8 cache, K is widened to bf16 instead (full-rate converts).
  constexpr bool kMxK = KF == FMX || KF == FMIX;  // K from an mxfp4 cache
  constexpr bool kSplitQ = QF == FBF16 && kMxK;
  // bf16 Q quantised here to fp8 with a static scale: raw bf16 fragments are
  // held until the loads have landed, then the rest is the fp8-Q kernel
  constexpr bool kQuantQ = QF == FQ8S;
  // bf16 Q quantised here to mxfp4 (per-block scales): likewise
  constexpr bool kQuantQ4 = QF == FQ4;
  constexpr int QFE = kQuantQ ? FFP8 : kQuantQ4 ? FMX : QF;  // the Q format the loop computes with
  bf16x8_t qb[QF == FBF16 && !kSplitQ ? NQ : 1];
  u32x4_t qraw[kSplitQ || kQuantQ || kQuantQ4 ? 4 * NQ : 1];
  i32x8_t q8[QFE == FFP8 || kSplitQ ? NQ : 1];
  i32x8_t ql[kSplitQ ? NQ : 1];
  uint32_t qhs[kSplitQ ? NQ : 1], qls[kSplitQ ? NQ : 1];
  i32x4_t q4[QFE == FMX ? NQ : 1];
  uint32_t q4s[QFE == FMX ? NQ : 1];
  float qs = 1.0f, ks = 1.0f;
  if constexpr (kSplitQ) {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (static_cast<size_t>(v) * kHeads + hq) * kDqk;
#pragma unroll
    for (int c = 0; c < NQ; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // the 4-bit K operand is contiguous per lane group (dims 128c + 32g +
        // [0, 32)), the 8-bit one puts byte half h of lane group g at K
        // position 64h + 16g: half h = j >> 1 takes dims 128c + 64h + 16g + [0, 16)
        const int d = 128 * c + 64 * (j >> 1) + 16 * g + 8 * (j & 1);
        qraw[4 * c + j] = u32x4_t{0u, 0u, 0u, 0u};
        if (d < kDqk) qraw[4 * c + j] = *reinterpret_cast<const u32x4_t*>(qrow + d);
      }
  } else if constexpr (kQuantQ || kQuantQ4) {
    // the fp8 B operand of chunk c holds dims 128c + 32g + [0, 32) in order,
    // as does the mxfp4 one (one 32-element block per lane); chunk 4: dims
    // 512 + 32g + [0, 32) for g < 2, zeros otherwise.  Where the waves share
    // the work a wave loads only the chunks it quantises (c mod waves = w).
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (static_cast<size_t>(v) * kHeads + hq) * kDqk;
#pragma unroll
    for (int c = 0; c < NQ; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 128 * c + 32 * g + 8 * j;
        qraw[4 * c + j] = u32x4_t{0u, 0u, 0u, 0u};
        if (d < kDqk && (!kShareQ || c % kWaves == w)) qraw[4 * c + j] = *reinterpret_cast<const u32x4_t*>(qrow + d);
      }
  }
  // Over the bf16 cache, Q is loaded after the first tiles' DMAs are issued
  // (below): Q does not feed the gather chain (kv_indptr -> page ids ->
  // tiles), and a wait for the page ids also waits for every load issued
  // before them (loads complete in issue order), so loading Q late lets its
  // latency overlap the 36 KB tiles' instead of delaying the page-id wait.
  // The smaller fp8 and mxfp4 tiles arrive before a late Q would (measured
  // 0.5 - 1.5 us slower there), so those formats load Q first, beside the
  // kv_indptr -> page-id chain.
  constexpr bool kLateQ = KF == FBF16;
  auto load_q = [&]() {
  if constexpr (kSplitQ || kQuantQ || kQuantQ4) {
  } else if constexpr (QF == FBF16) {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (static_cast<size_t>(v) * kHeads + hq) * kDqk;
#pragma unroll
    for (int m = 0; m < NQ; ++m) qb[m] = *reinterpret_cast<const bf16x8_t*>(qrow + qdim_bf16<KF>(m, g));
  } else if constexpr (QF == FFP8) {
    const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + (static_cast<size_t>(v) * kHeads + hq) * kDqk;
#pragma unroll
    for (int c = 0; c < 4; ++c) q8[c] = *reinterpret_cast<const i32x8_t*>(qrow + 128 * c + 32 * g);
    q8[4] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    if (g < 2) q8[4] = *reinterpret_cast<const i32x8_t*>(qrow + 512 + 32 * g);
  } else {
    const size_t qr = static_cast<size_t>(v) * kHeads + hq;
    const uint8_t* qrow = static_cast<const uint8_t*>(a.q) + qr * MLA_MXFP4_ROW_BYTES;
    const uint8_t* qsc = static_cast<const uint8_t*>(a.q_scale) + qr * MLA_MXFP4_ROW_SCALES;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      q4[c] = *reinterpret_cast<const i32x4_t*>(qrow + 64 * c + 16 * g);
      q4s[c] = qsc[4 * c + g];
    }
    q4[4] = i32x4_t{0, 0, 0, 0};
    q4s[4] = 127u;
    if (g < 2) {
      q4[4] = *reinterpret_cast<const i32x4_t*>(qrow + 256 + 16 * g);
      q4s[4] = qsc[16 + g];
    }
  }
  };
  // The compiler waits for the Q loads at these pins (everything issued
  // before them completes first), so no explicit vmcnt wait of the pipeline
  // below ever counts a Q load.
  auto pin_q = [&]() {
  if constexpr (QF == FBF16 && !kSplitQ) {
#pragma unroll
    for (int m = 0; m < NQ; ++m) asm volatile("" : "+v"(qb[m]));
  } else if constexpr (QF == FFP8) {
#pragma unroll
    for (int m = 0; m < NQ; ++m) asm volatile("" : "+v"(q8[m]));
  } else if constexpr (QF == FMX) {
#pragma unroll
    for (int m = 0; m < NQ; ++m) asm volatile("" : "+v"(q4[m]), "+v"(q4s[m]));
  }
  };
  if constexpr (!kLateQ) load_q();
  if constexpr (QFE == FFP8) qs = *static_cast<const float*>(a.q_scale);
  if constexpr (KF == FFP8) ks = *static_cast<const float*>(a.kv_scale);
  float vs = 1.0f;  // split cache: V scale, applied with the final division
  if constexpr (KF == FMIX) vs = *a.kv2_scale;
  const int kv0 = a.kv_indptr[b];
  const int Lr = a.kv_indptr[b + 1] - kv0;
  int t0, n;  // first token and token count of this workgroup's range
  if (a.items) {
    // clamped to the request, so a plan that disagrees with kv_indptr still
    // only touches this request's pages
    t0 = max(0, min(it_t0, Lr));
    n = max(0, min(it_n, Lr - t0));
  } else {
    const int chunk = (Lr + S - 1) / S;
    t0 = s * chunk;
    n = max(0, min(chunk, Lr - t0));
  }
  const int nsub = (n + kSub - 1) / kSub;
  const int nloc = w < nsub ? (nsub - w + kWaves - 1) / kWaves : 0;
  const uint32_t gbase = a.page_indptr ? static_cast<uint32_t>(t0) : static_cast<uint32_t>(kv0 + t0);
  const int32_t* ptab = a.page_table + (a.page_indptr ? a.page_indptr[b] : 0);
  const uint32_t P = static_cast<uint32_t>(a.page_size);
  // page index and slot of a stream position: shifts for power-of-two page
  // sizes (wave-uniform branch), a division otherwise
  const int plog = (P & (P - 1u)) == 0u ? __builtin_ctz(P) : -1;
  // (the opaque copy of P keeps the compiler from hoisting the division's
  // reciprocal out of the loop and then computing both forms every sub-tile)
  auto page_of = [&](uint32_t gp) -> uint32_t {
    if (plog >= 0) return gp >> plog;
    uint32_t p = P;
    asm volatile("" : "+s"(p));
    return gp / p;
  };
  auto slot_of = [&](uint32_t gp) -> uint32_t {
    if (plog >= 0) return gp & (P - 1u);
    uint32_t p = P;
    asm volatile("" : "+s"(p));
    return gp % p;
  };

  // ---- per-wave LDS ring
  const uint32_t wbase = smem0 + static_cast<uint32_t>(w) * L::kWaveBytes;
  auto slot_addr = [&](int x) { return wbase + static_cast<uint32_t>(x) * L::kSlot; };
  auto sc_addr = [&](int x) { return wbase + L::kScOff + static_cast<uint32_t>(x) * L::kScSlot; };
  auto par_addr = [&](int x) { return wbase + L::kParOff + static_cast<uint32_t>(x) * L::kParSlot; };
  auto pid_addr = [&](int y) { return wbase + L::kPidOff + static_cast<uint32_t>(y & (L::kNpid - 1)) * L::kPidSlot; };


  auto issue_pid = [&](int X) {
    const int xc = X < nloc ? X : (nloc > 0 ? nloc - 1 : 0);
    const int tok = min(kSub * (w + kWaves * xc) + (lane & 31), max(n - 1, 0));
    const uint32_t gpos = gbase + static_cast<uint32_t>(tok);
    dma_b32(ptab + page_of(gpos), pid_addr(X));
  };
  constexpr int U = Kv<KF>::kUnits;
  // Per DMA instruction i, this lane fills LDS chunk 64i + lane = token t,
  // stored unit k (stream unit k ^ tswz(t)), packed as (8t << 16) | 16*(stream
  // unit): the row-pointer table offset and the byte offset inside the row.
  // The split cache (25), fp8 (18) and mxfp4 (9 per lane) keep these in
  // registers; bf16 rows (36 instructions) recompute them from an opaque lane
  // index each sub-tile: 36 more live registers beside its 18 Q fragments
  // made the compiler spill inside the loop.
  constexpr bool kPre = Kv<KF>::kNdmaX4 <= 25;
  auto dma_pack = [](int i, int ln) {
    if constexpr (KF == FMIX) {
      // K rows: chunks 64i + ln of an 18-unit row-major stream; V rows: 32
      // units each, unit k stored at k ^ vswz(t), addressed through the
      // second row-pointer table
      constexpr int UK = Kv<FMIX>::kUnitsK, NK = Kv<FMIX>::kNdmaK;
      if (i < NK) {
        const int c = 64 * i + ln;
        const int t = c / UK;
        return ((8 * t) << 16) | (16 * (c - t * UK));
      }
      const int c = 64 * (i - NK) + ln;
      const int t = c >> 5;
      return ((8 * kSub + 8 * t) << 16) | (16 * ((c & 31) ^ vswz(t)));
    } else {
      const int c = 64 * i + ln;
      const int t = c / U;
      return ((8 * t) << 16) | (16 * ((c - t * U) ^ tswz<KF>(t)));
    }
  };
  int dmao[kPre ? Kv<KF>::kNdmaX4 : 1];
#pragma unroll
  for (int i = 0; i < (kPre ? Kv<KF>::kNdmaX4 : 1); ++i) dmao[i] = dma_pack(i, lane);
  // With two slots per wave (fp8), a tile's DMAs are issued in three parts:
  // the first KA right after the slot is freed, the rest interleaved with the
  // next sub-tile's compute.  The address unit accepts a 1 KB direct-to-LDS
  // load about every 16 clocks per CU, so a burst of 18 per wave (x4 waves per CU)
  // would hold the wave at issue for most of a microsecond.
  constexpr bool kSplitDma = NBUF == 2;
  constexpr int KA = kSplitDma ? 6 : Kv<KF>::kNdmaX4;
  constexpr int KB = kSplitDma ? KA + (Kv<KF>::kNdmaX4 - KA) / 2 : Kv<KF>::kNdmaX4;
  // DMAs [I0, I1) of tile X (row-pointer table already written)
  auto issue_part = [&](int X, auto i0c, auto i1c) {
    constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
    if constexpr (I1 > I0) {
      const int pt = static_cast<int>(wbase + L::kPtrOff);
      uint64_t rptr[I1 - I0];
#pragma unroll
      for (int i = I0; i < I1; ++i) rptr[i - I0] = lds_ld<uint64_t>(pt + (dmao[i] >> 16));
#pragma unroll
      for (int i = I0; i < I1; ++i)
        dma_x4_nt(reinterpret_cast<const char*>(rptr[i - I0]) + (dmao[i] & 0xffff), slot_addr(X % NBUF) + 1024u * i);
    }
  };
  // tile X goes to slot x (= X mod NBUF, tracked by the caller: a modulo
  // here would put a subtraction into every LDS address of the slot and keep
  // the compiler from folding the constant offsets)
  auto issue_tile = [&](int X, int x, bool full) {
    wait_lgkm0();  // every LDS read of the slot being refilled has completed
    const int ub = kSub * (w + kWaves * X);
    const int nv = min(kSub, n - ub);
    const int rt = static_cast<int>(wbase + L::kRowOff);
    const int pt = static_cast<int>(wbase + L::kPtrOff);
    // physical row (and its base address) of each of the 32 tokens; tokens
    // past the end repeat the last valid one, so a tail sub-tile stays finite
    // and in bounds
    uint32_t row = 0;
    if (lane < kSub) {
      const int tok = ub + min(lane, nv - 1);
      const uint32_t gpos = gbase + static_cast<uint32_t>(tok);
      const uint32_t pid = static_cast<uint32_t>(lds_ld<int>(static_cast<int>(pid_addr(X)) + 4 * lane));
      // a page id past the cache (a corrupt table) reads the last row rather
      // than memory outside the cache
      row = min(pid * P + slot_of(gpos), a.max_row);
      lds_st<uint32_t>(rt + 4 * lane, row);
      lds_st<uint64_t>(pt + 8 * lane, reinterpret_cast<uint64_t>(a.kv + static_cast<int64_t>(row) * ROW));
      if constexpr (KF == FMIX)
        lds_st<uint64_t>(pt + 8 * kSub + 8 * lane, reinterpret_cast<uint64_t>(a.kv2 + static_cast<int64_t>(row) * kDqk));
    }
    // mxfp4 scale rows are 18 bytes, staged as aligned dwords: bit t of the
    // slot's parity word says token t's row starts 2 bytes into its window
    if constexpr (kMxK) {
      const uint32_t pm = static_cast<uint32_t>(__ballot(lane < kSub && (row & 1u)));
      if (lane == 0) lds_st<uint32_t>(static_cast<int>(par_addr(x)), pm);
    }
    // Row-pointer reads in batches of up to 18 (one LDS latency per batch),
    // each batch followed by its DMA instructions.
    constexpr int NB = Kv<KF>::kNdmaX4 < 18 ? Kv<KF>::kNdmaX4 : 18;
    int lnv = lane;
    if constexpr (!kPre) asm volatile("" : "+v"(lnv));
    auto issue_x4 = [&](int x) {
      if constexpr (kSplitDma) {
        if (full) {
          issue_part(X, std::integral_constant<int, 0>(), std::integral_constant<int, Kv<KF>::kNdmaX4>());
        } else {
          issue_part(X, std::integral_constant<int, 0>(), std::integral_constant<int, KA>());
        }
        return;
      }
#pragma unroll
      for (int i0 = 0; i0 < Kv<KF>::kNdmaX4; i0 += NB) {
        constexpr int NT = Kv<KF>::kNdmaX4;
        uint64_t rptr[NB];
        int off[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          if (i0 + i < NT) {
            if constexpr (kPre) off[i] = dmao[i0 + i];
            else off[i] = dma_pack(i0 + i, lnv);
            rptr[i] = lds_ld<uint64_t>(pt + (off[i] >> 16));
          }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
          if (i0 + i < NT)
            dma_x4_nt(reinterpret_cast<const char*>(rptr[i]) + (off[i] & 0xffff), slot_addr(x) + 1024u * (i0 + i));
      }
    };
    if constexpr (kMxK) {
      const uint8_t* ksc = static_cast<const uint8_t*>(a.kv_scale);
      const uint8_t* sp[3];
#pragma unroll
      for (int i2 = 0; i2 < 3; ++i2) {
        const int d = 64 * i2 + lane;
        const int td = d < 160 ? d / 5 : 0;
        const int sw = d < 160 ? d - 5 * td : 0;
        const int64_t srow = lds_ld<uint32_t>(rt + 4 * td);
        sp[i2] = ksc + ((18 * srow) & ~static_cast<int64_t>(3)) + 4 * sw;
      }
      issue_x4(x);
#pragma unroll
      for (int i2 = 0; i2 < 3; ++i2) dma_b32(sp[i2], sc_addr(x) + 256u * i2);
    } else {
      issue_x4(x);
    }
  };

  // The first page-id gathers (overlapping the Q loads of the formats that
  // issue them first, which one wait covers too).
  if (nloc > 0) {
#pragma unroll
    for (int X = 0; X < D; ++X) issue_pid(X);
  }

  // log2-domain logit scale, kept positive: a zero Q or cache scale then
  // still gives every valid token the same weight (all logits vanish) and
  // masked ones none
  const float c_log2s = fmaxf(a.sm_scale_log2e * qs * ks, 0x1p-126f);
  const float out_mul = KF == FFP8 ? ks : KF == FMIX ? vs : 1.0f;
  // Wait for the page ids and an early Q together, and make the compiler see
  // that Q as complete here, so its own wait for Q cannot drain the
  // in-flight tiles later.
  wait_vm<0>();
  if constexpr (kSplitQ || kQuantQ || kQuantQ4) {
    // split or quantise after the first tile DMAs are issued (below): it
    // then overlaps their latency instead of delaying them
#pragma unroll
    for (int i = 0; i < 4 * NQ; ++i) asm volatile("" : "+v"(qraw[i]));
  } else if constexpr (!kLateQ) {
    pin_q();
  }

  // ---- running softmax state (head hq) and the O^T accumulators
  f32x4_t acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_huge_valf();
  float l_run = 0.0f;

  // Lane-constant LDS offsets used by the reads.
  const int tq0 = hq, tq1 = 16 + hq;  // QK A-operand rows: tokens of tile 0 / 1
  // P*V token slots of this lane group: slot kk <-> token (kk<4 ? 4g+kk : 16+4g+kk-4)
  // pend: tile whose DMAs [KA, 18) are still to be issued (split mode), or -1
  auto compute = [&](int x, int ntok, int pend) {
    const int tb = static_cast<int>(slot_addr(x));
    // mxfp4 scale-row parities of the slot's 32 tokens (one broadcast read)
    uint32_t pmask = 0;
    if constexpr (kMxK) pmask = lds_ld<uint32_t>(static_cast<int>(par_addr(x)));
#pragma unroll
    for (int c = 0; c < 32; c += 8) pin_acc8(acc + c);
    // fp8 V^T fragments for P*V, one transposing read per 16-column tile:
    // lane j of a 16-lane group addresses token T[j/2] (8 B at column 8*(j%2)),
    // T = {4g..4g+3, 16+4g..16+4g+3}; lane i then holds column i of all eight.
    constexpr bool kV8 = KF == FFP8 || KF == FMIX;  // fp8 V
    i32x2_t vv[kV8 ? 32 : 1];
    const int tvj = (lane & 15) >> 1;
    const int tv8 = tvj < 4 ? 4 * g + tvj : 16 + 4 * g + (tvj - 4);
    // unit c of token tv8 sits at chunk NVB(c / NVB) + ((c % NVB) ^ swizzle):
    // NVB lane bases (the swizzle flips the log2(NVB) low bits), the rest is
    // an immediate offset.  The split cache's V rows start after the K rows.
    constexpr int NVB = KF == FMIX ? 8 : 4;
    constexpr int UV = KF == FMIX ? Kv<FMIX>::kUnitsV : U;
    const int tbv = KF == FMIX ? tb + kSub * Kv<FMIX>::kUnitsK * 16 : tb;
    const int vsw = KF == FMIX ? vswz(tv8) : tswz<KF>(tv8);
    int vb[NVB];
#pragma unroll
    for (int r = 0; r < NVB; ++r) vb[r] = tbv + 16 * (tv8 * UV + (r ^ vsw)) + 8 * (lane & 1);
    auto tr8_frag = [&](int c) {
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<__attribute__((address_space(3))) i32x2_t*>(
          static_cast<uintptr_t>(vb[c % NVB] + 16 * NVB * (c / NVB))));
    };
    // QK fragment of token t, unit 4c + g (any unit index of that form keeps
    // the swizzle inside its low two bits); the split cache's K rows are
    // mxfp4 rows of 18 units
    constexpr int UK = KF == FMIX ? Kv<FMIX>::kUnitsK : U;
    const int qb0 = tb + 16 * (tq0 * UK + (g ^ tswz<KF>(tq0)));
    const int qb1 = tb + 16 * (tq1 * UK + (g ^ tswz<KF>(tq1)));
    auto qoff = [&](int t, int c) { return (t == tq0 ? qb0 : qb1) + 64 * c; };
    // ---------------- QK^T: both 16-token tiles at once (two independent
    // accumulator chains), every LDS fragment fetched before the MFMAs run.
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    // A dependent MFMA waits for its predecessor's result, so the K
    // dimension is spread over independent partial accumulators (four or
    // more chains in flight) that are summed once at the end.
    f32x4_t t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KF == FBF16) {
#pragma unroll
      for (int hh2 = 0; hh2 < 2; ++hh2) {
        bf16x8_t k0[9], k1[9];
#pragma unroll
        for (int i = 0; i < 9; ++i) {
          k0[i] = lds_ld<bf16x8_t>(qoff(tq0, 9 * hh2 + i));
          k1[i] = lds_ld<bf16x8_t>(qoff(tq1, 9 * hh2 + i));
        }
        sched_fence();
#pragma unroll
        for (int i = 0; i < 9; ++i) {
          pin2(k0[i], k1[i]);
          if (i & 1) {
            t0 = mfma_bf16(k0[i], qb[9 * hh2 + i], t0);
            t1 = mfma_bf16(k1[i], qb[9 * hh2 + i], t1);
          } else {
            s0 = mfma_bf16(k0[i], qb[9 * hh2 + i], s0);
            s1 = mfma_bf16(k1[i], qb[9 * hh2 + i], s1);
          }
        }
      }
    } else if constexpr (KF == FFP8 && QF == FBF16) {
      i32x4_t k0[9], k1[9];
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        k0[c] = lds_ld<i32x4_t>(qoff(tq0, c));
        k1[c] = lds_ld<i32x4_t>(qoff(tq1, c));
      }
      sched_fence();
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        pin2(k0[c], k1[c]);
        s0 = mfma_bf16(cvt_fp8x8(i32x2_t{k0[c].x, k0[c].y}), qb[2 * c], s0);
        s1 = mfma_bf16(cvt_fp8x8(i32x2_t{k1[c].x, k1[c].y}), qb[2 * c], s1);
        t0 = mfma_bf16(cvt_fp8x8(i32x2_t{k0[c].z, k0[c].w}), qb[2 * c + 1], t0);
        t1 = mfma_bf16(cvt_fp8x8(i32x2_t{k1[c].z, k1[c].w}), qb[2 * c + 1], t1);
      }
    } else if constexpr (KF == FFP8) {  // fp8 x fp8
      i32x8_t a0[5], a1[5];
#pragma unroll
      for (int c = 0; c < 5; ++c) {
        a0[c] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        a1[c] = a0[c];
        if (c < 4 || g < 2) {
          // units 8c + 2g + {0,1}: the swizzle touches only their low two bits
          const int f0 = tswz<KF>(tq0), f1 = tswz<KF>(tq1);
          const i32x4_t u0 = lds_ld<i32x4_t>(tb + 16 * (tq0 * U + 8 * c + ((2 * g) ^ f0)));
          const i32x4_t u1 = lds_ld<i32x4_t>(tb + 16 * (tq0 * U + 8 * c + ((2 * g + 1) ^ f0)));
          const i32x4_t w0 = lds_ld<i32x4_t>(tb + 16 * (tq1 * U + 8 * c + ((2 * g) ^ f1)));
          const i32x4_t w1 = lds_ld<i32x4_t>(tb + 16 * (tq1 * U + 8 * c + ((2 * g + 1) ^ f1)));
          a0[c] = i32x8_t{u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
          a1[c] = i32x8_t{w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        }
      }
      sched_fence();
#pragma unroll
      for (int c = 0; c < 5; ++c) {
        pin2(a0[c], a1[c]);
        if (c & 1) {
          t0 = mfma_fp8(a0[c], q8[c], t0);
          t1 = mfma_fp8(a1[c], q8[c], t1);
        } else {
          s0 = mfma_fp8(a0[c], q8[c], s0);
          s1 = mfma_fp8(a1[c], q8[c], s1);
        }
      }
    } else {  // mxfp4 K: block scales read once per (token, block)
      const int sb0 = static_cast<int>(sc_addr(x)) + 20 * tq0 + 2 * static_cast<int>(bit_of(pmask, tq0));
      const int sb1 = static_cast<int>(sc_addr(x)) + 20 * tq1 + 2 * static_cast<int>(bit_of(pmask, tq1));
      {
        i32x4_t u0[5], u1[5];
        uint32_t c0[5], c1[5];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u0[c] = lds_ld<i32x4_t>(qoff(tq0, c));
          u1[c] = lds_ld<i32x4_t>(qoff(tq1, c));
          c0[c] = lds_ld<uint8_t>(sb0 + 4 * c + g);
          c1[c] = lds_ld<uint8_t>(sb1 + 4 * c + g);
        }
        // dims 576..639 (lane groups 2 and 3 of the fifth chunk) are
        // padding: Q is zero there, and e2m1 codes are always finite, so
        // whatever the LDS holds past the row (the next row, or the wave's
        // scale area after the last slot) adds exactly zero.  Only the block
        // scale must stay finite: 2^0.
        u0[4] = lds_ld<i32x4_t>(tb + 16 * (tq0 * UK + 16 + g));
        u1[4] = lds_ld<i32x4_t>(tb + 16 * (tq1 * UK + 16 + g));
        c0[4] = lds_ld<uint8_t>(sb0 + 16 + g);
        c1[4] = lds_ld<uint8_t>(sb1 + 16 + g);
        if (g >= 2) {
          c0[4] = 127u;
          c1[4] = 127u;
        }
        sched_fence();
        if constexpr (kSplitQ) {
#pragma unroll
          for (int c = 0; c < 5; ++c) {
            // hi and lo terms into one chain per token tile: the two chains
            // alternate, so each 32-cycle MFMA's successor in its chain
            // issues a full MFMA later
            pin2(u0[c], u1[c]);
            s0 = mfma_fp4_fp8(u0[c], c0[c], q8[c], qhs[c], s0);
            s1 = mfma_fp4_fp8(u1[c], c1[c], q8[c], qhs[c], s1);
            s0 = mfma_fp4_fp8(u0[c], c0[c], ql[c], qls[c], s0);
            s1 = mfma_fp4_fp8(u1[c], c1[c], ql[c], qls[c], s1);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 5; ++c) {
            pin2(u0[c], u1[c]);
            if (c & 1) {
              t0 = mfma_fp4(u0[c], c0[c], q4[c], q4s[c], t0);
              t1 = mfma_fp4(u1[c], c1[c], q4[c], q4s[c], t1);
            } else {
              s0 = mfma_fp4(u0[c], c0[c], q4[c], q4s[c], s0);
              s1 = mfma_fp4(u1[c], c1[c], q4[c], q4s[c], s1);
            }
          }
        }
      }
    }
    if constexpr (kSplitDma) {
      if (pend >= 0) issue_part(pend, std::integral_constant<int, KA>(), std::integral_constant<int, KB>());
    }
    if constexpr (!kSplitQ) {  // bf16 Q over mxfp4 K accumulates in one chain per tile
      s0 += t0;
      s1 += t1;
    }
    // the logits are consumed by VALU code: keep them out of the AGPRs that
    // hold the O accumulator
    asm volatile("" : "+v"(s0), "+v"(s1));
    // ---------------- online softmax (log2 domain); lane holds head hq,
    // tokens 4g+r (tile 0) and 16+4g+r (tile 1).  The reference max is only
    // moved when a logit exceeds it by more than 2^kLazy, so the O rescale
    // (all 128 accumulators) runs a handful of times per request; the
    // weights stay <= 2^kLazy and the final division uses the same reference.
    // raw logits: the log2-domain scale c_log2s > 0 is applied to their
    // maximum once and to each logit inside its weight's fma (rounding is
    // monotonic, so the scaled maximum is the maximum of the scaled logits)
    float sv[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = s0[r];
      sv[4 + r] = s1[r];
    }
    if (ntok < kSub) {  // wave-uniform: only a range's last sub-tile is short
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (4 * g + r >= ntok) sv[r] = -__builtin_huge_valf();
        if (16 + 4 * g + r >= ntok) sv[4 + r] = -__builtin_huge_valf();
      }
    }
    float mx = vmax3(vmax3(sv[0], sv[1], sv[2]), vmax3(sv[3], sv[4], sv[5]), vmax2(sv[6], sv[7]));
    mx = group_max(mx) * c_log2s;
#pragma unroll
    for (int c = 0; c < 32; c += 8) pin_acc8(acc + c);
    if (__any(mx > m_run + kLazy)) {
      const float m_new = vmax2(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] *= alpha;
#pragma unroll
      for (int c = 0; c < 32; c += 8) pin_acc8(acc + c);
      m_run = m_new;
    }
    u32x4_t pw;
    float psum = 0.0f;
    const bf16x2_t kOnes2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2_t pr = {static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], c_log2s, -m_run))),
                           static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], c_log2s, -m_run)))};
      // the running sum takes the same bf16-rounded weights the MFMA sees
      psum = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, psum, false);
      pw[i] = bits(pr);
    }
    l_run += psum;
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
    if constexpr (kSplitDma) {
      if (pend >= 0) issue_part(pend, std::integral_constant<int, KB>(), std::integral_constant<int, Kv<KF>::kNdmaX4>());
    }
    // ---------------- P*V
    if constexpr (KF == FBF16) {
      const int j = lane & 15;
      const int kb = (j & 3) >> 1;
      const int ta = 4 * g + (j >> 2), tc = 16 + 4 * g + (j >> 2);

#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        i16x4_t v0[8], v1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v0[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<__attribute__((address_space(3))) i16x4_t*>(
                  static_cast<uintptr_t>(tb + 16 * (ta * U + 4 * ((8 * cg + e) >> 1) +
                                                   ((2 * ((8 * cg + e) & 1) + kb) ^ tswz<KF>(ta))) + 8 * (j & 1))));
          v1[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<__attribute__((address_space(3))) i16x4_t*>(
                  static_cast<uintptr_t>(tb + 16 * (tc * U + 4 * ((8 * cg + e) >> 1) +
                                                   ((2 * ((8 * cg + e) & 1) + kb) ^ tswz<KF>(tc))) + 8 * (j & 1))));
        }
        sched_fence();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0[e], v1[e], 0, 1, 2, 3, 4, 5, 6, 7));
          acc[8 * cg + e] = mfma_bf16(av, pb, acc[8 * cg + e]);
        }
      }
    } else if constexpr (kV8) {
      // four groups of eight 16-column tiles, two groups of reads in flight
#pragma unroll
      for (int c = 0; c < 16; ++c) vv[c] = tr8_frag(c);
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        pin8(vv + 8 * cg);
        if (cg < 2) {
#pragma unroll
          for (int c = 16 + 8 * cg; c < 24 + 8 * cg; ++c) vv[c] = tr8_frag(c);
        }
#pragma unroll
        for (int c = 8 * cg; c < 8 * cg + 8; ++c) acc[c] = mfma_bf16(cvt_fp8x8(vv[c]), pb, acc[c]);
      }
    } else {
      // mxfp4: lane (column block i = lane&15) decodes unit i of its 8 tokens;
      // output tile c row r <-> latent column 32*(4g+r) + c.
      const int i = lane & 15;
      // lane bases of token 4g, made opaque so that every read below adds
      // only an immediate offset (token 4g + kk is + 16 U kk bytes of codes
      // and + 20 kk bytes of scales; tokens 16 + 4g + kk are 16 further)
      int vbase = tb + 16 * (4 * g * U + i);
      int sbase = static_cast<int>(sc_addr(x)) + 20 * 4 * g + i;
      asm volatile("" : "+v"(vbase), "+v"(sbase));
      const uint32_t pl = pmask >> (4 * g);  // parity of token 4g + k at bit k
      uint32_t vw[8][4];
      float vsc[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int dt = kk < 4 ? kk : 16 + (kk - 4);  // token offset from 4g
        const i32x4_t u = lds_ld<i32x4_t>(vbase + 16 * U * dt);
        vw[kk][0] = u.x;
        vw[kk][1] = u.y;
        vw[kk][2] = u.z;
        vw[kk][3] = u.w;
        const int sa = sbase + 2 * static_cast<int>(bit_of(pl, dt));
        vsc[kk] = e8m0_f32(lds_ld<uint8_t>(sa + 20 * dt));
      }
      sched_fence();
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        uint32_t cv[8][4];  // token kk: bf16 pairs (cols 8qd + 2e, +1)
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8_t d = cvt_fp4x8(vw[kk][qd], vsc[kk]);
          const u32x4_t du = __builtin_bit_cast(u32x4_t, d);
          cv[kk][0] = du.x;
          cv[kk][1] = du.y;
          cv[kk][2] = du.z;
          cv[kk][3] = du.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          u32x4_t av;
#pragma unroll
          for (int p = 0; p < 4; ++p)
            av[p] = (e & 1) ? hi_pair(cv[2 * p][e >> 1], cv[2 * p + 1][e >> 1])
                            : lo_pair(cv[2 * p][e >> 1], cv[2 * p + 1][e >> 1]);
          acc[8 * qd + e] = mfma_bf16(__builtin_bit_cast(bf16x8_t, av), pb, acc[8 * qd + e]);
        }
      }
    }
  };

  // ---- bf16 Q quantised in the prologue: the first tile goes out, then Q
  // is quantised while it and the next page ids are in flight (the fill
  // below continues from the second tile).  Every wave takes part, streaming
  // or not, since where the work is shared each wave quantises only its
  // chunks (c mod waves = w) and reads the others' from LDS.
  if constexpr (kQuantQ || kQuantQ4) {
    if (nloc > 0) {
      issue_pid(D);
      issue_tile(0, 0, true);
    }
    const int qx = static_cast<int>(smem0) + L::kTotal;
    if constexpr (kQuantQ) {
      const float r = 1.0f / qs;
      const bool fast = qs >= 0x1p-60f && qs <= 0x1p60f;  // workgroup-uniform
      auto quant = [&](int c) {
        q8[c] = fast ? quant_q_fp8<false>(qraw + 4 * c, qs, r) : quant_q_fp8<true>(qraw + 4 * c, qs, r);
      };
      if constexpr (kShareQ) {
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
          if (c % kWaves == w) {
            quant(c);
            const u32x8_t u = __builtin_bit_cast(u32x8_t, q8[c]);
            lds_st<u32x4_t>(qx + (c * 64 + lane) * 32, u32x4_t{u[0], u[1], u[2], u[3]});
            lds_st<u32x4_t>(qx + (c * 64 + lane) * 32 + 16, u32x4_t{u[4], u[5], u[6], u[7]});
          }
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
          const u32x4_t a0 = lds_ld<u32x4_t>(qx + (c * 64 + lane) * 32);
          const u32x4_t a1 = lds_ld<u32x4_t>(qx + (c * 64 + lane) * 32 + 16);
          q8[c] = __builtin_bit_cast(i32x8_t, u32x8_t{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]});
        }
      } else {
#pragma unroll
        for (int c = 0; c < NQ; ++c) quant(c);
      }
    } else {
      // codes [c][lane] 16 B each, then scales [c][lane] 4 B each
      const int qsx = qx + NQ * 64 * 16;
#pragma unroll
      for (int c = 0; c < NQ; ++c) {
        if (c % kWaves == w) {
          quant_q_mxfp4(qraw + 4 * c, q4[c], q4s[c]);
          lds_st<i32x4_t>(qx + (c * 64 + lane) * 16, q4[c]);
          lds_st<uint32_t>(qsx + (c * 64 + lane) * 4, q4s[c]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < NQ; ++c) {
        q4[c] = lds_ld<i32x4_t>(qx + (c * 64 + lane) * 16);
        q4s[c] = lds_ld<uint32_t>(qsx + (c * 64 + lane) * 4);
      }
      // dims 576..639 are padding, as in the mxfp4-Q load: zero codes, 2^0
      if (g >= 2) {
        q4[4] = i32x4_t{0, 0, 0, 0};
        q4s[4] = 127u;
      }
    }
  }

  // ---- the asynchronous pipeline
  if (nloc > 0) {
    const int nfill = min(NBUF, nloc);
    int pend = -1;
    for (int X = kQuantQ || kQuantQ4 ? 1 : 0; X < nfill; ++X) {
      if (X >= D) wait_vm<D * NDMA + D - 1>();
      issue_pid(X + D);
      // split mode: the second fill tile leaves its rest to compute(0)
      const bool full = !kSplitDma || X == 0;
      issue_tile(X, X, full);
      if (!full) pend = X;
    }
    if constexpr (kSplitQ) {
#pragma unroll
      for (int c = 0; c < NQ; ++c) split_q_fp8(qraw + 4 * c, g, q8[c], ql[c], qhs[c], qls[c]);
    } else if constexpr (kLateQ) {
      load_q();
      pin_q();
    }
    int xs = 0;  // slot of tile jx
    for (int jx = 0; jx < nloc; ++jx) {
      const int ahead = min(nloc - 1, jx + NBUF - 1) - jx;
      if constexpr (NBUF == 1) {
        wait_vm<0>();
      } else if constexpr (NBUF == 2) {
        // issued after tile jx: the next page-id gather and the first KA
        // DMAs of tile jx + 1 (its rest went out during the previous compute)
        if (ahead >= 1) wait_vm<KA + 1>();
        else wait_vm<0>();
      } else {
        if (ahead >= 2) wait_vm<2 * (NDMA + 1)>();
        else if (ahead == 1) wait_vm<NDMA + 1>();
        else wait_vm<0>();
      }
      const int ubase = kSub * (w + kWaves * jx);
      compute(xs, min(kSub, n - ubase), pend);
      pend = -1;
      const int X = jx + NBUF;
      if (X < nloc) {
        wait_vm<D * NDMA + D - 1>();
        issue_pid(X + D);
        issue_tile(X, xs, !kSplitDma);
        if (kSplitDma) pend = X;
      }
      xs = xs + 1 == NBUF ? 0 : xs + 1;
    }
  }

  // ---- merge the waves (log2-domain weights), then write.  Every wave parks
  // its O^T fragments and (m, l) in LDS (the staging rings are idle now),
  // then wave v merges fragments F v .. F v + F - 1 (F = 32 / waves, its
  // share of the output columns) over all waves and stores them, so one
  // barrier separates the two halves and the output stores are spread over
  // the waves.
  constexpr int F = 32 / kWaves;
  l_run = group_sum(l_run);
  __syncthreads();
  const int ob0 = static_cast<int>(smem0);
  const int mlb = ob0 + kWaves * 32768;  // m[w][16], l[w][16]
#pragma unroll
  for (int c = 0; c < 32; ++c) lds_st<f32x4_t>(ob0 + w * 32768 + (c * 64 + lane) * 16, acc[c]);
  if (g == 0) {
    lds_st<float>(mlb + (w * kHeads + hq) * 4, m_run);
    lds_st<float>(mlb + (kWaves * kHeads + w * kHeads + hq) * 4, l_run);
  }
  __syncthreads();
  float mw[kWaves], lw[kWaves];
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    mw[v] = lds_ld<float>(mlb + (v * kHeads + hq) * 4);
    lw[v] = lds_ld<float>(mlb + (kWaves * kHeads + v * kHeads + hq) * 4);
  }
  f32x4_t part[kWaves][F];
#pragma unroll
  for (int v = 0; v < kWaves; ++v)
#pragma unroll
    for (int i = 0; i < F; ++i) part[v][i] = lds_ld<f32x4_t>(ob0 + v * 32768 + ((F * w + i) * 64 + lane) * 16);
  sched_fence();
  float M = mw[0];
#pragma unroll
  for (int v = 1; v < kWaves; ++v) M = fmaxf(M, mw[v]);
  float fv[kWaves];
  float lsum = 0.0f;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    fv[v] = mw[v] == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(mw[v] - M);
    lsum += lw[v] * fv[v];
  }
  f32x4_t o[F];
#pragma unroll
  for (int i = 0; i < F; ++i) {
    o[i] = part[0][i] * fv[0];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) o[i] += part[v][i] * fv[v];
  }

  const bool nonempty = lsum > 0.0f;
  const float mul = nonempty ? out_mul / lsum : 0.0f;
  const float lse = nonempty ? M + __builtin_amdgcn_logf(lsum) : -__builtin_huge_valf();
  const size_t orow = static_cast<size_t>(v) * kHeads + hq;
  const bool direct = a.items ? slot < 0 : S == 1;
  // fragment c = F w + i; non-mxfp4 row r of fragment c is output column
  // 16c + 4g + r, mxfp4 row r is column 32(4g + r) + c
  if (direct) {
    uint16_t* op = a.out + orow * kDv;
    if constexpr (KF == FMX) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int h4 = 0; h4 < F / 4; ++h4) {
          const bf16x2_t p0 = {static_cast<__bf16>(o[4 * h4 + 0][r] * mul), static_cast<__bf16>(o[4 * h4 + 1][r] * mul)};
          const bf16x2_t p1 = {static_cast<__bf16>(o[4 * h4 + 2][r] * mul), static_cast<__bf16>(o[4 * h4 + 3][r] * mul)};
          *reinterpret_cast<i32x2_t*>(op + 32 * (4 * g + r) + F * w + 4 * h4) =
              i32x2_t{static_cast<int>(bits(p0)), static_cast<int>(bits(p1))};
        }
    } else {
#pragma unroll
      for (int i = 0; i < F; ++i) {
        const bf16x2_t p0 = {static_cast<__bf16>(o[i][0] * mul), static_cast<__bf16>(o[i][1] * mul)};
        const bf16x2_t p1 = {static_cast<__bf16>(o[i][2] * mul), static_cast<__bf16>(o[i][3] * mul)};
        *reinterpret_cast<i32x2_t*>(op + 16 * (F * w + i) + 4 * g) =
            i32x2_t{static_cast<int>(bits(p0)), static_cast<int>(bits(p1))};
      }
    }
  } else {
    // the query group's 16 partial rows (head hq at row prow0 + hq).  A
    // single round of four-wave workgroups ends all at once, with every
    // partial still dirty in the L2s: written through, they drain during
    // the epilogue instead of between the two launches (bs=32 kv=1024 S=8:
    // 16.8 against 17.8 us per call; 1.5-2.4 % on the other one-round
    // shapes).  Two-wave workgroups keep write-back stores, which measured
    // faster there (bs=64 kv=8192 S=8: 62.0 against 63.0 us), and so do the
    // mxfp4 kernels, whose stores write 16-byte pieces 512 bytes apart: the
    // L2 must merge those into lines (written through, bs=4 kv=1024 S=8
    // took 14.4 against 12.4 us with mxfp4 Q).
    constexpr int kCp = kWaves == 4 && KF != FMX ? kCpolDev : 0;
    const size_t prow0 = ((a.items ? static_cast<size_t>(slot) : static_cast<size_t>(b) * S + s) * G + r) * kHeads;
    const __amdgpu_buffer_rsrc_t po = rsrc_of(a.part_o + prow0 * kDv, kHeads * kDv * 4);
    const uint32_t ob = static_cast<uint32_t>(hq * kDv * 4);
    if constexpr (KF == FMX) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int h4 = 0; h4 < F / 4; ++h4)
          st_pol<kCp>(po, ob + 4 * (32 * (4 * g + r) + F * w + 4 * h4),
                      f32x4_t{o[4 * h4][r], o[4 * h4 + 1][r], o[4 * h4 + 2][r], o[4 * h4 + 3][r]} * mul);
    } else {
#pragma unroll
      for (int i = 0; i < F; ++i) st_pol<kCp>(po, ob + 4 * (16 * (F * w + i) + 4 * g), o[i] * mul);
    }
    if (w == 0 && g == 0) st_pol<kCp>(rsrc_of(a.part_lse + prow0, kHeads * 4), 4 * hq, lse);
  }
}

// ------------------------------------------------------------------ stage 2
// A thread merges kC columns of one head over the S splits with base-2
// log-sum-exp weights (empty splits, LSE = -inf, are skipped; an all-empty
// request yields zeros); a workgroup covers four heads x 512 / kParts columns
// of one query group.  The LSEs and partial rows of kB splits are loaded
// together; with kPre the next kB are in flight while a batch is combined,
// and the running maximum moves with a rescale of the accumulator.  9 to 32
// splits are taken in a single batch of loads (one memory round trip), with
// four columns per thread so twice as many workgroups share the reads.
template <int kB, int kC, bool kPre>
__global__ __launch_bounds__(256) void stage2_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                                                     uint16_t* __restrict__ out, int S, const int32_t* __restrict__ req,
                                                     int G) {
  static_assert(kC == 4 || kC == 8, "four or eight columns per thread");
  constexpr int kParts = 8 / kC;  // column parts of a head row
  constexpr int kV = kC / 4;      // f32x4 per split per thread
  const int per_v = 4 * kParts;
  const int v = blockIdx.x / per_v;  // query group (request b, group r)
  const int hb = blockIdx.x - v * per_v;
  const int b = v / G;
  const int r = v - b * G;
  const int hq = 4 * (hb / kParts) + (threadIdx.x >> 6);
  const int col = (hb % kParts) * (kDv / kParts) + kC * (threadIdx.x & 63);
  // a request's partials: slots [base, base + S) (work list: from the plan;
  // a single-item request was written by stage 1); slot si of group r holds
  // rows ((base + si) * G + r) * 16 + [0, 16)
  size_t base = static_cast<size_t>(b) * S;
  if (req) {
    S = req[2 * b + 1];
    if (S <= 1) return;
    base = static_cast<size_t>(req[2 * b]);
  }
  const size_t stride = static_cast<size_t>(G) * kHeads;  // rows between consecutive splits
  const float* lse = part_lse + (base * G + r) * kHeads + hq;
  const float* po = part_o + ((base * G + r) * kHeads + hq) * kDv + col;
  constexpr float kNegInf = -__builtin_huge_valf();
  float M = kNegInf, ws = 0.0f;
  f32x4_t acc[kV];
#pragma unroll
  for (int k = 0; k < kV; ++k) acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // batch loads: splits [s0, s0 + kB), past the end weighted 0
  float l[kB], ln[kPre ? kB : 1];
  f32x4_t x[kB][kV], y[kPre ? kB : 1][kV];
  auto load = [&](int s0, float* lb, f32x4_t (*bx)[kV]) {
    if constexpr (kB > 8) {
      // a single wide batch: only the splits that exist are loaded
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        lb[i] = kNegInf;
#pragma unroll
        for (int k = 0; k < kV; ++k) bx[i][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (s0 + i < S) {
          lb[i] = lse[(s0 + i) * stride];
#pragma unroll
          for (int k = 0; k < kV; ++k)
            bx[i][k] = *reinterpret_cast<const f32x4_t*>(po + (s0 + i) * stride * kDv + 4 * k);
        }
      }
    } else {
      // all kB loads unconditional (past the end: the last split again, a
      // cache hit), so they are in flight together
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        const int si = min(s0 + i, S - 1);
        lb[i] = lse[si * stride];
#pragma unroll
        for (int k = 0; k < kV; ++k) bx[i][k] = *reinterpret_cast<const f32x4_t*>(po + si * stride * kDv + 4 * k);
      }
    }
  };
  load(0, l, x);
  for (int s0 = 0; s0 < S; s0 += kB) {
    const bool more = s0 + kB < S;
    if constexpr (kPre) {
      if (more) load(s0 + kB, ln, y);
    } else {
      if (s0 > 0) load(s0, l, x);
    }
#pragma unroll
    for (int i = 0; i < kB; ++i)
      if (s0 + i >= S) l[i] = kNegInf;
    float mb = l[0];
#pragma unroll
    for (int i = 1; i < kB; ++i) mb = fmax3(mb, l[i]);
    if (mb != kNegInf) {  // else every split of this batch is empty
      const float Mn = fmax3(M, mb);
      const float rs = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
#pragma unroll
      for (int k = 0; k < kV; ++k) acc[k] *= rs;
      ws *= rs;
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        const float wgt = l[i] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(l[i] - Mn);
#pragma unroll
        for (int k = 0; k < kV; ++k) acc[k] += x[i][k] * wgt;
        ws += wgt;
      }
      M = Mn;
    }
    if constexpr (kPre) {
      if (more) {
#pragma unroll
        for (int i = 0; i < kB; ++i) {
          l[i] = ln[i];
#pragma unroll
          for (int k = 0; k < kV; ++k) x[i][k] = y[i][k];
        }
      }
    }
  }
  const float inv = ws > 0.0f ? 1.0f / ws : 0.0f;
  uint32_t o[2 * kV];
#pragma unroll
  for (int k = 0; k < kV; ++k) {
    const f32x4_t a = acc[k] * inv;
    o[2 * k] = bits(bf16x2_t{static_cast<__bf16>(a.x), static_cast<__bf16>(a.y)});
    o[2 * k + 1] = bits(bf16x2_t{static_cast<__bf16>(a.z), static_cast<__bf16>(a.w)});
  }
  uint16_t* op = out + (static_cast<size_t>(v) * kHeads + hq) * kDv + col;
  if constexpr (kV == 2) {
    *reinterpret_cast<u32x4_t*>(op) = u32x4_t{o[0], o[1], o[2], o[3]};
  } else {
    *reinterpret_cast<i32x2_t*>(op) = i32x2_t{static_cast<int>(o[0]), static_cast<int>(o[1])};
  }
}

// -------------------------------------------------------------- quantisers
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

__global__ void zero_f32_kernel(float* p) { p[0] = 0.0f; }

// max |x| over bf16 inputs, as the bit pattern of a non-negative fp32 (NaN
// skipped).  16-byte loads over the aligned middle, element loads for the
// unaligned head and the tail; one atomic per workgroup, on a grid of at most
// a few hundred workgroups, so the single target word sees little contention.
__device__ __forceinline__ void amax_take(unsigned& m, uint32_t h) {
  const unsigned a = (h & 0x7fffu) << 16;
  if (a <= 0x7f800000u && a > m) m = a;
}

__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ x, int64_t n, unsigned* __restrict__ amax) {
  unsigned m = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t tid = blockIdx.x * 256ll + threadIdx.x;
  const int64_t head = min(n, static_cast<int64_t>((16u - (reinterpret_cast<uintptr_t>(x) & 15u)) & 15u) / 2);
  const int64_t nv = (n - head) >> 3;
  for (int64_t i = tid; i < head; i += stride) amax_take(m, x[i]);
  const u32x4_t* xv = reinterpret_cast<const u32x4_t*>(x + head);
  for (int64_t i = tid; i < nv; i += stride) {
    const u32x4_t u = xv[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      amax_take(m, u[k] & 0xffffu);
      amax_take(m, u[k] >> 16);
    }
  }
  for (int64_t i = head + 8 * nv + tid; i < n; i += stride) amax_take(m, x[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned v = __shfl_xor(m, o);
    m = v > m ? v : m;
  }
  __shared__ unsigned wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wm[0], wm[1]), max(wm[2], wm[3]));
    if (m) atomicMax(amax, m);
  }
}

__global__ void fp8_scale_kernel(float* scale) {
  const float a = scale[0];
  scale[0] = (a < 1e-12f ? 1e-12f : a) / 448.0f;
}

// Nearest OCP e4m3fn code to v, |v| <= 448, ties to even: with
// e = max(floor(log2|v|), -6) the code magnitude is 8(e+6) + rne(|v| * 2^(3-e));
// subnormals (e = -6) and the carry into the next binade fall out of the same
// formula because the code is the concatenation exponent|mantissa.
__device__ __forceinline__ uint8_t to_e4m3fn(float v) {
  const float av = __builtin_fabsf(v);
  int e = static_cast<int>((__float_as_uint(av) >> 23) & 0xff) - 127;
  e = e < -6 ? -6 : e;
  const int mag = 8 * (e + 6) + static_cast<int>(__builtin_rintf(__builtin_ldexpf(av, 3 - e)));
  return static_cast<uint8_t>((__float_as_uint(v) >> 24 & 0x80u) | static_cast<unsigned>(mag));
}

__device__ __forceinline__ uint8_t quant_fp8_one(uint32_t h, float sc) {
  float q = bf16_bits_to_f32(static_cast<uint16_t>(h)) / sc;
  q = q > 448.0f ? 448.0f : (q < -448.0f ? -448.0f : q);
  return to_e4m3fn(q);
}

// Eight elements per thread and step (16 bytes in, 8 out) when source and
// destination share their offset from a 16 / 8-byte boundary; element by
// element otherwise and for the tail.
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ x, int64_t n, const float* __restrict__ scale,
                                                        uint8_t* __restrict__ dst, int vec) {
  const float sc = scale[0];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t tid = blockIdx.x * 256ll + threadIdx.x;
  const int64_t nv = vec ? n >> 3 : 0;
  const u32x4_t* xv = reinterpret_cast<const u32x4_t*>(x);
  for (int64_t i = tid; i < nv; i += stride) {
    const u32x4_t u = xv[i];
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      lo |= static_cast<uint32_t>(quant_fp8_one(u[k] & 0xffffu, sc)) << (16 * k);
      lo |= static_cast<uint32_t>(quant_fp8_one(u[k] >> 16, sc)) << (16 * k + 8);
      hi |= static_cast<uint32_t>(quant_fp8_one(u[k + 2] & 0xffffu, sc)) << (16 * k);
      hi |= static_cast<uint32_t>(quant_fp8_one(u[k + 2] >> 16, sc)) << (16 * k + 8);
    }
    *reinterpret_cast<u32x2_t*>(dst + 8 * i) = u32x2_t{lo, hi};
  }
  for (int64_t i = 8 * nv + tid; i < n; i += stride) dst[i] = quant_fp8_one(x[i], sc);
}

// Nearest e2m1 code to v (ties to even, saturating at 6): thresholds are the
// midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5 with the tie going to the even code.
__device__ __forceinline__ uint32_t to_e2m1(float v) {
  const float a = __builtin_fabsf(v);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return c | ((__float_as_uint(v) >> 28) & 8u);
}

// one thread per 32-element block
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t* __restrict__ x, int64_t nblocks, int64_t cols,
                                                          uint8_t* __restrict__ packed, uint8_t* __restrict__ scales) {
  const int64_t blk = blockIdx.x * 256ll + threadIdx.x;
  if (blk >= nblocks) return;
  const int64_t nb = cols / 32;
  const int64_t row = blk / nb, bi = blk - row * nb;
  const uint16_t* xr = x + row * cols + bi * 32;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(xr + 8 * i);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * i + 2 * k] = __uint_as_float(u[k] << 16);
      v[8 * i + 2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float a = __builtin_fabsf(v[i]);
    amax = a > amax ? a : amax;  // NaN compares false and is skipped
  }
  int X;
  uint8_t sc;
  if (amax == 0.0f) {
    X = -127;
    sc = 0;
  } else {
    X = __builtin_amdgcn_frexp_expf(amax) - 1 - 2;  // floor(log2 amax) - emax(e2m1)
    X = X < -127 ? -127 : (X > 127 ? 127 : X);
    sc = static_cast<uint8_t>(X + 127);
  }
  scales[row * nb + bi] = sc;
  u32x4_t out;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) w |= to_e2m1(__builtin_ldexpf(v[8 * k + e], -X)) << (4 * e);
    out[k] = w;
  }
  *reinterpret_cast<u32x4_t*>(packed + row * (cols / 2) + bi * 16) = out;
}

// ------------------------------------------------------------------ launch
template <int QF, int KF>
hipError_t launch_stage1(const Stage1Args& a, unsigned grid, bool two_waves, hipStream_t st) {
  if (two_waves)
    hipLaunchKernelGGL((stage1_kernel<QF, KF, 2>), dim3(grid), dim3(128), 0, st, a);
  else
    hipLaunchKernelGGL((stage1_kernel<QF, KF, 4>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_stage1_any(const Stage1Args& a, int32_t q_dtype, int32_t kv_dtype, unsigned grid, bool two_waves,
                             hipStream_t st) {
  const bool qb = q_dtype == MLA_DTYPE_BF16;
  if (kv_dtype == MLA_DTYPE_BF16) return launch_stage1<FBF16, FBF16>(a, grid, two_waves, st);
  if (kv_dtype == MLA_DTYPE_FP8_E4M3FN)
    return qb                                 ? launch_stage1<FBF16, FFP8>(a, grid, two_waves, st)
           : q_dtype == MLA_Q_BF16_FP8_STATIC ? launch_stage1<FQ8S, FFP8>(a, grid, two_waves, st)
                                              : launch_stage1<FFP8, FFP8>(a, grid, two_waves, st);
  if (kv_dtype == MLA_KV_MXFP4_K_FP8_V)
    return qb ? launch_stage1<FBF16, FMIX>(a, grid, two_waves, st) : launch_stage1<FMX, FMIX>(a, grid, two_waves, st);
  return qb                            ? launch_stage1<FBF16, FMX>(a, grid, two_waves, st)
         : q_dtype == MLA_Q_BF16_MXFP4 ? launch_stage1<FQ4, FMX>(a, grid, two_waves, st)
                                       : launch_stage1<FMX, FMX>(a, grid, two_waves, st);
}

// Compute units of the current device (queried once per device; concurrent
// callers may both query, and store the same value).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Scratch of mla_decode_noalloc: the split partials in a file-scope device
// array (each GPU the library runs on holds its own copy until the process
// ends), for callers that cannot allocate.  Host code never uses the array's
// name as an address: its device address is looked up once per device.
__device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

void* scratch_ptr() {
  static std::atomic<void*> ptrs[64];
  static std::mutex init;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(init);
  p = ptrs[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    ptrs[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

int grid_for(int64_t n, int per) {
  int64_t g = (n + per - 1) / per;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return static_cast<int>(g);
}

// ---------------------------------------------------------------------------
// Streaming-read probe: each workgroup reads one contiguous chunk with 16-byte
// non-temporal loads, four per lane in flight, and folds them into one word.
// The word is stored only if it equals an improbable constant, so the loads
// stay live without adding writes.  Measures the HBM read ceiling that the
// decode kernels (which read their cache once) are compared against.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n16,
                                                          int64_t per_block, uint32_t* sink) {
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per_block;
  const int64_t b1 = min(b0 + per_block, n16);
  uint32_t acc = 0;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += 4 * 256) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + 256 * u;
      v[u] = j < b1 ? __builtin_nontemporal_load(src + j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Shared launcher: uniform splits (items == NULL) or a work-list plan, for
// q_rows query rows per request (G = q_rows / 16 query groups).  kv_dtype
// MLA_KV_MXFP4_K_FP8_V is the split cache: kv_cache / kv_scale are its mxfp4
// K side, v_cache / v_scale its fp8 V side (otherwise both NULL).
int decode_launch(const void* q, int32_t q_dtype, const void* q_scale, int32_t q_rows, const void* kv_cache,
                  int32_t kv_dtype, const void* kv_scale, int64_t num_kv_rows, const int32_t* kv_indptr,
                  int32_t batch, const int32_t* page_table, const int32_t* page_indptr, int32_t page_size,
                  int32_t num_splits, const int32_t* items, int32_t num_items, const int32_t* req, int32_t num_slots,
                  void* out, void* workspace, size_t workspace_bytes, void* stream, const void* v_cache = nullptr,
                  const void* v_scale = nullptr) {
  if (q_rows < kHeads || q_rows % kHeads || q_rows > MLA_MAX_Q_ROWS) return MLA_ERR_ARG;
  const int G = q_rows / kHeads;
  // the shared argument checks, without the workspace (sized per mode below)
  const bool mixed = kv_dtype == MLA_KV_MXFP4_K_FP8_V;
  int rc = mixed ? mla_validate_mixed(q, q_dtype, q_scale, q_rows, kv_cache, kv_scale, v_cache, v_scale, num_kv_rows,
                                      kv_indptr, batch, page_table, page_indptr, page_size,
                                      items ? 1 : num_splits, out, nullptr, 0)
                 : mla_validate(q, q_dtype, q_scale, kv_cache, kv_dtype, kv_scale, num_kv_rows, kv_indptr, batch,
                                page_table, page_indptr, page_size, items ? 1 : num_splits, out, nullptr, 0);
  if (rc == MLA_ERR_WORKSPACE) rc = MLA_OK;  // checked below
  if (rc != MLA_OK || batch == 0) return rc;
  if (items && (!req)) return MLA_ERR_NULL;
  if (items && (num_items < batch || num_slots < 0)) return MLA_ERR_ARG;
  const int64_t units = items ? static_cast<int64_t>(num_items) : static_cast<int64_t>(batch) * num_splits;
  // grid sizes must fit an unsigned 32-bit launch: stage 1 pads the units to
  // a multiple of 8 per query group, stage 2 takes up to 8 workgroups per group
  if ((units + 7) * G > 0x7fffffffLL || static_cast<int64_t>(batch) * G * 8 > 0x7fffffffLL) return MLA_ERR_ARG;
  const int64_t nslots = items ? num_slots : (num_splits > 1 ? static_cast<int64_t>(batch) * num_splits : 0);
  const size_t parts = static_cast<size_t>(nslots) * G * kHeads;
  const size_t need = parts * kDv * sizeof(float) + parts * sizeof(float);
  if (need) {
    if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return MLA_ERR_ALIGN;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so it is not misattributed
  Stage1Args a;
  a.q = q;
  a.q_scale = q_scale;
  a.kv = static_cast<const char*>(kv_cache);
  a.kv_scale = kv_scale;
  a.kv2 = static_cast<const char*>(v_cache);
  a.kv2_scale = static_cast<const float*>(v_scale);
  a.kv_indptr = kv_indptr;
  a.page_table = page_table;
  a.page_indptr = page_indptr;
  a.part_o = need ? static_cast<float*>(workspace) : nullptr;
  a.part_lse = need ? static_cast<float*>(workspace) + parts * kDv : nullptr;
  a.out = static_cast<uint16_t*>(out);
  a.items = items;
  a.batch = batch;
  a.groups = G;
  a.units = static_cast<int32_t>(units);
  a.page_size = page_size;
  a.num_splits = items ? 1 : num_splits;
  a.max_row = static_cast<uint32_t>(std::min<int64_t>(num_kv_rows - 1, 0xffffffffLL));
  a.sm_scale_log2e = static_cast<float>(1.4426950408889634 / 24.0);  // log2(e) / sqrt(576)
  const int64_t grid = G == 1 ? units : (units + 7) / 8 * 8 * G;
  // more workgroups than CUs: two-wave workgroups, two per CU, one round
  const bool two_waves = grid > device_cus();
  if (launch_stage1_any(a, q_dtype, kv_dtype, static_cast<unsigned>(grid), two_waves, st) != hipSuccess)
    return MLA_ERR_LAUNCH;
  if (need) {
    // 9 to 32 splits: one batch of loads (one memory round trip), four
    // columns per thread; other counts (and work lists, whose per-request
    // counts live on the device): batches of eight with the next batch in
    // flight.  (Measured at bs=4, S=16: 14.5 against 15.0 us per call with
    // two batches of eight; at S <= 8 four columns per thread were slower.)
    const int S2 = items ? 1 : num_splits;
    const int32_t* rq = items ? req : nullptr;
    uint16_t* o16 = static_cast<uint16_t*>(out);
    const unsigned vg = static_cast<unsigned>(batch) * G;
    if (!items && num_splits > 16 && num_splits <= 32)
      hipLaunchKernelGGL((stage2_kernel<32, 4, false>), dim3(vg * 8), dim3(256), 0, st, a.part_o, a.part_lse, o16, S2,
                         rq, G);
    else if (!items && num_splits > 8 && num_splits <= 16)
      hipLaunchKernelGGL((stage2_kernel<16, 4, false>), dim3(vg * 8), dim3(256), 0, st, a.part_o, a.part_lse, o16, S2,
                         rq, G);
    else
      hipLaunchKernelGGL((stage2_kernel<8, 8, true>), dim3(vg * 4), dim3(256), 0, st, a.part_o, a.part_lse, o16, S2,
                         rq, G);
    if (hipGetLastError() != hipSuccess) return MLA_ERR_LAUNCH;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode(const void* q, int32_t q_dtype, const void* q_scale, const void* kv_cache, int32_t kv_dtype,
               const void* kv_scale, int64_t num_kv_rows, const int32_t* kv_indptr, int32_t batch,
               const int32_t* page_table, const int32_t* page_indptr, int32_t page_size, int32_t num_splits, void* out,
               void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = mla_validate(q, q_dtype, q_scale, kv_cache, kv_dtype, kv_scale, num_kv_rows, kv_indptr, batch, page_table,
                              page_indptr, page_size, num_splits, out, workspace, workspace_bytes);
  if (rc != MLA_OK || batch == 0) return rc;
  return decode_launch(q, q_dtype, q_scale, kHeads, kv_cache, kv_dtype, kv_scale, num_kv_rows, kv_indptr, batch,
                       page_table, page_indptr, page_size, num_splits, nullptr, 0, nullptr, 0, out, workspace,
                       workspace_bytes, stream);
}

int mla_decode_noalloc(const void* q, int32_t q_dtype, const void* q_scale, const void* kv_cache, int32_t kv_dtype,
                       const void* kv_scale, int64_t num_kv_rows, const int32_t* kv_indptr, int32_t batch,
                       const int32_t* page_table, const int32_t* page_indptr, int32_t page_size, int32_t num_splits,
                       void* out, void* stream) {
  const size_t need = mla_workspace_bytes(batch, num_splits);
  if (need > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need) {
    ws = scratch_ptr();
    if (!ws) return MLA_ERR_DEVICE;
  }
  const int rc = mla_validate(q, q_dtype, q_scale, kv_cache, kv_dtype, kv_scale, num_kv_rows, kv_indptr, batch,
                              page_table, page_indptr, page_size, num_splits, out, ws, need ? MLA_NOALLOC_SCRATCH_BYTES : 0);
  if (rc != MLA_OK || batch == 0) return rc;
  return decode_launch(q, q_dtype, q_scale, kHeads, kv_cache, kv_dtype, kv_scale, num_kv_rows, kv_indptr, batch,
                       page_table, page_indptr, page_size, num_splits, nullptr, 0, nullptr, 0, out, ws,
                       need ? MLA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int mla_decode_rows(const void* q, int32_t q_dtype, const void* q_scale, int32_t q_rows, const void* kv_cache,
                    int32_t kv_dtype, const void* kv_scale, int64_t num_kv_rows, const int32_t* kv_indptr,
                    int32_t batch, const int32_t* page_table, const int32_t* page_indptr, int32_t page_size,
                    int32_t num_splits, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_launch(q, q_dtype, q_scale, q_rows, kv_cache, kv_dtype, kv_scale, num_kv_rows, kv_indptr, batch,
                       page_table, page_indptr, page_size, num_splits, nullptr, 0, nullptr, 0, out, workspace,
                       workspace_bytes, stream);
}

int mla_decode_worklist(const void* q, int32_t q_dtype, const void* q_scale, int32_t q_rows, const void* kv_cache,
                        int32_t kv_dtype, const void* kv_scale, int64_t num_kv_rows, const int32_t* kv_indptr,
                        int32_t batch, const int32_t* page_table, const int32_t* page_indptr, int32_t page_size,
                        const int32_t* items, int32_t num_items, const int32_t* req, int32_t num_slots, void* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (batch > 0 && !items) return MLA_ERR_NULL;
  return decode_launch(q, q_dtype, q_scale, q_rows, kv_cache, kv_dtype, kv_scale, num_kv_rows, kv_indptr, batch,
                       page_table, page_indptr, page_size, 1, items, num_items, req, num_slots, out, workspace,
                       workspace_bytes, stream);
}

int mla_decode_mixed(const void* q, int32_t q_dtype, const void* q_scale, int32_t q_rows, const void* k_cache,
                     const void* k_scale, const void* v_cache, const void* v_scale, int64_t num_kv_rows,
                     const int32_t* kv_indptr, int32_t batch, const int32_t* page_table, const int32_t* page_indptr,
                     int32_t page_size, int32_t num_splits, void* out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return decode_launch(q, q_dtype, q_scale, q_rows, k_cache, MLA_KV_MXFP4_K_FP8_V, k_scale, num_kv_rows, kv_indptr,
                       batch, page_table, page_indptr, page_size, num_splits, nullptr, 0, nullptr, 0, out, workspace,
                       workspace_bytes, stream, v_cache, v_scale);
}

int mla_quantize_fp8(const void* src_bf16, int64_t n, uint8_t* dst, float* scale, int32_t dynamic, void* stream) {
  if (n < 0) return MLA_ERR_ARG;
  if (!scale) return MLA_ERR_NULL;
  if (n > 0 && (!src_bf16 || !dst)) return MLA_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dynamic) {
    hipLaunchKernelGGL(zero_f32_kernel, dim3(1), dim3(1), 0, st, scale);
    if (n > 0)
      hipLaunchKernelGGL(amax_kernel, dim3(min(grid_for(n, 256 * 64), 2 * device_cus())), dim3(256), 0, st,
                         static_cast<const uint16_t*>(src_bf16), n, reinterpret_cast<unsigned*>(scale));
    hipLaunchKernelGGL(fp8_scale_kernel, dim3(1), dim3(1), 0, st, scale);
  }
  const int vec = (reinterpret_cast<uintptr_t>(src_bf16) & 15u) == 0 && (reinterpret_cast<uintptr_t>(dst) & 7u) == 0;
  if (n > 0)
    hipLaunchKernelGGL(quant_fp8_kernel, dim3(grid_for(n, 256 * 32)), dim3(256), 0, st, static_cast<const uint16_t*>(src_bf16),
                       n, scale, dst, vec);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int mla_quantize_mxfp4(const void* src_bf16, int64_t rows, int64_t cols, uint8_t* packed, uint8_t* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32) return MLA_ERR_ARG;
  if (rows == 0) return MLA_OK;
  if (!src_bf16 || !packed || !scales) return MLA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src_bf16) | reinterpret_cast<uintptr_t>(packed)) & 15u) return MLA_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t nblocks = rows * (cols / 32);
  const int64_t grid = (nblocks + 255) / 256;
  if (grid > 0x7fffffffLL) return MLA_ERR_ARG;
  hipLaunchKernelGGL(quant_mxfp4_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, static_cast<const uint16_t*>(src_bf16),
                     nblocks, cols, packed, scales);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

int mla_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16) return MLA_ERR_ARG;
  if (bytes == 0) return MLA_OK;
  if (!src || !sink) return MLA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(src) & 15u) return MLA_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t n16 = bytes / 16;
  // Many small chunks (at least 8 KB each, up to 131072 workgroups) keep the
  // most DRAM channels busy at once: on MI355X the rate still rose from
  // 16384 to 131072 workgroups over a 1.2 GB buffer (6.69 -> 7.06 TB/s).
  const int64_t grid = std::min<int64_t>(131072, (n16 + 511) / 512);
  const int64_t per_block = (n16 + grid - 1) / grid;
  hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                     static_cast<const u32x4_t*>(src), n16, per_block, sink);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

}  // extern "C"
