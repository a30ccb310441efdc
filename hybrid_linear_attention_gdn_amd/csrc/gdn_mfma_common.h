// MFMA kernel family (shared definitions): bf16 or fp8 (E4M3FN) q/k/v, d_k = d_v = 112, fp32 state, on gfx950.
//
// The gated delta rule (the frame-wise Gated DeltaNet of the "SANA-WM"
// cookbook page, table "Architecture & components") is evaluated chunk by
// chunk (80 tokens).  Per (batch, head) and chunk, with raw bf16 rows K, Q, V,
// fp32 scales rk = 1/||k||, rq = 1/||q||, beta, the chunk-local cumulative
// log-decay G, gamma = e^G, and T = (I + A)^{-1} where
//   A_ri = beta_r rk_r rk_i e^{G_r - G_i} (k_r . k_i)            (i < r),
// the recurrence over one chunk with entry state S (d_v x d_k) is exactly
//   Y      = K S^T                      R = diag(beta) V - diag(beta gamma rk) Y
//   O      = diag(gamma rq) Q S^T + P' R              P' = P T,
//            P_ri = rq_r rk_i e^{G_r - G_i} (q_r . k_i)   (i <= r)
//   S^T   <- gamma_n S^T + M R                        M  = K^T diag(s) T,
//            s_i = rk_i e^{G_n - G_i}
// (derivation: the chunked WY form U = T R, O = diag(gamma) Q^ S^T + P U,
// S_next = gamma_n S + U^T diag(e^{G_n - G}) K^, with the scales folded in).
// The state pass takes the normalised rows K^ = diag(rk) K, Q^ = diag(rq) Q
// with their scales folded in, K~ = -diag(beta gamma) K^ and Q~ = diag(gamma) Q^,
// so that R = diag(beta) V + K~ S^T.  Substituting R into O gives the form
// the output uses, in which R does not appear:
//   O = Q' S^T + P'' V,      Q' = Q~ + P' K~,      P'' = P' diag(beta).
//
// The intra-chunk step (gdn_intra.h, one group of four waves per (b, h,
// chunk), fully parallel) forms A and P from K K^T and K Q^T on the matrix
// cores, solves T in LDS (fp32), then M, P', P'' and Q' on the matrix cores.
// It stores them in the exact register order the state pass consumes, with
// the per-token scales.  The state pass (gdn_scan.hip, one workgroup per
// (b, h, pair of 16-column tiles of d_v), sequential over chunks) keeps its
// 112 x 16 slices of the fp32 state in registers and runs R = diag(beta) V +
// K~ S^T and the update per chunk, and the output O = Q' S^T + P'' V.
//
// Precision.  The intra-chunk step works from the exact bf16 rows: K K^T and
// K Q^T on bf16 matrix instructions, T by fp32 substitution and bf16 hi/lo
// block products (x = hi + lo, hi = bf16(x), lo = bf16(x - hi): about 16
// bits), M, P' and P' K~ from hi/lo operands, all accumulating in fp32.  The
// state pass then takes K~, Q', M and its own S and R as fp16 (11 significant
// bits, round to nearest even; |K~| <= 1) and P'' as a bf16 hi/lo pair against
// the exact bf16 rows of V.  S and R are scaled by a power of two per 112 x 16
// / 80 x 16 tile whenever the tile's largest magnitude leaves [2^-6, 2^15),
// which keeps fp16's range out of the way; the scale is undone exactly on the
// fp32 results.  Every product accumulates in fp32 and the state stays fp32.
// The intra-chunk term P'' V, which dominates o when the gates decay within a
// chunk, so carries no fp16 rounding of its own; an fp64 emulation of exactly
// these roundings gives 2.2e-3 to 2.5e-3 of rms(o) on the 241-frame clip and
// 0.7e-3 to 1.3e-3 with a gate on every token (against 7e-3 to 9e-3 if R
// entered the output as fp16).
//
// MFMA lane layouts (v_mfma_f32_16x16x32_bf16 / 16x16x16_bf16, lane l,
// g = l >> 4): A row l & 15 and B column l & 15 hold k = 8g..8g+7 (4g..4g+3
// for the 16-deep form); the accumulator holds column l & 15, rows 4g..4g+3.
// A 32-deep reduction block built from two accumulator tiles uses the
// k-order "pair": instruction slots 0-3 of group g are rows 4g..4g+3 of the
// first 16-row tile and slots 4-7 rows 4g..4g+3 of the second, so an
// accumulator pair becomes a B operand without any data movement; every A
// operand of such a product is read in the same order.
#pragma once
#include <type_traits>

#include "gdn_internal.h"

namespace gdn {
namespace mfma {

constexpr int D = kMfmaDim;  // 112
constexpr int C = kChunk;    // 80
constexpr int NT = D / 16;   // 7 column tiles of d_v (and row tiles of d_k)
constexpr int CT = C / 16;   // 5 token tiles per chunk

// One chunk-head record: the state pass's operands as fragment images (K~,
// Q', M in fp16; P'' as bf16 hi and lo) and fp32 scales a = beta (per token)
// and gamma_n.
constexpr int kKQBytes = CT * 3584;  // K~ or Q': per token tile 3 K32 blocks of 1 KB + 1 of 512 B
constexpr int kPBytes = 7680;        // lower-triangular token blocks of P'' (hi or lo)
constexpr int kCsFloats = 128;       // a[80], gamma_n, pad
constexpr int kMBytes = NT * 2560;   // 7 d_k tiles x (2 K32 blocks of 1 KB + 1 K16 block of 512 B)
constexpr int kRecK = 0, kRecQ = kKQBytes, kRecP = 2 * kKQBytes, kRecPl = kRecP + kPBytes;
constexpr int kRecCs = kRecPl + kPBytes;
constexpr int kRecM = kRecCs + kCsFloats * 4;  // 51,712
constexpr int kRecBytes = kRecM + kMBytes;     // 69,632
constexpr int kCsGammaN = 80;                  // index of gamma_n among the scales

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

struct F32 {  // 8 bf16 = one lane of a 32-deep operand
  uint32_t w[4];
};
struct F16 {  // 4 bf16 = one lane of a 16-deep operand
  uint32_t w[2];
};

__device__ __forceinline__ f32x4 mma(const F32 &a, const F32 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}
// A 16-deep block on the same 16x16x32 instruction with slots 4-7 of both
// operands zero: one MFMA opcode throughout keeps a dependent accumulation
// chain on a single instruction latency.
__device__ __forceinline__ f32x4 mma(const F16 &a, const F16 &b, f32x4 c) {
  const F32 a2{{a.w[0], a.w[1], 0u, 0u}}, b2{{b.w[0], b.w[1], 0u, 0u}};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a2), __builtin_bit_cast(bf16x8_t, b2),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// fp16 operands (eight per lane, packed in pairs) on the 16x16x32 fp16 instruction
__device__ __forceinline__ f32x4 mma_h(const F32 &a, const F32 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}
// four fp32 -> four fp16 (round to nearest even), element order kept
__device__ __forceinline__ uint2 pack_f16x4(const f32x4 &v) {
  return make_uint2(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]));
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi), both round-to-nearest-even;
// four consecutive k-slots -> two packed words of hi and two of lo
__device__ __forceinline__ void split4(const float *v, uint32_t *hi, uint32_t *lo) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t h = pack_bf16x2(v[2 * p], v[2 * p + 1]);
    hi[p] = h;
    lo[p] = pack_bf16x2(v[2 * p] - __uint_as_float(h << 16), v[2 * p + 1] - __uint_as_float(h & 0xffff0000u));
  }
}
__device__ __forceinline__ void split4(const f32x4 &v, uint32_t *hi, uint32_t *lo) {
  float t[4] = {v[0], v[1], v[2], v[3]};
  split4(t, hi, lo);
}

// Loads of input rows that are read once (q, k in the intra-chunk step), marked
// non-temporal so that they do not push the chunk-head records, which the
// next launch reads back, out of the caches (the 241-frame layer measured 9 %
// faster with these and the streaming stores of o than with neither).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ldg8(const void *p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ldg16(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// q, k, v given as OCP E4M3FN codes: every such value is exact in bf16, so the
// widened rows enter the same bf16 products (and give the same results) as
// bf16 inputs holding those values.  Four codes (code j in byte j of w) -> four
// bf16 in two packed words, element order kept.
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_to_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}
__device__ __forceinline__ uint2 fp8x4_to_bf16(uint32_t w) {
  return make_uint2(fp8x2_to_bf16<false>(w), fp8x2_to_bf16<true>(w));
}
// Eight consecutive input elements as loaded (16 bytes of bf16 or 8 bytes of
// codes), and widened to eight bf16.  Loads and conversions are separate
// steps so that a batch of loads can be issued before the first conversion
// waits on its data.
template <bool kFp8>
using Elems8 = std::conditional_t<kFp8, uint2, uint4>;
template <bool kFp8>
__device__ __forceinline__ Elems8<kFp8> ld_elems8(const char *p) {
  if constexpr (kFp8)
    return ldg8(p);
  else
    return ldg16(p);
}
template <bool kFp8>
__device__ __forceinline__ uint4 elems8_bf16(const Elems8<kFp8> &x) {
  if constexpr (kFp8) {
    const uint2 a = fp8x4_to_bf16(x.x), b = fp8x4_to_bf16(x.y);
    return make_uint4(a.x, a.y, b.x, b.y);
  } else {
    return x;
  }
}

// ---------------------------------------------------------------------------
// Byte offsets of the fragment-ordered fp16 operands inside their record parts.
// K~, Q': token tile t, block kb (d_k 32kb .. 32kb + 31 in the "pair" order of
//    the state's accumulator tiles, 16 B per lane; block 3 holds only its slots
//    0..3, d_k 96 + 4g .. + 3, 8 B per lane: d_k 112.. do not exist).
__device__ __forceinline__ constexpr int kq_off(int t, int kb) { return t * 3584 + kb * 1024; }
// M: tile mt (d_k rows 16mt..), blocks kb 0,1 (tokens 32kb.. paired, 16 B per
//    lane) and the 16-deep block of tokens 64..79 (8 B per lane).
__device__ __forceinline__ constexpr int m_off32(int mt, int kb) { return mt * 2560 + kb * 1024; }
__device__ __forceinline__ constexpr int m_off16(int mt) { return mt * 2560 + 2048; }
// P'' (hi and lo alike): row tile R (tokens 16R..) uses 32-deep blocks over token tiles (0,1),
// (2,3) below its diagonal and, for even R, the 16-deep block of tile R.
__device__ __forceinline__ constexpr int p_base(int R) {
  return R == 0 ? 0 : R == 1 ? 512 : R == 2 ? 1536 : R == 3 ? 3072 : 5120;
}
__device__ __forceinline__ constexpr int p_off32(int R, int kb) { return p_base(R) + kb * 1024; }
__device__ __forceinline__ constexpr int p_off16(int R) { return p_base(R) + (R / 2) * 1024; }
static_assert(p_base(4) + 2560 == kPBytes, "P' record layout");

// Raw buffer access (gfx9 descriptor, stride 0): an offset at or past
// `bytes` reads zero and drops a store.
constexpr uint32_t kOutOfRange = 0x7ffffff0u;
// cache-policy operand of a raw buffer store that streams (the non-temporal
// bit): outputs that nothing in the pass reads back
constexpr int kStreamStore = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), short(0), int(bytes), 0x00020000);
}
// 16 bytes per lane from buffer offset `off` into LDS at dst + 16 * lane
// (dst is wave-uniform); an out-of-range lane writes zeros.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, char *dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, int(off), 0, 0, 0);
}
// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier for waves that compute on LDS operands; it also keeps the
// scheduler from moving register-only work (the matrix products) across it,
// so each phase's products stay on their side of the barrier that hands
// buffers back.
__device__ __forceinline__ void compute_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}
// Barrier for the waves that touch LDS only through the copy engine (or not
// at all): no fence, so no wait on the copies still in flight is implied.
__device__ __forceinline__ void bare_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// lower-triangular 16x16 block index (I >= J)
__device__ __forceinline__ constexpr int tri(int I, int J) { return I * (I + 1) / 2 + J; }

}  // namespace mfma
}  // namespace gdn
