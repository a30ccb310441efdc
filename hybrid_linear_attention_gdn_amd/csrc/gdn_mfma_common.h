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
//
// Kernel "intra" (one workgroup per (b, h, chunk), fully parallel) forms A and
// P from K K^T and K Q^T on the matrix cores, solves T in LDS (fp32), and then
// M and P' on the matrix cores.  It stores M and P' already split into bf16
// hi + lo pairs in the exact register order the state pass consumes, and the
// per-token scales.  Kernel "chain" (one workgroup per (b, h, 16 columns of
// d_v), sequential over chunks) keeps its 16 x 112 slice of the fp32 state in
// registers and runs the four products above per chunk.
//
// Precision: q, k, v enter the matrix cores as the exact bf16 inputs; every
// derived operand (S, R, M, P', T) is split x = hi + lo with hi = bf16(x),
// lo = bf16(x - hi) and multiplied as hi*hi + hi*lo + lo*hi (or hi*raw +
// lo*raw), accumulating in fp32 -- a relative error near 2^-16 per operand
// instead of bf16's unit roundoff 2^-8.
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

// bytes per chunk-head of the precomputed operands
constexpr int kMBytes = NT * 5120;  // 7 d_k tiles x (2 K32 blocks + 1 K16 block) x hi/lo
constexpr int kPBytes = 15360;      // lower-triangular token blocks of P', hi/lo
constexpr int kCsFloats = 256;      // a[80], b[80], c[80], gamma_n, pad

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
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
// A 16-deep block runs on the same 16x16x32 instruction with slots 4-7 of
// both operands zero: one MFMA opcode throughout keeps every dependent
// accumulation chain on a single instruction latency.
__device__ __forceinline__ f32x4 mma(const F16 &a, const F16 &b, f32x4 c) {
  const F32 a2{{a.w[0], a.w[1], 0u, 0u}}, b2{{b.w[0], b.w[1], 0u, 0u}};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a2), __builtin_bit_cast(bf16x8_t, b2),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

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

__device__ __forceinline__ uint2 ldg8(const void *p) { return *reinterpret_cast<const uint2 *>(p); }
__device__ __forceinline__ uint4 ldg16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

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
// Byte offsets of the fragment-ordered operands inside one chunk-head record.
// M: tile mt (d_k rows 16mt..), blocks kb 0,1 (tokens 32kb.. paired, 16 B per
//    lane) and the 16-deep block of tokens 64..79 (8 B per lane); hi then lo.
__device__ __forceinline__ int m_off32(int mt, int kb, int hl) { return mt * 5120 + kb * 2048 + hl * 1024; }
__device__ __forceinline__ int m_off16(int mt, int hl) { return mt * 5120 + 4096 + hl * 512; }
// P': row tile R (tokens 16R..) uses 32-deep blocks over token tiles (0,1),
// (2,3) below its diagonal and, for even R, the 16-deep block of tile R.
__device__ __forceinline__ int p_base(int R) {
  return R == 0 ? 0 : R == 1 ? 1024 : R == 2 ? 3072 : R == 3 ? 6144 : 10240;
}
__device__ __forceinline__ int p_off32(int R, int kb, int hl) { return p_base(R) + kb * 2048 + hl * 1024; }
__device__ __forceinline__ int p_off16(int R, int hl) { return p_base(R) + (R / 2) * 2048 + hl * 512; }

// Raw buffer access (gfx9 descriptor, stride 0): an offset at or past
// `bytes` reads zero and drops a store.
constexpr uint32_t kOutOfRange = 0x7ffffff0u;
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

// Launches the intra kernel writing M, P' and the chunk scales of chunks
// c_first .. c_end - 1 of every (b, h) on `stream` (gdn_intra.hip).
hipError_t launch_intra(const Plan &p, const Args &a, char *M, char *P, float *cs, int c_first, int c_end,
                        hipStream_t stream);

}  // namespace mfma
}  // namespace gdn
