// Kernel "scan" of the MFMA family: the sequential state pass fused with the
// output, plus the intra-chunk step of the next chunk range, in one launch.
//
// A forward pass over N chunks of 80 tokens runs as a short sequence of
// launches of one kernel over chunk ranges r_0, r_1, ...:
//   launch 0:  intra(r_0)
//   launch j:  state pass(r_{j-1})  +  intra(r_j)       (j >= 1)
// Blocks [0, n_chain) run the state pass, the rest the intra-chunk step
// (gdn_intra.h, two chunk-heads per block).  The state-pass blocks come
// first, so they are placed first, one per CU (their LDS fills a CU); the
// intra blocks fill the remaining CUs.  No block waits on another: the
// records of range r_{j-1} were written by the previous launch, and stream
// order is the only synchronisation.  The state is carried from one range to
// the next in the workspace.
//
// State pass, per chunk (the algebra is in gdn_mfma_common.h), with the
// chunk's record (K~, Q', P'', M, a = beta, gamma_n):
//   R = diag(a) V + K~ S^T,   S^T <- gamma_n S^T + M R,   O = Q' S^T + P'' V.
// Each product accumulates onto the term before it (a V, gamma_n S^T, Q' S^T).
// The output needs S of the chunk's start and the chunk's own rows only, not R.
// One workgroup per (b, h, pair of 16-column tiles of d_v): 4 workgroups per
// head (tiles 0-1, 2-3, 4-5, 6).  Eight waves:
//   0, 2  "state" wave of local tile 0, 1: holds the tile's 112 x 16 fp32 slice
//         of S^T in registers (7 accumulator tiles of 16 x 16), computes R and
//         the update M R; publishes S as an fp16 operand image in LDS for the
//         output wave.
//   1, 3  "output" wave of local tile 0, 1: Q' S^T + P'' V, the output rows.
//   4-7   copy waves: buffer-to-LDS loads (16 bytes per lane, no register
//         round trip) of the chunk's record and of this workgroup's V columns.
// Two barriers per chunk: X opens chunk c (its record and V rows landed; S
// of chunk c published); by Y every wave has read what it needs of chunk c's
// buffer and of the S image into registers.
//
// Buffers: records and V rows are double-buffered, so chunk c + 2's record
// and rows are copied from Y(c) on; the S image is rewritten after Y(c).
//
// Operand orders.  All products use the "pair" k-order, in which two 16-row
// accumulator tiles (rows 4g .. 4g + 3 of each in lane group g) already are
// one 32-deep operand: S and R go from the accumulators to the next product
// without moving between lanes, and the record stores K~, Q', M and P'' in
// that order.
#include <algorithm>
#include <vector>

#include "gdn_intra.h"

namespace gdn {
namespace mfma {
namespace {

constexpr int kTPW = 2;                          // 16-column tiles of d_v per state-pass workgroup
constexpr int kGroups = (NT + kTPW - 1) / kTPW;  // workgroups per (b, h)
constexpr int kThreads = 512;
constexpr int kRecInstr = kRecBytes / 1024;  // 1 KB copies of one record (68)
static_assert(kRecBytes % 1024 == 0, "whole 1 KB record copies");
constexpr int kCopyWaves = 4;

// One buffer of chunk operands, for bf16 (kFp8 false) or E4M3FN (kFp8 true) V rows.
template <bool kFp8>
struct Buf {
  static constexpr int kElem = kFp8 ? 1 : 2;      // bytes per input element
  static constexpr int kVRow = kTPW * 16 * kElem; // bytes per staged V row: this workgroup's columns
  static constexpr int kVSlots = C * kVRow / 16;
  static constexpr int kVInstr = (kVSlots + 63) / 64;
  static constexpr int kRec = 0;                  // the record (parts A and B)
  static constexpr int kV = kRecBytes;
  static constexpr int kBytes = kV + C * kVRow;   // 74,752 / 72,192
  // after the two buffers: per local tile the S image (4 x 1 KB) and its scale
  // exponent
  static constexpr int kSImg = 2 * kBytes;
  static constexpr int kExp = kSImg + kTPW * 4096;  // per tile: S exponent
  static constexpr int kLds = kExp + 32;
  static_assert(kV % 16 == 0 && kBytes % 16 == 0 && kRecBytes % 16 == 0, "16-byte aligned copy targets");
};
constexpr int kScanLds = std::max({Buf<false>::kLds, Buf<true>::kLds, 2 * kLdsIntra});
static_assert(kScanLds <= 160 * 1024, "one CU's LDS");

// Arguments of one launch.
struct ScanArgs {
  const char *q, *k, *v;
  const float *g, *beta;
  const float *state_in;  // entry state of the state-pass range (NULL = zero)
  float *state_out;       // exit state of the range (NULL = not written)
  void *o;
  // state pass over chunks [cb, ce): the record of (u, c) at rec + ((c - cb) * units + u) * kRecBytes
  const char *rec;
  int cb, ce;
  // intra over chunks [ib, ie): records written at irec + ((c - ib) * units + u) * kRecBytes
  char *irec;
  int ib, ie;
  int T, H, units, n_chain;
  uint32_t flags;
};

// F32 of four packed words
__device__ __forceinline__ F32 f32_of(uint32_t a, uint32_t b, uint32_t c, uint32_t d) { return F32{{a, b, c, d}}; }

// largest |x| over the wave (DPP row reductions, then the two halves)
__device__ __forceinline__ float wave_max_abs(float x) {
  x = fabsf(x);
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, true)));  // quad_perm 1,0,3,2
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, true)));  // quad_perm 2,3,0,1
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, true)));  // row_half_mirror
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, true)));  // row_mirror
  const float r0 = lane_value(x, 0), r1 = lane_value(x, 16), r2 = lane_value(x, 32), r3 = lane_value(x, 48);
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The scaling code below runs only when a tile leaves fp16's comfortable
// range, which normal inputs never do.  Left alone, the compiler would
// evaluate it on every chunk (x 2^0 == x); the empty volatile statement makes
// the block a real, wave-uniform branch instead.
__device__ __forceinline__ bool rare_branch_mark() {
  asm volatile("");
  return true;
}
#define GDN_RARELY(cond) if (__builtin_expect(bool(cond), 0) && rare_branch_mark())

// Scale exponent of a tile whose largest magnitude is m: 0 while m lies in
// [2^-6, 2^15) (fp16 then holds the tile in its normal range); otherwise s with
// m 2^-s in [2^14, 2^15).  0 for m = 0, infinite or NaN (those pass unscaled).
__device__ __forceinline__ int range_exponent(float m) {
  const bool in_range = m >= 0x1p-6f && m < 0x1p15f;
  const bool finite = m > 0.f && m < __builtin_huge_valf();
  return (!in_range && finite) ? __builtin_amdgcn_frexp_expf(m) - 15 : 0;
}

// Scale exponent of a tile from each lane's largest magnitude m: a wave vote
// settles the common case (no lane at or above 2^15 and some lane at or above
// 2^-6, so the tile's maximum lies in [2^-6, 2^15) and the exponent is 0); only
// otherwise is the maximum reduced over the wave.
__device__ __forceinline__ int tile_exponent(float m) {
  int s = 0;
  GDN_RARELY(__builtin_amdgcn_ballot_w64(!(m < 0x1p15f)) != 0 || __builtin_amdgcn_ballot_w64(m >= 0x1p-6f) == 0) {
    s = range_exponent(wave_max_abs(m));
  }
  return s;
}

// One lane's K~ or Q~ fragment of token tile t, block kb (pair k-order over
// d_k) from a record image; block 3 holds slots 0..3 only (8 bytes per lane).
__device__ __forceinline__ F32 kq_frag(const char *img, int t, int kb, int lane) {
  if (kb < 3) {
    const uint4 x = *reinterpret_cast<const uint4 *>(img + kq_off(t, kb) + 16 * lane);
    return F32{{x.x, x.y, x.z, x.w}};
  }
  const uint2 x = *reinterpret_cast<const uint2 *>(img + kq_off(t, 3) + 8 * lane);
  return F32{{x.x, x.y, 0u, 0u}};
}
// acc[t] += rows(t) x S'^T over d_k for the five token tiles (fp16 operands):
// five independent chains of four products (a chain's next product issues
// five products later, past the instruction's dependent latency).  The
// 16-deep last block runs on the 16x16x32 instruction with zero slots 4-7.
__device__ __forceinline__ void rows_times_S(const char *img, int lane, const F32 *Sop, f32x4 *acc) {
  F32 f[4][CT];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int t = 0; t < CT; ++t) f[kb][t] = kq_frag(img, t, kb, lane);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int t = 0; t < CT; ++t)
      acc[t] = mma_h(f[kb][t], Sop[kb], acc[t]);
}

// ---------------------------------------------------------------------------
// State wave of local tile jl (d_v columns 16 j .. 16 j + 15, j = tile0 + jl).
template <bool kFp8>
__device__ __forceinline__ void state_role(const ScanArgs &a, int b, int h, int j, int jl, char *lds) {
  using G = Buf<kFp8>;
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const size_t u = size_t(b) * a.H + h;
  char *Simg = lds + G::kSImg + jl * 4096;
  int *exps = reinterpret_cast<int *>(lds + G::kExp) + jl;

  // S^T tile i: accumulator rows d_k = 16 i + 4 lg + e, column d_v = 16 j + ln
  f32x4 St[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    St[i] = zero4();
    if (a.state_in) {
      const float4 t = *reinterpret_cast<const float4 *>(a.state_in + (u * D + 16 * j + ln) * D + 16 * i + 4 * lg);
      St[i] = f32x4{t.x, t.y, t.z, t.w};
    }
  }
  // fp16 operand blocks of S 2^-sS (pair k-order: accumulator tiles 2kb, 2kb + 1
  // as they are), also published for the output wave
  F32 Sop[4];
  int sS = 0;
  auto build_S = [&]() {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(St[i][e]));
    sS = tile_exponent(m);
    uint2 x[8];
    f32x4 Ss[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) Ss[i] = St[i];
    GDN_RARELY(sS) {
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) Ss[i][e] = __builtin_ldexpf(Ss[i][e], -sS);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) x[i] = pack_f16x4(Ss[i]);
    x[7] = make_uint2(0u, 0u);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Sop[kb] = f32_of(x[2 * kb].x, x[2 * kb].y, x[2 * kb + 1].x, x[2 * kb + 1].y);
      *reinterpret_cast<uint4 *>(Simg + kb * 1024 + lane * 16) = make_uint4(Sop[kb].w[0], Sop[kb].w[1], Sop[kb].w[2], Sop[kb].w[3]);
    }
    if (lane == 0) exps[0] = sS;
  };
  build_S();

  for (int c = a.cb; c < a.ce; ++c) {
    const char *buf = lds + (c & 1) * G::kBytes;
    const float *cs = reinterpret_cast<const float *>(buf + kRecCs);
    compute_barrier();  // X(c)
    // ---- Y = K~ S'^T from zero accumulators, so that the products wait only
    // for the K~ fragments (read first), not for the V rows
    f32x4 Y[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) Y[t] = zero4();
    rows_times_S(buf + kRecK, lane, Sop, Y);
    // ---- R = a V + 2^sS Y
    f32x4 Racc[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      const float4 x = *reinterpret_cast<const float4 *>(cs + 16 * t + 4 * lg);
      const float xa[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * t + 4 * lg + e;
        float vv;
        if constexpr (kFp8)
          vv = __builtin_amdgcn_cvt_pk_f32_fp8(uint32_t(reinterpret_cast<const uint8_t *>(buf + G::kV)[r * G::kVRow + 16 * jl + ln]), false)[0];
        else
          vv = bf16_to_f32(reinterpret_cast<const uint16_t *>(buf + G::kV)[r * (G::kVRow / 2) + 16 * jl + ln]);
        Racc[t][e] = xa[e] * vv;
      }
    }
    // the update accumulates onto gamma_n S^T in place (gamma_n is 1 on every
    // chunk without a frame's first token)
    const float gamma_n = cs[kCsGammaN];
    GDN_RARELY(gamma_n != 1.f) {
#pragma unroll
      for (int i = 0; i < NT; ++i) St[i] = St[i] * gamma_n;
    }
    GDN_RARELY(sS) {
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) Racc[t][e] += __builtin_ldexpf(Y[t][e], sS);
    } else {
#pragma unroll
      for (int t = 0; t < CT; ++t) Racc[t] = Racc[t] + Y[t];
    }
    // M's fragments only now (before Y(c)): read earlier, they would queue in
    // front of K~'s in LDS and hold 84 more registers across the products
    __builtin_amdgcn_sched_barrier(0);
    const char *Mr = buf + kRecM;
    F32 mf[3][NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const uint4 x0 = *reinterpret_cast<const uint4 *>(Mr + m_off32(i, 0) + lane * 16);
      const uint4 x1 = *reinterpret_cast<const uint4 *>(Mr + m_off32(i, 1) + lane * 16);
      const uint2 x2 = *reinterpret_cast<const uint2 *>(Mr + m_off16(i) + lane * 8);
      mf[0][i] = f32_of(x0.x, x0.y, x0.z, x0.w);
      mf[1][i] = f32_of(x1.x, x1.y, x1.z, x1.w);
      mf[2][i] = f32_of(x2.x, x2.y, 0u, 0u);
    }
    // ---- R scaled by 2^-sR into fp16 pair-order operand blocks
    float mx = 0.f;
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(Racc[t][e]));
    const int sR = tile_exponent(mx);
    GDN_RARELY(sR) {
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) Racc[t][e] = __builtin_ldexpf(Racc[t][e], -sR);
    }
    uint2 rw[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) rw[t] = pack_f16x4(Racc[t]);
    const F32 Rb0 = f32_of(rw[0].x, rw[0].y, rw[1].x, rw[1].y);
    const F32 Rb1 = f32_of(rw[2].x, rw[2].y, rw[3].x, rw[3].y);
    const F32 Rb2 = f32_of(rw[4].x, rw[4].y, 0u, 0u);
    compute_barrier();  // Y(c): chunk c's record and V are no longer read
    // ---- S^T <- gamma_n S^T + 2^sR M R': seven chains of three products (the
    // 16-deep last one padded, as everywhere in this kernel)
    GDN_RARELY(sR) {
      f32x4 U[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) U[i] = zero4();
#pragma unroll
      for (int kb = 0; kb < 3; ++kb)
#pragma unroll
        for (int i = 0; i < NT; ++i)
          U[i] = mma_h(mf[kb][i], kb == 0 ? Rb0 : kb == 1 ? Rb1 : Rb2, U[i]);
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) St[i][e] += __builtin_ldexpf(U[i][e], sR);
    } else {
#pragma unroll
      for (int kb = 0; kb < 3; ++kb)
#pragma unroll
        for (int i = 0; i < NT; ++i)
          St[i] = mma_h(mf[kb][i], kb == 0 ? Rb0 : kb == 1 ? Rb1 : Rb2, St[i]);
    }
    // S of chunk c + 1: the output wave read S of chunk c before Y(c)
    build_S();
  }
  if (a.state_out) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
      *reinterpret_cast<float4 *>(a.state_out + (u * D + 16 * j + ln) * D + 16 * i + 4 * lg) =
          make_float4(St[i][0], St[i][1], St[i][2], St[i][3]);
  }
}

// ---------------------------------------------------------------------------
// Output wave of local tile jl: O = Q' S^T + P'' V.
template <bool kOutBf16, bool kFp8, bool kRev>
__device__ __forceinline__ void output_role(const ScanArgs &a, int b, int h, int j, int jl, char *lds) {
  using G = Buf<kFp8>;
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const char *Simg = lds + G::kSImg + jl * 4096;
  const int *exps = reinterpret_cast<const int *>(lds + G::kExp) + jl;
  const size_t rowstride = size_t(a.H) * D;
  auto ld128 = [](const char *p) {
    const uint4 x = *reinterpret_cast<const uint4 *>(p);
    return f32_of(x.x, x.y, x.z, x.w);
  };
  auto ld64 = [](const char *p) {
    const uint2 x = *reinterpret_cast<const uint2 *>(p);
    return f32_of(x.x, x.y, 0u, 0u);
  };
  for (int c = a.cb; c < a.ce; ++c) {
    const int t0 = c * C, nv = min(C, a.T - t0);
    const int p0 = kRev ? a.T - t0 - nv : t0;  // first physical row of the chunk
    const char *buf = lds + (c & 1) * G::kBytes;
    compute_barrier();  // X(c)
    F32 Sop[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Sop[kb] = ld128(Simg + kb * 1024 + lane * 16);
    const int sS = exps[0];
    // P'' fragments (hi and lo) and this tile's V columns as bf16 B operands in
    // pair order: token tiles (0, 1), (2, 3) and 4 alone; rows past the chunk's
    // end hold zeros
    const char *Ph = buf + kRecP, *Pl = buf + kRecPl;
    F32 ph[9], pl[9];
    {
      const int off[9] = {p_off16(0), p_off32(1, 0), p_off32(2, 0), p_off16(2), p_off32(3, 0),
                          p_off32(3, 1), p_off32(4, 0), p_off32(4, 1), p_off16(4)};
      const bool wide[9] = {false, true, true, false, true, true, true, true, false};
#pragma unroll
      for (int x = 0; x < 9; ++x) {
        ph[x] = wide[x] ? ld128(Ph + off[x] + lane * 16) : ld64(Ph + off[x] + lane * 8);
        pl[x] = wide[x] ? ld128(Pl + off[x] + lane * 16) : ld64(Pl + off[x] + lane * 8);
      }
    }
    uint32_t vw[CT][2];
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      float vv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * t + 4 * lg + e;
        if constexpr (kFp8)
          vv[e] = __builtin_amdgcn_cvt_pk_f32_fp8(uint32_t(reinterpret_cast<const uint8_t *>(buf + G::kV)[r * G::kVRow + 16 * jl + ln]), false)[0];
        else
          vv[e] = bf16_to_f32(reinterpret_cast<const uint16_t *>(buf + G::kV)[r * (G::kVRow / 2) + 16 * jl + ln]);
      }
      // exact: every value here is a bf16 (or an E4M3 code, exact in bf16)
      vw[t][0] = (__float_as_uint(vv[0]) >> 16) | (__float_as_uint(vv[1]) & 0xffff0000u);
      vw[t][1] = (__float_as_uint(vv[2]) >> 16) | (__float_as_uint(vv[3]) & 0xffff0000u);
    }
    const F32 Vb0 = f32_of(vw[0][0], vw[0][1], vw[1][0], vw[1][1]);
    const F32 Vb1 = f32_of(vw[2][0], vw[2][1], vw[3][0], vw[3][1]);
    const F32 Vh0 = f32_of(vw[0][0], vw[0][1], 0u, 0u), Vh2 = f32_of(vw[2][0], vw[2][1], 0u, 0u);
    const F32 Vh4 = f32_of(vw[4][0], vw[4][1], 0u, 0u);
    // ---- Q' S'^T (Q' S^T = 2^sS of it)
    f32x4 O[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) O[t] = zero4();
    rows_times_S(buf + kRecQ, lane, Sop, O);
    GDN_RARELY(sS) {
#pragma unroll
      for (int t = 0; t < CT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) O[t][e] = __builtin_ldexpf(O[t][e], sS);
    }
    compute_barrier();  // Y(c): chunk c's buffer and the S image are no longer read
    // ---- + P'' V (bf16 hi and lo against the exact rows)
    const F32 *vb[9] = {&Vh0, &Vb0, &Vb0, &Vh2, &Vb0, &Vb1, &Vb0, &Vb1, &Vh4};
    const int row_tile[9] = {0, 1, 2, 2, 3, 3, 4, 4, 4};
#pragma unroll
    for (int x = 0; x < 9; ++x) O[row_tile[x]] = mma(ph[x], *vb[x], O[row_tile[x]]);
#pragma unroll
    for (int x = 0; x < 9; ++x) O[row_tile[x]] = mma(pl[x], *vb[x], O[row_tile[x]]);
    // the chunk's rows of o: logical row r at physical row p0 + r (p0 + nv - 1 - r
    // reversed).  All values first, then the stores, each from its own register
    // (a store that reuses a register holds the next value back until it is sent).
    float val[CT][4];
    uint32_t ob[CT][4];
    constexpr uint32_t kOutBytes = kOutBf16 ? 2u : 4u;
#pragma unroll
    for (int t = 0; t < CT; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        val[t][e] = O[t][e];
        const int r = 16 * t + 4 * lg + e;
        // rows past the chunk's end are aimed outside the store descriptor and dropped
        const uint32_t oi = uint32_t(kRev ? nv - 1 - r : r) * uint32_t(rowstride) + uint32_t(h) * D + 16u * j + ln;
        ob[t][e] = r < nv ? oi * kOutBytes : kOutOfRange;
      }
    }
    const auto ro = make_rsrc(static_cast<char *>(a.o) + (size_t(b) * a.T + p0) * rowstride * kOutBytes,
                              uint32_t(nv) * uint32_t(rowstride) * kOutBytes);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < CT; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (kOutBf16)
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(val[t][e]), ro, int(ob[t][e]), 0, kStreamStore);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val[t][e]), ro, int(ob[t][e]), 0, kStreamStore);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Copy wave L (0..3): the chunk record's 1 KB pieces i with i % 4 == L and
// (L == 3) this workgroup's V columns.  Every read of chunk c's buffer happens
// before barrier Y(c), so chunk c + 2's copies may be issued from Y(c) on and
// must land before X(c + 2).  The copies of a chunk take about as long to
// issue as a chunk takes to compute (the memory pipeline accepts a load only
// as fast as earlier ones drain), so they are issued in two parts: part A of
// chunk c + 2 after Y(c), part B after X(c + 1); no barrier waits for a whole
// chunk's issue.  Loads complete in issue order, so each wait names the
// younger loads that may stay in flight (part A of the next chunk).  An
// instruction none of whose lanes is in range may complete ahead of older
// ones, so the loads a wait leaves in flight must each have a lane in range:
// part A holds record pieces only, which always lie in range.  (One-dword
// touches of later chunks' lines, issued to warm L2 ahead of the copies,
// measured 4.5 % slower than none.)
template <int L, bool kFp8, bool kRev>
__device__ __forceinline__ void copy_role(const ScanArgs &a, int b, int h, int tile0, int ntiles, char *lds) {
  using G = Buf<kFp8>;
  const int lane = threadIdx.x & 63;
  const size_t u = size_t(b) * a.H + h;
  const uint32_t row_bytes = uint32_t(a.H) * D * G::kElem;
  const uint32_t head_off = uint32_t(h) * D * G::kElem;
  constexpr int kLast = kCopyWaves - 1;
  // record pieces of this wave per chunk, the first kA of them in part A;
  // part B holds the rest and (L == 3) the V rows.  Part A is about a sixth
  // of the wave's copies (the 241-frame layer measured 0.515 / 0.513 / 0.502 /
  // 0.502 / 0.503 ms with a half / third / quarter / sixth / none in part A):
  // copies issued right after Y(c) slow the state waves' update that follows.
  constexpr int kPieces = (kRecInstr - L + kCopyWaves - 1) / kCopyWaves;
  constexpr int kA = (kPieces + (L == kLast ? G::kVInstr : 0)) / 6;
  constexpr int cN = kPieces + (L == kLast ? G::kVInstr : 0);
  static_assert(cN + kA < 64, "vmcnt holds 63");
  // part A (kPart 0) or B (kPart 1) of chunk c's copies
  auto copy_part = [&](int c, auto part) {
    constexpr int kPart = decltype(part)::value;
    const auto rr = make_rsrc(a.rec + (size_t(c - a.cb) * a.units + u) * kRecBytes, kRecBytes);
    char *dst = lds + (c & 1) * G::kBytes + G::kRec;
#pragma unroll
    for (int x = 0; x < kPieces; ++x) {
      const int i = L + kCopyWaves * x;
      if ((x < kA) == (kPart == 0)) copy16(rr, dst + 1024 * i, 1024u * i + 16u * lane);
    }
    if constexpr (L == kLast && kPart == 1) {
      // this workgroup's columns of each row; a missing second tile reads as zero
      const int t0 = c * C, nv = min(C, a.T - t0);
      const int p0 = kRev ? a.T - t0 - nv : t0;
      const auto rs = make_rsrc(a.v + (size_t(b) * a.T + p0) * row_bytes, uint32_t(nv) * row_bytes);
      char *vd = lds + (c & 1) * G::kBytes + G::kV;
#pragma unroll
      for (int i = 0; i < G::kVInstr; ++i) {
        constexpr int kPer = G::kVRow / 16;
        const int slot = 64 * i + lane, r = slot / kPer, p = slot % kPer;
        const int tile = tile0 + (p * 16) / (16 * G::kElem);
        const uint32_t off =
            (r < nv && tile < tile0 + ntiles)
                ? uint32_t(kRev ? nv - 1 - r : r) * row_bytes + head_off + uint32_t(tile0 * 16 * G::kElem) + 16u * p
                : kOutOfRange;
        if (slot < G::kVSlots) copy16(rs, vd + 1024 * i, off);
      }
    }
  };
  constexpr auto kPartA = std::integral_constant<int, 0>{};
  constexpr auto kPartB = std::integral_constant<int, 1>{};
  const int cb = a.cb, ce = a.ce;
  if (cb < ce) {
    copy_part(cb, kPartA);
    copy_part(cb, kPartB);
    if (cb + 1 < ce) copy_part(cb + 1, kPartA);
  }
  for (int c = cb; c < ce; ++c) {
    // issued after chunk c's last copy: part A of c + 1 (if c + 1 < ce)
    if (c + 1 < ce)
      wait_vm<kA>();
    else
      wait_vm<0>();
    bare_barrier();  // X(c)
    if (c + 1 < ce) copy_part(c + 1, kPartB);
    bare_barrier();  // Y(c)
    if (c + 2 < ce) copy_part(c + 2, kPartA);
  }
  wait_vm<0>();
}

// a wave with no tile (the last workgroup of a head has one): meets the barriers
__device__ __forceinline__ void idle_role(const ScanArgs &a) {
  for (int c = a.cb; c < a.ce; ++c) {
    bare_barrier();
    bare_barrier();
  }
}

template <bool kOutBf16, bool kFp8, bool kRev>
__global__ __launch_bounds__(kThreads, 1) void scan_kernel(ScanArgs a) {
  extern __shared__ __align__(16) char lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (int(blockIdx.x) < a.n_chain) {
    // Workgroup i runs on XCD i % 8: the four workgroups of a (b, h) share one
    // XCD, so its K, Q and records are fetched from HBM once into that L2.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int u = xcd + 8 * (slot / kGroups), gi = slot % kGroups;
    if (u >= a.units) return;
    const int b = u / a.H, h = u % a.H;
    const int tile0 = gi * kTPW, ntiles = min(kTPW, NT - tile0);
    if (wave < 2 * kTPW) {
      const int jl = wave >> 1;
      if (jl >= ntiles)
        idle_role(a);
      else if (wave & 1)
        output_role<kOutBf16, kFp8, kRev>(a, b, h, tile0 + jl, jl, lds);
      else
        state_role<kFp8>(a, b, h, tile0 + jl, jl, lds);
    } else if (wave == 4) {
      copy_role<0, kFp8, kRev>(a, b, h, tile0, ntiles, lds);
    } else if (wave == 5) {
      copy_role<1, kFp8, kRev>(a, b, h, tile0, ntiles, lds);
    } else if (wave == 6) {
      copy_role<2, kFp8, kRev>(a, b, h, tile0, ntiles, lds);
    } else {
      copy_role<3, kFp8, kRev>(a, b, h, tile0, ntiles, lds);
    }
    return;
  }
  // intra-chunk step: two chunk-heads per block (waves 0-3 and 4-7), heads
  // fastest, the range's chunks last to first
  const int group = wave >> 2;
  const int qi = 2 * (int(blockIdx.x) - a.n_chain) + group;
  const int n_r = a.ie - a.ib;
  const bool valid = qi < a.units * n_r;
  const int u = valid ? qi % a.units : 0;
  const int c = valid ? a.ie - 1 - qi / a.units : a.ib;
  char *rec = a.irec + (size_t(c - a.ib) * a.units + u) * kRecBytes;
  intra_chunk<kFp8>(lds + group * kLdsIntra, a.q, a.k, a.g, a.beta, rec, a.T, a.H, u / a.H, u % a.H, c, a.flags,
                    threadIdx.x & 255, valid);
}

template <bool kOutBf16, bool kFp8, bool kRev>
hipError_t launch_typed(const ScanArgs &a, unsigned blocks, hipStream_t st) {
  // more than the default 64 KB of dynamic LDS (gfx950 has 160 KB per CU), once per instantiation
  static const hipError_t lds_ok =
      hipFuncSetAttribute(reinterpret_cast<const void *>(&scan_kernel<kOutBf16, kFp8, kRev>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kScanLds);
  if (lds_ok != hipSuccess) return lds_ok;
  scan_kernel<kOutBf16, kFp8, kRev><<<dim3(blocks), dim3(kThreads), kScanLds, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_one(const Plan &p, const ScanArgs &a, unsigned blocks, hipStream_t st) {
  const bool rev = p.flags & kReverse;
  if (p.qkv_fp8) {
    if (rev) return p.o_bf16 ? launch_typed<true, true, true>(a, blocks, st) : launch_typed<false, true, true>(a, blocks, st);
    return p.o_bf16 ? launch_typed<true, true, false>(a, blocks, st) : launch_typed<false, true, false>(a, blocks, st);
  }
  if (rev) return p.o_bf16 ? launch_typed<true, false, true>(a, blocks, st) : launch_typed<false, false, true>(a, blocks, st);
  return p.o_bf16 ? launch_typed<true, false, false>(a, blocks, st) : launch_typed<false, false, false>(a, blocks, st);
}

}  // namespace
}  // namespace mfma

size_t mfma_record_bytes() { return mfma::kRecBytes; }

// Chunk ranges: a short first range (its intra-chunk step runs alone), then
// ranges of at most `cap` chunks.
void mfma_ranges(int N, int cap, std::vector<int> &bounds) {
  bounds.assign(1, 0);
  if (N <= 0) return;
  bounds.push_back(std::min(N, std::min(kFirstRange, cap)));
  while (bounds.back() < N) bounds.push_back(std::min(N, bounds.back() + cap));
}

hipError_t launch_mfma(const Plan &p, const Args &a) {
  std::vector<int> bounds;
  mfma_ranges(p.N, p.range_cap, bounds);
  const int R = int(bounds.size()) - 1;
  const int units = p.B * p.H;
  char *ring = a.ws + p.off_rec;
  const size_t slot_bytes = size_t(p.range_cap) * units * mfma::kRecBytes;
  float *carry = reinterpret_cast<float *>(a.ws + p.off_carry);
  mfma::ScanArgs sa{};
  sa.q = static_cast<const char *>(a.q);
  sa.k = static_cast<const char *>(a.k);
  sa.v = static_cast<const char *>(a.v);
  sa.g = a.g;
  sa.beta = a.beta;
  sa.o = a.o;
  sa.T = p.T;
  sa.H = p.H;
  sa.units = units;
  sa.flags = p.flags;
  const unsigned chain_blocks = 8u * mfma::kGroups * unsigned((units + 7) / 8);
  for (int j = 0; j <= R; ++j) {
    // state pass over range j - 1 (if any) and intra over range j (if any)
    sa.n_chain = 0;
    sa.cb = sa.ce = 0;
    if (j >= 1) {
      sa.n_chain = int(chain_blocks);
      sa.cb = bounds[j - 1];
      sa.ce = bounds[j];
      sa.rec = ring + ((j - 1) & 1) * slot_bytes;
      sa.state_in = j == 1 ? a.state_in : carry;
      sa.state_out = j == R ? a.state_out : carry;
    }
    unsigned intra_blocks = 0;
    sa.ib = sa.ie = 0;
    if (j < R) {
      sa.ib = bounds[j];
      sa.ie = bounds[j + 1];
      sa.irec = ring + (j & 1) * slot_bytes;
      intra_blocks = unsigned((size_t(units) * (sa.ie - sa.ib) + 1) / 2);
    }
    const hipError_t e = mfma::launch_one(p, sa, unsigned(sa.n_chain) + intra_blocks, a.stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
