// Kernel "chain" of the MFMA family: the sequential state pass fused with the
// output, one workgroup per (b, h, 16 columns of d_v).
//
// Per chunk (the algebra is in gdn_mfma_common.h):
//   Y = K S^T,  R = diag(beta) V - diag(beta gamma rk) Y,
//   O = diag(gamma rq) Q S^T + P' R,   S^T <- gamma_n S^T + M R.
// The 16 x 112 fp32 state slice S^T lives in accumulator registers as 7 row
// tiles spread over four compute waves.  Two barriers per chunk: X opens
// chunk c (S published as bf16 hi/lo B operands, the chunk's rows and record
// landed in LDS), Y follows phase A (R published; every other LDS operand
// of the chunk already read into registers).
//
// Wave roles (eight waves, two per SIMD):
//   0-3  compute: every operand comes from LDS; they issue no global load,
//        only the output stores.
//   4-6  copy: buffer-to-LDS loads (16 bytes per lane, no register round
//        trip) of the chunk's M and P' record, scales, K and Q rows and this
//        workgroup's 16 columns of V.  Each copy wave waits on exact counts of
//        its own loads, so later copies stay in flight across the barriers.
//   7    L2 warm-up of a chunk two steps ahead.
// With one wave per SIMD doing everything, a load that cannot issue blocks
// the matrix instructions queued behind it in that wave; split this way, the
// compute waves keep issuing while the copy waves wait on the memory system.
//
// Buffers.  Rows (K, Q, V, scales) are double-buffered and the M / P' record
// single-buffered.  Phase A reads all of them, so at barrier Y both the
// record buffer and row buffer c & 1 are free: the copy waves then issue
// chunk c + 1's record (due at X of c + 1) and chunk c + 2's rows.  With fp8
// rows there is room for a second record buffer: chunk c's record then sits
// in buffer c & 1 and is copied together with its rows, a chunk ahead.
//
// K and Q rows sit at a 256-byte stride with their 16-byte pieces permuted
// by row (slot = piece ^ (row & 15)), so the 16-byte fragment reads of 16
// consecutive rows hit 16 distinct bank groups.  With fp8 (E4M3FN) inputs the
// rows are staged as they are (112 bytes at a 128-byte stride, slot = piece ^
// (row & 7)) and widened to bf16 as the compute waves read their fragments:
// the copies move half the bytes and the products are those of bf16 inputs
// holding the same values.  The products K S^T and
// Q S^T use the instruction's natural k-order (lane group g holds k = 8g ..
// 8g + 7), which makes each K/Q fragment one contiguous 16-byte read; the
// state tiles are written to LDS in that order.  The products with R keep
// the "pair" k-order of the M and P' records.
#include "gdn_mfma_common.h"

#include <algorithm>
#include <mutex>
#include <vector>

namespace gdn {
namespace mfma {
namespace {

struct Roles {
  int nY, Y[2];    // token tiles whose Y = K S^T and R this wave computes (phase A)
  int nQA, QA[1];  // token tiles whose Q S^T it computes in phase A
  int nQB, QB[2];  // ... in phase B
  int nO, O[2];    // output tiles it finishes (uses its Q S^T of the same tile)
  int nS, S[3];    // d_k row tiles of the state it owns
};
// Phase A: every wave does 16 MFMAs; phase B is balanced as far as 7 state
// tiles and 5 token tiles allow.
__device__ constexpr Roles kRoles[4] = {
    {1, {0, 0}, 1, {0}, 0, {0, 0}, 1, {0, 0}, 3, {0, 1, 2}},
    {1, {1, 0}, 1, {1}, 0, {0, 0}, 1, {1, 0}, 2, {3, 4, 0}},
    {1, {2, 0}, 1, {2}, 0, {0, 0}, 1, {2, 0}, 2, {5, 6, 0}},
    {2, {3, 4}, 0, {0}, 2, {3, 4}, 2, {3, 4}, 0, {0, 0, 0}},
};
constexpr int kComputeWaves = 4;
constexpr int kThreads = 8 * 64;

// LDS map (bytes)
constexpr int kLdsS = 0;                         // S operand: hi/lo x (3 x 1 KB + 512 B)
constexpr int kLdsR = 2 * (3 * 1024 + 512);      // R operand: hi/lo x (2 x 1 KB + 512 B)
constexpr int kLdsMP = kLdsR + 2 * (2 * 1024 + 512);  // M then P' record of the current chunk
constexpr int kLdsRows = kLdsMP + kMBytes + kPBytes;  // two row buffers
constexpr int kMInstr = kMBytes / 1024;             // 35 one-KB copies of M
constexpr int kPInstr = kPBytes / 1024;             // 15 of P'

// One row buffer, for bf16 (kFp8 false) or E4M3FN (kFp8 true) inputs: K rows,
// Q rows, this workgroup's 16 columns of V and the chunk's 256 scale floats.
template <bool kFp8>
struct Rows {
  static constexpr int kElem = kFp8 ? 1 : 2;      // bytes per input element
  static constexpr int kStride = kFp8 ? 128 : 256;  // bytes per staged K/Q row (112 / 224 used)
  static constexpr int kSlots = kStride / 16;     // 16-byte slots per staged row
  static constexpr int kPieces = D * kElem / 16;  // 16-byte pieces per row (7 / 14); the rest read as zero
  static constexpr int kK = 0;
  static constexpr int kQ = C * kStride;
  static constexpr int kV = 2 * C * kStride;      // V tile: 80 rows x 16 elements, tail rows zero
  static constexpr int kVRow = 16 * kElem;
  static constexpr int kVInstr = kFp8 ? 2 : 3;    // 1 KB copies of the V tile
  static constexpr int kCs = kV + kVInstr * 1024;
  static constexpr int kBytes = kCs + kCsFloats * 4;  // 45,056 / 23,552
  // fp8 rows leave room for a second record buffer: chunk c's record sits in
  // buffer c & 1, so the copy of chunk c + 2's record starts a chunk earlier
  static constexpr bool kRec2 = kFp8;
  static constexpr int kRec1 = kLdsRows + 2 * kBytes;  // the second record buffer
  static constexpr int kLds = kRec1 + (kRec2 ? kMBytes + kPBytes : 0);  // 153,600 / 161,792
  static constexpr int rec_off(int c) { return kRec2 && (c & 1) ? kRec1 : kLdsMP; }
  static constexpr int kKQInstr = C * kStride / 1024;  // 20 / 10 one-KB copies per matrix
  // Copy split between the three copy waves, per chunk: waves 0 and 1 take
  // kMShare KB of M each and the K, resp. Q rows; wave 2 the rest of M, P',
  // the V tile and the scales.
  static constexpr int kMShare = kFp8 ? 14 : 17;
  static constexpr int rec_share(int L) { return L < 2 ? kMShare : kMInstr - 2 * kMShare + kPInstr; }
  static constexpr int row_share(int L) { return L < 2 ? kKQInstr : kVInstr + 1; }
  static_assert(kBytes % 1024 == 0 && kLds <= 160 * 1024, "1 KB aligned row buffers within one CU's LDS");
  static_assert(kVInstr * 1024 >= C * kVRow, "the V copies cover its 80 rows");
  static_assert(rec_share(0) + 2 * row_share(0) < 64 && rec_share(2) + 2 * row_share(2) < 64, "vmcnt holds 63");
};
static_assert(kMBytes % 1024 == 0 && kPBytes % 1024 == 0 && kCsFloats * 4 == 1024, "whole 1 KB copies");
// The reverse scan of the bidirectional layer (kAdd) adds the forward scan's
// fp32 output, which o already holds, to its own: copy wave 2 brings the
// chunk's 80 x 16 tile of o into one of two buffers after the row buffers
// (bf16 rows only: 153,600 + 2 x 5,120 bytes is all of the CU's LDS).
constexpr int kAddTile = C * 16 * 4;
template <bool kFp8, bool kAdd>
constexpr int chain_lds() { return Rows<kFp8>::kLds + (kAdd ? 2 * kAddTile : 0); }
template <bool kFp8>
constexpr int add_off(int c) { return Rows<kFp8>::kLds + (c & 1) * kAddTile; }
static_assert(chain_lds<false, true>() <= 160 * 1024, "the addend tiles fit beside bf16 row buffers");
static_assert(kLdsMP % 1024 == 0 && kLdsRows % 1024 == 0, "copy targets 1 KB aligned");

struct RowFrags {  // one lane's share of a 16-row tile of K or Q (A operand, k = d_k)
  F32 f[3];
  F16 t;
};

template <int W, bool kOutBf16, bool kFp8, bool kRev, bool kAdd>
__device__ __forceinline__ void compute_role(const float *__restrict__ state_in, float *state_out,
                                             void *__restrict__ o, int T, int H, int cb, int ce, int b, int h,
                                             int nt, char *lds) {
  using G = Rows<kFp8>;
  constexpr Roles ro = kRoles[W];
  constexpr int nA = ro.nY + ro.nQA;  // 16-row tiles of K or Q multiplied by S^T in phase A
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const size_t u = size_t(b) * H + h;
  const size_t rowstride = size_t(H) * D;
  char *Slds = lds + kLdsS;
  char *Rlds = lds + kLdsR;
  const char *MPlds = lds + kLdsMP;

  // ---- state slice: S^T tile j, accumulator rows d_k = 16j + 4lg + e, column d_v = 16nt + ln
  f32x4 S[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    S[s] = zero4();
    if (s < ro.nS && state_in) {
      const float4 t = *reinterpret_cast<const float4 *>(state_in + (u * D + 16 * nt + ln) * D + 16 * ro.S[s] + 4 * lg);
      S[s] = f32x4{t.x, t.y, t.z, t.w};
    }
  }
  // Where this lane's hi half of tile j goes in the B-operand image of S in
  // the natural k-order: the 16 bytes read by lane (ln, g) of 32-deep block kb
  // are rows 8(g & 1) .. + 7 of tile 2kb + (g >> 1), i.e. the 8-byte halves
  // written by lane groups 2(g & 1) and 2(g & 1) + 1 of that tile.
  auto s_slot = [&](int j) { return (j >> 1) * 1024 + (ln + 16 * (2 * (j & 1) + (lg >> 1))) * 16 + (lg & 1) * 8; };

  // A-operand fragments of a 16-row tile of the staged K (m = 0) or Q (m = 1):
  // lane (ln, lg) takes d_k = 32kb + 8lg .. + 7 of row 16 tile + ln per 32-deep
  // block and d_k = 96 + 4lg .. + 3 for the 16-deep block
  auto rows_frag = [&](const char *rb, int m, int tile) {
    const char *rowp = rb + (m ? G::kQ : G::kK) + (16 * tile + ln) * G::kStride;
    RowFrags rf;
    if constexpr (kFp8) {
      const int sw = ln & 7;  // (row & 7)
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) {
        const uint2 x = *reinterpret_cast<const uint2 *>(rowp + 16 * ((2 * kb + (lg >> 1)) ^ sw) + 8 * (lg & 1));
        const uint2 a = fp8x4_to_bf16(x.x), c = fp8x4_to_bf16(x.y);
        rf.f[kb] = F32{{a.x, a.y, c.x, c.y}};
      }
      const uint32_t x1 = *reinterpret_cast<const uint32_t *>(rowp + 16 * (6 ^ sw) + 4 * lg);
      const uint2 t = fp8x4_to_bf16(x1);
      rf.t = F16{{t.x, t.y}};
    } else {
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) {
        const uint4 x = *reinterpret_cast<const uint4 *>(rowp + 16 * ((4 * kb + lg) ^ ln));
        rf.f[kb] = F32{{x.x, x.y, x.z, x.w}};
      }
      const uint2 x2 = *reinterpret_cast<const uint2 *>(rowp + 16 * ((12 + (lg >> 1)) ^ ln) + 8 * (lg & 1));
      rf.t = F16{{x2.x, x2.y}};
    }
    return rf;
  };
  // element (row, column ln) of the staged V tile
  auto v_elem = [&](const char *vl, int row) {
    if constexpr (kFp8)
      return __builtin_amdgcn_cvt_pk_f32_fp8(uint32_t(reinterpret_cast<const uint8_t *>(vl)[row * 16 + ln]), false)[0];
    else
      return bf16_to_f32(reinterpret_cast<const uint16_t *>(vl)[row * 16 + ln]);
  };
  auto ldf4 = [](const float *p) {
    const float4 t = *reinterpret_cast<const float4 *>(p);
    return f32x4{t.x, t.y, t.z, t.w};
  };
  auto ld32 = [&](int off) {
    const uint4 x = *reinterpret_cast<const uint4 *>(MPlds + off + lane * 16);
    return F32{{x.x, x.y, x.z, x.w}};
  };
  auto ld16 = [&](int off) {
    const uint2 x = *reinterpret_cast<const uint2 *>(MPlds + off + lane * 8);
    return F16{{x.x, x.y}};
  };
  // tiles x (hi, lo) independent accumulation chains over the four k-blocks of d_k
  auto rows_times_S = [](const RowFrags *rf, int n, const F32 *Sh, const F32 *Sl, const F16 &Sth, const F16 &Stl,
                         f32x4 *out) {
    f32x4 ah[2] = {zero4(), zero4()}, al[2] = {zero4(), zero4()};
#pragma unroll
    for (int kb = 0; kb < 3; ++kb)
#pragma unroll
      for (int a = 0; a < 2; ++a)
        if (a < n) {
          ah[a] = mma(rf[a].f[kb], Sh[kb], ah[a]);
          al[a] = mma(rf[a].f[kb], Sl[kb], al[a]);
        }
#pragma unroll
    for (int a = 0; a < 2; ++a)
      if (a < n) {
        ah[a] = mma(rf[a].t, Sth, ah[a]);
        al[a] = mma(rf[a].t, Stl, al[a]);
        out[a] = ah[a] + al[a];
      }
  };

  // phase 0 of the first chunk: publish the entry state
  auto publish_S = [&]() {
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if (s < ro.nS) {
        const int j = ro.S[s];
        uint32_t hi[2], lo[2];
        split4(S[s], hi, lo);
        const int off = j < 6 ? s_slot(j) : 3072 + lane * 8;
        *reinterpret_cast<uint2 *>(Slds + off) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2 *>(Slds + 3584 + off) = make_uint2(lo[0], lo[1]);
      }
    }
  };
  publish_S();
  for (int c = cb; c < ce; ++c) {
    const int t0 = c * C, nv = min(C, T - t0);
    const char *rb = lds + kLdsRows + (c & 1) * G::kBytes;
    MPlds = lds + G::rec_off(c);
    const float *csl = reinterpret_cast<const float *>(rb + G::kCs);
    const char *vl = rb + G::kV;
    compute_barrier();  // X: chunk c opens (S published; its rows and record landed)
    // ---- phase A: every LDS operand of the chunk except R is read here, so
    // that both buffers are free once R is published
    F32 Sh[3], Sl[3];
    F16 Sth, Stl;
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) {
      const uint4 xh = *reinterpret_cast<const uint4 *>(Slds + kb * 1024 + lane * 16);
      const uint4 xl = *reinterpret_cast<const uint4 *>(Slds + 3584 + kb * 1024 + lane * 16);
      Sh[kb] = F32{{xh.x, xh.y, xh.z, xh.w}};
      Sl[kb] = F32{{xl.x, xl.y, xl.z, xl.w}};
    }
    {
      const uint2 xh = *reinterpret_cast<const uint2 *>(Slds + 3072 + lane * 8);
      const uint2 xl = *reinterpret_cast<const uint2 *>(Slds + 3584 + 3072 + lane * 8);
      Sth = F16{{xh.x, xh.y}};
      Stl = F16{{xl.x, xl.y}};
    }
    RowFrags fa[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
      if (a < nA) fa[a] = rows_frag(rb, a < ro.nY ? 0 : 1, a < ro.nY ? ro.Y[a] : ro.QA[0]);
    f32x4 aa[2], bb[2];
    float va[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < ro.nY) {
        const int tile = ro.Y[s];
        aa[s] = ldf4(csl + 16 * tile + 4 * lg);
        bb[s] = ldf4(csl + 80 + 16 * tile + 4 * lg);
#pragma unroll
        for (int e = 0; e < 4; ++e) va[s][e] = v_elem(vl, 16 * tile + 4 * lg + e);
      }
    const float gamma_n = csl[240];
    f32x4 ya[2];
    rows_times_S(fa, nA, Sh, Sl, Sth, Stl, ya);
    // The phase-B operands (Q tiles, M and P' fragments) are read only after
    // the Y products have issued: a wave tracks at most 15 LDS reads in
    // flight, so reading them first held the products back until most of
    // them had gone out.  They still land before barrier Y, which waits for
    // them, and they are in flight while the products run.
    __builtin_amdgcn_sched_barrier(0);
    RowFrags fb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < ro.nQB) fb[s] = rows_frag(rb, 1, ro.QB[s]);
    F32 Mf[3][2][2];
    F16 Mt[3][2];
#pragma unroll
    for (int s = 0; s < 3; ++s)
      if (s < ro.nS) {
        const int mt = ro.S[s];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) Mf[s][kb][hl] = ld32(m_off32(mt, kb, hl));
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) Mt[s][hl] = ld16(m_off16(mt, hl));
      }
    F32 Pf[2][2][2];
    F16 Pt[2][2];
    f32x4 cc[2];
    float adv[2][4];  // kAdd: o's elements of this wave's output tiles
    if constexpr (kAdd) {
      const float *at = reinterpret_cast<const float *>(lds + add_off<kFp8>(c));
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s < ro.nO)
#pragma unroll
          for (int e = 0; e < 4; ++e) adv[s][e] = at[(16 * ro.O[s] + 4 * lg + e) * 16 + ln];
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < ro.nO) {
        const int R = ro.O[s];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
            if (kb < (R + 1) / 2) Pf[s][kb][hl] = ld32(kMBytes + p_off32(R, kb, hl));
        if (!(R & 1))
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) Pt[s][hl] = ld16(kMBytes + p_off16(R, hl));
        cc[s] = ldf4(csl + 160 + 16 * R + 4 * lg);
      }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < ro.nY) {
        const int tile = ro.Y[s];
        float r4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = aa[s][e] * va[s][e] - bb[s][e] * ya[s][e];
        uint32_t hi[2], lo[2];
        split4(r4, hi, lo);
        if (tile < 4) {
          const int kb = tile >> 1, half = tile & 1;
          *reinterpret_cast<uint2 *>(Rlds + kb * 1024 + lane * 16 + half * 8) = make_uint2(hi[0], hi[1]);
          *reinterpret_cast<uint2 *>(Rlds + 2560 + kb * 1024 + lane * 16 + half * 8) = make_uint2(lo[0], lo[1]);
        } else {
          *reinterpret_cast<uint2 *>(Rlds + 2048 + lane * 8) = make_uint2(hi[0], hi[1]);
          *reinterpret_cast<uint2 *>(Rlds + 2560 + 2048 + lane * 8) = make_uint2(lo[0], lo[1]);
        }
      }
    }
    f32x4 QS[2] = {zero4(), zero4()};
    if (ro.nQA) QS[0] = ya[ro.nY];
    compute_barrier();  // Y: R published; the record and row buffer c & 1 may be refilled
    // ---- phase B: R operands, the state update, S published for chunk c + 1,
    // then the outputs
    F32 Rh[2], Rl[2];
    F16 Rth, Rtl;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint4 xh = *reinterpret_cast<const uint4 *>(Rlds + kb * 1024 + lane * 16);
      const uint4 xl = *reinterpret_cast<const uint4 *>(Rlds + 2560 + kb * 1024 + lane * 16);
      Rh[kb] = F32{{xh.x, xh.y, xh.z, xh.w}};
      Rl[kb] = F32{{xl.x, xl.y, xl.z, xl.w}};
    }
    {
      const uint2 xh = *reinterpret_cast<const uint2 *>(Rlds + 2048 + lane * 8);
      const uint2 xl = *reinterpret_cast<const uint2 *>(Rlds + 2560 + 2048 + lane * 8);
      Rth = F16{{xh.x, xh.y}};
      Rtl = F16{{xl.x, xl.y}};
    }
    // S^T tile update: gamma_n S + Mhi Rhi + Mhi Rlo + Mlo Rhi as three chains
    f32x4 a0[3], a1[3], a2[3];
#pragma unroll
    for (int s = 0; s < 3; ++s)
      if (s < ro.nS) {
        a0[s] = S[s] * gamma_n;
        a1[s] = zero4();
        a2[s] = zero4();
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 3; ++s)
        if (s < ro.nS) {
          a0[s] = mma(Mf[s][kb][0], Rh[kb], a0[s]);
          a1[s] = mma(Mf[s][kb][0], Rl[kb], a1[s]);
          a2[s] = mma(Mf[s][kb][1], Rh[kb], a2[s]);
        }
#pragma unroll
    for (int s = 0; s < 3; ++s)
      if (s < ro.nS) {
        a0[s] = mma(Mt[s][0], Rth, a0[s]);
        a1[s] = mma(Mt[s][0], Rtl, a1[s]);
        a2[s] = mma(Mt[s][1], Rth, a2[s]);
        S[s] = a0[s] + a1[s] + a2[s];
      }
    // S written for chunk c + 1: every wave read S of chunk c before Y
    publish_S();
    if (ro.nQB) {
      f32x4 qb[2];
      rows_times_S(fb, ro.nQB, Sh, Sl, Sth, Stl, qb);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s < ro.nQB) QS[s] = qb[s];
    }
    // outputs: diag(gamma rq) Q S^T + P'hi Rhi + P'hi Rlo + P'lo Rhi
    f32x4 o0[2], o1[2], o2[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < ro.nO) {
        o0[s] = cc[s] * QS[s];
        o1[s] = zero4();
        o2[s] = zero4();
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s < ro.nO && kb < (ro.O[s] + 1) / 2) {
          o0[s] = mma(Pf[s][kb][0], Rh[kb], o0[s]);
          o1[s] = mma(Pf[s][kb][0], Rl[kb], o1[s]);
          o2[s] = mma(Pf[s][kb][1], Rh[kb], o2[s]);
        }
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < ro.nO && !(ro.O[s] & 1)) {
        // the 16-deep block covers token tile R (tile 4: the shared 16-deep R slot;
        // tiles 0 and 2: first halves of the 32-deep R slots)
        const int R = ro.O[s];
        F16 rh, rl;
        if (R == 4) {
          rh = Rth;
          rl = Rtl;
        } else {
          rh = F16{{Rh[R >> 1].w[0], Rh[R >> 1].w[1]}};
          rl = F16{{Rl[R >> 1].w[0], Rl[R >> 1].w[1]}};
        }
        o0[s] = mma(Pt[s][0], rh, o0[s]);
        o1[s] = mma(Pt[s][0], rl, o1[s]);
        o2[s] = mma(Pt[s][1], rh, o2[s]);
      }
    // the chunk's rows of o: physical rows p0 .. p0 + nv - 1 (logical row r at
    // p0 + r, or at p0 + nv - 1 - r in the reverse scan)
    const int p0 = kRev ? T - t0 - nv : t0;
    constexpr uint32_t kOutBytes = kOutBf16 ? 2u : 4u;
    const auto ro_ = make_rsrc(static_cast<char *>(o) + (size_t(b) * T + p0) * rowstride * kOutBytes,
                               uint32_t(nv) * uint32_t(rowstride) * kOutBytes);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < ro.nO) {
        const int R = ro.O[s];
        f32x4 acc = o0[s] + o1[s] + o2[s];
        if constexpr (kAdd)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += adv[s][e];
        // rows past the chunk's end are aimed outside the store descriptor and dropped
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * R + 4 * lg + e;
          const uint32_t oi = uint32_t(kRev ? nv - 1 - r : r) * uint32_t(rowstride) + uint32_t(h) * D + 16u * nt + ln;
          const uint32_t ob = !kRev || r < nv ? oi * kOutBytes : kOutOfRange;
          if constexpr (kOutBf16)
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[e]), ro_, int(ob), 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[e]), ro_, int(ob), 0, 0);
        }
      }
    }
  }
  if (state_out) {
#pragma unroll
    for (int s = 0; s < 3; ++s)
      if (s < ro.nS)
        *reinterpret_cast<float4 *>(state_out + (u * D + 16 * nt + ln) * D + 16 * ro.S[s] + 4 * lg) =
            make_float4(S[s][0], S[s][1], S[s][2], S[s][3]);
  }
}

// Copy wave L (0, 1 or 2).  Before barrier X of chunk c its rows and record
// must have landed; after barrier Y (phase A has read both buffers) the wave
// issues its share of chunk c + 1's record and of chunk c + 2's rows.  Loads
// complete in issue order, so each wait names the number of younger copies
// that may still be in flight (at most a record share and two row shares:
// 57 of the 63 the counter holds).
template <int L, bool kFp8, bool kRev, bool kAdd>
__device__ __forceinline__ void copy_role(const char *__restrict__ q, const char *__restrict__ k,
                                          const char *__restrict__ v, const char *__restrict__ Mws,
                                          const char *__restrict__ Pws, const float *__restrict__ CS,
                                          const float *addend, int T, int H, int N, int cb, int ce, int b, int h,
                                          int nt, char *lds) {
  using G = Rows<kFp8>;
  constexpr int kRow = G::row_share(L) + (kAdd && L == 2 ? kAddTile / 1024 : 0);
  const int lane = threadIdx.x & 63;
  const size_t u = size_t(b) * H + h;
  const uint32_t row_bytes = uint32_t(H) * D * G::kElem;
  const uint32_t head_off = uint32_t(h) * D * G::kElem;
  // Logical row r of a chunk with nv rows sits at physical row p0 + r (p0 + nv
  // - 1 - r in the reverse scan) of the buffer that starts at row p0; rows at
  // or past nv read as zero (forward: they lie past the buffer's end).
  auto row_ok = [&](int r, int nv) { return !kRev || r < nv; };
  auto row_at = [&](int r, int nv) { return uint32_t(kRev ? nv - 1 - r : r) * row_bytes; };
  auto row_at_f32 = [&](int r, int nv) { return uint32_t(kRev ? nv - 1 - r : r) * uint32_t(H) * D * 4u; };
  // K / Q: copy i fills 1 KB of LDS rows, lane -> (row, slot lane % kSlots)
  // holding piece slot ^ (row % kSlots); slots past the row's pieces read as zero
  auto kq_off = [&](int i, int nv) {
    constexpr int kRowsPerCopy = 64 / G::kSlots;
    const int r = kRowsPerCopy * i + lane / G::kSlots, p = (lane % G::kSlots) ^ (r % G::kSlots);
    return p < G::kPieces && row_ok(r, nv) ? row_at(r, nv) + head_off + 16u * p : kOutOfRange;
  };
  // V: copy i fills 1 KB of the tile's rows (kVRow bytes each: this tile's 16 columns)
  auto v_off = [&](int i, int nv) {
    constexpr int kLanesPerRow = G::kVRow / 16;
    const int r = (64 / kLanesPerRow) * i + lane / kLanesPerRow;
    return r < C && row_ok(r, nv) ? row_at(r, nv) + head_off + uint32_t(G::kVRow) * nt + 16u * (lane % kLanesPerRow)
                                  : kOutOfRange;
  };
  // wave 0: K rows; wave 1: Q rows; wave 2: the V tile and the scales
  auto copy_rows = [&](int c) {
    const int t0 = c * C, nv = min(C, T - t0);
    const int p0 = kRev ? T - t0 - nv : t0;  // first physical row of the chunk
    const size_t base = (size_t(b) * T + p0) * size_t(H) * D * G::kElem;
    const uint32_t bytes = uint32_t(nv) * row_bytes;
    char *rb = lds + kLdsRows + (c & 1) * G::kBytes;
    if constexpr (L < 2) {
      const auto rs = make_rsrc((L == 0 ? k : q) + base, bytes);
#pragma unroll
      for (int i = 0; i < G::kKQInstr; ++i) copy16(rs, rb + (L == 0 ? G::kK : G::kQ) + 1024 * i, kq_off(i, nv));
    } else {
      const auto rv = make_rsrc(v + base, bytes);
#pragma unroll
      for (int i = 0; i < G::kVInstr; ++i) copy16(rv, rb + G::kV + 1024 * i, v_off(i, nv));
      copy16(make_rsrc(CS + (u * N + c) * kCsFloats, kCsFloats * 4), rb + G::kCs, 16u * lane);
      if constexpr (kAdd) {  // o's 80 x 16 fp32 tile: copy i, lane l -> row 16 i + l / 4, columns 4 (l % 4) ..
        const uint32_t orow = uint32_t(H) * D * 4u;
        const auto ra = make_rsrc(addend + (size_t(b) * T + p0) * size_t(H) * D, uint32_t(nv) * orow);
#pragma unroll
        for (int i = 0; i < kAddTile / 1024; ++i) {
          const int r = 16 * i + lane / 4;
          const uint32_t off = row_ok(r, nv) ? row_at_f32(r, nv) + uint32_t(h * D + 16 * nt + 4 * (lane % 4)) * 4u
                                             : kOutOfRange;
          copy16(ra, lds + add_off<kFp8>(c) + 1024 * i, off);
        }
      }
    }
  };
  // waves 0, 1: kMShare KB of M each; wave 2: the rest of M and P'
  auto copy_record = [&](int c) {
    const auto rm = make_rsrc(Mws + (u * N + c) * size_t(kMBytes), kMBytes);
    constexpr int kMShare = G::kMShare;
    constexpr int m0 = L == 0 ? 0 : (L == 1 ? kMShare : 2 * kMShare), m1 = L == 2 ? kMInstr : m0 + kMShare;
    char *rd = lds + G::rec_off(c);
#pragma unroll
    for (int i = m0; i < m1; ++i) copy16(rm, rd + 1024 * i, 1024u * i + 16u * lane);
    if constexpr (L == 2) {
      const auto rp = make_rsrc(Pws + (u * N + c) * size_t(kPBytes), kPBytes);
#pragma unroll
      for (int i = 0; i < kPInstr; ++i) copy16(rp, rd + kMBytes + 1024 * i, 1024u * i + 16u * lane);
    }
  };
  if constexpr (G::kRec2) {
    constexpr int kRec = G::rec_share(L);
    static_assert(2 * (kRow + kRec) < 64, "vmcnt holds 63");
    if (cb < ce) {
      copy_rows(cb);
      copy_record(cb);
      if (cb + 1 < ce) {
        copy_rows(cb + 1);
        copy_record(cb + 1);
      }
    }
    for (int c = cb; c < ce; ++c) {
      // in flight, oldest first: rows(c), record(c), then rows(c + 1), record(c + 1) if c + 1 < ce
      if (c + 1 < ce)
        wait_vm<kRow + kRec>();
      else
        wait_vm<0>();
      bare_barrier();  // X: chunk c opens
      bare_barrier();  // Y: chunk c's record and rows have been read
      if (c + 2 < ce) {
        copy_rows(c + 2);
        copy_record(c + 2);
      }
    }
  } else {
    if (cb < ce) {
      copy_rows(cb);
      copy_record(cb);
      if (cb + 1 < ce) copy_rows(cb + 1);
    }
    for (int c = cb; c < ce; ++c) {
      // in flight, oldest first: rows(c), record(c), rows(c + 1) if c + 1 < ce
      if (c + 1 < ce)
        wait_vm<kRow>();
      else
        wait_vm<0>();
      bare_barrier();  // X: chunk c opens
      bare_barrier();  // Y: chunk c's record and rows have been read
      if (c + 1 < ce) copy_record(c + 1);
      if (c + 2 < ce) copy_rows(c + 2);
    }
  }
  wait_vm<0>();
}

// L2 warm-up of chunk c + kAhead: the head's 7 column-tile workgroups (on
// one XCD) split its cache lines -- 280 of M, 120 of P', 8 of scales and
// 3 per 224-byte row of K, Q, V (2 per 112-byte fp8 row) -- so that the copies of that chunk hit L2
// instead of all waiting on the same HBM misses.  Four dword loads per lane
// per chunk, each at a fixed per-lane base plus a per-chunk stride, consumed a
// chunk later.
constexpr int kAhead = 2;
template <bool kFp8, bool kRev>
__device__ __forceinline__ void warm_role(const char *__restrict__ q, const char *__restrict__ k,
                                          const char *__restrict__ v, const char *__restrict__ Mws,
                                          const char *__restrict__ Pws, const float *__restrict__ CS,
                                          void *__restrict__ o, int T, int H, int N, int cb, int ce, int b, int h,
                                          int nt) {
  const int lane = threadIdx.x & 63;
  const size_t u = size_t(b) * H + h;
  constexpr int kElem = kFp8 ? 1 : 2, kParts = kFp8 ? 2 : 3;  // touches per row: every 128-byte line of it
  const size_t row_bytes = size_t(H) * D * kElem;
  const char *base[4];
  size_t stride[4];
  int prow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int pe = nt + NT * (64 * j + lane);  // 0 .. 1791, cache-line task
    prow[j] = -1;
    if (pe < 280) {
      base[j] = Mws + u * N * size_t(kMBytes) + 128 * pe;
      stride[j] = kMBytes;
    } else if (pe < 400) {
      base[j] = Pws + u * N * size_t(kPBytes) + 128 * (pe - 280);
      stride[j] = kPBytes;
    } else if (pe < 408) {
      base[j] = reinterpret_cast<const char *>(CS + u * N * kCsFloats) + 128 * (pe - 400);
      stride[j] = kCsFloats * sizeof(float);
    } else {
      const int r = min(pe - 408, 3 * kParts * C - 1), t = r / (kParts * C), part = r % kParts;
      prow[j] = (r % (kParts * C)) / kParts;
      const char *src = t == 0 ? k : (t == 1 ? q : v);
      base[j] = src + (size_t(b) * T * H + h) * D * kElem +
                (part == 0 ? 0 : (kFp8 ? 108 : (part == 1 ? 128 : 220)));
      stride[j] = 0;  // rows: addressed by physical row below
    }
  }
  uint32_t pf[4] = {0u, 0u, 0u, 0u}, sink = 0;
  for (int c = cb; c < ce; ++c) {
    const int cp = min(c + kAhead, ce - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sink ^= pf[j];  // consumed a chunk after its load was issued
      // a row past the end of the last chunk touches the chunk's last row instead
      const size_t off = prow[j] < 0 ? size_t(cp) * stride[j]
                                     : size_t(phys_token(min(cp * C + prow[j], T - 1), T, kRev)) * row_bytes;
      pf[j] = *reinterpret_cast<const uint32_t *>(base[j] + off);
    }
    bare_barrier();
    bare_barrier();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) sink ^= pf[j];
  if (T < 0 && sink != 0u) static_cast<uint32_t *>(o)[0] = sink;  // never taken: keeps the touches alive
}

template <bool kOutBf16, bool kFp8, bool kRev, bool kAdd>
__global__ __launch_bounds__(kThreads) void chain_kernel(const char *__restrict__ q,
                                                         const char *__restrict__ k,
                                                         const char *__restrict__ v,
                                                         const char *__restrict__ Mws,
                                                         const char *__restrict__ Pws,
                                                         const float *__restrict__ CS, const float *addend,
                                                         const float *state_in,
                                                         float *state_out, void *__restrict__ o, int T, int H,
                                                         int N, int cb, int ce, int units) {
  extern __shared__ __align__(16) char lds[];
  // Workgroup i runs on XCD i % 8: keep the 7 column tiles of a (b, h) on one
  // XCD so that its K, Q, M and P' are fetched from HBM once into that L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int u = xcd + 8 * (slot / NT), nt = slot % NT;
  if (u >= units) return;
  const int b = u / H, h = u % H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  switch (wave) {
    case 0: compute_role<0, kOutBf16, kFp8, kRev, kAdd>(state_in, state_out, o, T, H, cb, ce, b, h, nt, lds); break;
    case 1: compute_role<1, kOutBf16, kFp8, kRev, kAdd>(state_in, state_out, o, T, H, cb, ce, b, h, nt, lds); break;
    case 2: compute_role<2, kOutBf16, kFp8, kRev, kAdd>(state_in, state_out, o, T, H, cb, ce, b, h, nt, lds); break;
    case 3: compute_role<3, kOutBf16, kFp8, kRev, kAdd>(state_in, state_out, o, T, H, cb, ce, b, h, nt, lds); break;
    case 4: copy_role<0, kFp8, kRev, kAdd>(q, k, v, Mws, Pws, CS, addend, T, H, N, cb, ce, b, h, nt, lds); break;
    case 5: copy_role<1, kFp8, kRev, kAdd>(q, k, v, Mws, Pws, CS, addend, T, H, N, cb, ce, b, h, nt, lds); break;
    case 6: copy_role<2, kFp8, kRev, kAdd>(q, k, v, Mws, Pws, CS, addend, T, H, N, cb, ce, b, h, nt, lds); break;
    default: warm_role<kFp8, kRev>(q, k, v, Mws, Pws, CS, o, T, H, N, cb, ce, b, h, nt); break;
  }
}

}  // namespace
}  // namespace mfma

size_t mfma_chunk_bytes_M() { return mfma::kMBytes; }
size_t mfma_chunk_bytes_P() { return mfma::kPBytes; }
size_t mfma_chunk_bytes_cs() { return mfma::kCsFloats * sizeof(float); }

namespace {

// A second stream per device on which the intra kernel of later chunk ranges
// runs while the state pass works through earlier ones, plus the events that
// order them.  Used when the state pass has more workgroups (7 per (b, h))
// than the device has CUs: it then runs in more than one round of workgroups,
// and the intra kernel fills the CUs its last round leaves free.  (With one
// round, intra workgroups that start first take CUs the state pass is waiting
// for, and the two kernels only slow each other down.)
struct SideResources {
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> ev;
  int cus = -1;
};
std::mutex g_side_mu;
SideResources g_side[64];

// Chunk ranges: a short first range (the intra kernel runs alone on it), then
// ranges growing by 30% each, so that the intra kernel of range s + 1 (on the
// CUs the state pass leaves free) finishes while the state pass works on range s.
void segment_bounds(int N, std::vector<int> &bounds) {
  bounds.assign(1, 0);
  int len = 16;
  while (bounds.back() < N) {
    bounds.push_back(std::min(N, bounds.back() + len));
    len = len + (len * 3 + 9) / 10;
  }
}
constexpr int kSegmentMinChunks = 64;

template <bool kOutBf16, bool kFp8, bool kRev, bool kAdd = false>
hipError_t launch_chain_typed(const Plan &p, const Args &a, const char *M, const char *P, const float *cs, int cb,
                              int ce, const float *sin, float *sout, hipStream_t st) {
  const char *q = static_cast<const char *>(a.q), *k = static_cast<const char *>(a.k),
             *v = static_cast<const char *>(a.v);
  const int units = p.B * p.H;
  const dim3 grid(8u * mfma::NT * unsigned((units + 7) / 8)), block(mfma::kThreads);
  constexpr int lds = mfma::chain_lds<kFp8, kAdd>();
  // more than the default 64 KB of dynamic LDS (gfx950 has 160 KB per CU), once per instantiation
  static const hipError_t lds_ok = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&mfma::chain_kernel<kOutBf16, kFp8, kRev, kAdd>),
      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (lds_ok != hipSuccess) return lds_ok;
  mfma::chain_kernel<kOutBf16, kFp8, kRev, kAdd><<<grid, block, lds, st>>>(
      q, k, v, M, P, cs, kAdd ? static_cast<const float *>(a.o) : nullptr, sin, sout, a.o, p.T, p.H,
                                                                     p.N, cb, ce, units);
  return hipGetLastError();
}

template <bool kOutBf16, bool kFp8>
hipError_t launch_chain_rev(const Plan &p, const Args &a, const char *M, const char *P, const float *cs, int cb,
                            int ce, const float *sin, float *sout, hipStream_t st) {
  if (!(p.flags & kReverse)) return launch_chain_typed<kOutBf16, kFp8, false>(p, a, M, P, cs, cb, ce, sin, sout, st);
  // the bidirectional layer's reverse scan adds o (the forward scan's fp32 output) to its own
  if constexpr (!kOutBf16 && !kFp8)
    if (p.o_add) return launch_chain_typed<false, false, true, true>(p, a, M, P, cs, cb, ce, sin, sout, st);
  return launch_chain_typed<kOutBf16, kFp8, true>(p, a, M, P, cs, cb, ce, sin, sout, st);
}

hipError_t launch_chain(const Plan &p, const Args &a, const char *M, const char *P, const float *cs, int cb, int ce,
                        const float *sin, float *sout, hipStream_t st) {
  if (p.qkv_fp8)
    return p.o_bf16 ? launch_chain_rev<true, true>(p, a, M, P, cs, cb, ce, sin, sout, st)
                    : launch_chain_rev<false, true>(p, a, M, P, cs, cb, ce, sin, sout, st);
  return p.o_bf16 ? launch_chain_rev<true, false>(p, a, M, P, cs, cb, ce, sin, sout, st)
                  : launch_chain_rev<false, false>(p, a, M, P, cs, cb, ce, sin, sout, st);
}


// the current device and its CU count (cached per device)
hipError_t device_cus(int *dev, int *cus) {
  hipError_t e;
  if ((e = hipGetDevice(dev)) != hipSuccess) return e;
  if (*dev < 0 || *dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_side_mu);
  if (g_side[*dev].cus < 0 &&
      hipDeviceGetAttribute(&g_side[*dev].cus, hipDeviceAttributeMultiprocessorCount, *dev) != hipSuccess)
    g_side[*dev].cus = 0;
  *cus = g_side[*dev].cus;
  return hipSuccess;
}

// the side stream and at least `n` events of device `dev` (caller holds g_side_mu)
hipError_t side_resources(int dev, int n) {
  SideResources &R = g_side[dev];
  hipError_t e;
  if (!R.side && (e = hipStreamCreateWithFlags(&R.side, hipStreamNonBlocking)) != hipSuccess) {
    R.side = nullptr;
    return e;
  }
  while (int(R.ev.size()) < n) {
    hipEvent_t ev;
    if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return e;
    R.ev.push_back(ev);
  }
  return hipSuccess;
}

}  // namespace

bool mfma_bidir_overlaps(const Plan &p) {
  int dev = 0, cus = 0;
  if (device_cus(&dev, &cus) != hipSuccess) return false;
  return long(p.B) * p.H * mfma::NT <= cus;
}

hipError_t launch_mfma_bidir(const Plan &F, const Args &af, const Plan &R, const Args &ar) {
  char *Mf = af.ws + F.off_M, *Pf = af.ws + F.off_P, *Mr = ar.ws + R.off_M, *Pr = ar.ws + R.off_P;
  float *csf = reinterpret_cast<float *>(af.ws + F.off_cs), *csr = reinterpret_cast<float *>(ar.ws + R.off_cs);
  hipError_t e;
  int dev = 0, cus = 0;
  if ((e = device_cus(&dev, &cus)) != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_side_mu);
  if ((e = side_resources(dev, 2)) != hipSuccess) return e;
  SideResources &S = g_side[dev];
  // intra (forward) on the caller's stream; the reverse scan's intra on the
  // side stream once it is done, next to the forward state pass
  stage_begin(af, kStageIntra);
  if ((e = mfma::launch_intra(F, af, Mf, Pf, csf, 0, F.N, af.stream)) != hipSuccess) return e;
  stage_end(af, kStageIntra);
  if ((e = hipEventRecord(S.ev[0], af.stream)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(S.side, S.ev[0], 0)) != hipSuccess) return e;
  stage_begin(af, kStageState);
  if ((e = launch_chain(F, af, Mf, Pf, csf, 0, F.N, af.state_in, af.state_out, af.stream)) != hipSuccess) return e;
  stage_end(af, kStageState);
  stage_begin(ar, kStageIntra, S.side);
  if ((e = mfma::launch_intra(R, ar, Mr, Pr, csr, 0, R.N, S.side)) != hipSuccess) return e;
  stage_end(ar, kStageIntra, S.side);
  if ((e = hipEventRecord(S.ev[1], S.side)) != hipSuccess) return e;
  // the reverse state pass after both (this wait also joins the side stream back)
  if ((e = hipStreamWaitEvent(ar.stream, S.ev[1], 0)) != hipSuccess) return e;
  stage_begin(ar, kStageState);
  e = launch_chain(R, ar, Mr, Pr, csr, 0, R.N, ar.state_in, ar.state_out, ar.stream);
  stage_end(ar, kStageState);
  return e;
}

hipError_t launch_mfma(const Plan &p, const Args &a) {
  char *M = a.ws + p.off_M;
  char *P = a.ws + p.off_P;
  float *cs = reinterpret_cast<float *>(a.ws + p.off_cs);
  float *seg_state = reinterpret_cast<float *>(a.ws + p.off_Sseg);
  hipError_t e;
  int dev = 0, cus = 0;
  if ((e = device_cus(&dev, &cus)) != hipSuccess) return e;
  const long chain_blocks = long(p.B) * p.H * mfma::NT;
  if (p.N < kSegmentMinChunks || chain_blocks <= cus) {
    stage_begin(a, kStageIntra);
    e = mfma::launch_intra(p, a, M, P, cs, 0, p.N, a.stream);
    stage_end(a, kStageIntra);
    if (e != hipSuccess) return e;
    stage_begin(a, kStageState);
    e = launch_chain(p, a, M, P, cs, 0, p.N, a.state_in, a.state_out, a.stream);
    stage_end(a, kStageState);
    return e;
  }
  std::vector<int> bounds;
  segment_bounds(p.N, bounds);
  const int segs = int(bounds.size()) - 1;
  // one caller at a time per device enqueues on the shared side stream and events
  std::lock_guard<std::mutex> lk(g_side_mu);
  if ((e = side_resources(dev, segs + 1)) != hipSuccess) return e;
  SideResources &R = g_side[dev];
  // fork: the side stream starts after the caller's earlier work (the inputs)
  if ((e = hipEventRecord(R.ev[segs], a.stream)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(R.side, R.ev[segs], 0)) != hipSuccess) return e;
  stage_begin(a, kStageIntra, R.side);
  for (int s = 0; s < segs; ++s) {
    if ((e = mfma::launch_intra(p, a, M, P, cs, bounds[s], bounds[s + 1], R.side)) != hipSuccess) return e;
    if ((e = hipEventRecord(R.ev[s], R.side)) != hipSuccess) return e;
  }
  stage_end(a, kStageIntra, R.side);
  // the state pass: range s after the intra kernel of range s; the state is
  // carried between ranges in the workspace (each workgroup reads and writes
  // only its own slice, so in place is safe).  The last wait joins the side
  // stream back into the caller's stream.
  stage_begin(a, kStageState);
  for (int s = 0; s < segs; ++s) {
    if ((e = hipStreamWaitEvent(a.stream, R.ev[s], 0)) != hipSuccess) return e;
    const float *sin = s == 0 ? a.state_in : seg_state;
    float *sout = s == segs - 1 ? a.state_out : seg_state;
    if ((e = launch_chain(p, a, M, P, cs, bounds[s], bounds[s + 1], sin, sout, a.stream)) != hipSuccess) return e;
  }
  stage_end(a, kStageState);
  return hipSuccess;
}

}  // namespace gdn
