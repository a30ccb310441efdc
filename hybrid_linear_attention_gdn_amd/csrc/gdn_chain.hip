// Kernel "chain" of the MFMA family: the sequential state pass fused with the
// output, one workgroup (4 waves) per (b, h, 16 columns of d_v).
//
// Per chunk (the algebra is in gdn_mfma_common.h):
//   Y = K S^T,  R = diag(beta) V - diag(beta gamma rk) Y,
//   O = diag(gamma rq) Q S^T + P' R,   S^T <- gamma_n S^T + M R.
// The 16 x 112 fp32 state slice S^T lives in accumulator registers as 7 row
// tiles spread over the waves.  Per chunk, two barriers exchange the bf16
// hi/lo operands S (after phase 0) and R (after phase A) through LDS.
//
// Operand traffic.  K, Q and this workgroup's 16 columns of V are loaded two
// chunks ahead by all 256 threads with 16-byte row loads (a 224-byte bf16 row
// is 14 such pieces) into a register set, and written to one of two LDS
// staging buffers a step later; each wave then reads its
// fragments from LDS (rows padded to 232 bytes so the 8-byte fragment reads
// of 16 consecutive rows fall in distinct banks).  The chunk's 1 KB record of
// per-token scales is staged with the rows (one load by wave 0).  The
// fragment-ordered M and P' records are read straight into registers, two
// chunks ahead: every such load is a contiguous 1 KB per instruction.
#include "gdn_mfma_common.h"

#include <algorithm>
#include <mutex>
#include <vector>

namespace gdn {
namespace mfma {
namespace {

// Raw buffer access (gfx9 descriptor, stride 0): an offset at or past
// `bytes` reads zero and drops a store.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
constexpr uint32_t kOutOfRange = 0x7ffffff0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), short(0), int(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
  return make_uint4(x.x, x.y, x.z, x.w);
}

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

constexpr int kRowPad = 116;  // bf16 per staged K/Q row (232 B)
constexpr int kVtPad = 84;    // bf16 per staged V^T row (168 B)
constexpr int kLdsS = 0;                                 // S operand: hi/lo x (3 x 1 KB + 512 B)
constexpr int kLdsR = 2 * (3 * 1024 + 512);              // R operand: hi/lo x (2 x 1 KB + 512 B)
constexpr int kLdsStage = kLdsR + 2 * (2 * 1024 + 512);  // two K/Q/V^T buffers
constexpr int kStageK = 0;
constexpr int kStageQ = C * kRowPad * 2;                 // 18,560
constexpr int kStageV = 2 * C * kRowPad * 2;             // 37,120
constexpr int kStageCs = kStageV + 16 * kVtPad * 2;     // 39,808: the chunk's 256 scale floats
constexpr int kStageBytes = kStageCs + kCsFloats * 4;    // 40,832
constexpr int kLdsChain = kLdsStage + 2 * kStageBytes;   // 93,952
static_assert(kStageBytes % 16 == 0, "stage buffers stay 16-byte aligned");

// Everything one wave reads from global memory for one chunk, besides the
// staged rows: independent of the state, so the next chunk's set is in flight
// while the current one is consumed.
struct ChunkOps {
  F32 Mf[3][2][2];           // M fragments of the owned state tiles [tile][block][hi/lo]
  F16 Mt[3][2];
  F32 Pf[2][2][2];           // P' fragments of the output tiles
  F16 Pt[2][2];
};

struct RowFrags {  // one lane's share of a 16-row tile of K or Q (A operand, k = d_k)
  F32 f[3];
  F16 t;
};

template <int W, bool kOutBf16>
__device__ __forceinline__ void chain_role(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                           const uint16_t *__restrict__ v, const char *__restrict__ Mws,
                                           const char *__restrict__ Pws, const float *__restrict__ CS,
                                           const float *state_in, float *state_out, void *__restrict__ o, int T,
                                           int H, int N, int cb, int ce, int b, int h, int nt, char *lds) {
  constexpr Roles ro = kRoles[W];
  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
  const size_t u = size_t(b) * H + h;
  const size_t rowstride = size_t(H) * D;
  char *Slds = lds + kLdsS;
  char *Rlds = lds + kLdsR;

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

  // ---- cooperative staging of K, Q rows and this tile's V columns (all 256 threads).
  // Thread tid takes 16-byte piece (tid & 15) of rows (tid >> 4) + 16 i of K and of Q
  // (pieces 14, 15 of a 224-byte row do not exist), and, for tid < 160, half (tid & 1)
  // of row tid >> 1 of the V tile: every address is a fixed per-thread offset plus the chunk base.
  // The loads are buffer loads through a descriptor that covers exactly the
  // chunk's valid rows: rows past the end (and the non-existent pieces 14, 15)
  // read as zero with no branch, so every wave issues the same memory
  // instructions on every path and the in-order load counter never forces a
  // wait on the next chunk's prefetch.
  const int sp = tid & 15, sr = tid >> 4;
  const bool sp_ok = sp < 14;
  const uint32_t row_bytes = uint32_t(rowstride) * 2u;
  const uint32_t offKQ = sp_ok ? uint32_t(sr) * row_bytes + uint32_t(h) * (D * 2) + 16u * sp : kOutOfRange;
  const uint32_t offV = tid < 2 * C ? uint32_t(tid >> 1) * row_bytes + uint32_t(h) * (D * 2) + 32u * nt + 16u * (tid & 1)
                                    : kOutOfRange;
  struct Staged {
    uint4 k[CT], q[CT], v, cs;  // cs: wave 0 only
  };
  auto stage_issue = [&](Staged &st, int c) {
    const int t0 = c * C, nv = min(C, T - t0);
    const size_t base = (size_t(b) * T + t0) * rowstride;
    const uint32_t bytes = uint32_t(nv) * row_bytes;
    const auto rk_ = make_rsrc(k + base, bytes), rq_ = make_rsrc(q + base, bytes), rv_ = make_rsrc(v + base, bytes);
#pragma unroll
    for (int i = 0; i < CT; ++i) {
      const uint32_t off = offKQ == kOutOfRange ? kOutOfRange : offKQ + uint32_t(16 * i) * row_bytes;
      st.k[i] = buf_load16(rk_, off);
      st.q[i] = buf_load16(rq_, off);
    }
    st.v = buf_load16(rv_, offV);
    if (W == 0) st.cs = ldg16(CS + (u * N + c) * kCsFloats + 4 * lane);  // the chunk's scales: one 1 KB load
  };
  auto stage_store = [&](const Staged &st, int buf) {
    char *sb = lds + kLdsStage + buf * kStageBytes;
    if (sp_ok) {
#pragma unroll
      for (int i = 0; i < CT; ++i) {
        const int off = (sr + 16 * i) * (kRowPad * 2) + 16 * sp;
        uint2 *dk = reinterpret_cast<uint2 *>(sb + kStageK + off);
        uint2 *dq = reinterpret_cast<uint2 *>(sb + kStageQ + off);
        dk[0] = make_uint2(st.k[i].x, st.k[i].y);
        dk[1] = make_uint2(st.k[i].z, st.k[i].w);
        dq[0] = make_uint2(st.q[i].x, st.q[i].y);
        dq[1] = make_uint2(st.q[i].z, st.q[i].w);
      }
    }
    if (tid < 2 * C) {
      uint16_t *vt = reinterpret_cast<uint16_t *>(sb + kStageV);
      const int vr = tid >> 1, half = tid & 1;
      const uint32_t w[4] = {st.v.x, st.v.y, st.v.z, st.v.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) vt[(8 * half + j) * kVtPad + vr] = uint16_t(w[j >> 1] >> (16 * (j & 1)));
    }
    if (W == 0) *reinterpret_cast<uint4 *>(sb + kStageCs + 16 * lane) = st.cs;
  };
  // A-operand fragments of a 16-row tile of the staged K (m = 0) or Q (m = 1), "pair" k-order
  auto rows_frag = [&](int buf, int m, int tile) {
    const char *rowp = lds + kLdsStage + buf * kStageBytes + (m ? kStageQ : kStageK) + (16 * tile + ln) * (kRowPad * 2);
    RowFrags rf;
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) {
      const uint2 x0 = *reinterpret_cast<const uint2 *>(rowp + 64 * kb + 8 * lg);
      const uint2 x1 = *reinterpret_cast<const uint2 *>(rowp + 64 * kb + 32 + 8 * lg);
      rf.f[kb] = F32{{x0.x, x0.y, x1.x, x1.y}};
    }
    const uint2 x2 = *reinterpret_cast<const uint2 *>(rowp + 192 + 8 * lg);
    rf.t = F16{{x2.x, x2.y}};
    return rf;
  };

  // ---- L2 warm-up of chunk c + kAhead: the head's 7 column-tile workgroups
  // (on one XCD) split its cache lines -- 280 of M, 120 of P', 8 of scales and
  // 3 per 224-byte row of K, Q, V -- so that the staging and operand loads of
  // that chunk hit L2 instead of all waiting on the same HBM misses.  One
  // dword load per lane, at a fixed per-lane base plus a per-chunk stride.
  constexpr int kAhead = 4;
  const char *pe_base;
  size_t pe_stride;
  int pe_row = -1;
  {
    const int pe = nt + NT * (64 * (tid >> 6) + lane);  // 0 .. 1791, cache-line task
    if (pe < 280) {
      pe_base = Mws + u * N * size_t(kMBytes) + 128 * pe;
      pe_stride = kMBytes;
    } else if (pe < 400) {
      pe_base = Pws + u * N * size_t(kPBytes) + 128 * (pe - 280);
      pe_stride = kPBytes;
    } else if (pe < 408) {
      pe_base = reinterpret_cast<const char *>(CS + u * N * kCsFloats) + 128 * (pe - 400);
      pe_stride = kCsFloats * sizeof(float);
    } else {
      const int r = min(pe - 408, 3 * 3 * C - 1), t = r / (3 * C), part = r % 3;
      pe_row = (r % (3 * C)) / 3;
      const uint16_t *src = t == 0 ? k : (t == 1 ? q : v);
      pe_base = reinterpret_cast<const char *>(src + (size_t(b) * T * H + h) * D) + (part == 0 ? 0 : (part == 1 ? 128 : 220));
      pe_stride = size_t(C) * row_bytes;
    }
  }
  auto l2_touch = [&](int c) -> uint32_t {
    const int cp = min(c + kAhead, ce - 1);
    // a row past the end of the last chunk touches the chunk's last row instead
    const int rr = pe_row < 0 ? 0 : min(pe_row, T - 1 - cp * C);
    const char *a = pe_base + size_t(cp) * pe_stride + size_t(rr) * row_bytes;
    return *reinterpret_cast<const uint32_t *>(a);
  };

  auto load_ops = [&](ChunkOps &op, int c) {
    const char *Mr = Mws + (u * N + c) * size_t(kMBytes);
    const char *Pr = Pws + (u * N + c) * size_t(kPBytes);
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if (s < ro.nS) {
        const int mt = ro.S[s];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) {
            const uint4 x = ldg16(Mr + m_off32(mt, kb, hl) + lane * 16);
            op.Mf[s][kb][hl] = F32{{x.x, x.y, x.z, x.w}};
          }
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
          const uint2 x = ldg8(Mr + m_off16(mt, hl) + lane * 8);
          op.Mt[s][hl] = F16{{x.x, x.y}};
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < ro.nO) {
        const int R = ro.O[s];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) {
            if (kb < (R + 1) / 2) {
              const uint4 x = ldg16(Pr + p_off32(R, kb, hl) + lane * 16);
              op.Pf[s][kb][hl] = F32{{x.x, x.y, x.z, x.w}};
            }
          }
        if (!(R & 1))
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) {
            const uint2 x = ldg8(Pr + p_off16(R, hl) + lane * 8);
            op.Pt[s][hl] = F16{{x.x, x.y}};
          }
      }
    }
  };

  // one chunk: consume `cur` and staging buffer c & 1; put chunk c + 1 in flight
  auto step = [&](int c, const ChunkOps &cur, ChunkOps &ahead, Staged &st_issue, const Staged &st_store) {
    const int t0 = c * C, nv = min(C, T - t0), buf = c & 1;
    // ---- phase 0: publish this wave's state tiles as bf16 hi/lo B operands
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if (s < ro.nS) {
        const int j = ro.S[s];
        uint32_t hi[2], lo[2];
        split4(S[s], hi, lo);
        if (j < 6) {
          const int kb = j >> 1, half = j & 1;
          *reinterpret_cast<uint2 *>(Slds + kb * 1024 + lane * 16 + half * 8) = make_uint2(hi[0], hi[1]);
          *reinterpret_cast<uint2 *>(Slds + 3584 + kb * 1024 + lane * 16 + half * 8) = make_uint2(lo[0], lo[1]);
        } else {
          *reinterpret_cast<uint2 *>(Slds + 3072 + lane * 8) = make_uint2(hi[0], hi[1]);
          *reinterpret_cast<uint2 *>(Slds + 3584 + 3072 + lane * 8) = make_uint2(lo[0], lo[1]);
        }
      }
    }
    __syncthreads();
    const auto ro_ = make_rsrc(static_cast<char *>(o) + (size_t(b) * T + t0) * rowstride * (kOutBf16 ? 2 : 4),
                               uint32_t(nv) * uint32_t(rowstride) * (kOutBf16 ? 2u : 4u));
    // ---- phase A: S operands, Y = K S^T -> R (published), Q S^T for phase-A tiles
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
    auto rows_times_S = [&](const RowFrags &rf) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) {
        acc = mma(rf.f[kb], Sh[kb], acc);
        acc = mma(rf.f[kb], Sl[kb], acc);
      }
      acc = mma(rf.t, Sth, acc);
      acc = mma(rf.t, Stl, acc);
      return acc;
    };
    const uint16_t *vt = reinterpret_cast<const uint16_t *>(lds + kLdsStage + buf * kStageBytes + kStageV);
    const float *csl = reinterpret_cast<const float *>(lds + kLdsStage + buf * kStageBytes + kStageCs);
    auto ldf4 = [](const float *p) {
      const float4 t = *reinterpret_cast<const float4 *>(p);
      return f32x4{t.x, t.y, t.z, t.w};
    };
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < ro.nY) {
        const int tile = ro.Y[s];
        const f32x4 y = rows_times_S(rows_frag(buf, 0, tile));
        const uint2 vv = *reinterpret_cast<const uint2 *>(vt + ln * kVtPad + 16 * tile + 4 * lg);
        const float va[4] = {__uint_as_float(vv.x << 16), __uint_as_float(vv.x & 0xffff0000u),
                             __uint_as_float(vv.y << 16), __uint_as_float(vv.y & 0xffff0000u)};
        float r4[4];
        const f32x4 aa = ldf4(csl + 16 * tile + 4 * lg), bb = ldf4(csl + 80 + 16 * tile + 4 * lg);
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = aa[e] * va[e] - bb[e] * y[e];
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
    if (ro.nQA) QS[0] = rows_times_S(rows_frag(buf, 1, ro.QA[0]));
    __syncthreads();
    // ---- phase B: R operands; state update and outputs.  The operand
    // fragments of chunk c + 2 are requested here (past the end, the last
    // chunk is fetched again: the same instructions issue on every chunk).
    load_ops(ahead, min(c + 2, ce - 1));
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
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < ro.nQB) QS[s] = rows_times_S(rows_frag(buf, 1, ro.QB[s]));
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if (s < ro.nS) {
        f32x4 acc = S[s] * csl[240];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          acc = mma(cur.Mf[s][kb][0], Rh[kb], acc);
          acc = mma(cur.Mf[s][kb][0], Rl[kb], acc);
          acc = mma(cur.Mf[s][kb][1], Rh[kb], acc);
        }
        acc = mma(cur.Mt[s][0], Rth, acc);
        acc = mma(cur.Mt[s][0], Rtl, acc);
        acc = mma(cur.Mt[s][1], Rth, acc);
        S[s] = acc;
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < ro.nO) {
        const int R = ro.O[s];
        f32x4 acc;
        const f32x4 cc = ldf4(csl + 160 + 16 * R + 4 * lg);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = cc[e] * QS[s][e];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb < (R + 1) / 2) {
            acc = mma(cur.Pf[s][kb][0], Rh[kb], acc);
            acc = mma(cur.Pf[s][kb][0], Rl[kb], acc);
            acc = mma(cur.Pf[s][kb][1], Rh[kb], acc);
          }
        }
        if (!(R & 1)) {
          // the 16-deep block covers token tile R (tile 4: the shared 16-deep R slot;
          // tiles 0 and 2: first halves of the 32-deep R slots)
          F16 rh, rl;
          if (R == 4) {
            rh = Rth;
            rl = Rtl;
          } else {
            const int kb = R >> 1;
            rh = F16{{Rh[kb].w[0], Rh[kb].w[1]}};
            rl = F16{{Rl[kb].w[0], Rl[kb].w[1]}};
          }
          acc = mma(cur.Pt[s][0], rh, acc);
          acc = mma(cur.Pt[s][0], rl, acc);
          acc = mma(cur.Pt[s][1], rh, acc);
        }
        // rows past the chunk's end fall outside the store descriptor and are dropped
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t oi = uint32_t(16 * R + 4 * lg + e) * uint32_t(rowstride) + uint32_t(h) * D + 16u * nt + ln;
          if constexpr (kOutBf16)
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(acc[e]), ro_, int(oi * 2u), 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[e]), ro_, int(oi * 4u), 0, 0);
        }
      }
    }
    // K/Q/V rows two chunks ahead go into the register set freed by the last
    // store; the set loaded one step ago (chunk c + 1) goes to staging buffer
    // (c + 1) & 1, last read in chunk c - 1, before this chunk's first barrier.
    stage_issue(st_issue, min(c + 2, ce - 1));
    stage_store(st_store, buf ^ 1);
  };

  // Three operand sets and three staging register sets rotate with the chunk
  // index mod 3 (chunk c + 1 landed, c + 2 in flight, c being consumed).
  ChunkOps op0, op1, op2;
  Staged st0, st1, st2;
  stage_issue(st0, cb);
  load_ops(op0, cb);
  stage_store(st0, cb & 1);
  stage_issue(st1, min(cb + 1, ce - 1));
  load_ops(op1, min(cb + 1, ce - 1));
  uint32_t pf = 0, sink = 0;
  auto touch = [&](int c) {
    sink ^= pf;  // consumed a step after its load was issued
    pf = l2_touch(c);
  };
  for (int c = cb; c < ce; c += 3) {
    step(c, op0, op2, st2, st1);
    touch(c);
    if (c + 1 < ce) {
      step(c + 1, op1, op0, st0, st2);
      touch(c + 1);
    }
    if (c + 2 < ce) {
      step(c + 2, op2, op1, st1, st0);
      touch(c + 2);
    }
  }
  sink ^= pf;
  if (T < 0 && sink != 0u) static_cast<uint32_t *>(o)[0] = sink;  // never taken: keeps the touches alive
  if (state_out) {
#pragma unroll
    for (int s = 0; s < 3; ++s)
      if (s < ro.nS)
        *reinterpret_cast<float4 *>(state_out + (u * D + 16 * nt + ln) * D + 16 * ro.S[s] + 4 * lg) =
            make_float4(S[s][0], S[s][1], S[s][2], S[s][3]);
  }
}

template <bool kOutBf16>
__global__ __launch_bounds__(256) void chain_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                    const uint16_t *__restrict__ v, const char *__restrict__ Mws,
                                                    const char *__restrict__ Pws, const float *__restrict__ CS,
                                                    const float *state_in, float *state_out,
                                                    void *__restrict__ o, int T, int H, int N, int cb, int ce,
                                                    int units) {
  extern __shared__ __align__(16) char lds[];
  // Workgroup i runs on XCD i % 8: keep the 7 column tiles of a (b, h) on one
  // XCD so that its K, Q, M and P' are fetched from HBM once into that L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int u = xcd + 8 * (slot / NT), nt = slot % NT;
  if (u >= units) return;
  const int b = u / H, h = u % H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  switch (wave) {
    case 0: chain_role<0, kOutBf16>(q, k, v, Mws, Pws, CS, state_in, state_out, o, T, H, N, cb, ce, b, h, nt, lds); break;
    case 1: chain_role<1, kOutBf16>(q, k, v, Mws, Pws, CS, state_in, state_out, o, T, H, N, cb, ce, b, h, nt, lds); break;
    case 2: chain_role<2, kOutBf16>(q, k, v, Mws, Pws, CS, state_in, state_out, o, T, H, N, cb, ce, b, h, nt, lds); break;
    default: chain_role<3, kOutBf16>(q, k, v, Mws, Pws, CS, state_in, state_out, o, T, H, N, cb, ce, b, h, nt, lds); break;
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

hipError_t launch_chain(const Plan &p, const Args &a, const char *M, const char *P, const float *cs, int cb, int ce,
                        const float *sin, float *sout, hipStream_t st) {
  const uint16_t *q = static_cast<const uint16_t *>(a.q), *k = static_cast<const uint16_t *>(a.k),
                 *v = static_cast<const uint16_t *>(a.v);
  const int units = p.B * p.H;
  const unsigned grid = 8u * mfma::NT * unsigned((units + 7) / 8);
  if (p.o_bf16)
    mfma::chain_kernel<true><<<dim3(grid), dim3(256), mfma::kLdsChain, st>>>(q, k, v, M, P, cs, sin, sout, a.o, p.T,
                                                                           p.H, p.N, cb, ce, units);
  else
    mfma::chain_kernel<false><<<dim3(grid), dim3(256), mfma::kLdsChain, st>>>(q, k, v, M, P, cs, sin, sout, a.o, p.T,
                                                                            p.H, p.N, cb, ce, units);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const Plan &p, const Args &a) {
  char *M = a.ws + p.off_M;
  char *P = a.ws + p.off_P;
  float *cs = reinterpret_cast<float *>(a.ws + p.off_cs);
  float *seg_state = reinterpret_cast<float *>(a.ws + p.off_Sseg);
  static const hipError_t lds0 = hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma::chain_kernel<false>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, mfma::kLdsChain);
  static const hipError_t lds1 = hipFuncSetAttribute(reinterpret_cast<const void *>(&mfma::chain_kernel<true>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, mfma::kLdsChain);
  if (lds0 != hipSuccess) return lds0;
  if (lds1 != hipSuccess) return lds1;
  hipError_t e;
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int cus;
  {
    std::lock_guard<std::mutex> lk(g_side_mu);
    if (g_side[dev].cus < 0 &&
        hipDeviceGetAttribute(&g_side[dev].cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      g_side[dev].cus = 0;
    cus = g_side[dev].cus;
  }
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
  SideResources &R = g_side[dev];
  if (!R.side && (e = hipStreamCreateWithFlags(&R.side, hipStreamNonBlocking)) != hipSuccess) {
    R.side = nullptr;
    return e;
  }
  while (int(R.ev.size()) < segs + 1) {
    hipEvent_t ev;
    if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return e;
    R.ev.push_back(ev);
  }
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
