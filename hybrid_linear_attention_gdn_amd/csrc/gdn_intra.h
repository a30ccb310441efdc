// Intra-chunk work of the MFMA family: the per-chunk operands of the state
// pass for one (b, h, chunk), run by a group of four waves (256 threads).  It
// is a device function: the scan kernel (gdn_scan.hip) runs it in the blocks
// that do not run the state pass.
//
// With raw bf16 rows K, Q of the chunk (fp8 inputs are widened to bf16 exactly
// on load) and fp32 scales (all derived here from the raw inputs: rk = 1/||k||,
// rq = 1/||q||, beta = sigmoid(logit), G = the chunk-local inclusive cumulative
// floored log-decay):
//   A_ri = beta_r rk_r rk_i e^{G_r - G_i} (k_r . k_i)   (i < r)
//   P_ri = rq_r rk_i e^{G_r - G_i} (q_r . k_i)          (i <= r)
//   T    = (I + A)^{-1}
//   M    = K^T diag(s) T,  s_i = rk_i e^{G_n - G_i};     P' = P T
//   P''  = P' diag(beta),  Q' = Q~ + P' K~  (K~ = -diag(beta gamma rk) K,
//                                             Q~ = diag(gamma rq) Q)
// (the algebra behind these is written out in gdn_mfma_common.h).
//
// Steps:
//  1. K rows -> LDS (row-major and transposed); squared norms of K and Q rows.
//  2. K K^T and K Q^T on the matrix cores.  Wave w owns block-row I = 4 - w of
//     T: it forms the blocks A_IK (K < I) transposed, so that each accumulator
//     tile is directly the A-operand fragment A_IK needs below.  P goes to LDS.
//  3. T, blocked: the diagonal blocks D_I = (I + A_II)^{-1} by forward
//     substitution (fp32, one column per thread), then block distance L = 1..4:
//     T_IJ = -D_I sum_{K=J}^{I-1} A_IK T_KJ on the matrix cores with bf16 hi/lo
//     operands and fp32 accumulation, one block per wave per level.
//  4. M^T = T^T diag(s) K and P'^T = T^T P^T on the matrix cores (bf16 hi/lo
//     operands, fp32 accumulation), each wave owning whole token-row tiles;
//     the accumulators are exactly the A-operand fragments the state pass
//     reads.  M is rounded once to fp16 (round to nearest even) and stored;
//     P'' = P' diag(beta) is stored as a bf16 hi/lo pair, and P' itself
//     (fp32) goes to LDS for step 5.
//  5. Q'^T = Q~^T + K^T (P' diag(w))^T, w = -beta gamma rk, on the matrix cores
//     (exact bf16 K^T against hi/lo P' diag(w)), accumulating onto Q~^T; the
//     accumulators are again the state pass's A-operand fragments of Q', rounded
//     to fp16 and stored.
// T, P and P' live in LDS as 16 x 16 fp32 blocks with 16-byte aligned rows, so
// every operand fragment is one 128-bit LDS read.
#pragma once
#include "gdn_mfma_common.h"

namespace gdn {
namespace mfma {

constexpr int kKrRow = 116;  // bf16 per K row (232 B): 8-byte reads of 16 rows hit distinct banks
constexpr int kKtRow = 84;   // bf16 per K^T row (168 B)
constexpr int kBs = 20;      // floats per row of a stored 16 x 16 block (80 B)
constexpr int kBlkF = 16 * kBs;
constexpr int kLdsT = 0;                              // 15 blocks of T^T, over the dead K rows
constexpr int kLdsKr = 0;
constexpr int kLdsKt = 15 * kBlkF * 4;                // 19,200: Q rows until step 2 ends, then K^T
constexpr int kLdsQr = kLdsKt;
constexpr int kLdsP = kLdsKt + 112 * kKtRow * 2;      // +18,816
constexpr int kLdsAd = kLdsP + 15 * kBlkF * 4;        // +19,200: diagonal blocks of A
constexpr int kLdsD = kLdsAd + 5 * kBlkF * 4;         // +6,400: diagonal blocks of T, row-major
constexpr int kLdsPp = kLdsAd;                        // step 4 on: 15 blocks of P', over the dead A and D blocks
constexpr int kLdsSc = kLdsPp + 15 * kBlkF * 4;       // +19,200
constexpr int kLdsIntra = kLdsSc + 8 * 80 * 4;        // +2,560 = 78,976: two workgroups per CU
static_assert(80 * kKrRow * 2 <= kLdsKt, "K rows fit under the T blocks");
static_assert(2 * 80 * 14 * 4 <= 15 * kBlkF * 4, "norm partial sums fit in the P region");

__device__ __forceinline__ F16 f16_of(const uint32_t *w) { return F16{{w[0], w[1]}}; }

// inclusive prefix sum over the 64 lanes of a wave (DPP row shifts within rows
// of 16 lanes, then row broadcasts across them)
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xf, true));
}
__device__ __forceinline__ float wave_scan(float x) {
  x += dpp<0x111>(x);       // row_shr:1
  x += dpp<0x112>(x);       // row_shr:2
  x += dpp<0x114>(x);       // row_shr:4
  x += dpp<0x118>(x);       // row_shr:8
  x += dpp<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}
__device__ __forceinline__ float lane_value(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
// e^x on the hardware exp2 (relative error a few ulp for |x| up to ~100)
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

// One chunk-head: q, k bf16 or (kFp8) E4M3FN elements, addressed in bytes.
// `lds` is this group's kLdsIntra bytes; `tid` its thread index 0..255.  Every
// __syncthreads() here is reached by all threads of the block, whatever their
// group: a group with valid == false (a block's spare half) runs the same
// steps on zero rows and stores nothing.
template <bool kFp8>
__device__ __forceinline__ void intra_chunk(char *lds, const char *__restrict__ q, const char *__restrict__ k,
                                            const float *__restrict__ g, const float *__restrict__ beta,
                                            char *__restrict__ rec, int T, int H, int b, int h, int c,
                                            uint32_t flags, int tid, bool valid) {
  char *Mrec = rec + kRecM, *Prec = rec + kRecP, *Plrec = rec + kRecPl;
  float *cs = reinterpret_cast<float *>(rec + kRecCs);
  uint16_t *Kr = reinterpret_cast<uint16_t *>(lds + kLdsKr);
  uint16_t *Kt = reinterpret_cast<uint16_t *>(lds + kLdsKt);
  float *Tt = reinterpret_cast<float *>(lds + kLdsT);   // block (I, J), I >= J: [jj][m] = T[16I+m][16J+jj]
  float *Pb = reinterpret_cast<float *>(lds + kLdsP);   // block (R, K), R >= K: [rr][kk] = P[16R+rr][16K+kk]
  float *Ad = reinterpret_cast<float *>(lds + kLdsAd);  // block I: [ii][kk] = A[16I+ii][16I+kk]
  float *Dm = reinterpret_cast<float *>(lds + kLdsD);   // block I: [ii][jj] = T[16I+ii][16I+jj]
  float *Pp = reinterpret_cast<float *>(lds + kLdsPp);  // block (R, I), R >= I: [rr][ii] = P'[16R+rr][16I+ii]
  float *sc = reinterpret_cast<float *>(lds + kLdsSc);
  float *sbeta = sc, *srq = sc + 80, *srk = sc + 160, *sG = sc + 240, *ss = sc + 320, *sw = sc + 400;
  auto blk = [](float *base, int I, int J) { return base + tri(I, J) * kBlkF; };

  const int t0 = c * C;
  const int n = valid ? min(C, T - t0) : 0;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
  const int ln = lane & 15, lg = lane >> 4;
  const size_t rowstride = size_t(H) * D;  // elements between consecutive tokens

  // ---- (0) raw decays and beta inputs of this chunk (scratch in the D region).
  // The reverse scan reads its tokens last to first and takes each token's
  // decay from its successor in the original order (none for the last token).
  const bool rev = flags & kReverse;
  float *gl = Dm, *bl = Dm + 80;
  if (tid < C) {
    const bool ok = tid < n;
    const int tau = t0 + tid;
    const size_t th = (size_t(b) * T + phys_token(tau, T, rev)) * H + h;
    float gv = 0.f;
    if (ok) gv = !rev ? g[th] : (tau > 0 ? g[th + H] : 0.f);
    gl[tid] = ok ? floor_log_decay(gv) : 0.f;
    bl[tid] = ok ? beta[th] : 0.f;
  }
  // ---- (1) K and Q rows -> LDS (row-major); partial sums of squares over 14
  // slices of 8, summed below in a fixed order.  All row loads are issued
  // before any is used.
  float *sqk = Pb, *sqq = Pb + C * 14;
  uint16_t *Qr = reinterpret_cast<uint16_t *>(lds + kLdsQr);
  constexpr size_t kElem = kFp8 ? 1 : 2;  // bytes per input element
  const char *kbase = k + (size_t(b) * T * rowstride + size_t(h) * D) * kElem;
  const char *qbase = q + (size_t(b) * T * rowstride + size_t(h) * D) * kElem;
  constexpr int kRowPieces = (C * 14 + 255) / 256;  // 5 pieces of 8 elements per thread and matrix
  Elems8<kFp8> kraw[kRowPieces], qraw[kRowPieces];
#pragma unroll
  for (int i = 0; i < kRowPieces; ++i) {
    const int idx = tid + 256 * i, r = idx / 14, cc = idx % 14;
    const bool ok = idx < C * 14 && r < n;
    const size_t off = (size_t(phys_token(t0 + r, T, rev)) * rowstride + cc * 8) * kElem;
    kraw[i] = ok ? ld_elems8<kFp8>(kbase + off) : Elems8<kFp8>{};
    qraw[i] = ok ? ld_elems8<kFp8>(qbase + off) : Elems8<kFp8>{};
  }
#pragma unroll
  for (int i = 0; i < kRowPieces; ++i) {
    const int idx = tid + 256 * i, r = idx / 14, cc = idx % 14;
    if (idx < C * 14) {
      const uint4 kv = elems8_bf16<kFp8>(kraw[i]), qv = elems8_bf16<kFp8>(qraw[i]);
      uint2 *kr = reinterpret_cast<uint2 *>(Kr + r * kKrRow + cc * 8);
      uint2 *qr = reinterpret_cast<uint2 *>(Qr + r * kKrRow + cc * 8);
      kr[0] = make_uint2(kv.x, kv.y);
      kr[1] = make_uint2(kv.z, kv.w);
      qr[0] = make_uint2(qv.x, qv.y);
      qr[1] = make_uint2(qv.z, qv.w);
      const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
      const uint32_t wq[4] = {qv.x, qv.y, qv.z, qv.w};
      float pk = 0.f, pq = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float fk = bf16_to_f32(uint16_t(w[j >> 1] >> (16 * (j & 1))));
        const float fq = bf16_to_f32(uint16_t(wq[j >> 1] >> (16 * (j & 1))));
        pk = fmaf(fk, fk, pk);
        pq = fmaf(fq, fq, pq);
      }
      sqk[r * 14 + cc] = pk;
      sqq[r * 14 + cc] = pq;
    }
  }
  __syncthreads();
  // step 5's operand: q_r[16 Dt + 4 lg .. + 3] for this wave's d_k tiles Dt = wave, wave + 4 and
  // rows r = 16 Rt + ln (four bf16 per tile), kept in registers from here: the Q rows' LDS is
  // reused after step 2
  uint2 q5[2][CT];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass)
#pragma unroll
    for (int Rt = 0; Rt < CT; ++Rt) {
      const int Dt = min(wave + 4 * pass, NT - 1);
      q5[pass][Rt] = *reinterpret_cast<const uint2 *>(Qr + (16 * Rt + ln) * kKrRow + 16 * Dt + 4 * lg);
    }
  // per-token scalars: beta, 1/||k||, 1/||q||, G; chunk scalars for the state pass.
  // Waves 0 and 1 take tokens 64 w + lane; G, the inclusive prefix sum of the
  // floored log-decays over the chunk, comes from wave scans of its two parts.
  // The hardware reciprocal square root, reciprocal and exp2 are within a few
  // ulp (the bf16 path's error budget is 1e-2 of rms(o)).
  if (wave < 2) {
    const float G0 = wave_scan(gl[lane]);                               // tokens 0 .. 63
    const float G1 = wave_scan(lane < C - 64 ? gl[64 + lane] : 0.f);   // tokens 64 .. 79, local
    const float G0_last = lane_value(G0, 63);
    const float Gl = G0_last + lane_value(G1, C - 65);  // G at the chunk's last token
    const int t = 64 * wave + lane;
    if (t < C) {
      const bool ok = t < n;
      float nk = 0.f, nq = 0.f;
#pragma unroll
      for (int cc = 0; cc < 14; ++cc) {
        nk += sqk[t * 14 + cc];
        nq += sqq[t * 14 + cc];
      }
      const float rk = (flags & kQkPrenormalized) ? 1.f : __builtin_amdgcn_rsqf(fmaxf(nk, 1e-12f));
      const float rq = (flags & kQkPrenormalized) ? 1.f : __builtin_amdgcn_rsqf(fmaxf(nq, 1e-12f));
      const float bt = (flags & kBetaIsProb) ? bl[t] : __builtin_amdgcn_rcpf(1.f + fexp(-bl[t]));
      const float G = wave == 0 ? G0 : G0_last + G1;
      const float bo = ok ? bt : 0.f, rko = ok ? rk : 0.f, rqo = ok ? rq : 0.f;
      sbeta[t] = bo;
      srq[t] = rqo;
      srk[t] = rko;
      sG[t] = G;
      ss[t] = rko * fexp(Gl - G);
      sw[t] = -(bo * fexp(G)) * rko;  // K~ = diag(w) K
      if (valid) cs[t] = bo;
    }
    if (valid && wave == 0 && lane == 0) cs[kCsGammaN] = fexp(Gl);
  }
  __syncthreads();

  // ---- (1b) the state pass's key operand, rounded to fp16, as a fragment
  // image: K~ = -diag(beta gamma) K^, where K^ = diag(rk) K are the normalised
  // rows (so that R = diag(beta) V + K~ S^T comes straight out of the matrix
  // product).  Per token tile t, blocks kb = 0..2 hold d_k 32 kb + 8 g .. + 7
  // of row 16 t + (lane & 15) (g = lane >> 4) for all 64 lanes.  Within a
  // block the lane's eight d_k are in the "pair" order of the state's
  // accumulator tiles: d_k 32 kb + 4 g .. + 3, then 32 kb + 16 + 4 g .. + 3; block
  // 3 stores only d_k 96 + 4 g .. + 3 (8 bytes per lane).
  if (valid) {
    constexpr int kPerTile = 4 * 64;
    for (int idx = tid; idx < CT * kPerTile; idx += 256) {
      const int t = idx / kPerTile, x = idx % kPerTile;
      const int kb = x / 64, l = x % 64, lg4 = l >> 4;
      const int row = 16 * t + (l & 15);
      const uint16_t *src = Kr + row * kKrRow + 32 * kb + 4 * lg4;
      const float sc = sw[row];
      // d_k 32 kb + 4 g .. + 3 and, below d_k 112, 32 kb + 16 + 4 g .. + 3
      const uint2 lo = *reinterpret_cast<const uint2 *>(src);
      const uint2 hi = kb < 3 ? *reinterpret_cast<const uint2 *>(src + 16) : make_uint2(0u, 0u);
      const uint32_t wd[4] = {lo.x, lo.y, hi.x, hi.y};
      uint32_t pk[4];
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2)
        pk[i2] = pack_f16x2(sc * __uint_as_float(wd[i2] << 16), sc * __uint_as_float(wd[i2] & 0xffff0000u));
      char *dst = rec + kRecK + kq_off(t, kb);
      if (kb < 3)
        *reinterpret_cast<uint4 *>(dst + 16 * l) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      else
        *reinterpret_cast<uint2 *>(dst + 8 * l) = make_uint2(pk[0], pk[1]);
    }
  }

  // ---- (2) K K^T (transposed A blocks of this wave's block-row) and K Q^T
  // K fragments over d in "pair" k-order: one tile = 3 x 32-deep + 1 x 16-deep
  auto kfrag32 = [&](int row, int kb) {
    const uint16_t *p = Kr + row * kKrRow + 32 * kb + 4 * lg;
    const uint2 a = *reinterpret_cast<const uint2 *>(p), bq = *reinterpret_cast<const uint2 *>(p + 16);
    return F32{{a.x, a.y, bq.x, bq.y}};
  };
  auto kfrag16 = [&](int row) {
    const uint2 a = *reinterpret_cast<const uint2 *>(Kr + row * kKrRow + 96 + 4 * lg);
    return F16{{a.x, a.y}};
  };
  auto qfrag32 = [&](int row, int kb) {
    const uint16_t *p = Qr + row * kKrRow + 32 * kb + 4 * lg;
    const uint2 a = *reinterpret_cast<const uint2 *>(p), bq = *reinterpret_cast<const uint2 *>(p + 16);
    return F32{{a.x, a.y, bq.x, bq.y}};
  };
  auto qfrag16 = [&](int row) {
    const uint2 a = *reinterpret_cast<const uint2 *>(Qr + row * kKrRow + 96 + 4 * lg);
    return F16{{a.x, a.y}};
  };
  // decay factor e^{x}, x = G_r - G_i <= 0, on the hardware exp2
  auto decay = [](float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); };
  auto ld4 = [](const float *p) {
    const float4 t = *reinterpret_cast<const float4 *>(p);
    return f32x4{t.x, t.y, t.z, t.w};
  };
  // Steps 2 and 3 depend on the wave's block-row I = 4 - wave; they are
  // instantiated per wave so that the block loops unroll with constant bounds
  // and the independent tiles' products and loads interleave.
  auto blockrow = [&](auto wc) {
    constexpr int W = decltype(wc)::value;
    constexpr int I = 4 - W;  // block-row of T owned by this wave (4, 3, 2, 1)
    // K tile I: the B operand of every A_IK (K < I) and both operands of A_II
    F32 kI[3];
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) kI[kb] = kfrag32(16 * I + ln, kb);
    const F16 kIt = kfrag16(16 * I + ln);
    // tile with rows from tile Ka of K and the columns held in (b, bt): acc[e] = k_{16Ka+4lg+e} . col_{ln}
    auto rows_times = [&](int Ka, const F32 *b, const F16 &bt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) acc = mma(kfrag32(16 * Ka + ln, kb), b[kb], acc);
      return mma(kfrag16(16 * Ka + ln), bt, acc);
    };
    // A_{r i} = beta_r rk_r rk_i e^{G_r - G_i} (k_r . k_i) for i < r, with r = 16Ir + ln, i = 16K + 4lg + e
    auto a_scale = [&](const f32x4 &acc, int Ir, int K, float *out) {
      const int r = 16 * Ir + ln;
      const float fr = sbeta[r] * srk[r], Gr = sG[r];
      const f32x4 rk4 = ld4(srk + 16 * K + 4 * lg), G4 = ld4(sG + 16 * K + 4 * lg);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * K + 4 * lg + e;
        out[e] = (i < r) ? fr * rk4[e] * decay(Gr - G4[e]) * acc[e] : 0.f;
      }
    };
    F16 Ah[4], Al[4];  // A_IK, K < I, as 16-deep A-operand fragments (hi, lo)
#pragma unroll
    for (int K = 0; K < 4; ++K) {
      Ah[K] = F16{{0, 0}};
      Al[K] = F16{{0, 0}};
      if (K < I) {
        float v[4];
        a_scale(rows_times(K, kI, kIt), I, K, v);
        uint32_t hi[2], lo[2];
        split4(v, hi, lo);
        Ah[K] = f16_of(hi);
        Al[K] = f16_of(lo);
      }
    }
    // diagonal blocks A_II (and A_00 by the last wave) -> LDS, row-major
    {
      float v[4];
      a_scale(rows_times(I, kI, kIt), I, I, v);
      *reinterpret_cast<float4 *>(Ad + I * kBlkF + ln * kBs + 4 * lg) = make_float4(v[0], v[1], v[2], v[3]);
      if constexpr (W == 3) {
        F32 k0[3];
#pragma unroll
        for (int kb = 0; kb < 3; ++kb) k0[kb] = kfrag32(ln, kb);
        a_scale(rows_times(0, k0, kfrag16(ln)), 0, 0, v);
        *reinterpret_cast<float4 *>(Ad + ln * kBs + 4 * lg) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    // P^T tiles (kk-tile It <= query tile Rt): acc[e] = k_{16It+4lg+e} . q_{16Rt+ln}
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int tix = W + 4 * s2;
      if (tix < 15) {
        int Rt = 0;
        while (tri(Rt + 1, 0) <= tix) ++Rt;
        const int It = tix - tri(Rt, 0);
        F32 qR[3];
#pragma unroll
        for (int kb = 0; kb < 3; ++kb) qR[kb] = qfrag32(16 * Rt + ln, kb);
        const f32x4 acc = rows_times(It, qR, qfrag16(16 * Rt + ln));
        const int r = 16 * Rt + ln;
        const float fr = srq[r], Gr = sG[r];
        const f32x4 rk4 = ld4(srk + 16 * It + 4 * lg), G4 = ld4(sG + 16 * It + 4 * lg);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * It + 4 * lg + e;
          v[e] = (i <= r) ? fr * rk4[e] * decay(Gr - G4[e]) * acc[e] : 0.f;
        }
        *reinterpret_cast<float4 *>(blk(Pb, Rt, It) + ln * kBs + 4 * lg) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    __syncthreads();
    // Q rows are dead: K^T (d-major, for step 4) takes their place, built from the
    // K rows two tokens at a time (one 32-bit LDS write per d), consecutive lanes
    // on consecutive token pairs of the same 8 columns
    for (int idx = tid; idx < (C / 2) * 14; idx += 256) {
      const int r = 2 * (idx % (C / 2)), cc = idx / (C / 2);
      const uint2 *k0 = reinterpret_cast<const uint2 *>(Kr + r * kKrRow + cc * 8);
      const uint2 *k1 = reinterpret_cast<const uint2 *>(Kr + (r + 1) * kKrRow + cc * 8);
      const uint2 a0 = k0[0], a1 = k0[1], b0 = k1[0], b1 = k1[1];
      const uint32_t wa[4] = {a0.x, a0.y, a1.x, a1.y}, wb[4] = {b0.x, b0.y, b1.x, b1.y};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t lo = (wa[j >> 1] >> (16 * (j & 1))) & 0xffffu, hi = (wb[j >> 1] >> (16 * (j & 1))) & 0xffffu;
        *reinterpret_cast<uint32_t *>(Kt + (cc * 8 + j) * kKtRow + r) = lo | (hi << 16);
      }
    }
    __syncthreads();  // K rows are dead from here on: their LDS now holds the T blocks

    // ---- (3a) diagonal blocks of T by forward substitution, one column per thread
    if (tid < C) {
      const int Ib = tid >> 4, cc = tid & 15;
      const float *A = Ad + Ib * kBlkF;
      float xv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) s = fmaf(A[r * kBs + m], xv[m], s);
        xv[r] = (r < cc) ? 0.f : (r == cc ? 1.f : -s);
      }
      float *Dr = Dm + Ib * kBlkF;
#pragma unroll
      for (int r = 0; r < 16; ++r) Dr[r * kBs + cc] = xv[r];
      float4 *Tr = reinterpret_cast<float4 *>(blk(Tt, Ib, Ib) + cc * kBs);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) Tr[q4] = make_float4(xv[4 * q4], xv[4 * q4 + 1], xv[4 * q4 + 2], xv[4 * q4 + 3]);
    }
    __syncthreads();
    // ---- (3b) off-diagonal blocks, one block-distance per step
#pragma unroll
    for (int L = 1; L < CT; ++L) {
      const int J = I - L;
      if (J >= 0) {
        f32x4 X = zero4();
#pragma unroll
        for (int K = 0; K < 4; ++K) {
          if (K >= J && K < I) {
            // B operand T_KJ: lane (column jj = ln, group lg) holds T[16K + 4lg + j][16J + ln]
            uint32_t th[2], tl[2];
            split4(ld4(blk(Tt, K, J) + ln * kBs + 4 * lg), th, tl);
            const F16 bh = f16_of(th), bl = f16_of(tl);
            X = mma(Ah[K], bh, X);
            X = mma(Ah[K], bl, X);
            X = mma(Al[K], bh, X);
          }
        }
        uint32_t xh[2], xl[2], dh[2], dl[2];
        split4(X, xh, xl);
        split4(ld4(Dm + I * kBlkF + ln * kBs + 4 * lg), dh, dl);
        f32x4 Tij = zero4();
        Tij = mma(f16_of(dh), f16_of(xh), Tij);
        Tij = mma(f16_of(dh), f16_of(xl), Tij);
        Tij = mma(f16_of(dl), f16_of(xh), Tij);
        // accumulator: column jj = ln, rows ii = 4lg + e -> T[16I + 4lg + e][16J + ln]
        *reinterpret_cast<float4 *>(blk(Tt, I, J) + ln * kBs + 4 * lg) = make_float4(-Tij[0], -Tij[1], -Tij[2], -Tij[3]);
      }
      __syncthreads();
    }
  };
  switch (wave) {
    case 0: blockrow(std::integral_constant<int, 0>{}); break;
    case 1: blockrow(std::integral_constant<int, 1>{}); break;
    case 2: blockrow(std::integral_constant<int, 2>{}); break;
    default: blockrow(std::integral_constant<int, 3>{}); break;
  }

  // ---- (4) M^T = T^T diag(s) K  and  P'^T = T^T P^T, split and stored.
  // Each wave owns whole token-row tiles, so it builds their bf16 hi/lo
  // A-operand fragments once and sweeps the other dimension:
  //   M rows Rt (over the 7 d tiles): wave 0: 0, wave 1: 1, wave 2: 2, wave 3: 3 and 4;
  //   P' rows It (over query tiles Rt >= It): wave 0: 4, wave 1: 2 and 3, wave 2: 1, wave 3: 0.
  // Row r of T^T over columns i = 16p + 4lg .. +3 (p >= r / 16): one 128-bit read.
  auto tt4 = [&](int r, int p) { return ld4(blk(Tt, p, r >> 4) + (r & 15) * kBs + 4 * lg); };
  auto pair = [](const F16 &a, const F16 &b) { return F32{{a.w[0], a.w[1], b.w[0], b.w[1]}}; };
  auto m_rows = [&](int Rt) {
    const int r = 16 * Rt + ln;
    F16 uh[CT], ul[CT];  // (T^T diag(s)) rows r over token tile p, hi/lo
#pragma unroll
    for (int p = 0; p < CT; ++p) {
      if (p >= Rt) {
        const f32x4 t = tt4(r, p), s4 = ld4(ss + 16 * p + 4 * lg);
        const float v[4] = {t[0] * s4[0], t[1] * s4[1], t[2] * s4[2], t[3] * s4[3]};
        uint32_t hi[2], lo[2];
        split4(v, hi, lo);
        uh[p] = f16_of(hi);
        ul[p] = f16_of(lo);
      }
    }
#pragma unroll
    for (int Dt = 0; Dt < NT; ++Dt) {
      const uint16_t *kt = Kt + (16 * Dt + ln) * kKtRow + 4 * lg;
      f32x4 acc = zero4();
#pragma unroll
      for (int p = 0; p < CT; ++p) {
        if (p >= Rt && !((p - Rt) & 1)) {
          if (p + 1 < CT) {  // 32-deep block over token tiles p, p + 1
            const uint2 k0 = *reinterpret_cast<const uint2 *>(kt + 16 * p), k1 = *reinterpret_cast<const uint2 *>(kt + 16 * p + 16);
            const F32 bk{{k0.x, k0.y, k1.x, k1.y}};
            acc = mma(pair(uh[p], uh[p + 1]), bk, acc);
            acc = mma(pair(ul[p], ul[p + 1]), bk, acc);
          } else {  // 16-deep block over tile p
            const uint2 k0 = *reinterpret_cast<const uint2 *>(kt + 16 * p);
            const F16 bk{{k0.x, k0.y}};
            acc = mma(uh[p], bk, acc);
            acc = mma(ul[p], bk, acc);
          }
        }
      }
      // accumulator: column d = 16Dt + ln, rows r = 16Rt + 4lg + e -> M[d][r], the state pass's A-operand order
      if (valid) {
        const uint2 w = pack_f16x4(acc);
        if (Rt < 4)
          *reinterpret_cast<uint2 *>(Mrec + m_off32(Dt, Rt >> 1) + lane * 16 + (Rt & 1) * 8) = w;
        else
          *reinterpret_cast<uint2 *>(Mrec + m_off16(Dt) + lane * 8) = w;
      }
    }
  };
  // P'^T[i][r] = sum_{kk=i}^{r} T^T[i][kk] P^T[kk][r]: A rows i = 16It + ln, B columns r = 16Rt + ln
  auto p_rows = [&](int It) {
    const int i = 16 * It + ln;
    F16 th[CT], tl[CT];
#pragma unroll
    for (int p = 0; p < CT; ++p) {
      if (p >= It) {
        uint32_t hi[2], lo[2];
        split4(tt4(i, p), hi, lo);
        th[p] = f16_of(hi);
        tl[p] = f16_of(lo);
      }
    }
#pragma unroll
    for (int Rt = 0; Rt < CT; ++Rt) {
      if (Rt < It) continue;
      f32x4 acc = zero4();
#pragma unroll
      for (int p = 0; p < CT; ++p) {
        if (p >= It && p <= Rt && !((p - It) & 1)) {
          if (p + 1 <= Rt) {
            F32 bh, bl;
            split4(ld4(blk(Pb, Rt, p) + ln * kBs + 4 * lg), bh.w, bl.w);
            split4(ld4(blk(Pb, Rt, p + 1) + ln * kBs + 4 * lg), bh.w + 2, bl.w + 2);
            const F32 ah = pair(th[p], th[p + 1]), al = pair(tl[p], tl[p + 1]);
            acc = mma(ah, bh, acc);
            acc = mma(ah, bl, acc);
            acc = mma(al, bh, acc);
          } else {
            uint32_t bh[2], bl[2];
            split4(ld4(blk(Pb, Rt, p) + ln * kBs + 4 * lg), bh, bl);
            acc = mma(th[p], f16_of(bh), acc);
            acc = mma(th[p], f16_of(bl), acc);
            acc = mma(tl[p], f16_of(bh), acc);
          }
        }
      }
      // accumulator: column r = 16Rt + ln, rows i = 16It + 4lg + e -> P'[r][i], the state pass's
      // A-operand order.  P'' = P' diag(beta) goes out as a bf16 hi/lo pair, P' to LDS.
      if (valid) {
        const f32x4 b4 = ld4(sbeta + 16 * It + 4 * lg);
        const float v[4] = {acc[0] * b4[0], acc[1] * b4[1], acc[2] * b4[2], acc[3] * b4[3]};
        uint32_t hi[2], lo[2];
        split4(v, hi, lo);
        const int off = (It == Rt && !(Rt & 1)) ? p_off16(Rt) + lane * 8 : p_off32(Rt, It >> 1) + lane * 16 + (It & 1) * 8;
        *reinterpret_cast<uint2 *>(Prec + off) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2 *>(Plrec + off) = make_uint2(lo[0], lo[1]);
      }
      *reinterpret_cast<float4 *>(blk(Pp, Rt, It) + ln * kBs + 4 * lg) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  };
  switch (wave) {
    case 0: m_rows(0); p_rows(4); break;
    case 1: m_rows(1); p_rows(2); p_rows(3); break;
    case 2: m_rows(2); p_rows(1); break;
    default: m_rows(3); m_rows(4); p_rows(0); break;
  }
  __syncthreads();  // P' complete in LDS

  // ---- (5) Q'^T = Q~^T + K^T (P' diag(w))^T, w = -beta gamma rk: A rows d = 16Dt + ln from
  // K^T (exact bf16), B columns r = 16Rt + ln over tokens i <= r from P' diag(w) (bf16 hi/lo),
  // accumulating onto Q~^T[d][r] = gamma_r rq_r q_r[d].  The accumulator of (Dt, Rt) holds
  // Q'[r][16Dt + 4lg + e] for column r: the state pass's A-operand fragment of Q' (pair order
  // over d_k, like K~).  Wave w takes the d_k tiles w and w + 4.
  {
    F16 bh[CT][CT], bl[CT][CT];  // [Rt][p], p <= Rt: tokens 16p + 4lg .. + 3 of column r = 16Rt + ln
#pragma unroll
    for (int Rt = 0; Rt < CT; ++Rt)
#pragma unroll
      for (int p = 0; p <= Rt; ++p) {
        const f32x4 x = ld4(blk(Pp, Rt, p) + ln * kBs + 4 * lg), w4 = ld4(sw + 16 * p + 4 * lg);
        const float v[4] = {x[0] * w4[0], x[1] * w4[1], x[2] * w4[2], x[3] * w4[3]};
        uint32_t hi[2], lo[2];
        split4(v, hi, lo);
        bh[Rt][p] = f16_of(hi);
        bl[Rt][p] = f16_of(lo);
      }
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int Dt = wave + 4 * pass;
      if (Dt < NT) {
        // Q~^T of the five tiles from the q elements kept since step 1
        f32x4 acc[CT];
#pragma unroll
        for (int Rt = 0; Rt < CT; ++Rt) {
          const int r = 16 * Rt + ln;
          const float f = fexp(sG[r]) * srq[r];  // 0 past the chunk's end
          const uint2 w = q5[pass][Rt];  // rows past the chunk's end are zero in LDS
          const float x[4] = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                              __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
          acc[Rt] = f32x4{f * x[0], f * x[1], f * x[2], f * x[3]};
        }
        const uint16_t *kt = Kt + (16 * Dt + ln) * kKtRow + 4 * lg;
#pragma unroll
        for (int Rt = 0; Rt < CT; ++Rt) {
#pragma unroll
          for (int p = 0; p <= Rt; p += 2) {
            if (p + 1 <= Rt) {  // 32-deep block over token tiles p, p + 1
              const uint2 k0 = *reinterpret_cast<const uint2 *>(kt + 16 * p), k1 = *reinterpret_cast<const uint2 *>(kt + 16 * p + 16);
              const F32 ak{{k0.x, k0.y, k1.x, k1.y}};
              acc[Rt] = mma(ak, pair(bh[Rt][p], bh[Rt][p + 1]), acc[Rt]);
              acc[Rt] = mma(ak, pair(bl[Rt][p], bl[Rt][p + 1]), acc[Rt]);
            } else {  // 16-deep block over tile p
              const uint2 k0 = *reinterpret_cast<const uint2 *>(kt + 16 * p);
              const F16 ak{{k0.x, k0.y}};
              acc[Rt] = mma(ak, bh[Rt][p], acc[Rt]);
              acc[Rt] = mma(ak, bl[Rt][p], acc[Rt]);
            }
          }
          if (valid) {
            const uint2 w = pack_f16x4(acc[Rt]);
            if (Dt < 6)
              *reinterpret_cast<uint2 *>(rec + kRecQ + kq_off(Rt, Dt >> 1) + lane * 16 + (Dt & 1) * 8) = w;
            else
              *reinterpret_cast<uint2 *>(rec + kRecQ + kq_off(Rt, 3) + lane * 8) = w;
          }
        }
      }
    }
  }
}

}  // namespace mfma
}  // namespace gdn
