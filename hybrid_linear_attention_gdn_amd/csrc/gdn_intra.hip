// Kernel "intra" of the MFMA family: per (b, h, chunk) operands of the state pass.
// (The chunked algebra and the operand layouts are described in gdn_mfma_common.h.)
#include "gdn_mfma_common.h"

namespace gdn {
namespace mfma {
namespace {

// ============================================================================
// Kernel "intra": one workgroup (4 waves) per (b, h, chunk).
// ============================================================================
constexpr int kKrStride = 120;  // bf16 per row of K (row-major), 240 B
constexpr int kKtStride = 88;   // bf16 per row of K^T (d-major), 176 B
constexpr int kBlk = 16 * 17;   // floats per padded 16x16 block
constexpr int kLdsKr = 0;                                 // K rows, later the A blocks
constexpr int kLdsKt = kLdsKr + 80 * kKrStride * 2;       // 19,200
constexpr int kLdsP = kLdsKt + 112 * kKtStride * 2;       // +19,712
constexpr int kLdsT = kLdsP + 15 * kBlk * 4;              // +16,320
constexpr int kLdsX = kLdsT + 15 * kBlk * 4;              // +16,320
constexpr int kLdsSc = kLdsX + 4 * kBlk * 4;              // +4,352
constexpr int kLdsIntra = kLdsSc + 8 * 80 * 4;            // +2,560
static_assert(15 * kBlk * 4 <= 80 * kKrStride * 2, "A blocks must fit in the K region");

__global__ __launch_bounds__(256, 2) void intra_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                       const float *__restrict__ g, const float *__restrict__ beta,
                                                       char *__restrict__ Mout, char *__restrict__ Pout,
                                                       float *__restrict__ CSout, int T, int H, int N,
                                                       uint32_t flags) {
  extern __shared__ __align__(16) char lds[];
  uint16_t *Kr = reinterpret_cast<uint16_t *>(lds + kLdsKr);
  float *Ab = reinterpret_cast<float *>(lds + kLdsKr);  // aliases Kr after the K K^T products
  uint16_t *Kt = reinterpret_cast<uint16_t *>(lds + kLdsKt);
  float *Pb = reinterpret_cast<float *>(lds + kLdsP);
  float *Tb = reinterpret_cast<float *>(lds + kLdsT);  // block (I,J) holds (T_IJ)^T: [jj][ii]
  float *Xb = reinterpret_cast<float *>(lds + kLdsX);
  float *sc = reinterpret_cast<float *>(lds + kLdsSc);
  float *sbeta = sc, *srq = sc + 80, *srk = sc + 160, *sG = sc + 240, *ss = sc + 320;

  // block -> (b, c, h) with h fastest: neighbouring workgroups read neighbouring rows
  int x = blockIdx.x;
  const int h = x % H;
  x /= H;
  const int c = x % N;
  const int b = x / N;
  const int t0 = c * C;
  const int n = min(C, T - t0);
  const size_t u = size_t(b) * H + h;
  const size_t rec = u * N + c;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;

  // ---- (0) per-token prep fused in: raw decays and beta inputs of this chunk
  const size_t rowstride = size_t(H) * D;  // elements between consecutive tokens
  float *gl = Xb, *bl = Xb + 80;           // scratch until the triangular solve
  if (tid < C) {
    const bool ok = tid < n;
    const size_t th = (size_t(b) * T + t0 + tid) * H + h;
    gl[tid] = ok ? fmaxf(g[th], kLogDecayFloor) : 0.f;
    bl[tid] = ok ? beta[th] : 0.f;
  }
  // ---- (1) K rows -> LDS, row-major and transposed; per-row partial sums of
  // squares of K and Q (14 slices of 8) for the norms, summed in a fixed order
  float *sqk = Pb, *sqq = Pb + C * 14;  // the P blocks are written only after the norms
  const uint16_t *kbase = k + (size_t(b) * T + t0) * rowstride + size_t(h) * D;
  const uint16_t *qrow0 = q + (size_t(b) * T + t0) * rowstride + size_t(h) * D;
  for (int idx = tid; idx < C * 14; idx += 256) {
    const int r = idx / 14, cc = idx % 14;
    uint4 val = make_uint4(0, 0, 0, 0), qv = make_uint4(0, 0, 0, 0);
    if (r < n) {
      val = ldg16(kbase + size_t(r) * rowstride + cc * 8);
      qv = ldg16(qrow0 + size_t(r) * rowstride + cc * 8);
    }
    *reinterpret_cast<uint4 *>(Kr + r * kKrStride + cc * 8) = val;
    const uint32_t w[4] = {val.x, val.y, val.z, val.w};
    const uint32_t wq[4] = {qv.x, qv.y, qv.z, qv.w};
    float pk = 0.f, pq = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint16_t e = uint16_t(w[j >> 1] >> (16 * (j & 1)));
      Kt[(cc * 8 + j) * kKtStride + r] = e;
      const float fk = bf16_to_f32(e), fq = bf16_to_f32(uint16_t(wq[j >> 1] >> (16 * (j & 1))));
      pk = fmaf(fk, fk, pk);
      pq = fmaf(fq, fq, pq);
    }
    sqk[r * 14 + cc] = pk;
    sqq[r * 14 + cc] = pq;
  }
  __syncthreads();
  // per-token scalars: beta, 1/||k||, 1/||q||, chunk-local cumulative decay G
  if (tid < C) {
    const bool ok = tid < n;
    float nk = 0.f, nq = 0.f;
#pragma unroll
    for (int cc = 0; cc < 14; ++cc) {
      nk += sqk[tid * 14 + cc];
      nq += sqq[tid * 14 + cc];
    }
    const float rk = (flags & kQkPrenormalized) ? 1.f : 1.f / fmaxf(sqrtf(nk), 1e-6f);
    const float rq = (flags & kQkPrenormalized) ? 1.f : 1.f / fmaxf(sqrtf(nq), 1e-6f);
    const float bt = (flags & kBetaIsProb) ? bl[tid] : 1.f / (1.f + expf(-bl[tid]));
    // inclusive prefix in token order (the same additions as a sequential scan)
    float G = 0.f, Gl = 0.f;
    for (int j = 0; j < C; ++j) {
      Gl += gl[j];
      if (j == tid) G = Gl;
    }
    const float bo = ok ? bt : 0.f, rko = ok ? rk : 0.f, rqo = ok ? rq : 0.f;
    const float gam = expf(G);
    sbeta[tid] = bo;
    srq[tid] = rqo;
    srk[tid] = rko;
    sG[tid] = G;
    ss[tid] = rko * expf(Gl - G);
    float *cs = CSout + rec * kCsFloats;
    cs[tid] = bo;
    cs[80 + tid] = bo * gam * rko;
    cs[160 + tid] = gam * rqo;
    if (tid == 0) cs[240] = expf(Gl);
  }
  __syncthreads();

  // ---- (2) A (from K K^T) and P (from K Q^T), 15 lower tiles each
  // A-operand rows of K from LDS in "pair" k-order; one tile = 3 x 32-deep + 1 x 16-deep.
  auto kfrag32 = [&](int row, int kb) {
    const uint16_t *p = Kr + row * kKrStride + 32 * kb + 4 * lg;
    const uint2 a = *reinterpret_cast<const uint2 *>(p), bq = *reinterpret_cast<const uint2 *>(p + 16);
    return F32{{a.x, a.y, bq.x, bq.y}};
  };
  auto kfrag16 = [&](int row) {
    const uint2 a = *reinterpret_cast<const uint2 *>(Kr + row * kKrStride + 96 + 4 * lg);
    return F16{{a.x, a.y}};
  };
  const uint16_t *qbase = q + (size_t(b) * T + t0) * rowstride + size_t(h) * D;
  auto qfrag32 = [&](int row, int kb) {
    if (row >= n) return F32{{0, 0, 0, 0}};
    const uint16_t *p = qbase + size_t(row) * rowstride + 32 * kb + 4 * lg;
    const uint2 a = ldg8(p), bq = ldg8(p + 16);
    return F32{{a.x, a.y, bq.x, bq.y}};
  };
  auto qfrag16 = [&](int row) {
    if (row >= n) return F16{{0, 0}};
    const uint2 a = ldg8(qbase + size_t(row) * rowstride + 96 + 4 * lg);
    return F16{{a.x, a.y}};
  };
  // A tiles: wave w takes tiles w, w+4, w+8, w+12 of the 15 (R >= I) in tri order
  f32x4 aacc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    aacc[s] = zero4();
    const int tix = wave + 4 * s;
    if (tix < 15) {
      int R = 0;
      while (tri(R + 1, 0) <= tix) ++R;
      const int I = tix - tri(R, 0);
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) aacc[s] = mma(kfrag32(16 * R + ln, kb), kfrag32(16 * I + ln, kb), aacc[s]);
      aacc[s] = mma(kfrag16(16 * R + ln), kfrag16(16 * I + ln), aacc[s]);
    }
  }
  // P^T tiles (I <= R): accumulator rows = key tokens i, columns = query tokens r
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int tix = wave + 4 * s;
    if (tix < 15) {
      int R = 0;
      while (tri(R + 1, 0) <= tix) ++R;
      const int I = tix - tri(R, 0);
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) acc = mma(kfrag32(16 * I + ln, kb), qfrag32(16 * R + ln, kb), acc);
      acc = mma(kfrag16(16 * I + ln), qfrag16(16 * R + ln), acc);
      // P[r][i] for i <= r into block (R, I) row-major
      const int r = 16 * R + ln;
      float *blk = Pb + tri(R, I) * kBlk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * I + 4 * lg + e;
        const float val = (i <= r) ? srq[r] * srk[i] * expf(sG[r] - sG[i]) * acc[e] : 0.f;
        blk[ln * 17 + 4 * lg + e] = val;
      }
    }
  }
  __syncthreads();  // every read of Kr is done: the A blocks may overwrite it
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int tix = wave + 4 * s;
    if (tix < 15) {
      int R = 0;
      while (tri(R + 1, 0) <= tix) ++R;
      const int I = tix - tri(R, 0);
      // accumulator: column i = 16I + ln, rows r = 16R + 4lg + e
      const int i = 16 * I + ln;
      float *blk = Ab + tri(R, I) * kBlk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + 4 * lg + e;
        const float val = (i < r) ? sbeta[r] * srk[r] * srk[i] * expf(sG[r] - sG[i]) * aacc[s][e] : 0.f;
        blk[(4 * lg + e) * 17 + ln] = val;
      }
    }
  }
  __syncthreads();

  // ---- (3) T = (I + A)^{-1}: diagonal blocks by forward substitution ...
  if (tid < C) {
    const int I = tid >> 4, cc = tid & 15;
    const float *Ad = Ab + tri(I, I) * kBlk;
    float xv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) s = fmaf(Ad[r * 17 + m], xv[m], s);
      xv[r] = (r < cc) ? 0.f : (r == cc ? 1.f : -s);
    }
    float *Td = Tb + tri(I, I) * kBlk;
#pragma unroll
    for (int r = 0; r < 16; ++r) Td[cc * 17 + r] = xv[r];
  }
  __syncthreads();
  // ... then block rows by distance L: T_IJ = -D_I sum_{K=J}^{I-1} A_IK T_KJ
  for (int L = 1; L < CT; ++L) {
    const int nb = CT - L;
    for (int e = tid; e < nb * 256; e += 256) {
      const int J = e >> 8, I = J + L, ii = (e >> 4) & 15, jj = e & 15;
      float s = 0.f;
      for (int K = J; K < I; ++K) {
        const float *Aik = Ab + tri(I, K) * kBlk + ii * 17;
        const float *Tkj = Tb + tri(K, J) * kBlk + jj * 17;  // (T_KJ)^T row jj
#pragma unroll
        for (int m = 0; m < 16; ++m) s = fmaf(Aik[m], Tkj[m], s);
      }
      Xb[J * kBlk + ii * 17 + jj] = s;
    }
    __syncthreads();
    for (int e = tid; e < nb * 256; e += 256) {
      const int J = e >> 8, I = J + L, ii = (e >> 4) & 15, jj = e & 15;
      const float *Dt = Tb + tri(I, I) * kBlk;  // (D_I)^T: Dt[m][ii] = D_I[ii][m]
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) s = fmaf(Dt[m * 17 + ii], Xb[J * kBlk + m * 17 + jj], s);
      Tb[tri(I, J) * kBlk + jj * 17 + ii] = -s;
    }
    __syncthreads();
  }

  // ---- (4) M^T = T^T diag(s) K  and  P'^T = T^T P^T, split and stored
  // Tt(r, i) = T[i][r] for i >= r lives in block (tile(i), tile(r)) at [r%16][i%16]
  auto tt = [&](int r, int i) { return Tb[tri(i >> 4, r >> 4) * kBlk + (r & 15) * 17 + (i & 15)]; };
  char *Mrec = Mout + rec * size_t(kMBytes);
  char *Prec = Pout + rec * size_t(kPBytes);
  // task list: 35 M^T tiles (Rt, Dt) then 15 P'^T tiles (It <= Rt)
  for (int task = wave; task < 50; task += 4) {
    if (task < 35) {
      const int Rt = task / NT, Dt = task % NT;
      const int r = 16 * Rt + ln;  // A-operand row (output token row of M^T)
      f32x4 acc = zero4();
      int p = Rt;
      while (p < CT) {
        if (p + 1 < CT) {  // 32-deep block over token tiles p, p+1
          float v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 16 * (p + (j >> 2)) + 4 * lg + (j & 3);
            v[j] = (i >= r) ? tt(r, i) * ss[i] : 0.f;
          }
          F32 ah, al;
          split4(v, ah.w, al.w);
          split4(v + 4, ah.w + 2, al.w + 2);
          const uint16_t *kt = Kt + (16 * Dt + ln) * kKtStride + 16 * p + 4 * lg;
          const uint2 k0 = *reinterpret_cast<const uint2 *>(kt), k1 = *reinterpret_cast<const uint2 *>(kt + 16);
          const F32 bk{{k0.x, k0.y, k1.x, k1.y}};
          acc = mma(ah, bk, acc);
          acc = mma(al, bk, acc);
          p += 2;
        } else {  // 16-deep block over tile p
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 16 * p + 4 * lg + j;
            v[j] = (i >= r) ? tt(r, i) * ss[i] : 0.f;
          }
          F16 ah, al;
          split4(v, ah.w, al.w);
          const uint2 k0 = *reinterpret_cast<const uint2 *>(Kt + (16 * Dt + ln) * kKtStride + 16 * p + 4 * lg);
          const F16 bk{{k0.x, k0.y}};
          acc = mma(ah, bk, acc);
          acc = mma(al, bk, acc);
          p += 1;
        }
      }
      // accumulator: column d = 16Dt + ln, rows r = 16Rt + 4lg + e -> M[d][r], chain A-operand order
      uint32_t hi[2], lo[2];
      split4(acc, hi, lo);
      if (Rt < 4) {
        const int kb = Rt >> 1, half = Rt & 1;
        *reinterpret_cast<uint2 *>(Mrec + m_off32(Dt, kb, 0) + lane * 16 + half * 8) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2 *>(Mrec + m_off32(Dt, kb, 1) + lane * 16 + half * 8) = make_uint2(lo[0], lo[1]);
      } else {
        *reinterpret_cast<uint2 *>(Mrec + m_off16(Dt, 0) + lane * 8) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2 *>(Mrec + m_off16(Dt, 1) + lane * 8) = make_uint2(lo[0], lo[1]);
      }
    } else {
      int tix = task - 35, Rt = 0;
      while (tri(Rt + 1, 0) <= tix) ++Rt;
      const int It = tix - tri(Rt, 0);
      // P'^T[i][r] = sum_{k=i}^{r} T[k][i] P[r][k]; A rows i = 16It + ln, B columns r = 16Rt + ln
      const int i = 16 * It + ln, r = 16 * Rt + ln;
      const float *prow = Pb + ln * 17;  // row r of P inside block (Rt, kt)
      f32x4 acc = zero4();
      int p = It;
      while (p <= Rt) {
        if (p + 1 <= Rt) {
          float va[8], vb[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int kk = 16 * (p + (j >> 2)) + 4 * lg + (j & 3);
            va[j] = (kk >= i) ? tt(i, kk) : 0.f;
            vb[j] = (kk <= r) ? prow[tri(Rt, kk >> 4) * kBlk + (kk & 15)] : 0.f;
          }
          F32 ah, al, bh, bl;
          split4(va, ah.w, al.w);
          split4(va + 4, ah.w + 2, al.w + 2);
          split4(vb, bh.w, bl.w);
          split4(vb + 4, bh.w + 2, bl.w + 2);
          acc = mma(ah, bh, acc);
          acc = mma(ah, bl, acc);
          acc = mma(al, bh, acc);
          p += 2;
        } else {
          float va[4], vb[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kk = 16 * p + 4 * lg + j;
            va[j] = (kk >= i) ? tt(i, kk) : 0.f;
            vb[j] = (kk <= r) ? prow[tri(Rt, kk >> 4) * kBlk + (kk & 15)] : 0.f;
          }
          F16 ah, al, bh, bl;
          split4(va, ah.w, al.w);
          split4(vb, bh.w, bl.w);
          acc = mma(ah, bh, acc);
          acc = mma(ah, bl, acc);
          acc = mma(al, bh, acc);
          p += 1;
        }
      }
      // accumulator: column r = 16Rt + ln, rows i = 16It + 4lg + e -> P'[r][i], chain A-operand order
      uint32_t hi[2], lo[2];
      split4(acc, hi, lo);
      if (It == Rt && !(Rt & 1)) {
        *reinterpret_cast<uint2 *>(Prec + p_off16(Rt, 0) + lane * 8) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2 *>(Prec + p_off16(Rt, 1) + lane * 8) = make_uint2(lo[0], lo[1]);
      } else {
        const int kb = It >> 1, half = It & 1;
        *reinterpret_cast<uint2 *>(Prec + p_off32(Rt, kb, 0) + lane * 16 + half * 8) = make_uint2(hi[0], hi[1]);
        *reinterpret_cast<uint2 *>(Prec + p_off32(Rt, kb, 1) + lane * 16 + half * 8) = make_uint2(lo[0], lo[1]);
      }
    }
  }
}

}  // namespace

hipError_t launch_intra(const Plan &p, const Args &a, char *M, char *P, float *cs) {
  const uint16_t *q = static_cast<const uint16_t *>(a.q), *k = static_cast<const uint16_t *>(a.k);
  const unsigned chunks = unsigned(p.B) * p.H * p.N;
  // the intra kernel needs more than the default 64 KB of dynamic LDS (gfx950 has 160 KB per CU)
  static const hipError_t lds_ok = hipFuncSetAttribute(reinterpret_cast<const void *>(&intra_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsIntra);
  if (lds_ok != hipSuccess) return lds_ok;
  stage_begin(a, kStageIntra);
  intra_kernel<<<dim3(chunks), dim3(256), kLdsIntra, a.stream>>>(q, k, a.g, a.beta, M, P, cs, p.T, p.H, p.N,
                                                                 p.flags);
  stage_end(a, kStageIntra);
  return hipGetLastError();
}

}  // namespace mfma
}  // namespace gdn
