// MFMA kernel family: bf16 q/k/v, d_k = d_v = 112, fp32 state, on gfx950.
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
// lo*raw), accumulating in fp32 -- a relative error near 2^-16 per product
// instead of bf16's 2^-9.
//
// MFMA lane layouts (v_mfma_f32_16x16x32_bf16 / 16x16x16_bf16, lane l,
// g = l >> 4): A row l & 15 and B column l & 15 hold k = 8g..8g+7 (4g..4g+3
// for the 16-deep form); the accumulator holds column l & 15, rows 4g..4g+3.
// A 32-deep reduction block built from two accumulator tiles uses the
// k-order "pair": instruction slots 0-3 of group g are rows 4g..4g+3 of the
// first 16-row tile and slots 4-7 rows 4g..4g+3 of the second, so an
// accumulator pair becomes a B operand without any data movement; every A
// operand of such a product is read in the same order.
#include "gdn_internal.h"

namespace gdn {
namespace {

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

// x = hi + lo, both bf16 (RNE); non-finite x keeps lo = 0
__device__ __forceinline__ void split1(float x, uint32_t &h, uint32_t &l) {
  const uint16_t hb = f32_to_bf16(x);
  float r = x - bf16_to_f32(hb);
  if (!(fabsf(r) <= 3.0e38f)) r = 0.f;
  h = hb;
  l = f32_to_bf16(r);
}
// four consecutive k-slots -> two packed words of hi and of lo
__device__ __forceinline__ void split4(const float *v, uint32_t *hi, uint32_t *lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split1(v[j], h[j], l[j]);
  hi[0] = h[0] | (h[1] << 16);
  hi[1] = h[2] | (h[3] << 16);
  lo[0] = l[0] | (l[1] << 16);
  lo[1] = l[2] | (l[3] << 16);
}
__device__ __forceinline__ void split4(const f32x4 &v, uint32_t *hi, uint32_t *lo) {
  float t[4] = {v[0], v[1], v[2], v[3]};
  split4(t, hi, lo);
}

__device__ __forceinline__ uint2 ldg8(const void *p) { return *reinterpret_cast<const uint2 *>(p); }
__device__ __forceinline__ uint4 ldg16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

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

// lower-triangular 16x16 block index (I >= J)
__device__ __forceinline__ constexpr int tri(int I, int J) { return I * (I + 1) / 2 + J; }

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
                                                       const float *__restrict__ s_beta,
                                                       const float *__restrict__ s_rq,
                                                       const float *__restrict__ s_rk,
                                                       const float *__restrict__ s_gcum, char *__restrict__ Mout,
                                                       char *__restrict__ Pout, float *__restrict__ CSout, int T,
                                                       int H, int N) {
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

  // ---- (0) per-token scalars
  if (tid < C) {
    const size_t sb = u * T + t0;
    const float Gl = s_gcum[sb + n - 1];
    const bool ok = tid < n;
    const float bt = ok ? s_beta[sb + tid] : 0.f;
    const float rq = ok ? s_rq[sb + tid] : 0.f;
    const float rk = ok ? s_rk[sb + tid] : 0.f;
    const float G = ok ? s_gcum[sb + tid] : Gl;
    const float gam = expf(G);
    sbeta[tid] = bt;
    srq[tid] = rq;
    srk[tid] = rk;
    sG[tid] = G;
    ss[tid] = rk * expf(Gl - G);
    float *cs = CSout + rec * kCsFloats;
    cs[tid] = bt;
    cs[80 + tid] = bt * gam * rk;
    cs[160 + tid] = gam * rq;
    if (tid == 0) cs[240] = expf(Gl);
  }
  // ---- (1) K rows -> LDS, row-major and transposed
  const size_t rowstride = size_t(H) * D;  // elements between consecutive tokens
  const uint16_t *kbase = k + (size_t(b) * T + t0) * rowstride + size_t(h) * D;
  for (int idx = tid; idx < C * 14; idx += 256) {
    const int r = idx / 14, cc = idx % 14;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (r < n) val = ldg16(kbase + size_t(r) * rowstride + cc * 8);
    *reinterpret_cast<uint4 *>(Kr + r * kKrStride + cc * 8) = val;
    const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) Kt[(cc * 8 + j) * kKtStride + r] = uint16_t(w[j >> 1] >> (16 * (j & 1)));
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

// ============================================================================
// Kernel "chain": one workgroup (4 waves) per (b, h, 16 columns of d_v).
// The state slice S^T (112 x 16, fp32) lives in accumulator registers, 7 row
// tiles spread over the waves; per chunk two barriers exchange the bf16
// hi/lo operands S (after phase 0) and R (after phase A) through LDS.
// ============================================================================
struct Roles {
  int nY, Y[2];    // token tiles whose Y = K S^T and R this wave computes (phase A)
  int nQA, QA[1];  // token tiles whose Q S^T it computes in phase A
  int nQB, QB[2];  // ... in phase B
  int nO, O[2];    // output tiles it finishes (uses its Q S^T of the same tile)
  int nS, S[3];    // d_k row tiles of the state it owns
};
__device__ constexpr Roles kRoles[4] = {
    {1, {0, 0}, 1, {0}, 0, {0, 0}, 1, {0, 0}, 3, {0, 1, 2}},
    {1, {1, 0}, 1, {1}, 0, {0, 0}, 1, {1, 0}, 2, {3, 4, 0}},
    {1, {2, 0}, 1, {2}, 0, {0, 0}, 1, {2, 0}, 2, {5, 6, 0}},
    {2, {3, 4}, 0, {0}, 2, {3, 4}, 2, {3, 4}, 0, {0, 0, 0}},
};

constexpr int kLdsS = 0;                      // S operand: hi/lo x (3 x 1 KB + 512 B)
constexpr int kLdsR = 2 * (3 * 1024 + 512);   // R operand: hi/lo x (2 x 1 KB + 512 B)
constexpr int kLdsChain = kLdsR + 2 * (2 * 1024 + 512);

struct RowFrags {  // one lane's share of a 16-row tile of K or Q (A operand, k = d_k)
  F32 f[3];
  F16 t;
};

template <int W, bool kOutBf16>
__device__ __forceinline__ void chain_role(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                           const uint16_t *__restrict__ v, const char *__restrict__ Mws,
                                           const char *__restrict__ Pws, const float *__restrict__ CS,
                                           const float *state_in, float *state_out, void *__restrict__ o, int T,
                                           int H, int N, int b, int h, int nt, char *lds) {
  constexpr Roles ro = kRoles[W];
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
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

  // operands of phase A (K rows for Y, Q rows for Q S^T, V and scales for R)
  RowFrags Kf[2], Qf[2];
  float Va[2][4], Aa[2][4], Bb[2][4];
  auto load_rows = [&](const uint16_t *src, int tok0, int nvalid, int tile, RowFrags &rf) {
    const int row = 16 * tile + ln;
    if (row < nvalid) {
      const uint16_t *p = src + (size_t(b) * T + tok0 + row) * rowstride + size_t(h) * D + 4 * lg;
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) {
        const uint2 x0 = ldg8(p + 32 * kb), x1 = ldg8(p + 32 * kb + 16);
        rf.f[kb] = F32{{x0.x, x0.y, x1.x, x1.y}};
      }
      const uint2 x2 = ldg8(p + 96);
      rf.t = F16{{x2.x, x2.y}};
    } else {
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) rf.f[kb] = F32{{0, 0, 0, 0}};
      rf.t = F16{{0, 0}};
    }
  };
  auto load_phaseA = [&](int c) {
    const int t0 = c * C, nv = min(C, T - t0);
    const float *cs = CS + (u * N + c) * kCsFloats;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < ro.nY) {
        const int tile = ro.Y[s];
        load_rows(k, t0, nv, tile, Kf[s]);
        const float4 a4 = *reinterpret_cast<const float4 *>(cs + 16 * tile + 4 * lg);
        const float4 b4 = *reinterpret_cast<const float4 *>(cs + 80 + 16 * tile + 4 * lg);
        Aa[s][0] = a4.x, Aa[s][1] = a4.y, Aa[s][2] = a4.z, Aa[s][3] = a4.w;
        Bb[s][0] = b4.x, Bb[s][1] = b4.y, Bb[s][2] = b4.z, Bb[s][3] = b4.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * tile + 4 * lg + e;
          Va[s][e] = row < nv ? bf16_to_f32(v[(size_t(b) * T + t0 + row) * rowstride + size_t(h) * D + 16 * nt + ln])
                              : 0.f;
        }
      }
    }
    if (ro.nQA) load_rows(q, t0, nv, ro.QA[0], Qf[0]);
  };
  // operands of phase B (M and P' fragments, output scales, Q rows of phase-B tiles)
  F32 Mf[3][2][2];
  F16 Mt[3][2];
  F32 Pf[2][2][2];
  F16 Pt[2][2];
  float Cc[2][4];
  float gC = 0.f;
  auto load_phaseB = [&](int c) {
    const int t0 = c * C, nv = min(C, T - t0);
    const char *Mr = Mws + (u * N + c) * size_t(kMBytes);
    const char *Pr = Pws + (u * N + c) * size_t(kPBytes);
    const float *cs = CS + (u * N + c) * kCsFloats;
    gC = cs[240];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if (s < ro.nS) {
        const int mt = ro.S[s];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) {
            const uint4 x = ldg16(Mr + m_off32(mt, kb, hl) + lane * 16);
            Mf[s][kb][hl] = F32{{x.x, x.y, x.z, x.w}};
          }
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) {
          const uint2 x = ldg8(Mr + m_off16(mt, hl) + lane * 8);
          Mt[s][hl] = F16{{x.x, x.y}};
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
              Pf[s][kb][hl] = F32{{x.x, x.y, x.z, x.w}};
            }
          }
        if (!(R & 1))
#pragma unroll
          for (int hl = 0; hl < 2; ++hl) {
            const uint2 x = ldg8(Pr + p_off16(R, hl) + lane * 8);
            Pt[s][hl] = F16{{x.x, x.y}};
          }
        const float4 c4 = *reinterpret_cast<const float4 *>(cs + 160 + 16 * R + 4 * lg);
        Cc[s][0] = c4.x, Cc[s][1] = c4.y, Cc[s][2] = c4.z, Cc[s][3] = c4.w;
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (s < ro.nQB) load_rows(q, t0, nv, ro.QB[s], Qf[s]);
  };

  load_phaseA(0);
  for (int c = 0; c < N; ++c) {
    const int t0 = c * C, nv = min(C, T - t0);
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
    load_phaseB(c);
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
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < ro.nY) {
        const int tile = ro.Y[s];
        const f32x4 y = rows_times_S(Kf[s]);
        float r4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r4[e] = Aa[s][e] * Va[s][e] - Bb[s][e] * y[e];
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
    if (ro.nQA) QS[0] = rows_times_S(Qf[0]);
    __syncthreads();
    if (c + 1 < N) load_phaseA(c + 1);
    // ---- phase B: R operands; state update and outputs
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
      if (s < ro.nQB) QS[s] = rows_times_S(Qf[s]);
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if (s < ro.nS) {
        f32x4 acc = S[s] * gC;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          acc = mma(Mf[s][kb][0], Rh[kb], acc);
          acc = mma(Mf[s][kb][0], Rl[kb], acc);
          acc = mma(Mf[s][kb][1], Rh[kb], acc);
        }
        acc = mma(Mt[s][0], Rth, acc);
        acc = mma(Mt[s][0], Rtl, acc);
        acc = mma(Mt[s][1], Rth, acc);
        S[s] = acc;
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < ro.nO) {
        const int R = ro.O[s];
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = Cc[s][e] * QS[s][e];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb < (R + 1) / 2) {
            acc = mma(Pf[s][kb][0], Rh[kb], acc);
            acc = mma(Pf[s][kb][0], Rl[kb], acc);
            acc = mma(Pf[s][kb][1], Rh[kb], acc);
          }
        }
        if (!(R & 1)) {
          // the 16-deep block covers token tile R: operand rows 4lg.. of R tile R
          // (tile 4 is in the shared 16-deep slot; tiles 0 and 2 are halves of 32-deep slots)
          F16 rh, rl;
          if (R == 4) {
            rh = Rth;
            rl = Rtl;
          } else {
            const int kb = R >> 1;
            rh = F16{{Rh[kb].w[0], Rh[kb].w[1]}};
            rl = F16{{Rl[kb].w[0], Rl[kb].w[1]}};
          }
          acc = mma(Pt[s][0], rh, acc);
          acc = mma(Pt[s][0], rl, acc);
          acc = mma(Pt[s][1], rh, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * R + 4 * lg + e;
          if (row < nv) {
            const size_t oi = (size_t(b) * T + t0 + row) * rowstride + size_t(h) * D + 16 * nt + ln;
            if constexpr (kOutBf16)
              static_cast<uint16_t *>(o)[oi] = f32_to_bf16(acc[e]);
            else
              static_cast<float *>(o)[oi] = acc[e];
          }
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

template <bool kOutBf16>
__global__ __launch_bounds__(256) void chain_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                    const uint16_t *__restrict__ v, const char *__restrict__ Mws,
                                                    const char *__restrict__ Pws, const float *__restrict__ CS,
                                                    const float *state_in, float *state_out,
                                                    void *__restrict__ o, int T, int H, int N, int units) {
  __shared__ __align__(16) char lds[kLdsChain];
  // Workgroup i runs on XCD i % 8: keep the 7 column tiles of a (b, h) on one
  // XCD so that its K, Q, M and P' are fetched from HBM once into that L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int u = xcd + 8 * (slot / NT), nt = slot % NT;
  if (u >= units) return;
  const int b = u / H, h = u % H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  switch (wave) {
    case 0: chain_role<0, kOutBf16>(q, k, v, Mws, Pws, CS, state_in, state_out, o, T, H, N, b, h, nt, lds); break;
    case 1: chain_role<1, kOutBf16>(q, k, v, Mws, Pws, CS, state_in, state_out, o, T, H, N, b, h, nt, lds); break;
    case 2: chain_role<2, kOutBf16>(q, k, v, Mws, Pws, CS, state_in, state_out, o, T, H, N, b, h, nt, lds); break;
    default: chain_role<3, kOutBf16>(q, k, v, Mws, Pws, CS, state_in, state_out, o, T, H, N, b, h, nt, lds); break;
  }
}

}  // namespace

size_t mfma_chunk_bytes_M() { return kMBytes; }
size_t mfma_chunk_bytes_P() { return kPBytes; }
size_t mfma_chunk_bytes_cs() { return kCsFloats * sizeof(float); }

hipError_t launch_mfma(const Plan &p, const Args &a) {
  const uint16_t *q = static_cast<const uint16_t *>(a.q), *k = static_cast<const uint16_t *>(a.k),
                 *v = static_cast<const uint16_t *>(a.v);
  const float *beta = reinterpret_cast<const float *>(a.ws + p.off_beta);
  const float *rq = reinterpret_cast<const float *>(a.ws + p.off_rq);
  const float *rk = reinterpret_cast<const float *>(a.ws + p.off_rk);
  const float *gc = reinterpret_cast<const float *>(a.ws + p.off_gcum);
  char *M = a.ws + p.off_M;
  char *P = a.ws + p.off_P;
  float *cs = reinterpret_cast<float *>(a.ws + p.off_cs);
  const unsigned chunks = unsigned(p.B) * p.H * p.N;
  // the intra kernel needs more than the default 64 KB of dynamic LDS (gfx950 has 160 KB per CU)
  static const hipError_t lds_ok = hipFuncSetAttribute(reinterpret_cast<const void *>(&intra_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsIntra);
  if (lds_ok != hipSuccess) return lds_ok;
  stage_begin(a, kStageIntra);
  intra_kernel<<<dim3(chunks), dim3(256), kLdsIntra, a.stream>>>(q, k, beta, rq, rk, gc, M, P, cs, p.T, p.H, p.N);
  stage_end(a, kStageIntra);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int units = p.B * p.H;
  const unsigned grid = 8u * NT * unsigned((units + 7) / 8);
  stage_begin(a, kStageState);
  if (p.o_bf16)
    chain_kernel<true><<<dim3(grid), dim3(256), 0, a.stream>>>(q, k, v, M, P, cs, a.state_in, a.state_out, a.o, p.T,
                                                               p.H, p.N, units);
  else
    chain_kernel<false><<<dim3(grid), dim3(256), 0, a.stream>>>(q, k, v, M, P, cs, a.state_in, a.state_out, a.o,
                                                                p.T, p.H, p.N, units);
  stage_end(a, kStageState);
  return hipGetLastError();
}

}  // namespace gdn
