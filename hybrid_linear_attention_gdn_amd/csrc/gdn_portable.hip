// Portable kernels: the chunked gated delta rule in fp32 on the vector ALUs.
//
// They serve fp32 inputs (any 1 <= d_k, d_v <= 128); fed the values of a bf16
// workload as fp32, they are a second, independent evaluation of what the
// MFMA path computes.  Per (batch,
// head) and per chunk of n <= 80 tokens with entry state S0 (d_v x d_k), the
// chunked form of the recurrence is (normalised q, k; G = chunk-local
// inclusive cumsum of the log-decay; gamma = exp(G)):
//   A_ri   = beta_r e^{G_r - G_i} (k_r . k_i),  i < r      (strictly lower)
//   Tm     = (I + A)^{-1}
//   W      = Tm diag(beta gamma) K,   Ut = Tm diag(beta) V
//   U      = Ut - W S0^T                                    (state pass)
//   S_next = gamma_n S0 + U^T diag(e^{G_n - G_i}) K
//   O      = diag(gamma) Q S0^T + (L o Gamma o Q K^T) U     (L: i <= r)
// This is the gated delta rule (named by the "SANA-WM" cookbook page, table
// "Architecture & components", row "Attention") solved chunk by chunk; it
// reproduces the token recurrence exactly in exact arithmetic.
//
//   K2 intra  : grid (b, h, chunk)  -> W, Ut                 [B,H,N,80,d]
//   K3 state  : grid (b, h, 16 rows of d_v), sequential over chunks
//               -> U [B,H,N,80,d_v], S0 per chunk [B,H,N,d_v,d_k], state_out
//   K4 output : grid (b, h, chunk)  -> o
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int C = kChunk;

struct ChunkIdx {
  int b, h, c, t0, n;
};

__device__ __forceinline__ ChunkIdx chunk_of_block(int H, int N, int T) {
  ChunkIdx r;
  int x = blockIdx.x;
  r.c = x % N;
  x /= N;
  r.h = x % H;
  r.b = x / H;
  r.t0 = r.c * C;
  r.n = min(C, T - r.t0);
  return r;
}

// Rows 0 .. rows-1 of an fp32 [*, d] source into LDS rows of stride ld (rows
// at and past n are zero).  The loads of a batch are all issued before any LDS
// store, so a block waits for one memory latency per batch rather than one per
// element; rows of a multiple of 4 floats move as 16-byte loads (the sources
// are 16-byte aligned).
template <typename RowPtr>
__device__ __forceinline__ void stage_rows(float *dst, int ld, int rows, int d, int n, RowPtr rowptr) {
  constexpr int kBatch = 8;
  if ((d & 3) == 0) {
    const int q4 = d >> 2, total = rows * q4;
    for (int base = threadIdx.x; base < total; base += blockDim.x * kBatch) {
      float4 t[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int idx = base + int(blockDim.x) * j, r = idx / q4, pc = idx % q4;
        t[j] = (idx < total && r < n) ? reinterpret_cast<const float4 *>(rowptr(r))[pc] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int idx = base + int(blockDim.x) * j, r = idx / q4, pc = idx % q4;
        if (idx < total) {
          float *o = dst + r * ld + 4 * pc;
          o[0] = t[j].x;
          o[1] = t[j].y;
          o[2] = t[j].z;
          o[3] = t[j].w;
        }
      }
    }
  } else {
    const int total = rows * d;
    for (int base = threadIdx.x; base < total; base += blockDim.x * kBatch) {
      float t[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int idx = base + int(blockDim.x) * j, r = idx / d;
        t[j] = (idx < total && r < n) ? rowptr(r)[idx % d] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int idx = base + int(blockDim.x) * j;
        if (idx < total) dst[(idx / d) * ld + idx % d] = t[j];
      }
    }
  }
}

// Each kernel first stages the rows it multiplies in LDS (row stride d + 1
// floats, so that threads walking rows hit distinct banks), then forms its
// products from LDS; global loads are coalesced row copies.  The reduction
// loops are unrolled so that their LDS reads are in flight together (the
// solve's serial chains are otherwise bound by one LDS latency per term).
__host__ __device__ constexpr size_t intra_lds_floats(int dk, int dv) {
  return size_t(C) * (dk + 1) + size_t(C) * (dv + 1) + 2 * size_t(C) * (C + 1) + 4 * C + (C / 16 - 1) * 256;
}
__host__ __device__ constexpr size_t state_lds_floats(int dk) {
  return 16 * size_t(dk + 1) + 2 * size_t(C) * (dk + 1) + size_t(C) * 17 + C + 1;
}
__host__ __device__ constexpr size_t output_lds_floats(int dk, int dv) {
  return size_t(C) * (dk + 1) + size_t(dv > C ? dv : C) * (dk + 1) + size_t(C) * (C + 1) + C;
}
constexpr size_t kLdsFloats = 160 * 1024 / 4;  // one CU's LDS
// the output kernel also stages the chunk's U rows when they fit
__host__ __device__ constexpr bool output_u_in_lds(int dk, int dv) {
  return output_lds_floats(dk, dv) + size_t(C) * (dv + 1) <= kLdsFloats;
}
__host__ __device__ constexpr size_t output_lds_launch_floats(int dk, int dv) {
  return output_lds_floats(dk, dv) + (output_u_in_lds(dk, dv) ? size_t(C) * (dv + 1) : 0);
}
static_assert(C % 16 == 0, "the blocked solve works on 16 x 16 blocks");
static_assert(intra_lds_floats(kMaxPortableDim, kMaxPortableDim) * 4 <= 160 * 1024 &&
                  state_lds_floats(kMaxPortableDim) * 4 <= 160 * 1024 &&
                  output_lds_floats(kMaxPortableDim, kMaxPortableDim) * 4 <= 160 * 1024,
              "every portable kernel fits one CU's LDS at the largest head dims");

// out[r][d] = sum_{i <= r, i < n} (L[r][i] w[i]) X[i][d] for the chunk's C rows
// and the d < nd columns (L lower triangular in LDS, stride ldl; X rows in LDS,
// stride ldx; out row-major with nd columns).  Thread (rg, dg) forms rows
// rg + 16 a and columns dg + 16 b (up to 128 columns): per term it reads five
// L entries and eight X entries for forty products.  Each entry is summed in
// increasing i, the order of one dot product.
__device__ __forceinline__ void tri_times_rows(const float *L, int ldl, const float *w, const float *X, int ldx,
                                               int nd, int n, float *__restrict__ out) {
  constexpr int RB = C / 16, DB = 8;
  const int rg = threadIdx.x / 16, dg = threadIdx.x % 16;
  float acc[RB][DB];
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[a][b] = 0.f;
  const int iend = min(rg + 16 * (RB - 1) + 1, n);  // the last row's terms
  for (int i = 0; i < iend; ++i) {
    float x[DB], l[RB];
#pragma unroll
    for (int b = 0; b < DB; ++b) x[b] = dg + 16 * b < nd ? X[i * ldx + dg + 16 * b] : 0.f;
#pragma unroll
    for (int a = 0; a < RB; ++a) l[a] = L[(rg + 16 * a) * ldl + i] * w[i];
#pragma unroll
    for (int a = 0; a < RB; ++a) {
      const bool in = i <= rg + 16 * a;
#pragma unroll
      for (int b = 0; b < DB; ++b) acc[a][b] = in ? fmaf(l[a], x[b], acc[a][b]) : acc[a][b];
    }
  }
#pragma unroll
  for (int a = 0; a < RB; ++a)
#pragma unroll
    for (int b = 0; b < DB; ++b)
      if (dg + 16 * b < nd) out[(rg + 16 * a) * nd + dg + 16 * b] = acc[a][b];
}

__global__ __launch_bounds__(256) void intra_kernel(const float *__restrict__ k, const float *__restrict__ v,
                                                    const float *__restrict__ s_beta,
                                                    const float *__restrict__ s_rk,
                                                    const float *__restrict__ s_gcum, float *__restrict__ W,
                                                    float *__restrict__ Ut, int T, int H, int dk, int dv,
                                                    int N, bool rev) {
  extern __shared__ float sm[];
  const int ldk = dk + 1, ldv = dv + 1, ldc = C + 1;
  float *Ks = sm;              // [C][ldk] raw k rows
  float *Vs = Ks + C * ldk;    // [C][ldv] v rows
  float *A = Vs + C * ldv;     // [C][ldc]
  float *Tm = A + C * ldc;     // [C][ldc]
  float *sb = Tm + C * ldc, *srk = sb + C, *sG = srk + C, *cw = sG + C;
  float *X = cw + C;           // [4][16][16] off-diagonal products of the solve
  const ChunkIdx ci = chunk_of_block(H, N, T);
  const size_t sbase = (size_t(ci.b) * H + ci.h) * T + ci.t0;
  for (int r = threadIdx.x; r < C; r += blockDim.x) {
    const bool ok = r < ci.n;
    sb[r] = ok ? s_beta[sbase + r] : 0.f;
    srk[r] = ok ? s_rk[sbase + r] : 0.f;
    sG[r] = ok ? s_gcum[sbase + r] : 0.f;
    cw[r] = ok ? sb[r] * expf(sG[r]) * srk[r] : 0.f;  // beta gamma rk
  }
  auto row = [&](int r, int d) { return ((size_t(ci.b) * T + phys_token(ci.t0 + r, T, rev)) * H + ci.h) * size_t(d); };
  stage_rows(Ks, ldk, C, dk, ci.n, [&](int r) { return k + row(r, dk); });
  stage_rows(Vs, ldv, C, dv, ci.n, [&](int r) { return v + row(r, dv); });
  __syncthreads();
  // A (strictly lower), padded rows/cols are zero.  Thread (rg, ig) forms the
  // 5 x 5 entries (rg + 16 a, ig + 16 b): ten row reads per step for 25 products
  {
    const int rg = threadIdx.x / 16, ig = threadIdx.x % 16;
    float dot[C / 16][C / 16];
#pragma unroll
    for (int a = 0; a < C / 16; ++a)
#pragma unroll
      for (int b = 0; b < C / 16; ++b) dot[a][b] = 0.f;
    #pragma unroll 2
    for (int d = 0; d < dk; ++d) {
      float kr[C / 16], ki[C / 16];
#pragma unroll
      for (int a = 0; a < C / 16; ++a) {
        kr[a] = Ks[(rg + 16 * a) * ldk + d];
        ki[a] = Ks[(ig + 16 * a) * ldk + d];
      }
#pragma unroll
      for (int a = 0; a < C / 16; ++a)
#pragma unroll
        for (int b = 0; b < C / 16; ++b) dot[a][b] = fmaf(kr[a], ki[b], dot[a][b]);
    }
#pragma unroll
    for (int a = 0; a < C / 16; ++a)
#pragma unroll
      for (int b = 0; b < C / 16; ++b) {
        const int r = rg + 16 * a, i = ig + 16 * b;
        A[r * ldc + i] = (i < r && r < ci.n) ? sb[r] * expf(sG[r] - sG[i]) * srk[r] * srk[i] * dot[a][b] : 0.f;
      }
  }
  __syncthreads();
  // Tm = (I + A)^{-1} by 16 x 16 blocks (A is strictly lower, so Tm is unit
  // lower triangular): the diagonal blocks by forward substitution, one column
  // per thread, then the blocks at distance 1 .. 4 below the diagonal,
  // Tm_IJ = -Tm_II X_IJ with X_IJ = sum_{K=J}^{I-1} A_IK Tm_KJ, whose blocks
  // Tm_KJ all lie closer to the diagonal.
  constexpr int NB = C / 16;
  for (int idx = threadIdx.x; idx < C * C; idx += blockDim.x) Tm[(idx / C) * ldc + idx % C] = 0.f;
  __syncthreads();
  if (threadIdx.x < C) {
    const int c0 = 16 * (threadIdx.x / 16), jj = threadIdx.x % 16, j = c0 + jj;
    for (int rr = jj; rr < 16; ++rr) {
      const int r = c0 + rr;
      float s = 0.f;
#pragma unroll 8
      for (int i = j; i < r; ++i) s = fmaf(A[r * ldc + i], Tm[i * ldc + j], s);
      Tm[r * ldc + j] = rr == jj ? 1.f : -s;
    }
  }
  __syncthreads();
  for (int dist = 1; dist < NB; ++dist) {
    const int nb = NB - dist;  // blocks (J + dist, J), J = 0 .. nb - 1
    for (int idx = threadIdx.x; idx < nb * 256; idx += blockDim.x) {
      const int J = idx / 256, I = J + dist, r = 16 * I + (idx % 256) / 16, j = 16 * J + idx % 16;
      float s = 0.f;
#pragma unroll 8
      for (int i = 16 * J; i < 16 * I; ++i) s = fmaf(A[r * ldc + i], Tm[i * ldc + j], s);
      X[idx] = s;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nb * 256; idx += blockDim.x) {
      const int J = idx / 256, I = J + dist, rr = (idx % 256) / 16, jj = idx % 16, r = 16 * I + rr;
      float s = 0.f;
#pragma unroll 8
      for (int kk = 0; kk <= rr; ++kk) s = fmaf(Tm[r * ldc + 16 * I + kk], X[J * 256 + kk * 16 + jj], s);
      Tm[r * ldc + 16 * J + jj] = -s;
    }
    __syncthreads();
  }
  const size_t cbase = ((size_t(ci.b) * H + ci.h) * N + ci.c) * C;
  // W = Tm diag(beta gamma rk) K_raw,  Ut = Tm diag(beta) V
  tri_times_rows(Tm, ldc, cw, Ks, ldk, dk, ci.n, W + cbase * dk);
  tri_times_rows(Tm, ldc, sb, Vs, ldv, dv, ci.n, Ut + cbase * dv);
}

// Sequential state pass: one block per (b, h, 16 rows of the state).
__global__ __launch_bounds__(256) void state_kernel(const float *__restrict__ k, const float *__restrict__ s_rk,
                                                    const float *__restrict__ s_gcum,
                                                    const float *__restrict__ W, const float *__restrict__ Ut,
                                                    const float *state_in, float *state_out,
                                                    float *__restrict__ U, float *__restrict__ S0, int T, int H,
                                                    int dk, int dv, int N, bool rev) {
  constexpr int R = 16;
  extern __shared__ float sm[];
  const int ldk = dk + 1;
  float *S = sm;                // [R][ldk] this block's rows of the state
  float *Ws = S + R * ldk;      // [C][ldk] W rows of the chunk
  float *Ks = Ws + C * ldk;     // [C][ldk] raw k rows of the chunk
  float *Us = Ks + C * ldk;     // [C][R + 1]
  float *coef = Us + C * (R + 1);
  float *gammaC = coef + C;
  const int tiles = (dv + R - 1) / R;
  const int tile = blockIdx.x % tiles;
  const int h = (blockIdx.x / tiles) % H;
  const int b = blockIdx.x / (tiles * H);
  const int i0 = tile * R;
  const int nrows = min(R, dv - i0);
  const size_t bh = size_t(b) * H + h;
  for (int idx = threadIdx.x; idx < R * dk; idx += blockDim.x) {
    const int ii = idx / dk, d = idx % dk;
    S[ii * ldk + d] = (ii < nrows && state_in) ? state_in[(bh * dv + i0 + ii) * dk + d] : 0.f;
  }
  for (int c = 0; c < N; ++c) {
    const int t0 = c * C, n = min(C, T - t0);
    __syncthreads();  // the previous chunk's update of S is complete; Ws, Ks, Us are free
    const size_t sb = bh * T + t0;
    if (threadIdx.x < C) {
      const int r = threadIdx.x;
      const float Gl = s_gcum[sb + n - 1];
      coef[r] = r < n ? s_rk[sb + r] * expf(Gl - s_gcum[sb + r]) : 0.f;
      if (r == 0) gammaC[0] = expf(Gl);
    }
    // entry state of this chunk, for the output kernel
    for (int idx = threadIdx.x; idx < nrows * dk; idx += blockDim.x) {
      const int ii = idx / dk, d = idx % dk;
      S0[((bh * N + c) * dv + i0 + ii) * dk + d] = S[ii * ldk + d];
    }
    const size_t cb = (bh * N + c) * C;
    stage_rows(Ws, ldk, C, dk, n, [&](int r) { return W + (cb + r) * dk; });
    stage_rows(Ks, ldk, C, dk, n, [&](int r) { return k + ((size_t(b) * T + phys_token(t0 + r, T, rev)) * H + h) * size_t(dk); });
    __syncthreads();
    // U = Ut - W S0^T for this tile's columns: thread (rg, ii) forms rows
    // rg, rg + 16, ... of column ii, reading each S element once for five rows
    {
      const int ii = threadIdx.x % R, rg = threadIdx.x / R;
      float acc[C / 16];
#pragma unroll
      for (int j = 0; j < C / 16; ++j) acc[j] = 0.f;
      #pragma unroll 4
      for (int d = 0; d < dk; ++d) {
        const float sv = S[ii * ldk + d];
#pragma unroll
        for (int j = 0; j < C / 16; ++j) acc[j] = fmaf(Ws[(rg + 16 * j) * ldk + d], sv, acc[j]);
      }
#pragma unroll
      for (int j = 0; j < C / 16; ++j) {
        const int r = rg + 16 * j;
        float u = 0.f;
        if (r < n && ii < nrows) {
          u = Ut[(cb + r) * dv + i0 + ii] - acc[j];
          U[(cb + r) * dv + i0 + ii] = u;
        }
        Us[r * (R + 1) + ii] = u;
      }
    }
    __syncthreads();
    // S <- gamma_n S + U^T diag(rk e^{G_n - G}) K_raw, one element per thread step
    // (a register-blocked form of this product measured slower)
    for (int idx = threadIdx.x; idx < R * dk; idx += blockDim.x) {
      const int ii = idx / dk, d = idx % dk;
      float s = 0.f;
      #pragma unroll 8
      for (int r = 0; r < n; ++r) s = fmaf(Us[r * (R + 1) + ii] * coef[r], Ks[r * ldk + d], s);
      S[ii * ldk + d] = fmaf(gammaC[0], S[ii * ldk + d], s);
    }
  }
  __syncthreads();
  if (state_out)
    for (int idx = threadIdx.x; idx < nrows * dk; idx += blockDim.x) {
      const int ii = idx / dk, d = idx % dk;
      state_out[(bh * dv + i0 + ii) * dk + d] = S[ii * ldk + d];
    }
}

template <typename TOut>
__global__ __launch_bounds__(256) void output_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                     const float *__restrict__ s_rq,
                                                     const float *__restrict__ s_rk,
                                                     const float *__restrict__ s_gcum,
                                                     const float *__restrict__ U, const float *__restrict__ S0,
                                                     TOut *__restrict__ o, int T, int H, int dk, int dv, int N,
                                                     bool rev) {
  extern __shared__ float sm[];
  const int ldk = dk + 1, ldc = C + 1;
  float *Qs = sm;                                // [C][ldk] raw q rows
  float *KS = Qs + C * ldk;                      // [C][ldk] raw k rows, then [dv][ldk] the entry state
  float *P = KS + (dv > C ? dv : C) * ldk;       // [C][ldc]
  float *sc = P + C * ldc;
  const ChunkIdx ci = chunk_of_block(H, N, T);
  const size_t sbase = (size_t(ci.b) * H + ci.h) * T + ci.t0;
  auto row = [&](int r, int d) { return ((size_t(ci.b) * T + phys_token(ci.t0 + r, T, rev)) * H + ci.h) * size_t(d); };
  stage_rows(Qs, ldk, C, dk, ci.n, [&](int r) { return q + row(r, dk); });
  stage_rows(KS, ldk, C, dk, ci.n, [&](int r) { return k + row(r, dk); });
  for (int r = threadIdx.x; r < C; r += blockDim.x)
    sc[r] = r < ci.n ? expf(s_gcum[sbase + r]) * s_rq[sbase + r] : 0.f;
  __syncthreads();
  {  // P: thread (rg, ig) forms the 5 x 5 entries (rg + 16 a, ig + 16 b)
    const int rg = threadIdx.x / 16, ig = threadIdx.x % 16;
    float dot[C / 16][C / 16];
#pragma unroll
    for (int a = 0; a < C / 16; ++a)
#pragma unroll
      for (int b = 0; b < C / 16; ++b) dot[a][b] = 0.f;
    #pragma unroll 2
    for (int d = 0; d < dk; ++d) {
      float qr[C / 16], ki[C / 16];
#pragma unroll
      for (int a = 0; a < C / 16; ++a) {
        qr[a] = Qs[(rg + 16 * a) * ldk + d];
        ki[a] = KS[(ig + 16 * a) * ldk + d];
      }
#pragma unroll
      for (int a = 0; a < C / 16; ++a)
#pragma unroll
        for (int b = 0; b < C / 16; ++b) dot[a][b] = fmaf(qr[a], ki[b], dot[a][b]);
    }
#pragma unroll
    for (int a = 0; a < C / 16; ++a)
#pragma unroll
      for (int b = 0; b < C / 16; ++b) {
        const int r = rg + 16 * a, i = ig + 16 * b;
        P[r * ldc + i] = (i <= r && r < ci.n)
                             ? expf(s_gcum[sbase + r] - s_gcum[sbase + i]) * s_rq[sbase + r] * s_rk[sbase + i] * dot[a][b]
                             : 0.f;
      }
  }
  __syncthreads();  // the k rows are no longer read: the entry state takes their place
  const size_t bhc = (size_t(ci.b) * H + ci.h) * N + ci.c;
  const float *S0c = S0 + bhc * size_t(dv) * dk;
  stage_rows(KS, ldk, dv, dk, dv, [&](int e) { return S0c + size_t(e) * dk; });
  // the chunk's U rows go to LDS too when they fit beside the rest (d_v <= 112
  // at d_k = d_v); otherwise the products read them from the workspace
  const float *Uc = U + bhc * C * size_t(dv);
  const bool u_lds = output_u_in_lds(dk, dv);
  float *Us = sc + C;  // [C][dv + 1] when u_lds
  if (u_lds) stage_rows(Us, dv + 1, C, dv, ci.n, [&](int i) { return Uc + size_t(i) * dv; });
  __syncthreads();
  if (u_lds) {
    // thread (rg, eg) forms rows rg + 16 a and columns eg + 16 b: per term five
    // reads of one operand and eight of the other for forty products; each
    // entry is summed in the order of one dot product (over d, then over i)
    constexpr int RB = C / 16, EB = 8;
    const int rg = threadIdx.x / 16, eg = threadIdx.x % 16;
    float acc[RB][EB];
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int b = 0; b < EB; ++b) acc[a][b] = 0.f;
    for (int d = 0; d < dk; ++d) {
      float qv[RB], sv[EB];
#pragma unroll
      for (int a = 0; a < RB; ++a) qv[a] = Qs[(rg + 16 * a) * ldk + d];
#pragma unroll
      for (int b = 0; b < EB; ++b) sv[b] = eg + 16 * b < dv ? KS[(eg + 16 * b) * ldk + d] : 0.f;
#pragma unroll
      for (int a = 0; a < RB; ++a)
#pragma unroll
        for (int b = 0; b < EB; ++b) acc[a][b] = fmaf(qv[a], sv[b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < RB; ++a)
#pragma unroll
      for (int b = 0; b < EB; ++b) acc[a][b] = sc[rg + 16 * a] * acc[a][b];
    const int iend = min(rg + 16 * (RB - 1) + 1, ci.n);
    for (int i = 0; i < iend; ++i) {
      float pv[RB], uv[EB];
#pragma unroll
      for (int a = 0; a < RB; ++a) pv[a] = P[(rg + 16 * a) * ldc + i];
#pragma unroll
      for (int b = 0; b < EB; ++b) uv[b] = eg + 16 * b < dv ? Us[i * (dv + 1) + eg + 16 * b] : 0.f;
#pragma unroll
      for (int a = 0; a < RB; ++a) {
        const bool in = i <= rg + 16 * a;
#pragma unroll
        for (int b = 0; b < EB; ++b) acc[a][b] = in ? fmaf(pv[a], uv[b], acc[a][b]) : acc[a][b];
      }
    }
#pragma unroll
    for (int a = 0; a < RB; ++a) {
      const int r = rg + 16 * a;
      if (r >= ci.n) continue;
#pragma unroll
      for (int b = 0; b < EB; ++b) {
        const int e = eg + 16 * b;
        if (e >= dv) continue;
        const size_t oi = row(r, dv) + e;
        if constexpr (sizeof(TOut) == 2)
          o[oi] = f32_to_bf16(acc[a][b]);
        else
          o[oi] = acc[a][b];
      }
    }
    return;
  }
  for (int idx = threadIdx.x; idx < ci.n * dv; idx += blockDim.x) {
    const int r = idx / dv, e = idx % dv;
    float qs = 0.f;
    #pragma unroll 8
    for (int d = 0; d < dk; ++d) qs = fmaf(Qs[r * ldk + d], KS[e * ldk + d], qs);
    float acc = sc[r] * qs;
    if (u_lds) {
      #pragma unroll 8
      for (int i = 0; i <= r; ++i) acc = fmaf(P[r * ldc + i], Us[i * (dv + 1) + e], acc);
    } else {
      #pragma unroll 8
      for (int i = 0; i <= r; ++i) acc = fmaf(P[r * ldc + i], Uc[size_t(i) * dv + e], acc);
    }
    const size_t oi = row(r, dv) + e;
    if constexpr (sizeof(TOut) == 2)
      o[oi] = f32_to_bf16(acc);
    else
      o[oi] = acc;
  }
}

// more than the default 64 KB of dynamic LDS, once per instantiation, sized for the largest head dims
template <typename F>
hipError_t allow_lds(F *kernel, size_t floats) {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             int(floats * sizeof(float)));
}

hipError_t launch_fp32(const Plan &p, const Args &a) {
  const float *q = static_cast<const float *>(a.q), *k = static_cast<const float *>(a.k),
              *v = static_cast<const float *>(a.v);
  const float *beta = reinterpret_cast<const float *>(a.ws + p.off_beta);
  const float *rq = reinterpret_cast<const float *>(a.ws + p.off_rq);
  const float *rk = reinterpret_cast<const float *>(a.ws + p.off_rk);
  const float *gc = reinterpret_cast<const float *>(a.ws + p.off_gcum);
  float *W = reinterpret_cast<float *>(a.ws + p.off_W);
  float *Ut = reinterpret_cast<float *>(a.ws + p.off_Ut);
  float *U = reinterpret_cast<float *>(a.ws + p.off_U);
  float *S0 = reinterpret_cast<float *>(a.ws + p.off_S0);
  const unsigned chunks = unsigned(p.B) * p.H * p.N;
  const bool rev = p.flags & kReverse;
  constexpr int kD = kMaxPortableDim;
  static const hipError_t lds_ok[4] = {
      allow_lds(&intra_kernel, intra_lds_floats(kD, kD)), allow_lds(&state_kernel, state_lds_floats(kD)),
      allow_lds(&output_kernel<uint16_t>, kLdsFloats), allow_lds(&output_kernel<float>, kLdsFloats)};
  for (hipError_t le : lds_ok)
    if (le != hipSuccess) return le;
  intra_kernel<<<dim3(chunks), dim3(256), intra_lds_floats(p.dk, p.dv) * sizeof(float), a.stream>>>(
      k, v, beta, rk, gc, W, Ut, p.T, p.H, p.dk, p.dv, p.N, rev);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned tiles = unsigned(p.B) * p.H * ((p.dv + 15) / 16);
  state_kernel<<<dim3(tiles), dim3(256), state_lds_floats(p.dk) * sizeof(float), a.stream>>>(
      k, rk, gc, W, Ut, a.state_in, a.state_out, U, S0, p.T, p.H, p.dk, p.dv, p.N, rev);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.o_bf16)
    output_kernel<uint16_t><<<dim3(chunks), dim3(256), output_lds_launch_floats(p.dk, p.dv) * sizeof(float), a.stream>>>(
        q, k, rq, rk, gc, U, S0, static_cast<uint16_t *>(a.o), p.T, p.H, p.dk, p.dv, p.N, rev);
  else
    output_kernel<float><<<dim3(chunks), dim3(256), output_lds_launch_floats(p.dk, p.dv) * sizeof(float), a.stream>>>(
        q, k, rq, rk, gc, U, S0, static_cast<float *>(a.o), p.T, p.H, p.dk, p.dv, p.N, rev);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_portable(const Plan &p, const Args &a) {
  // bf16 and fp8 inputs always take the MFMA kernels (make_plan): only fp32 here
  if (p.qkv_bf16 || p.qkv_fp8) return hipErrorInvalidValue;
  return launch_fp32(p, a);
}

}  // namespace gdn
