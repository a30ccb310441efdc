// Portable kernels: the chunked gated delta rule in fp32 on the vector ALUs.
//
// They serve fp32 inputs (and any 1 <= d_k, d_v <= 128) and, on request, bf16
// inputs as a second, independent evaluation of the MFMA path.  Per (batch,
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

template <typename TIn>
__global__ __launch_bounds__(256) void intra_kernel(const TIn *__restrict__ k, const TIn *__restrict__ v,
                                                    const float *__restrict__ s_beta,
                                                    const float *__restrict__ s_rk,
                                                    const float *__restrict__ s_gcum, float *__restrict__ W,
                                                    float *__restrict__ Ut, int T, int H, int dk, int dv,
                                                    int N, bool rev) {
  __shared__ float A[C][C + 1];
  __shared__ float Tm[C][C + 1];
  __shared__ float sb[C], srk[C], sG[C];
  const ChunkIdx ci = chunk_of_block(H, N, T);
  const size_t sbase = (size_t(ci.b) * H + ci.h) * T + ci.t0;
  for (int r = threadIdx.x; r < C; r += blockDim.x) {
    const bool ok = r < ci.n;
    sb[r] = ok ? s_beta[sbase + r] : 0.f;
    srk[r] = ok ? s_rk[sbase + r] : 0.f;
    sG[r] = ok ? s_gcum[sbase + r] : 0.f;
  }
  __syncthreads();
  auto krow = [&](int r) { return ((size_t(ci.b) * T + phys_token(ci.t0 + r, T, rev)) * H + ci.h) * size_t(dk); };
  auto vrow = [&](int r) { return ((size_t(ci.b) * T + phys_token(ci.t0 + r, T, rev)) * H + ci.h) * size_t(dv); };
  // A (strictly lower), padded rows/cols are zero
  for (int idx = threadIdx.x; idx < C * C; idx += blockDim.x) {
    const int r = idx / C, i = idx % C;
    float val = 0.f;
    if (i < r && r < ci.n) {
      const size_t kr = krow(r), ki = krow(i);
      float dot = 0.f;
      for (int d = 0; d < dk; ++d) dot = fmaf(load_f32(k, kr + d), load_f32(k, ki + d), dot);
      val = sb[r] * expf(sG[r] - sG[i]) * srk[r] * srk[i] * dot;
    }
    A[r][i] = val;
  }
  __syncthreads();
  // Tm = (I + A)^{-1} by forward substitution, one column per thread
  if (threadIdx.x < C) {
    const int j = threadIdx.x;
    for (int r = 0; r < C; ++r) {
      float x;
      if (r < j) {
        x = 0.f;
      } else if (r == j) {
        x = 1.f;
      } else {
        float s = 0.f;
        for (int i = j; i < r; ++i) s = fmaf(A[r][i], Tm[i][j], s);
        x = -s;
      }
      Tm[r][j] = x;
    }
  }
  __syncthreads();
  const size_t cbase = ((size_t(ci.b) * H + ci.h) * N + ci.c) * C;
  // W = Tm diag(beta gamma rk) K_raw
  for (int idx = threadIdx.x; idx < C * dk; idx += blockDim.x) {
    const int r = idx / dk, d = idx % dk;
    float s = 0.f;
    for (int i = 0; i <= r && i < ci.n; ++i)
      s = fmaf(Tm[r][i] * (sb[i] * expf(sG[i]) * srk[i]), load_f32(k, krow(i) + d), s);
    W[(cbase + r) * dk + d] = s;
  }
  // Ut = Tm diag(beta) V
  for (int idx = threadIdx.x; idx < C * dv; idx += blockDim.x) {
    const int r = idx / dv, e = idx % dv;
    float s = 0.f;
    for (int i = 0; i <= r && i < ci.n; ++i) s = fmaf(Tm[r][i] * sb[i], load_f32(v, vrow(i) + e), s);
    Ut[(cbase + r) * dv + e] = s;
  }
}

// Sequential state pass: one block per (b, h, 16 rows of the state).
template <typename TIn>
__global__ __launch_bounds__(256) void state_kernel(const TIn *__restrict__ k, const float *__restrict__ s_rk,
                                                    const float *__restrict__ s_gcum,
                                                    const float *__restrict__ W, const float *__restrict__ Ut,
                                                    const float *state_in, float *state_out,
                                                    float *__restrict__ U, float *__restrict__ S0, int T, int H,
                                                    int dk, int dv, int N, bool rev) {
  constexpr int R = 16;
  __shared__ float S[R][kMaxPortableDim + 1];
  __shared__ float Us[C][R + 1];
  __shared__ float coef[C];
  __shared__ float gammaC;
  const int tiles = (dv + R - 1) / R;
  const int tile = blockIdx.x % tiles;
  const int h = (blockIdx.x / tiles) % H;
  const int b = blockIdx.x / (tiles * H);
  const int i0 = tile * R;
  const int nrows = min(R, dv - i0);
  const size_t bh = size_t(b) * H + h;
  for (int idx = threadIdx.x; idx < R * dk; idx += blockDim.x) {
    const int ii = idx / dk, d = idx % dk;
    S[ii][d] = (ii < nrows && state_in) ? state_in[(bh * dv + i0 + ii) * dk + d] : 0.f;
  }
  for (int c = 0; c < N; ++c) {
    const int t0 = c * C, n = min(C, T - t0);
    __syncthreads();
    const size_t sb = bh * T + t0;
    if (threadIdx.x < C) {
      const int r = threadIdx.x;
      const float Gl = s_gcum[sb + n - 1];
      coef[r] = r < n ? s_rk[sb + r] * expf(Gl - s_gcum[sb + r]) : 0.f;
      if (r == 0) gammaC = expf(Gl);
    }
    // entry state of this chunk, for the output kernel
    for (int idx = threadIdx.x; idx < nrows * dk; idx += blockDim.x) {
      const int ii = idx / dk, d = idx % dk;
      S0[((bh * N + c) * dv + i0 + ii) * dk + d] = S[ii][d];
    }
    // U = Ut - W S0^T for this tile's columns
    const size_t cb = (bh * N + c) * C;
    for (int idx = threadIdx.x; idx < C * R; idx += blockDim.x) {
      const int r = idx / R, ii = idx % R;
      float u = 0.f;
      if (r < n && ii < nrows) {
        float s = 0.f;
        const float *wr = W + (cb + r) * dk;
        for (int d = 0; d < dk; ++d) s = fmaf(wr[d], S[ii][d], s);
        u = Ut[(cb + r) * dv + i0 + ii] - s;
        U[(cb + r) * dv + i0 + ii] = u;
      }
      Us[r][ii] = u;
    }
    __syncthreads();
    // S <- gamma_n S + U^T diag(rk e^{G_n - G}) K_raw
    for (int idx = threadIdx.x; idx < R * dk; idx += blockDim.x) {
      const int ii = idx / dk, d = idx % dk;
      float s = 0.f;
      for (int r = 0; r < n; ++r)
        s = fmaf(Us[r][ii] * coef[r], load_f32(k, ((size_t(b) * T + phys_token(t0 + r, T, rev)) * H + h) * size_t(dk) + d),
                 s);
      S[ii][d] = fmaf(gammaC, S[ii][d], s);
    }
  }
  __syncthreads();
  if (state_out)
    for (int idx = threadIdx.x; idx < nrows * dk; idx += blockDim.x) {
      const int ii = idx / dk, d = idx % dk;
      state_out[(bh * dv + i0 + ii) * dk + d] = S[ii][d];
    }
}

template <typename TIn, typename TOut>
__global__ __launch_bounds__(256) void output_kernel(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                     const float *__restrict__ s_rq,
                                                     const float *__restrict__ s_rk,
                                                     const float *__restrict__ s_gcum,
                                                     const float *__restrict__ U, const float *__restrict__ S0,
                                                     TOut *__restrict__ o, int T, int H, int dk, int dv, int N,
                                                     bool rev) {
  __shared__ float P[C][C + 1];
  __shared__ float sc[C];
  const ChunkIdx ci = chunk_of_block(H, N, T);
  const size_t sbase = (size_t(ci.b) * H + ci.h) * T + ci.t0;
  auto row = [&](int r, int d) { return ((size_t(ci.b) * T + phys_token(ci.t0 + r, T, rev)) * H + ci.h) * size_t(d); };
  for (int idx = threadIdx.x; idx < C * C; idx += blockDim.x) {
    const int r = idx / C, i = idx % C;
    float val = 0.f;
    if (i <= r && r < ci.n) {
      float dot = 0.f;
      const size_t qr = row(r, dk), ki = row(i, dk);
      for (int d = 0; d < dk; ++d) dot = fmaf(load_f32(q, qr + d), load_f32(k, ki + d), dot);
      val = expf(s_gcum[sbase + r] - s_gcum[sbase + i]) * s_rq[sbase + r] * s_rk[sbase + i] * dot;
    }
    P[r][i] = val;
  }
  for (int r = threadIdx.x; r < C; r += blockDim.x)
    sc[r] = r < ci.n ? expf(s_gcum[sbase + r]) * s_rq[sbase + r] : 0.f;
  __syncthreads();
  const size_t bhc = (size_t(ci.b) * H + ci.h) * N + ci.c;
  const float *S0c = S0 + bhc * size_t(dv) * dk;
  const float *Uc = U + bhc * C * size_t(dv);
  for (int idx = threadIdx.x; idx < ci.n * dv; idx += blockDim.x) {
    const int r = idx / dv, e = idx % dv;
    float qs = 0.f;
    const size_t qr = row(r, dk);
    for (int d = 0; d < dk; ++d) qs = fmaf(load_f32(q, qr + d), S0c[size_t(e) * dk + d], qs);
    float acc = sc[r] * qs;
    for (int i = 0; i <= r; ++i) acc = fmaf(P[r][i], Uc[size_t(i) * dv + e], acc);
    const size_t oi = row(r, dv) + e;
    if constexpr (sizeof(TOut) == 2)
      o[oi] = f32_to_bf16(acc);
    else
      o[oi] = acc;
  }
}

template <typename TIn>
hipError_t launch_typed(const Plan &p, const Args &a) {
  const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k),
            *v = static_cast<const TIn *>(a.v);
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
  stage_begin(a, kStageIntra);
  intra_kernel<TIn><<<dim3(chunks), dim3(256), 0, a.stream>>>(k, v, beta, rk, gc, W, Ut, p.T, p.H, p.dk, p.dv,
                                                              p.N, rev);
  stage_end(a, kStageIntra);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned tiles = unsigned(p.B) * p.H * ((p.dv + 15) / 16);
  stage_begin(a, kStageState);
  state_kernel<TIn><<<dim3(tiles), dim3(256), 0, a.stream>>>(k, rk, gc, W, Ut, a.state_in, a.state_out, U, S0,
                                                             p.T, p.H, p.dk, p.dv, p.N, rev);
  stage_end(a, kStageState);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  stage_begin(a, kStageOutput);
  if (p.o_bf16)
    output_kernel<TIn, uint16_t><<<dim3(chunks), dim3(256), 0, a.stream>>>(
        q, k, rq, rk, gc, U, S0, static_cast<uint16_t *>(a.o), p.T, p.H, p.dk, p.dv, p.N, rev);
  else
    output_kernel<TIn, float><<<dim3(chunks), dim3(256), 0, a.stream>>>(
        q, k, rq, rk, gc, U, S0, static_cast<float *>(a.o), p.T, p.H, p.dk, p.dv, p.N, rev);
  stage_end(a, kStageOutput);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_portable(const Plan &p, const Args &a) {
  return p.qkv_bf16 ? launch_typed<uint16_t>(p, a) : launch_typed<float>(p, a);
}

}  // namespace gdn
