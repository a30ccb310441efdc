// K1 "prep": per token-head scalars of the gated delta rule, shared by both
// kernel families.
//
// For every (b, t, h) it writes, in head-major [B, H, T] fp32 arrays:
//   beta = sigmoid(beta logit)             (or the input itself: BETA_IS_PROB)
//   rq   = 1 / max(||q||_2, 1e-6)          (1 with QK_PRENORMALIZED)
//   rk   = 1 / max(||k||_2, 1e-6)
//   gcum = inclusive cumulative sum of max(g, -80) within the token's chunk
// Normalisation, sigmoid and the log-decay are the readings stated in
// include/sanawm_gdn.h of the gated delta rule the "SANA-WM" cookbook page
// (table "Architecture & components") names as its attention.  q and k stay
// raw in HBM: later kernels apply rq / rk as fp32 scales, so the bf16 inputs
// enter the matrix cores unrounded.
#include "gdn_internal.h"

namespace gdn {
namespace {

template <typename TIn>
__global__ __launch_bounds__(256) void prep_kernel(const TIn *__restrict__ q, const TIn *__restrict__ k,
                                                   const float *__restrict__ g,
                                                   const float *__restrict__ beta, float *__restrict__ o_beta,
                                                   float *__restrict__ o_rq, float *__restrict__ o_rk,
                                                   float *__restrict__ o_gcum, int T, int H, int dk, int N,
                                                   uint32_t flags) {
  const int b = blockIdx.x / N, c = blockIdx.x % N;
  const int t0 = c * kChunk;
  const int n = min(kChunk, T - t0);
  const bool rev = flags & kReverse;
  // 16 lanes per token-head row: lane l sums d = l, l + 16, ... (coalesced 64-byte
  // pieces), then the 16 partial sums are added by butterfly shuffles
  const int sub = threadIdx.x & 15;
  for (int idx = threadIdx.x >> 4; idx < n * H; idx += blockDim.x >> 4) {
    const int tt = idx / H, h = idx % H;
    const size_t th = (size_t(b) * T + phys_token(t0 + tt, T, rev)) * H + h;
    float rq = 1.f, rk = 1.f;
    if (!(flags & kQkPrenormalized)) {
      float sq = 0.f, sk = 0.f;
      const size_t row = th * size_t(dk);
      for (int d = sub; d < dk; d += 16) {
        const float a = load_f32(q, row + d), e = load_f32(k, row + d);
        sq = fmaf(a, a, sq);
        sk = fmaf(e, e, sk);
      }
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) {
        sq += __shfl_xor(sq, m, 16);
        sk += __shfl_xor(sk, m, 16);
      }
      rq = 1.f / fmaxf(sqrtf(sq), 1e-6f);
      rk = 1.f / fmaxf(sqrtf(sk), 1e-6f);
    }
    if (sub == 0) {
      const float bl = beta[th];
      const float bt = (flags & kBetaIsProb) ? bl : 1.f / (1.f + expf(-bl));
      const size_t out = (size_t(b) * H + h) * T + t0 + tt;
      o_beta[out] = bt;
      o_rq[out] = rq;
      o_rk[out] = rk;
    }
  }
  // chunk-local inclusive cumsum of the floored log-decay: the chunk's decays
  // of up to 64 heads are staged in LDS (coalesced over heads), then one
  // thread per head scans them.  The reverse scan takes each token's decay
  // from its successor in the original order (the same frame boundary), and
  // none for the last token.
  __shared__ float gs[kChunk][65];
  for (int h0 = 0; h0 < H; h0 += 64) {
    const int nh = min(64, H - h0);
    __syncthreads();  // the previous group's scan is done with gs
    for (int idx = threadIdx.x; idx < n * nh; idx += blockDim.x) {
      const int tt = idx / nh, hh = idx % nh, tau = t0 + tt;
      const float gv = !rev ? g[(size_t(b) * T + tau) * H + h0 + hh]
                            : (tau > 0 ? g[(size_t(b) * T + T - tau) * H + h0 + hh] : 0.f);
      gs[tt][hh] = floor_log_decay(gv);
    }
    __syncthreads();
    if (threadIdx.x < nh) {
      const int h = h0 + threadIdx.x;
      float G = 0.f;
      const size_t out = (size_t(b) * H + h) * T + t0;
      for (int tt = 0; tt < n; ++tt) {
        G += gs[tt][threadIdx.x];
        o_gcum[out + tt] = G;
      }
    }
  }
}

// o = x + y (the forward and reverse scans of the bidirectional layer): four
// elements per thread and step, the last n % 4 one by one
// (x may be o itself: each element is read before it is written, by the same thread)
template <bool kBf16>
__global__ __launch_bounds__(256) void combine_kernel(const float *x, const float *__restrict__ y, void *o,
                                                      size_t n) {
  const size_t n4 = n / 4;
  const float4 *x4 = reinterpret_cast<const float4 *>(x), *y4 = reinterpret_cast<const float4 *>(y);
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < n4; i += size_t(gridDim.x) * blockDim.x) {
    const float4 a = x4[i], b = y4[i];
    const float4 s = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    if constexpr (kBf16)
      static_cast<uint2 *>(o)[i] = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
    else
      reinterpret_cast<float4 *>(o)[i] = s;
  }
  if (blockIdx.x == 0 && threadIdx.x < n - 4 * n4) {
    const size_t i = 4 * n4 + threadIdx.x;
    if constexpr (kBf16)
      static_cast<uint16_t *>(o)[i] = f32_to_bf16(x[i] + y[i]);
    else
      static_cast<float *>(o)[i] = x[i] + y[i];
  }
}

// state_out = state_in (or 0) for an empty sequence
__global__ void state_passthrough_kernel(const float *__restrict__ sin, float *__restrict__ sout, size_t n) {
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < n; i += size_t(gridDim.x) * blockDim.x)
    sout[i] = sin ? sin[i] : 0.f;
}

}  // namespace

hipError_t launch_prep(const Plan &p, const Args &a) {
  float *beta = reinterpret_cast<float *>(a.ws + p.off_beta);
  float *rq = reinterpret_cast<float *>(a.ws + p.off_rq);
  float *rk = reinterpret_cast<float *>(a.ws + p.off_rk);
  float *gc = reinterpret_cast<float *>(a.ws + p.off_gcum);
  dim3 grid(unsigned(p.B) * unsigned(p.N)), block(256);
  if (p.qkv_bf16)
    prep_kernel<uint16_t><<<grid, block, 0, a.stream>>>(static_cast<const uint16_t *>(a.q),
                                                        static_cast<const uint16_t *>(a.k), a.g, a.beta, beta,
                                                        rq, rk, gc, p.T, p.H, p.dk, p.N, p.flags);
  else
    prep_kernel<float><<<grid, block, 0, a.stream>>>(static_cast<const float *>(a.q),
                                                     static_cast<const float *>(a.k), a.g, a.beta, beta, rq,
                                                     rk, gc, p.T, p.H, p.dk, p.N, p.flags);
  return hipGetLastError();
}

hipError_t launch_combine(const float *x, const float *y, void *o, bool o_bf16, size_t n, hipStream_t stream) {
  // every pointer is 16-byte aligned
  const size_t want = (n / 4 + 255) / 256;
  const dim3 grid(unsigned(want < 8192 ? (want ? want : 1) : 8192)), block(256);
  if (o_bf16)
    combine_kernel<true><<<grid, block, 0, stream>>>(x, y, o, n);
  else
    combine_kernel<false><<<grid, block, 0, stream>>>(x, y, o, n);
  return hipGetLastError();
}

hipError_t launch_state_passthrough(const Plan &p, const Args &a) {
  if (!a.state_out || a.state_out == a.state_in) return hipSuccess;
  const size_t n = size_t(p.B) * p.H * p.dv * p.dk;
  state_passthrough_kernel<<<dim3(unsigned((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)), dim3(256), 0,
                             a.stream>>>(a.state_in, a.state_out, n);
  return hipGetLastError();
}

}  // namespace gdn
