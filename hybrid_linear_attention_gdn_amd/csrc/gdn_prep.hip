// K1 "prep": per token-head scalars of the gated delta rule for the fp32
// kernels (the MFMA kernels form them inside their intra-chunk step).
//
// For every (b, t, h) it writes, in head-major [B, H, T] fp32 arrays:
//   beta = sigmoid(beta logit)             (or the input itself: BETA_IS_PROB)
//   rq   = 1 / max(||q||_2, 1e-6)          (1 with QK_PRENORMALIZED)
//   rk   = 1 / max(||k||_2, 1e-6)
//   gcum = inclusive cumulative sum of max(g, -80) within the token's chunk
// Normalisation, sigmoid and the log-decay are the readings stated in
// include/sanawm_gdn.h of the gated delta rule the "SANA-WM" cookbook page
// (table "Architecture & components") names as its attention.  q and k stay
// raw in HBM: later kernels apply rq / rk as fp32 scales.
#include "gdn_internal.h"

namespace gdn {
namespace {

// One block per (b, chunk, h): 16 lanes per token row (coalesced 64-byte
// pieces, partial sums added by butterfly shuffles), 16 rows at a time; then
// the chunk's floored decays are scanned in LDS (log-step inclusive scan).
__global__ __launch_bounds__(256) void prep_kernel(const float *__restrict__ q, const float *__restrict__ k,
                                                   const float *__restrict__ g, const float *__restrict__ beta,
                                                   float *__restrict__ o_beta, float *__restrict__ o_rq,
                                                   float *__restrict__ o_rk, float *__restrict__ o_gcum, int T, int H,
                                                   int dk, int N, uint32_t flags) {
  const int h = blockIdx.x % H, c = (blockIdx.x / H) % N, b = blockIdx.x / (H * N);
  const int t0 = c * kChunk;
  const int n = min(kChunk, T - t0);
  const bool rev = flags & kReverse;
  const size_t out = (size_t(b) * H + h) * T + t0;
  const int sub = threadIdx.x & 15;
  for (int tt = threadIdx.x >> 4; tt < n; tt += blockDim.x >> 4) {
    const size_t th = (size_t(b) * T + phys_token(t0 + tt, T, rev)) * H + h;
    float rq = 1.f, rk = 1.f;
    if (!(flags & kQkPrenormalized)) {
      float sq = 0.f, sk = 0.f;
      const size_t row = th * size_t(dk);
#pragma unroll 8
      for (int d = sub; d < dk; d += 16) {
        const float x = q[row + d], e = k[row + d];
        sq = fmaf(x, x, sq);
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
      o_beta[out + tt] = (flags & kBetaIsProb) ? bl : 1.f / (1.f + expf(-bl));
      o_rq[out + tt] = rq;
      o_rk[out + tt] = rk;
    }
  }
  // chunk-local inclusive cumsum of the floored log-decay, summed left to right
  // by one thread (so that G_r - G_i carries only the rounding of the terms
  // between i and r, as in a running sum).  The reverse scan takes each token's
  // decay from its successor in the original order (the same frame boundary),
  // and none for the last token.
  __shared__ float gs[kChunk];
  const int t = threadIdx.x;
  if (t < n) {
    const int tau = t0 + t;
    gs[t] = floor_log_decay(!rev ? g[(size_t(b) * T + tau) * H + h] : (tau > 0 ? g[(size_t(b) * T + T - tau) * H + h] : 0.f));
  }
  __syncthreads();
  if (t == 0) {
    float G = 0.f;
    for (int tt = 0; tt < n; ++tt) {
      G += gs[tt];
      o_gcum[out + tt] = G;
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
  // the fp32 kernels only (bf16 and fp8 inputs take the MFMA kernels, whose
  // intra-chunk step forms these scalars itself)
  if (p.qkv_bf16 || p.qkv_fp8) return hipErrorInvalidValue;
  const dim3 grid(unsigned(p.B) * unsigned(p.N) * unsigned(p.H)), block(256);
  prep_kernel<<<grid, block, 0, a.stream>>>(static_cast<const float *>(a.q), static_cast<const float *>(a.k), a.g,
                                            a.beta, beta, rq, rk, gc, p.T, p.H, p.dk, p.N, p.flags);
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
