// The GDN layer's projections on the matrix cores: C = A W^T with A [M, K]
// (tokens x features, bf16) and W [N, K] (the weight in output-major order,
// bf16), fp32 accumulation, and an epilogue that writes C where the layer
// wants it (see include/sanawm_gdn.h, "The layer around the scan").
//
//   in-projection : [q | k | v | beta | a] = x W_in^T, written as q, k, v
//                   [B, T, H, 112] bf16 and beta, g [B, T, H] fp32, with the
//                   frame-wise log-decay g = -softplus(a) on a frame's first
//                   token and 0 elsewhere
//   out-projection: y = o W_out^T, fp32 or bf16
//
// One workgroup computes a 256 x 256 tile of C with eight waves (2 x 4, each
// 128 x 64 = 8 x 4 accumulator tiles of v_mfma_f32_16x16x32_bf16).  K runs in
// steps of 64: the step's A and W rows (32 KB each) are brought into LDS with
// buffer-to-LDS loads, double-buffered.  The two waves on each SIMD belong to
// two groups that run half a step apart (ping-pong): while one multiplies,
// the other reads its next fragments from LDS and issues copies, so the matrix
// pipe is not left idle during the reads.  A staged row is 128 bytes, its
// 16-byte pieces permuted by row (slot = piece ^ ((row >> 1) & 7)), so the
// 16-byte fragment reads of 16 consecutive rows fall on distinct banks.
// Rows past M or N and pieces past K are read as zeros (buffer range checks)
// and never stored.  Workgroups are mapped XCD by XCD to consecutive tile
// indices, and tile indices run over groups of eight M bands, M fastest, so
// the ~32 tiles one XCD runs at a time share both their A bands and their W
// tiles in that XCD's L2.
#include "gdn_mfma_common.h"

namespace gdn {
namespace proj {
namespace {

using mfma::compute_barrier;
using mfma::copy16;
using mfma::F32;
using mfma::f32x4;
using mfma::kOutOfRange;
using mfma::make_rsrc;
using mfma::mma;
using mfma::wait_vm;
using mfma::zero4;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kNS = 2;                         // stages in the ring
constexpr int kGroupM = 8;                     // M bands per tile group
constexpr int kThreads = 512;                  // 8 waves: 2 along M x 4 along N
constexpr int TM = 8, TN = 4;                  // accumulator tiles per wave (128 x 64)
constexpr int kRow = BK * 2;                   // 128 bytes per staged row
constexpr int kPieces = kRow / 16;             // 8
constexpr int kStage = (BM + BN) * kRow;       // 64 KB: A rows, then W rows
constexpr int kOutRow = BN * 4 + 16;           // staged fp32 output row (padded: lane groups on distinct banks)
constexpr int kLds = 128 * kOutRow;            // 130 KB: two K stages, or half of the output tile
static_assert(kLds >= kNS * kStage, "the output staging reuses the K stages");
constexpr int kCopies = kStage / 1024 / 8;     // 8 one-KB copies per wave and step
constexpr int kRowsPerCopy = 1024 / kRow;      // 8
constexpr int kCopiesA = BM / kRowsPerCopy;    // 32 copies of A rows, then 32 of W rows

// Workgroup barrier that waits for this wave's LDS reads but not for its
// buffer-to-LDS copies in flight (those are waited for with wait_vm).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// staged rows sharing one 256-byte bank line get different slots
__device__ __forceinline__ int slot_of(int row, int piece) { return piece ^ ((row / (256 / kRow)) % kPieces); }

// ---- epilogues: store(m, n, x) writes C[m][n .. n + 3] = x[0 .. 3] (m < M,
// n < N; columns past N are dropped), n a multiple of 4 ----
// The epilogues' outputs are written once and read by the next kernel, not by
// this one, so they are stored non-temporal: they then leave the A bands and
// W tiles this GEMM re-reads in the caches (the layer measured 1.4 % faster).
typedef unsigned int st_u32x2 __attribute__((ext_vector_type(2)));
typedef float st_f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_bf16x4(uint16_t *p, float4 x) {
  __builtin_nontemporal_store(st_u32x2{pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w)}, reinterpret_cast<st_u32x2 *>(p));
}

struct StoreOut {  // y [M, N] fp32 or bf16, N a multiple of 4
  void *y;
  int ldy;
  bool bf16;
  __device__ void store(int m, int n, int N, float4 x) const {
    const size_t i = size_t(m) * ldy + n;
    if (bf16)
      store_bf16x4(static_cast<uint16_t *>(y) + i, x);
    else
      __builtin_nontemporal_store(st_f32x4{x.x, x.y, x.z, x.w}, reinterpret_cast<st_f32x4 *>(static_cast<float *>(y) + i));
  }
};

struct InProj {  // columns: q, k, v (HD each, HD a multiple of 4), beta (H), a (H)
  uint16_t *q, *k, *v;
  float *beta, *g;
  int HD, H, T, frame_tokens;
  __device__ void one(int m, int n, float x) const {
    if (n < 3 * HD + H) {
      beta[size_t(m) * H + (n - 3 * HD)] = x;
    } else {
      // softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(e^-|x|)
      const bool first = (m % T) % frame_tokens == 0;
      g[size_t(m) * H + (n - 3 * HD - H)] = first ? -(fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)))) : 0.f;
    }
  }
  __device__ void store(int m, int n, int N, float4 x) const {
    if (n < 3 * HD) {  // four columns of one of q, k, v
      const int which = n / HD, c = n - which * HD;
      uint16_t *dst = which == 0 ? q : (which == 1 ? k : v);
      store_bf16x4(dst + size_t(m) * HD + c, x);
    } else {
      const float e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < N) one(m, n + i, e[i]);
    }
  }
};

template <class Epi>
__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(const uint16_t *__restrict__ A,
                                                           const uint16_t *__restrict__ W, int M, int N, int K,
                                                           int tiles_m, int tiles_n, Epi epi) {
  extern __shared__ __align__(16) char lds[];
  // workgroup i runs on XCD i % 8: XCD x takes tiles [x * per, (x + 1) * per)
  const int per = int(gridDim.x) / 8;
  const int t = int(blockIdx.x & 7) * per + int(blockIdx.x >> 3);
  if (t >= tiles_m * tiles_n) return;
  const int group = t / (kGroupM * tiles_n), in_group = t % (kGroupM * tiles_n);
  const int gm = min(kGroupM, tiles_m - group * kGroupM);
  const int tm = group * kGroupM + in_group % gm, tn = in_group / gm;
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 2, wn = wave & 3;

  const uint32_t row_bytes = uint32_t(K) * 2u;
  const auto ra = make_rsrc(A + size_t(tm) * BM * K, uint32_t(min(BM, M - tm * BM)) * row_bytes);
  const auto rw = make_rsrc(W + size_t(tn) * BN * K, uint32_t(min(BN, N - tn * BN)) * row_bytes);
  // Copy c (0 .. 63) of a step fills staged rows 8 c' .. 8 c' + 7 of A
  // (c' = c < 32) or W (c' = c - 32); lane l takes row 8 c' + l / 8.  The
  // slot permutation of a row depends on c' only through its parity, so each
  // lane keeps two byte offsets (even / odd c') and adds the copy's row and
  // the step's k as wave-uniform terms.
  const int lrow = lane / kPieces;
  const int piece_e[2] = {(lane % kPieces) ^ (lrow >> 1), (lane % kPieces) ^ (4 + (lrow >> 1))};
  const uint32_t lane_off[2] = {uint32_t(lrow) * row_bytes + 16u * uint32_t(piece_e[0]),
                                uint32_t(lrow) * row_bytes + 16u * uint32_t(piece_e[1])};
  auto issue_copy = [&](int step, int c) {
    char *buf = lds + (step % kNS) * kStage;
    const int k0 = step * BK;
    const bool isw = c >= kCopiesA;
    const int cc = isw ? c - kCopiesA : c;
    const int e = cc & 1;
    const uint32_t off = k0 + 8 * piece_e[e] < K
                             ? lane_off[e] + uint32_t(cc) * (kRowsPerCopy * row_bytes) + uint32_t(k0) * 2u
                             : kOutOfRange;
    copy16(isw ? rw : ra, buf + (isw ? BM * kRow : 0) + 1024 * cc, off);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero4();

  // Ping-pong.  The lead group (wm 0) and the lag group (wm 1) each hold one
  // wave on every SIMD, and a barrier opens every half step ("period"):
  //   period 2s    : lead reads the fragments of step s, then issues all
  //                  copies of step s + 1;  lag multiplies step s - 1;
  //   period 2s + 1: lead multiplies step s;  lag reads step s.
  // The stage of step s + 1 holds step s - 1, whose last reads (lag, period
  // 2s - 1) end before period 2s.  Only the lead copies inside the loop: the
  // compiler makes a wave's LDS reads wait for that wave's copies in flight,
  // so copies from the lag would stall its reads one period later.
  const int steps = (K + BK - 1) / BK;
  const bool lead = wm == 0;
  F32 af[BK / 32][TM], bfr[BK / 32][TN];
  auto read = [&](int s) {
    const char *buf = lds + (s % kNS) * kStage;
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * 64 + 16 * j + ln;
        const uint4 x =
            *reinterpret_cast<const uint4 *>(buf + BM * kRow + row * kRow + 16 * slot_of(row, 4 * kb + lg));
        bfr[kb][j] = F32{{x.x, x.y, x.z, x.w}};
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * 128 + 16 * i + ln;
        const uint4 x = *reinterpret_cast<const uint4 *>(buf + row * kRow + 16 * slot_of(row, 4 * kb + lg));
        af[kb][i] = F32{{x.x, x.y, x.z, x.w}};
      }
    }
  };
  auto multiply = [&]() {
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mma(af[kb][i], bfr[kb][j], acc[i][j]);
  };
  // steps 0 and 1 before the loop, an eighth from each wave
#pragma unroll
  for (int st = 0; st < 2; ++st)
    if (st < steps) {
#pragma unroll
      for (int i = 0; i < kCopies; ++i) issue_copy(st, kCopies * wave + i);
    }
  if (steps > 1)
    wait_vm<kCopies>();  // this wave's copies of step 0 have landed
  else
    wait_vm<0>();
  if (lead) {
    for (int s = 0; s < steps; ++s) {
      lds_barrier();  // period 2s
      read(s);
      if (s >= 1 && s + 1 < steps) {
#pragma unroll
        for (int i = 0; i < 2 * kCopies; ++i) issue_copy(s + 1, 2 * kCopies * wave + i);
      }
      lds_barrier();  // period 2s + 1
      multiply();
      __builtin_amdgcn_sched_barrier(0);  // the wait stays behind the products
      wait_vm<0>();  // the copies of step s + 1 are in LDS before period 2s + 2
    }
    lds_barrier();  // period 2 steps
  } else {
    lds_barrier();  // period 0
    for (int s = 0; s < steps; ++s) {
      lds_barrier();  // period 2s + 1
      read(s);
      wait_vm<0>();  // (step 1's copies from before the loop)
      lds_barrier();  // period 2s + 2
      multiply();
    }
  }
  // Output through LDS, half a tile (128 rows x 256 columns, fp32) at a time:
  // the waves of that half write their accumulators -- tile (i, j) holds rows
  // 16 i + 4 lg + e of the wave's 128, column 16 j + ln of its 64 -- then every
  // wave stores whole rows, 16 bytes per lane.
  float *out = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    compute_barrier();  // the K stages (or the previous half) are no longer read
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            out[(16 * i + 4 * lg + e) * (kOutRow / 4) + wn * 64 + 16 * j + ln] = acc[i][j][e];
    }
    compute_barrier();
    const int n = tn * BN + 4 * lane;
#pragma unroll 4
    for (int r = wave; r < 128; r += 8) {
      const int m = tm * BM + half * 128 + r;
      if (m < M && n < N) epi.store(m, n, N, *reinterpret_cast<const float4 *>(out + r * (kOutRow / 4) + 4 * lane));
    }
  }
}

template <class Epi>
hipError_t launch_gemm(const uint16_t *A, const uint16_t *W, int M, int N, int K, const Epi &epi,
                       hipStream_t stream) {
  static const hipError_t lds_ok = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_nt_kernel<Epi>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (lds_ok != hipSuccess) return lds_ok;
  if (M <= 0 || N <= 0) return hipSuccess;
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  const unsigned grid = 8u * unsigned((tiles_m * tiles_n + 7) / 8);
  gemm_nt_kernel<Epi><<<dim3(grid), dim3(kThreads), kLds, stream>>>(A, W, M, N, K, tiles_m, tiles_n, epi);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_in_proj(const uint16_t *x, const uint16_t *w_in, int M, int H, int T, int frame_tokens,
                          uint16_t *q, uint16_t *k, uint16_t *v, float *beta, float *g, hipStream_t stream) {
  const int HD = H * kMfmaDim;
  InProj epi{q, k, v, beta, g, HD, H, T, frame_tokens};
  return launch_gemm(x, w_in, M, 3 * HD + 2 * H, HD, epi, stream);
}

hipError_t launch_out_proj(const uint16_t *o, const uint16_t *w_out, int M, int HD, void *y, bool y_bf16,
                           hipStream_t stream) {
  StoreOut epi{y, HD, y_bf16};
  return launch_gemm(o, w_out, M, HD, HD, epi, stream);
}

}  // namespace proj
}  // namespace gdn
