// Streaming chunk-causal softmax attention block (see include/sanawm_attn.h).
//
// Two kernels per call:
//   stage: writes the block's k and v into its ring slot of the cache (and
//          its sink frames, if any, into the sink slot): K as rows of 112 bf16,
//          V transposed (per slot, 112 rows of the slot's keys), so that the
//          attention kernel's V operand is a run of consecutive keys.
//   attn:  flash attention over the context segments (sink slot, the ring
//          slots of the cached blocks, the current block's slot), one
//          workgroup per (b, h, 224 queries): seven compute waves (32 queries
//          each, two per SIMD) and a copy wave that brings 64-key tiles of K
//          and V^T into LDS with buffer-to-LDS loads, two barriers per tile
//          (the two waves of a SIMD trade matrix and vector work at the
//          second).  The compute waves are software-pipelined: step j forms
//          S^T of tile j while it accumulates P V of tile j - 1 (independent
//          products) and takes the softmax of tile j in the other half.  K
//          tiles therefore run one tile ahead of V^T tiles; each kind is
//          double-buffered.
//
// The compute waves work in transposed form.  S^T = K Q^T puts one query per
// lane (the accumulator column), so the running max and sum of a query stay
// in its lanes; its four 16-key row groups sit in lane groups g = 0..3 and
// are combined with two lane exchanges per tile.  O^T = V^T P^T then takes P^T
// straight from the S^T accumulators: two 16-key accumulator tiles are one
// 32-deep B operand in the "pair" k-order (slots 0-3: keys 4g..4g+3 of the
// first tile, slots 4-7: the same of the second), and V^T fragments are read
// in that order.  Each O^T accumulator lane again holds one query, so the
// per-tile rescale by e^(m_old - m_new) is lane-local.
//
// V^T layout: within every 32-key group of a slot, position 8g + s holds key
// 4g + s (s < 4) or 16 + 4g + (s - 4) (s >= 4), so that the eight keys a lane
// needs in the pair order are one 16-byte read.  Slot rows are padded to a
// multiple of 64 keys, the padding zero-filled by the stage kernel.
//
// Running maximum: each tile's maximum of a query is reduced over its four
// lane groups with two lane swaps (v_permlane16_swap / v_permlane32_swap,
// register-only), so P is taken against the exact running maximum and the
// query's largest weight is exactly 1 (a stale maximum would leave that
// dominant weight to bf16 rounding).  The accumulators are rescaled only when
// some query of the wave has a new maximum (a wave-uniform branch).
//
// Precision: q, k, v enter the matrix cores as the exact bf16 inputs; scores
// and the softmax are fp32; P is rounded to bf16 (relative 2^-8 at most per weight)
// for the P V product, accumulated in fp32.
#include "gdn_mfma_common.h"

#include <algorithm>

namespace gdn {
namespace attn {
namespace {

using mfma::bare_barrier;
using mfma::compute_barrier;
using mfma::copy16;
using mfma::F16;
using mfma::F32;
using mfma::f32x4;
using mfma::kOutOfRange;
using mfma::make_rsrc;
using mfma::mma;
using mfma::wait_vm;
using mfma::zero4;

constexpr int D = 112;
constexpr int KT = 64;                      // keys per tile
constexpr int kComputeWaves = 7;            // two per SIMD (one SIMD shares with the copy wave)
constexpr int QW = 32;                      // queries per compute wave (two 16-query tiles)
constexpr int QB = QW * kComputeWaves;      // 224 queries per workgroup
constexpr int kThreads = (kComputeWaves + 1) * 64;
constexpr int kKRow = 256;                  // bytes per staged K row (224 used)
constexpr int kKTile = KT * kKRow;          // 16 KB
constexpr int kVTile = D * KT * 2;          // 14 KB: V^T rows of 64 keys (128 B)
constexpr int kLdsV = 2 * kKTile;           // two K tile buffers, then two V^T tile buffers
constexpr int kLds = kLdsV + 2 * kVTile;    // 60 KB
constexpr int kKInstr = kKTile / 1024;      // 16 copies of 1 KB per K tile
constexpr int kVInstr = kVTile / 1024;      // 14 per V^T tile

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups of a column)
__device__ __forceinline__ float lanes4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ---------------------------------------------------------------------------
// stage: one workgroup (256 threads) per (b, h, 64 tokens of the block)
// position of key kk of a slot in its V^T rows (a permutation inside each 32-key group)
__device__ __forceinline__ int vt_pos(int kk) {
  const int g = kk & 31, hi = g >> 4, r = g & 15;
  return (kk & ~31) + 8 * (r >> 2) + 4 * hi + (r & 3);
}

__global__ __launch_bounds__(256) void stage_kernel(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                                    char *__restrict__ cache, int Lb, int H, int units,
                                                    size_t bh_bytes, int ring_koff, size_t ring_vt, int ring_pad,
                                                    int sink_koff, size_t sink_vt, int sink_keys, int sink_pad,
                                                    int sink_len, int block_tok0) {
  __shared__ uint16_t vs[KT][D + 2];  // the tile's V rows (row pitch 228 B)
  const int tiles = (Lb + KT - 1) / KT;
  const int u = blockIdx.x / tiles, t0 = (blockIdx.x % tiles) * KT;
  if (u >= units) return;
  const int b = u / H, h = u % H;
  const int n = min(KT, Lb - t0);
  const int tid = threadIdx.x;
  char *base = cache + size_t(u) * bh_bytes;
  const size_t rowstride = size_t(H) * D;
  const uint16_t *ksrc = k + (size_t(b) * Lb + t0) * rowstride + size_t(h) * D;
  const uint16_t *vsrc = v + (size_t(b) * Lb + t0) * rowstride + size_t(h) * D;
  // tokens of this block that are also sink tokens: block-local t < sink_len
  for (int idx = tid; idx < n * 14; idx += 256) {
    const int t = idx / 14, p = idx % 14;
    const uint4 kx = *reinterpret_cast<const uint4 *>(ksrc + size_t(t) * rowstride + 8 * p);
    *reinterpret_cast<uint4 *>(base + size_t(ring_koff + t0 + t) * (D * 2) + 16 * p) = kx;
    if (t0 + t < sink_len)
      *reinterpret_cast<uint4 *>(base + size_t(sink_koff + block_tok0 + t0 + t) * (D * 2) + 16 * p) = kx;
    const uint4 vx = *reinterpret_cast<const uint4 *>(vsrc + size_t(t) * rowstride + 8 * p);
    const uint32_t w[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) vs[t][8 * p + j] = uint16_t(w[j >> 1] >> (16 * (j & 1)));
  }
  __syncthreads();
  // V^T of a slot (row d: the slot's keys, permuted, rows of `pad` keys); this
  // tile fills keys key0 .. key0 + limit - 1, and the workgroup holding the
  // slot's last key also zero-fills the padding keys len .. pad - 1
  auto put_vt = [&](size_t vt_off, int pad, int len, int key0, int limit) {
    uint16_t *vt = reinterpret_cast<uint16_t *>(base + vt_off);
    for (int idx = tid; idx < D * limit; idx += 256) {
      const int d = idx / limit, t = idx % limit;
      vt[size_t(d) * pad + vt_pos(key0 + t)] = vs[t][d];
    }
    if (key0 + limit == len) {
      const int np = pad - len;
      for (int idx = tid; idx < D * np; idx += 256) {
        const int d = idx / np, t = idx % np;
        vt[size_t(d) * pad + vt_pos(len + t)] = 0;
      }
    }
  };
  // ring slot: the tile's keys t0 .. t0 + 63 fill positions t0 .. t0 + 63 of
  // every row (t0 is a multiple of 64); one 16-byte store per 8 positions,
  // keys past the block zero (the last tile covers the row padding)
  {
    uint16_t *vt = reinterpret_cast<uint16_t *>(base + ring_vt);
    for (int idx = tid; idx < D * (KT / 8); idx += 256) {
      const int d = idx / (KT / 8), gp = idx % (KT / 8);
      const int kb = 32 * (gp >> 2) + 4 * (gp & 3);  // keys kb .. kb + 3 and kb + 16 .. kb + 19
      uint32_t w[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const int ka = kb + (s2 < 2 ? 2 * s2 : 16 + 2 * (s2 - 2)), kc = ka + 1;
        const uint32_t lo = ka < n ? vs[ka][d] : 0u, hi = kc < n ? vs[kc][d] : 0u;
        w[s2] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4 *>(vt + size_t(d) * ring_pad + t0 + 8 * gp) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  if (t0 < sink_len) put_vt(sink_vt, sink_pad, sink_keys, block_tok0 + t0, min(n, sink_len - t0));
}

// ---------------------------------------------------------------------------
// attention: context segments, each a run of keys in one cache slot
struct Segs {
  int n;              // segments (1 .. 4)
  int koff[4];        // first key of the segment's slot in the per-(b, h) key space
  int len[4];         // keys of the segment (a prefix of the slot)
  int pad[4];         // keys per V^T row of the slot (a multiple of 64)
  int vt_off[4];      // byte offset of the slot's V^T in the per-(b, h) cache slice
  int tiles0[5];      // tiles before segment s; tiles0[n] = all tiles
};

__device__ __forceinline__ void tile_of(const Segs &sg, int j, int &s, int &key0, int &nvalid) {
  s = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < sg.n && j >= sg.tiles0[i]) s = i;
  key0 = KT * (j - sg.tiles0[s]);
  nvalid = min(KT, sg.len[s] - key0);
}

// Copy wave L (0: K tile, 1: V^T tile): tile j into buffer j & 1.
__device__ __forceinline__ void copy_role(const char *__restrict__ bh, const Segs &sg, char *lds) {
  const int lane = threadIdx.x & 63;
  const int ntiles = sg.tiles0[sg.n];
  auto issue_k = [&](int j) {
    int s, key0, nvalid;
    tile_of(sg, j, s, key0, nvalid);
    {
      // key r = 4i + lane / 16 of the tile, LDS slot lane % 16 holds piece slot ^ (r & 15)
      char *buf = lds + (j & 1) * kKTile;
      const auto rs = make_rsrc(bh + size_t(sg.koff[s] + key0) * (D * 2), uint32_t(nvalid) * (D * 2));
#pragma unroll
      for (int i = 0; i < kKInstr; ++i) {
        const int r = 4 * i + (lane >> 4), p = (lane & 15) ^ (r & 15);
        copy16(rs, buf + 1024 * i, p < 14 ? uint32_t(r) * (D * 2) + 16u * p : kOutOfRange);
      }
    }
  };
  auto issue_v = [&](int j) {
    int s, key0, nvalid;
    tile_of(sg, j, s, key0, nvalid);
    {
      // V^T row d = 8i + lane / 8, LDS slot lane % 8 holds positions 8 (slot ^ ((d >> 1) & 7)) .. + 7:
      // the sixteen 16-byte reads of rows d = 0..15 at one position hit distinct bank groups.
      // Positions past the segment hold other keys of the slot or the zero padding (masked)
      char *buf = lds + kLdsV + (j & 1) * kVTile;
      const auto rs = make_rsrc(bh + sg.vt_off[s], uint32_t(sg.pad[s]) * (D * 2));
#pragma unroll
      for (int i = 0; i < kVInstr; ++i) {
        const int d = 8 * i + (lane >> 3), p = (lane & 7) ^ ((d >> 1) & 7);
        copy16(rs, buf + 1024 * i, (uint32_t(d) * sg.pad[s] + key0 + 8 * p) * 2u);
      }
    }
  };
  // barrier j (j = 0 .. ntiles) opens step j, which reads K tile j and V^T
  // tile j - 1; after it, K tile j + 1 and V^T tile j are issued (their
  // buffers were last read in step j - 1).  K tile j + 1 has landed by the
  // mid-step turn, so the compute waves can read its first key tile during
  // their vector half.
  issue_k(0);
  for (int j = 0; j <= ntiles; ++j) {
    wait_vm<0>();
    bare_barrier();  // step j opens
    if (j + 1 < ntiles) issue_k(j + 1);
    if (j < ntiles) issue_v(j);
    if (j + 1 < ntiles) {  // K tile j + 1 lands by the mid-step turn (V^T tile j may stay in flight)
      if (j < ntiles)
        wait_vm<kVInstr>();
      else
        wait_vm<0>();
    }
    bare_barrier();  // the compute waves' mid-step turn
  }
}

template <bool kOutBf16>
__device__ __forceinline__ void compute_role(int W, const uint16_t *__restrict__ q, void *__restrict__ o, int Lb,
                                             int H, int b, int h, int qt, const Segs &sg, char *lds) {
  const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
  const size_t rowstride = size_t(H) * D;
  const int q0 = qt * QB + W * QW;  // first query of this wave
  // Q^T fragments (B operand of S^T = K Q^T, natural k-order): lane (ln, g) of
  // query tile qq holds q[q0 + 16 qq + ln][32 kb + 8 g .. + 7], tail [96 + 4 g .. + 3]
  F32 qf[2][3];
  F16 qtl[2];
  {
    const auto rq = make_rsrc(q + size_t(b) * Lb * rowstride, uint32_t(Lb) * uint32_t(rowstride) * 2u);
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const uint32_t row = (uint32_t(q0 + 16 * qq + ln) * uint32_t(rowstride) + uint32_t(h) * D) * 2u;
      const uint32_t rowo = q0 + 16 * qq + ln < Lb ? row : kOutOfRange;
#pragma unroll
      for (int kb = 0; kb < 3; ++kb) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(
            rq, int(rowo == kOutOfRange ? kOutOfRange : rowo + 64u * kb + 16u * lg), 0, 0);
        qf[qq][kb] = F32{{x.x, x.y, x.z, x.w}};
      }
      const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(
          rq, int(rowo == kOutOfRange ? kOutOfRange : rowo + 192u + 8u * lg), 0, 0);
      qtl[qq] = F16{{x.x, x.y}};
    }
  }
  // raw scores q . k to the log2 domain of the softmax: / sqrt(d) * log2(e)
  const float scale2 = 1.44269504088896341f / __builtin_sqrtf(float(D));
  f32x4 oacc[7][2];
#pragma unroll
  for (int dt = 0; dt < 7; ++dt) oacc[dt][0] = oacc[dt][1] = zero4();
  // running maximum of the raw scores per query tile, and the softmax
  // denominators: sum of the bf16 weights, formed on the matrix cores (an
  // all-ones A operand), so they are exactly the weights the numerator uses
  float m[2] = {-__builtin_inff(), -__builtin_inff()};
  f32x4 lacc[2] = {zero4(), zero4()};
  constexpr uint32_t kOnes = 0x3f803f80u;  // two bf16 1.0
  const F32 ones{{kOnes, kOnes, kOnes, kOnes}};
  const int ntiles = sg.tiles0[sg.n];
  f32x4 sacc[4][2];
  F32 pf[2][2];  // P^T B operands [qq][key pair] of the previous tile
  // ---- S^T = K Q^T of tile j: key tile t (16 keys), query tile qq
  // fragments of key tile t of K tile j
  auto kfrag = [&](int j, int t, F32 *kf, F16 &kt) {
    const char *rowp = lds + (j & 1) * kKTile + (16 * t + ln) * kKRow;
#pragma unroll
    for (int kb = 0; kb < 3; ++kb) {
      const uint4 x = *reinterpret_cast<const uint4 *>(rowp + 16 * ((4 * kb + lg) ^ ln));
      kf[kb] = F32{{x.x, x.y, x.z, x.w}};
    }
    const uint2 x2 = *reinterpret_cast<const uint2 *>(rowp + 16 * ((12 + (lg >> 1)) ^ ln) + 8 * (lg & 1));
    kt = F16{{x2.x, x2.y}};
  };
  F32 kpf[3];  // key tile 0 of the next K tile, read in the vector half before its scores
  F16 kpt;
  auto scores = [&](int j, bool pre) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      F32 kf[3];
      F16 kt;
      if (t == 0 && pre) {
        kf[0] = kpf[0];
        kf[1] = kpf[1];
        kf[2] = kpf[2];
        kt = kpt;
      } else {
        kfrag(j, t, kf, kt);
      }
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 3; ++kb) acc = mma(kf[kb], qf[qq][kb], acc);
        sacc[t][qq] = mma(kt, qtl[qq], acc);
      }
    }
  };
  // ---- O^T += V^T P^T of tile j: d tile dt, key pair pp (keys 32 pp .. 32 pp + 31)
  auto pv = [&](int j) {
    const char *vb_ = lds + kLdsV + (j & 1) * kVTile;
#pragma unroll
    for (int dt = 0; dt < 7; ++dt) {
      const int d = 16 * dt + ln;
      const char *vrow = vb_ + d * (KT * 2);
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        // positions 32 pp + 8 g .. + 7 hold this lane's pair-order keys
        const uint4 a = *reinterpret_cast<const uint4 *>(vrow + 16 * ((4 * pp + lg) ^ ((d >> 1) & 7)));
        const F32 vf{{a.x, a.y, a.z, a.w}};
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) oacc[dt][qq] = mma(vf, pf[qq][pp], oacc[dt][qq]);
      }
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) lacc[qq] = mma(ones, pf[qq][pp], lacc[qq]);
  };
  // ---- softmax of tile j per query (one query per lane column), exact running
  // maximum.  m holds the maximum raw score q . k; the weights are
  // 2^(scale2 (s - m)) = e^((s - m) / sqrt(d)), one FMA and one exp2 per score.
  auto softmax = [&](int j) {
    int s_, key0, nvalid;
    tile_of(sg, j, s_, key0, nvalid);
    if (nvalid < KT) {  // a segment's last tile: keys past it score -inf (wave-uniform)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * t + 4 * lg + e >= nvalid) sacc[t][qq][e] = -__builtin_inff();
    }
    float mnew[2];
    bool grow = false;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[t][qq][e]);
      mnew[qq] = fmaxf(m[qq], lanes4_max(mx));
      grow |= mnew[qq] > m[qq];
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {  // some query of the wave has a new maximum
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const float alpha = __builtin_amdgcn_exp2f((m[qq] - mnew[qq]) * scale2);  // 0 on the first tile
        lacc[qq] = lacc[qq] * alpha;
#pragma unroll
        for (int dt = 0; dt < 7; ++dt) oacc[dt][qq] = oacc[dt][qq] * alpha;
      }
    }
    m[0] = mnew[0];
    m[1] = mnew[1];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const float mo = -m[qq] * scale2;
      float pv_[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv_[t][e] = __builtin_amdgcn_exp2f(fmaf(sacc[t][qq][e], scale2, mo));
        }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
        pf[qq][pp] = F32{{pack_bf16x2(pv_[2 * pp][0], pv_[2 * pp][1]), pack_bf16x2(pv_[2 * pp][2], pv_[2 * pp][3]),
                          pack_bf16x2(pv_[2 * pp + 1][0], pv_[2 * pp + 1][1]),
                          pack_bf16x2(pv_[2 * pp + 1][2], pv_[2 * pp + 1][3])}};
    }
  };
  // Step j reads K tile j and V^T tile j - 1, in two halves separated by a
  // barrier.  Waves 0-3 ("lead") run the scores of tile j with P V of tile
  // j - 1 in the first half and the softmax of tile j in the second; waves 4-6
  // ("lag", the second wave on SIMDs 0-2) run the softmax of tile j - 1 in the
  // first half and the scores of tile j with P V of tile j - 1 in the second.
  // The two waves of a SIMD thus take turns on the matrix core while the other
  // works on the vector ALU; the mid-step barrier keeps them in turn (left
  // free-running they drifted into overlapping matrix phases), and the wave in
  // its matrix phase runs at raised priority so its MFMAs issue ahead of the
  // other wave's vector work.
  if (W < 4) {
    compute_barrier();
    scores(0, false);
    compute_barrier();
    softmax(0);
    if (1 < ntiles) kfrag(1, 0, kpf, kpt);
    for (int j = 1; j < ntiles; ++j) {
      compute_barrier();
      __builtin_amdgcn_s_setprio(2);
      scores(j, true);
      pv(j - 1);
      __builtin_amdgcn_s_setprio(0);
      compute_barrier();
      softmax(j);
      if (j + 1 < ntiles) kfrag(j + 1, 0, kpf, kpt);  // K tile j + 1 landed by the mid-step turn
    }
    compute_barrier();
    pv(ntiles - 1);
    compute_barrier();
  } else {
    compute_barrier();
    compute_barrier();
    scores(0, false);
    for (int j = 1; j < ntiles; ++j) {
      compute_barrier();
      softmax(j - 1);
      kfrag(j, 0, kpf, kpt);
      compute_barrier();
      __builtin_amdgcn_s_setprio(2);
      scores(j, true);
      pv(j - 1);
      __builtin_amdgcn_s_setprio(0);
    }
    compute_barrier();
    softmax(ntiles - 1);
    compute_barrier();
    pv(ntiles - 1);
  }
  // ---- normalise and store: lane (ln, g) of query tile qq holds d = 16 dt + 4 g .. + 3
  const auto ro = make_rsrc(static_cast<char *>(o) + size_t(b) * Lb * rowstride * (kOutBf16 ? 2 : 4),
                            uint32_t(Lb) * uint32_t(rowstride) * (kOutBf16 ? 2u : 4u));
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const float inv = 1.f / lacc[qq][0];  // every row of the denominator tile holds the same sum
    const int qi = q0 + 16 * qq + ln;
    const uint32_t row = qi < Lb ? uint32_t(qi) * uint32_t(rowstride) + uint32_t(h) * D : kOutOfRange;
#pragma unroll
    for (int dt = 0; dt < 7; ++dt) {
      const f32x4 w = oacc[dt][qq] * inv;
      const uint32_t el = row == kOutOfRange ? kOutOfRange : row + 16u * dt + 4u * lg;
      if constexpr (kOutBf16) {
        const u32x2_t pk = {pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3])};
        __builtin_amdgcn_raw_buffer_store_b64(pk, ro, int(el == kOutOfRange ? kOutOfRange : el * 2u), 0, 0);
      } else {
        const u32x4_t pk = {__float_as_uint(w[0]), __float_as_uint(w[1]), __float_as_uint(w[2]),
                            __float_as_uint(w[3])};
        __builtin_amdgcn_raw_buffer_store_b128(pk, ro, int(el == kOutOfRange ? kOutOfRange : el * 4u), 0, 0);
      }
    }
  }
}

template <bool kOutBf16>
__global__ __launch_bounds__(kThreads) void attn_kernel(const uint16_t *__restrict__ q,
                                                        const char *__restrict__ cache, void *__restrict__ o,
                                                        int Lb, int H, int units, int nqt, size_t bh_bytes,
                                                        Segs sg) {
  extern __shared__ __align__(16) char lds[];
  // workgroup i runs on XCD i % 8; each XCD takes a contiguous range of the
  // (b, h, query tile) list, so a (b, h)'s K and V^T are fetched into at most
  // two L2s and every XCD gets the same number of workgroups
  const int per_xcd = int((gridDim.x + 7) / 8);
  const int g = (blockIdx.x & 7) * per_xcd + int(blockIdx.x >> 3);
  if (g >= units * nqt) return;
  const int u = g / nqt, qt = g % nqt;
  const int b = u / H, h = u % H;
  const char *bh = cache + size_t(u) * bh_bytes;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  switch (wave) {
    case kComputeWaves: copy_role(bh, sg, lds); break;
    default: compute_role<kOutBf16>(wave, q, o, Lb, H, b, h, qt, sg, lds); break;
  }
}

}  // namespace

hipError_t launch_attn(const AttnPlan &p, int block, const void *q, const void *k, const void *v, void *cache,
                       void *o, hipStream_t stream) {
  const int units = p.B * p.H;
  const int ring = block % (p.C + 1);
  const int ring_koff = p.Ls + ring * p.Lb;
  const int block_tok0 = block * p.Lb;                           // first token of the block in the stream
  const int sink_len = std::max(0, std::min(p.Lb, p.Ls - block_tok0));  // block tokens that are sink tokens
  char *c = static_cast<char *>(cache);
  // V^T slots follow the K rows: the sink slot, then the ring slots
  auto ring_vt = [&](int r) { return p.vt0 + size_t(224) * (size_t(p.Ls_pad) + size_t(r) * p.Lb_pad); };
  {
    const unsigned grid = unsigned(units) * unsigned((p.Lb + KT - 1) / KT);
    stage_kernel<<<dim3(grid), dim3(256), 0, stream>>>(static_cast<const uint16_t *>(k),
                                                       static_cast<const uint16_t *>(v), c, p.Lb, p.H, units,
                                                       p.bh_bytes, ring_koff, ring_vt(ring), p.Lb_pad, 0, p.vt0, p.Ls,
                                                       p.Ls_pad, sink_len, block_tok0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // context segments: uncovered sink frames, the cached blocks (oldest first), the current block
  Segs sg{};
  const int first_block = std::max(0, block - p.C);
  const int sink_uncovered = std::min(p.Ls, first_block * p.Lb);  // sink keys below the window
  auto add = [&](int koff, int len, int pad, size_t vt_off) {
    sg.koff[sg.n] = koff;
    sg.len[sg.n] = len;
    sg.pad[sg.n] = pad;
    sg.vt_off[sg.n] = int(vt_off);
    sg.tiles0[sg.n + 1] = sg.tiles0[sg.n] + (len + KT - 1) / KT;
    ++sg.n;
  };
  if (sink_uncovered > 0) add(0, sink_uncovered, p.Ls_pad, p.vt0);
  for (int nb = first_block; nb <= block; ++nb) {
    const int r = nb % (p.C + 1);
    add(p.Ls + r * p.Lb, p.Lb, p.Lb_pad, ring_vt(r));
  }
  static const hipError_t lds0 = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_kernel<false>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  static const hipError_t lds1 = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_kernel<true>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (lds0 != hipSuccess) return lds0;
  if (lds1 != hipSuccess) return lds1;
  const int nqt = (p.Lb + QB - 1) / QB;
  const unsigned grid = 8u * unsigned((units * nqt + 7) / 8);
  if (p.o_bf16)
    attn_kernel<true><<<dim3(grid), dim3(kThreads), kLds, stream>>>(static_cast<const uint16_t *>(q), c, o, p.Lb,
                                                                   p.H, units, nqt, p.bh_bytes, sg);
  else
    attn_kernel<false><<<dim3(grid), dim3(kThreads), kLds, stream>>>(static_cast<const uint16_t *>(q), c, o, p.Lb,
                                                                    p.H, units, nqt, p.bh_bytes, sg);
  return hipGetLastError();
}

}  // namespace attn
}  // namespace gdn
