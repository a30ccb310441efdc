// Internal declarations shared by the host front-end and the kernel files of
// libsanawm_gdn.  Not part of the public ABI (include/sanawm_gdn.h is).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace gdn {

constexpr int kChunk = 80;        // tokens per chunk (divides the 880-token latent frame)
constexpr int kMaxPortableDim = 128;
constexpr int kMfmaDim = 112;     // head_dim of the SANA-WM DiT (20 heads x 112 = 2240)
constexpr float kLogDecayFloor = -80.0f;
// MFMA path: chunks in the first range (its intra-chunk step runs alone: 25
// chunks of 20 heads are 250 blocks of two chunk-heads, one round of a
// 256-CU GPU) and the default length of the later ranges (the workspace ring
// holds two ranges)
constexpr int kFirstRange = 25;
constexpr int kRangeCap = 48;
constexpr bool kHaveMfmaPath = true;

enum : uint32_t { kBetaIsProb = 1u, kQkPrenormalized = 2u, kReverse = 8u };

// Everything a launch sequence needs: the problem, the selected kernels and
// where each intermediate lives inside the caller's workspace.
struct Plan {
  int B = 0, T = 0, H = 0, dk = 0, dv = 0, N = 0;  // N = ceil(T / kChunk)
  int qkv_bf16 = 0, qkv_fp8 = 0, o_bf16 = 0;
  uint32_t flags = 0;
  bool mfma = false;
  // byte offsets into the workspace
  size_t off_beta = 0, off_rq = 0, off_rk = 0, off_gcum = 0;       // fp32 [B,H,T]
  size_t off_W = 0, off_Ut = 0, off_U = 0, off_S0 = 0;              // portable path
  // MFMA path: a ring of two slots of range_cap x B*H chunk-head records
  // (K~ | Q' | P'' hi | P'' lo | scales | M, mfma_record_bytes() each) and the fp32 [B, H, d_v, d_k]
  // state carried from one chunk range to the next
  size_t off_rec = 0, off_carry = 0;
  int range_cap = 0;
  size_t total = 0;
};

struct Args {
  const void *q, *k, *v;
  const float *g, *beta, *state_in;
  float *state_out;
  void *o;
  char *ws;
  hipStream_t stream;
};

// Kernel launch sequences (each returns the first launch error, if any).
hipError_t launch_prep(const Plan &p, const Args &a);
hipError_t launch_portable(const Plan &p, const Args &a);
hipError_t launch_mfma(const Plan &p, const Args &a);
hipError_t launch_state_passthrough(const Plan &p, const Args &a);
// The layer's projections (proj.hip): x [M, H*112] -> q, k, v [M, H*112] bf16,
// beta, g [M, H] fp32; o [M, HD] bf16 -> y [M, HD].  Weights are [out, in] bf16.
namespace proj {
hipError_t launch_in_proj(const uint16_t *x, const uint16_t *w_in, int M, int H, int T, int frame_tokens,
                          uint16_t *q, uint16_t *k, uint16_t *v, float *beta, float *g, hipStream_t stream);
hipError_t launch_out_proj(const uint16_t *o, const uint16_t *w_out, int M, int HD, void *y, bool y_bf16,
                           hipStream_t stream);
}  // namespace proj
// o = o_type(x + y) over n elements (fp32 x, y; o fp32 or bf16): the two scans of the bidirectional layer
hipError_t launch_combine(const float *x, const float *y, void *o, bool o_bf16, size_t n, hipStream_t stream);

// Streaming attention block (attn.hip): the validated geometry of one call.
struct AttnPlan {
  int B = 0, H = 0;
  int ft = 0, fpb = 0, C = 0, S = 0;  // frame tokens, frames per block, cached blocks, sink frames
  int Lb = 0, Ls = 0;                 // tokens per block, sink tokens
  int total_keys = 0;                 // keys per (b, h) in the cache: sink slot + C + 1 ring slots
  int Ls_pad = 0, Lb_pad = 0;         // V^T row lengths of the sink and ring slots (multiples of 64)
  size_t vt0 = 0;                     // byte offset of the V^T slots in a (b, h) slice (after the K rows)
  size_t bh_bytes = 0;                // cache bytes per (b, h)
  bool o_bf16 = false;
};
namespace attn {
hipError_t launch_attn(const AttnPlan &p, int block, const void *q, const void *k, const void *v, void *cache,
                       void *o, hipStream_t stream);
}

// bytes of one chunk-head record of the MFMA path (K~ | Q' | P'' hi, lo | scales | M)
size_t mfma_record_bytes();

// ---- small device helpers shared by the kernel files ----
// Physical token index of logical token tau: the reverse scan (kReverse)
// walks the tokens from last to first, every kernel indexing its chunks and
// rows by the logical order.
__device__ __forceinline__ int phys_token(int tau, int T, bool rev) { return rev ? T - 1 - tau : tau; }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's v_cvt_pk_bf16_f32
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
// two fp32 -> packed bf16 pair (first value in the low half), one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
// two fp32 -> packed fp16 pair (first value in the low half), round to nearest even
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}

// The log-decay floor: g below -80 is read as -80 (a decay factor changes by at
// most e^-80); NaN passes through unchanged, so a NaN gate propagates like any
// other NaN input.
__device__ __forceinline__ float floor_log_decay(float g) { return g < kLogDecayFloor ? kLogDecayFloor : g; }

template <typename T> __device__ __forceinline__ float load_f32(const T *p, size_t i);
template <> __device__ __forceinline__ float load_f32<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t *p, size_t i) {
  return bf16_to_f32(p[i]);
}

}  // namespace gdn
