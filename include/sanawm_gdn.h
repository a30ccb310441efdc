/*
 * libsanawm_gdn -- frame-wise Gated DeltaNet (GDN) forward on AMD Instinct
 * MI355X (CDNA4, gfx950).  Plain C ABI: no HIP, C++ or framework types.
 *
 * The operation.  The SGLang-diffusion cookbook page "SANA-WM" (table
 * "Architecture & components", row "Attention") and the blog post on SANA-WM
 * (section "core idea / structure") name the DiT's token mixer a frame-wise
 * Gated DeltaNet whose bounded state carries the causal history across
 * streaming chunks.  The pages print no formula; this library computes the
 * published gated delta rule (Yang, Kautz & Hatamizadeh, ICLR 2025), for
 * every batch row b and head h independently, over tokens t in the order
 * given (frame-major):
 *
 *     S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t * v_t k_t^T
 *     o_t = S_t q_t
 *
 * S is a d_v x d_k fp32 matrix (row i = value channel i).  Readings where
 * the pages are silent:
 *   - q_t and k_t are L2-normalised inside: x / max(||x||_2, 1e-6);
 *   - beta_t = sigmoid(beta[t]) (beta holds logits; +-inf give exactly 1, 0);
 *   - alpha_t = exp(g[t]); g is the per-token log-decay.  "Frame-wise" gating
 *     is carried by the data: g is non-zero on a frame's first token only.
 *     g is floored at -80 before use (changes a decay by at most e^-80);
 *   - the output reads the state after the token's own update, unscaled.
 *
 * Layouts (all contiguous, row-major, 16-byte aligned base pointers):
 *   q, k      [B, T, H, d_k]  qkv_dtype
 *   v         [B, T, H, d_v]  qkv_dtype
 *   g, beta   [B, T, H]       fp32
 *   state     [B, H, d_v, d_k] fp32
 *   o         [B, T, H, d_v]  o_dtype
 *
 * Ownership: the caller owns every buffer, including the workspace (size it
 * with gdn_workspace_bytes).  The library allocates and frees no device
 * memory and keeps no pointer after the enqueued work completes.
 *
 * Asynchrony: gdn_fwd / gdn_chunk_step validate their arguments on the host,
 * enqueue kernels on `hip_stream` (a hipStream_t; NULL = the default stream)
 * and return.  Device faults surface at the caller's next synchronisation.
 *
 * Errors: every function returns a status; no exception or abort crosses the
 * ABI.  All argument checks run before the first launch, so a call that
 * returns anything but GDN_OK or GDN_ERR_HIP has enqueued nothing.  A
 * thread-local message with the detail is available from gdn_last_error().
 *
 * Determinism: identical inputs give bitwise identical outputs (no atomics,
 * fixed reduction orders).
 */
#ifndef SANAWM_GDN_H
#define SANAWM_GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARGUMENT = 1, /* NULL/misaligned pointer, bad shape or dtype */
    GDN_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. head size) */
    GDN_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required */
    GDN_ERR_HIP = 4,              /* a HIP call failed; gdn_last_error has its text */
    GDN_ERR_INTERNAL = 5
} gdn_status_t;

/* GDN_FP8_E4M3: OCP 8-bit float E4M3FN (1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, max 448), for q, k, v only, unit scale.  A
 * per-tensor scale needs no argument: q and k are normalised inside (their
 * scale cancels) and o and the state are linear in v (a scale on v factors
 * out of both). */
typedef enum { GDN_F32 = 0, GDN_BF16 = 1, GDN_FP8_E4M3 = 2 } gdn_dtype_t;

enum {
    GDN_FLAG_BETA_IS_PROB = 1u,     /* beta already holds probabilities: no sigmoid */
    GDN_FLAG_QK_PRENORMALIZED = 2u, /* q, k already unit length: no normalisation */
    GDN_FLAG_REVERSE = 8u           /* the reverse scan (gdn_fwd only; see below) */
};

typedef struct {
    int32_t batch;      /* B >= 1 */
    int32_t seq_len;    /* T >= 0 tokens per call */
    int32_t num_heads;  /* H >= 1 */
    int32_t head_dim_k; /* d_k */
    int32_t head_dim_v; /* d_v */
    int32_t qkv_dtype;  /* gdn_dtype_t of q, k, v */
    int32_t o_dtype;    /* gdn_dtype_t of o */
    uint32_t flags;     /* GDN_FLAG_* */
} gdn_problem_t;

/*
 * Supported problems.  qkv_dtype = GDN_BF16 or GDN_FP8_E4M3 with d_k = d_v =
 * 112 (20 x 112 = the DiT's hidden 2240) runs the MFMA kernels; fp8 inputs
 * are widened exactly to bf16 inside them (the SGLang cookbook's FP8 Stage-1
 * precision), the state stays fp32.  On these kernels the state enters its
 * products split into two bf16 halves, and the other derived operands (the
 * chunk's M = K^T diag(s) T, P' = P T and the new values R) enter as fp16, R
 * scaled by a power of two per 80 x 16 tile; every product accumulates in
 * fp32.  The output's error is near 2e-3 of rms(o) on N(0,1) inputs of the
 * 241-frame clip.  qkv_dtype = GDN_F32 runs fp32 vector-ALU kernels (error near
 * 1e-6 of rms(o)), which take any 1 <= d_k, d_v <= 128.  Other combinations
 * return GDN_ERR_UNSUPPORTED.
 */

/* Chunk length of the chunked evaluation (80 tokens: it divides the 880
 * tokens of a 704 x 1280 latent frame). */
int32_t gdn_chunk_len(void);

/* Bytes of device workspace that gdn_fwd / gdn_chunk_step need for `p`. */
gdn_status_t gdn_workspace_bytes(const gdn_problem_t *p, size_t *bytes);

/*
 * One forward pass over T tokens.
 *   state_in  NULL = zero initial state.
 *   state_out NULL = final state not written; may equal state_in (in place).
 *   o         written for every token.
 * Same streaming semantics as running the recurrence token by token: a
 * sequence split into calls, each call's state_out fed as the next call's
 * state_in, gives the outputs of one pass.
 */
gdn_status_t gdn_fwd(const gdn_problem_t *p, const void *q, const void *k, const void *v,
                     const float *g, const float *beta, const float *state_in, float *state_out,
                     void *o, void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * One streaming call (a chunk of the causal rollout, e.g. 3 latent frames =
 * 2,640 tokens): the same mathematics as gdn_fwd, with a stricter contract --
 * state_in must be non-NULL and seq_len a multiple of gdn_chunk_len(), which
 * makes a rollout of calls bitwise equal to one gdn_fwd pass over the
 * concatenation.  state_out may be NULL (a denoising step that must not
 * commit the state) or equal state_in.
 */
gdn_status_t gdn_chunk_step(const gdn_problem_t *p, const void *q, const void *k, const void *v,
                            const float *g, const float *beta, const float *state_in,
                            float *state_out, void *o, void *workspace, size_t workspace_bytes,
                            void *hip_stream);

/*
 * gdn_fwd_no_alloc: gdn_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same problem, arguments, flags and results as gdn_fwd (the
 * outputs equal gdn_fwd's bit for bit), but no workspace argument: the
 * workspace is a fixed array of GDN_NO_ALLOC_SCRATCH_BYTES inside the library,
 * one per device, allocated when the library's code is loaded on that device
 * and held until the process ends.  The call allocates and frees nothing.
 * Limit: on the bf16/fp8 kernels the chunk ranges shrink to fit (B*H up to
 * 354 at 64 MiB); the fp32 kernels need their whole gdn_workspace_bytes.  A
 * problem that does not fit returns GDN_ERR_WORKSPACE before any HIP call.
 * The current device must be the stream's device (else
 * GDN_ERR_INVALID_ARGUMENT).  Calls that overlap on one device (two streams,
 * two threads) share the array and race: serialise them.
 */
#define GDN_NO_ALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status_t gdn_fwd_no_alloc(const gdn_problem_t *p, const void *q, const void *k, const void *v,
                              const float *g, const float *beta, const float *state_in,
                              float *state_out, void *o, void *hip_stream);

/*
 * The reverse scan (GDN_FLAG_REVERSE, gdn_fwd only).  The same recurrence run
 * over the tokens from last to first: S'_t = alpha'_t S'_{t+1} (I - beta_t k_t
 * k_t^T) + beta_t v_t k_t^T, o_t = S'_t q_t, where alpha'_t = exp(g[t + 1])
 * for t < T - 1 and alpha'_{T-1} = 1, so that the decays sit on the same
 * frame boundaries as the forward scan's (with frame-wise g, a token's
 * contribution to another decays by the gates of the frame starts between
 * them, on either side).  state_in is the state after the last token, o and
 * state_out (the state after token 0) keep the layouts above and the original
 * token order.  gdn_chunk_step rejects the flag: a call's last decay would
 * come from the next call.
 *
 * The bidirectional layer of the dense checkpoint (the SGLang cookbook page
 * "SANA-WM", serving-mode table, row "Dense bidirectional": one-shot
 * generation with full bidirectional context).  The pages do not say how the
 * recurrent mixer is made bidirectional; this library takes the reading
 *     o_t = o_t(forward scan) + o_t(reverse scan),
 * both scans from a zero state, on the same q, k, v, g, beta.  A caller that
 * wants another combination (other inputs per direction, a weighted sum) runs
 * gdn_fwd with and without GDN_FLAG_REVERSE itself.
 *
 * gdn_bidir_fwd: o [B, T, H, d_v] (fp32 or bf16) for every token; the flags
 * may not include GDN_FLAG_REVERSE.  Both scans accumulate in fp32; for bf16
 * o the sum is rounded once; either way each element is one fp32 add of the
 * two scans' outputs.  Size the workspace with
 * gdn_bidir_workspace_bytes: the scan's workspace (the two scans run one
 * after the other and share it) plus the reverse scan's fp32 output and, for
 * bf16 o, the forward scan's.  Same validation, ownership and asynchrony contract as gdn_fwd.
 */
gdn_status_t gdn_bidir_workspace_bytes(const gdn_problem_t *p, size_t *bytes);
gdn_status_t gdn_bidir_fwd(const gdn_problem_t *p, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, void *o, void *workspace,
                           size_t workspace_bytes, void *hip_stream);

/*
 * The layer around the scan (projections of the DiT's token mixer).  The
 * SGLang cookbook page "SANA-WM" (table "Architecture & components") gives
 * the DiT's width, hidden 2240 = 20 heads x 112, and names the mixer; it does
 * not print the layer's projections.  Readings taken (plain linear maps, no
 * biases, weights in [out, in] order, bf16, fp32 accumulation):
 *   [q | k | v | b | a] = x W_in^T,  W_in [3 H 112 + 2 H, H 112]
 *     q, k, v  [B, T, H, 112] bf16   (the scan normalises q and k itself)
 *     beta     = b (the logits the scan passes through its sigmoid)
 *     g        = -softplus(a) on a frame's first token (t % frame_tokens == 0),
 *                0 on the others: one log-decay per (frame, head), read from
 *                the frame's first token -- the frame-wise gate
 *   o = scan(q, k, v, g, beta)  (bf16, causal with state; or bidirectional)
 *   y = o W_out^T,  W_out [H 112, H 112],  y [B, T, H 112] fp32 or bf16
 * Both projections run on hand-written MFMA kernels (256 x 256 tiles).
 */
typedef struct {
    int32_t batch;        /* B >= 1 */
    int32_t seq_len;      /* T >= 0 */
    int32_t num_heads;    /* H >= 1; the model width is H * 112 */
    int32_t frame_tokens; /* tokens per latent frame (880 at 704 x 1280), >= 1 */
    int32_t y_dtype;      /* GDN_F32 or GDN_BF16 */
    uint32_t flags;       /* 0, or GDN_LAYER_BIDIRECTIONAL */
} gdn_layer_t;
#define GDN_LAYER_BIDIRECTIONAL 16u /* the scan is gdn_bidir_fwd's (no state in or out) */

/* x [B, T, H 112] bf16, w_in [3 H 112 + 2 H, H 112] bf16 -> q, k, v [B, T, H,
 * 112] bf16 and beta, g [B, T, H] fp32 (all device pointers, 16-byte aligned). */
gdn_status_t gdn_in_proj(const gdn_layer_t *L, const void *x, const void *w_in, void *q, void *k, void *v,
                         float *beta, float *g, void *hip_stream);
/* o [B, T, H 112] bf16, w_out [H 112, H 112] bf16 -> y [B, T, H 112] (y_dtype). */
gdn_status_t gdn_out_proj(const gdn_layer_t *L, const void *o, const void *w_out, void *y, void *hip_stream);
/* The whole layer: in-projection, scan, out-projection.  state_in / state_out
 * as in gdn_fwd (both NULL for the bidirectional layer).  Workspace: q, k, v,
 * beta, g and o of the layer plus the scan's own (gdn_layer_workspace_bytes). */
gdn_status_t gdn_layer_workspace_bytes(const gdn_layer_t *L, size_t *bytes);
gdn_status_t gdn_layer_fwd(const gdn_layer_t *L, const void *x, const void *w_in, const void *w_out,
                           const float *state_in, float *state_out, void *y, void *workspace,
                           size_t workspace_bytes, void *hip_stream);

/* Where the intermediates live inside the workspace (byte offsets; 0 = not
 * used by the selected kernels).  For tests and profiling. */
typedef struct {
    size_t beta, rq, rk, gcum; /* fp32 kernels: fp32 [B, H, T] each: sigmoid(beta), 1/||q||,
                                  1/||k||, chunk-local inclusive cumsum of the floored g */
    size_t rec;                /* MFMA kernels: a ring of two slots, each range_cap x B*H
                                  chunk-head records of rec_bytes, in the state pass's operand
                                  fragment order: K~ = -diag(beta gamma / ||k||) K (fp16,
                                  17,920 B), Q' = diag(gamma / ||q||) Q + P' K~ (fp16, 17,920 B),
                                  P'' = P T diag(beta) as a bf16 hi and a bf16 lo part (7,680 B
                                  each), 128 fp32 chunk scalars (beta[80], gamma_n), and
                                  M = K^T diag(s) T (fp16, 17,920 B).  The chunks run in ranges
                                  of first_range, then range_cap chunks; range j's records sit
                                  in slot j % 2, record (chunk c, unit b*H + h) at index
                                  (c - range start) * B*H + b*H + h.  After a call, the last two
                                  ranges' records remain. */
    size_t rec_bytes;          /* 69,632 */
    size_t carry;              /* MFMA kernels: fp32 [B, H, d_v, d_k] state between ranges */
    int32_t range_cap, first_range;
    size_t total;              /* == gdn_workspace_bytes */
    int32_t mfma;              /* 1 = MFMA kernels selected, 0 = fp32 kernels */
} gdn_workspace_layout_t;
gdn_status_t gdn_workspace_layout(const gdn_problem_t *p, gdn_workspace_layout_t *layout);

const char *gdn_status_string(gdn_status_t s);
const char *gdn_last_error(void); /* thread-local detail of the last failing call */
int32_t gdn_version(void);        /* GDN_ABI_VERSION */

#ifdef __cplusplus
}
#endif

#endif /* SANAWM_GDN_H */
