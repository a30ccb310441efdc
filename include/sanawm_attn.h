/*
 * Streaming chunk-causal softmax attention block of the SANA-WM Stage-1 DiT
 * on AMD Instinct MI355X (gfx950).  Part of libsanawm_gdn; plain C ABI.
 *
 * The operation.  The DiT interleaves softmax attention blocks with its
 * Gated DeltaNet layers (SGLang-diffusion cookbook page "SANA-WM", table
 * "Architecture & components", row "Attention"; WorldFoundry guide, method
 * overview).  In streaming mode video is produced block by block with
 * chunk-causal context, a rolling KV cache of the last `cached_blocks`
 * blocks and `sink_frames` sink frames (cookbook, "Configuration reference":
 * num_frame_per_block 3, num_cached_blocks 2, sink_size 1).  For block n,
 * per batch row b and head h,
 *
 *     o_t = sum_j softmax_j(q_t . k_j / sqrt(d)) v_j
 *
 * over the keys j of the context frames: the frames of blocks
 * max(0, n - cached_blocks) .. n (the current block included) and the first
 * `sink_frames` frames of the stream, each frame once.  Readings where the
 * pages are silent: the 1/sqrt(d) scale; no bias or mask inside the context;
 * q and k enter as given (positional encodings and norms belong to the
 * projections around this op); a sink frame still inside the cached window
 * is not counted twice.
 *
 * Layouts (contiguous, 16-byte aligned):
 *   q, k, v  [B, L, H, 112]  bf16, L = frames_per_block * frame_tokens
 *   o        [B, L, H, 112]  fp32 or bf16
 *   cache    attn_cache_bytes() bytes, laid out by the library: per (b, h),
 *            the keys of a sink slot (sink_frames frames) and of
 *            cached_blocks + 1 ring slots (one block each), as K rows and as
 *            V transposed.  Block n lives in ring slot n mod (cached_blocks + 1).
 *
 * Streaming contract.  attn_block_fwd(block n) first writes block n's k and
 * v into its ring slot (and its sink frames, if it holds any, into the sink
 * slot), then attends.  Blocks are called in order 0, 1, 2, ...; a block may
 * be called several times (the denoising steps of one block), each call
 * replacing the block's cached k and v, so the cache keeps what the last call
 * for a block passed (the clean pass).  Calls on one cache must be ordered on
 * one stream; the library keeps no state between calls.
 *
 * Ownership, asynchrony, errors: as in sanawm_gdn.h.  The caller owns the
 * cache and the output; the library allocates nothing and only enqueues work
 * on `hip_stream`.  Argument errors are reported before any launch.
 */
#ifndef SANAWM_ATTN_H
#define SANAWM_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include "sanawm_gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch;            /* B >= 1 */
  int32_t num_heads;        /* H >= 1 */
  int32_t head_dim;         /* must be 112 */
  int32_t frame_tokens;     /* tokens per latent frame (880 for 704 x 1280), >= 1 */
  int32_t frames_per_block; /* latent frames per streaming block (3), >= 1 */
  int32_t cached_blocks;    /* past blocks kept in the rolling cache (2), >= 0 */
  int32_t sink_frames;      /* leading frames of the stream always attended (1), >= 0 */
  int32_t o_dtype;          /* GDN_F32 or GDN_BF16 (q, k, v are bf16) */
} attn_problem_t;

/* Bytes of the KV cache for `p` (written to *bytes; 0 on error). */
gdn_status_t attn_cache_bytes(const attn_problem_t *p, size_t *bytes);

/* Stage block `block` (>= 0) into `cache` and compute its attention output
 * `o`.  q, k, v, o: device pointers with the layouts above; cache: device
 * pointer of at least attn_cache_bytes() bytes, 256-byte aligned; hip_stream:
 * a hipStream_t (NULL = default stream).  Errors: GDN_ERR_INVALID_ARGUMENT
 * (NULL or misaligned pointer, bad shape, negative block), GDN_ERR_UNSUPPORTED
 * (head_dim != 112, sizes past the 32-bit offsets used inside),
 * GDN_ERR_WORKSPACE (cache too small), GDN_ERR_HIP (launch failure). */
gdn_status_t attn_block_fwd(const attn_problem_t *p, int32_t block, const void *q, const void *k, const void *v,
                            void *cache, size_t cache_bytes, void *o, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SANAWM_ATTN_H */
