// Host front-end of libsanawm_gdn: the C ABI declared in include/sanawm_gdn.h.
//
// Every check runs on the host before the first launch; the functions only
// enqueue work on the caller's stream and never synchronise, allocate or free
// device memory.
#include "sanawm_gdn.h"
#include "sanawm_attn.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <limits>
#include <mutex>
#include <vector>

#include "gdn_internal.h"

namespace {

thread_local char g_last_error[512] = "";

gdn_status_t fail(gdn_status_t s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool mul_ok(size_t a, size_t b, size_t *out) {
  if (a != 0 && b > std::numeric_limits<size_t>::max() / a) return false;
  *out = a * b;
  return true;
}

// Validates the problem descriptor and lays out the workspace.  `ws_limit`:
// the most workspace the caller can offer (the MFMA path then shortens its
// chunk ranges to fit; every other path needs its full size).
gdn_status_t make_plan(const gdn_problem_t *p, gdn::Plan *pl, size_t ws_limit = SIZE_MAX) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "problem descriptor is NULL");
  if (p->batch < 1 || p->num_heads < 1 || p->seq_len < 0 || p->head_dim_k < 1 || p->head_dim_v < 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "bad shape: batch=%d seq_len=%d heads=%d d_k=%d d_v=%d", p->batch,
                p->seq_len, p->num_heads, p->head_dim_k, p->head_dim_v);
  if ((p->qkv_dtype != GDN_F32 && p->qkv_dtype != GDN_BF16 && p->qkv_dtype != GDN_FP8_E4M3) ||
      (p->o_dtype != GDN_F32 && p->o_dtype != GDN_BF16))
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown dtype (qkv=%d, o=%d)", p->qkv_dtype, p->o_dtype);
  const uint32_t known = GDN_FLAG_BETA_IS_PROB | GDN_FLAG_QK_PRENORMALIZED | GDN_FLAG_REVERSE;
  if (p->flags & ~known) return fail(GDN_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", p->flags & ~known);

  gdn::Plan P;
  P.B = p->batch;
  P.T = p->seq_len;
  P.H = p->num_heads;
  P.dk = p->head_dim_k;
  P.dv = p->head_dim_v;
  P.N = (P.T + gdn::kChunk - 1) / gdn::kChunk;
  P.qkv_bf16 = p->qkv_dtype == GDN_BF16;
  P.qkv_fp8 = p->qkv_dtype == GDN_FP8_E4M3;
  P.o_bf16 = p->o_dtype == GDN_BF16;
  P.flags = p->flags;
  P.mfma = gdn::kHaveMfmaPath && (P.qkv_bf16 || P.qkv_fp8);
  if (P.mfma) {
    if (P.dk != gdn::kMfmaDim || P.dv != gdn::kMfmaDim)
      return fail(GDN_ERR_UNSUPPORTED, "the MFMA kernels need d_k = d_v = %d (got %d, %d)", gdn::kMfmaDim, P.dk,
                  P.dv);
    // one chunk of rows of o (fp32) must stay addressable by a 31-bit buffer offset
    if (size_t(gdn::kChunk) * P.H * gdn::kMfmaDim * sizeof(float) >= (size_t(1) << 31))
      return fail(GDN_ERR_UNSUPPORTED, "too many heads for the MFMA kernels (%d)", P.H);
  } else if (P.dk > gdn::kMaxPortableDim || P.dv > gdn::kMaxPortableDim) {
    return fail(GDN_ERR_UNSUPPORTED, "portable kernels take d_k, d_v <= %d (got %d, %d)", gdn::kMaxPortableDim,
                P.dk, P.dv);
  }
  // grid sizes are 1-D: keep every block count and index product far from overflow
  const size_t units = size_t(P.B) * size_t(P.H);
  if (units * size_t(P.N) > (size_t(1) << 31) - 1 || units > (size_t(1) << 24))
    return fail(GDN_ERR_UNSUPPORTED, "problem too large (B*H*ceil(T/%d) = %zu)", gdn::kChunk, units * P.N);

  size_t off = 0, sz = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  size_t bht;
  if (!mul_ok(units, size_t(P.T), &bht) || !mul_ok(bht, sizeof(float), &sz))
    return fail(GDN_ERR_UNSUPPORTED, "problem too large");
  const size_t chunks = units * size_t(P.N);
  if (P.mfma) {  // the MFMA path computes its per-token scalars inside the intra-chunk step
    P.range_cap = std::max(1, std::min(P.N, gdn::kRangeCap));
    if (ws_limit != SIZE_MAX) {  // two record slots of range_cap chunks per unit, then the carried state
      const size_t carry = align_up(units * size_t(P.dv) * P.dk * sizeof(float));
      const size_t per_chunk = 2 * units * gdn::mfma_record_bytes();
      const size_t fit = ws_limit > carry ? (ws_limit - carry) / per_chunk : 0;
      if (fit < 1)
        return fail(GDN_ERR_WORKSPACE, "B*H = %zu needs at least %zu bytes of workspace, more than the %zu "
                    "available", units, carry + per_chunk, ws_limit);
      P.range_cap = int(std::min<size_t>(size_t(P.range_cap), fit));
    }
    P.off_rec = take(2 * size_t(P.range_cap) * units * gdn::mfma_record_bytes());
    P.off_carry = take(units * size_t(P.dv) * P.dk * sizeof(float));
  } else {
    P.off_beta = take(sz);
    P.off_rq = take(sz);
    P.off_rk = take(sz);
    P.off_gcum = take(sz);
    const size_t rowsk = chunks * gdn::kChunk * size_t(P.dk) * sizeof(float);
    const size_t rowsv = chunks * gdn::kChunk * size_t(P.dv) * sizeof(float);
    P.off_W = take(rowsk);
    P.off_Ut = take(rowsv);
    P.off_U = take(rowsv);
    P.off_S0 = take(chunks * size_t(P.dv) * P.dk * sizeof(float));
  }
  P.total = P.T == 0 ? 0 : off;
  if (P.total > ws_limit)
    return fail(GDN_ERR_WORKSPACE, "the problem needs %zu bytes of workspace, more than the %zu available", P.total,
                ws_limit);
  *pl = P;
  return GDN_OK;
}

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// The launch sequence of one validated scan.
hipError_t enqueue(const gdn::Plan &P, const gdn::Args &a) {
  if (P.T == 0) return gdn::launch_state_passthrough(P, a);
  if (P.mfma) return gdn::launch_mfma(P, a);
  hipError_t e = gdn::launch_prep(P, a);
  if (e == hipSuccess) e = gdn::launch_portable(P, a);
  return e;
}

gdn_status_t run(const gdn_problem_t *p, const void *q, const void *k, const void *v, const float *g,
                 const float *beta, const float *state_in, float *state_out, void *o, void *workspace,
                 size_t workspace_bytes, void *hip_stream, bool chunk_step, size_t ws_limit = SIZE_MAX) {
  gdn::Plan P;
  gdn_status_t s = make_plan(p, &P, ws_limit);
  if (s != GDN_OK) return s;
  if (chunk_step) {
    if (P.flags & GDN_FLAG_REVERSE)
      return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_chunk_step takes no REVERSE flag (the reverse scan needs the "
                  "next call's first decay)");
    if (!state_in) return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_chunk_step needs a non-NULL state_in");
    if (P.T % gdn::kChunk)
      return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_chunk_step needs seq_len %% %d == 0 (got %d)", gdn::kChunk, P.T);
  }
  const struct {
    const void *ptr;
    const char *name;
  } need[] = {{q, "q"}, {k, "k"}, {v, "v"}, {g, "g"}, {beta, "beta"}, {o, "o"}};
  if (P.T > 0)
    for (const auto &n : need) {
      if (!n.ptr) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is NULL", n.name);
      if (!aligned16(n.ptr)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n.name);
    }
  if (state_in && !aligned16(state_in)) return fail(GDN_ERR_INVALID_ARGUMENT, "state_in is not 16-byte aligned");
  if (state_out && !aligned16(state_out))
    return fail(GDN_ERR_INVALID_ARGUMENT, "state_out is not 16-byte aligned");
  if (P.total > 0) {
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", P.total);
    if (workspace_bytes < P.total)
      return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, P.total);
    if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
      return fail(GDN_ERR_INVALID_ARGUMENT, "workspace is not %zu-byte aligned", kAlign);
  }

  gdn::Args a{q,
              k,
              v,
              g,
              beta,
              state_in,
              state_out,
              o,
              static_cast<char *>(workspace),
              static_cast<hipStream_t>(hip_stream)};
  const hipError_t e = enqueue(P, a);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error[0] = '\0';
  return GDN_OK;
}

// Workspace of the bidirectional layer: one scan's workspace (the two scans
// run one after the other and share it), then the reverse scan's fp32 output
// and, for bf16 o, the forward scan's fp32 output.
struct BidirPlan {
  gdn::Plan scan;
  size_t off_rev = 0, off_fwd = 0, total = 0;
};

gdn_status_t make_bidir_plan(const gdn_problem_t *p, BidirPlan *bp) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "problem descriptor is NULL");
  if (p->flags & GDN_FLAG_REVERSE)
    return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_bidir_fwd runs both scans itself: no REVERSE flag");
  BidirPlan B;
  gdn_status_t s = make_plan(p, &B.scan);
  if (s != GDN_OK) return s;
  const gdn::Plan &P = B.scan;
  size_t n, bytes;
  if (!mul_ok(size_t(P.B) * size_t(P.H), size_t(P.T), &n) || !mul_ok(n, size_t(P.dv) * sizeof(float), &bytes))
    return fail(GDN_ERR_UNSUPPORTED, "problem too large");
  B.off_rev = align_up(P.total);
  B.off_fwd = align_up(B.off_rev + bytes);
  B.total = P.T == 0 ? 0 : (P.o_bf16 ? align_up(B.off_fwd + bytes) : B.off_fwd);
  *bp = B;
  return GDN_OK;
}

gdn_status_t run_bidir(const gdn_problem_t *p, const void *q, const void *k, const void *v, const float *g,
                       const float *beta, void *o, void *workspace, size_t workspace_bytes, void *hip_stream) {
  BidirPlan B;
  gdn_status_t s = make_bidir_plan(p, &B);
  if (s != GDN_OK) return s;
  gdn::Plan &P = B.scan;
  if (P.T == 0) {
    g_last_error[0] = '\0';
    return GDN_OK;
  }
  const struct {
    const void *ptr;
    const char *name;
  } need[] = {{q, "q"}, {k, "k"}, {v, "v"}, {g, "g"}, {beta, "beta"}, {o, "o"}};
  for (const auto &n : need) {
    if (!n.ptr) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is NULL", n.name);
    if (!aligned16(n.ptr)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n.name);
  }
  if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", B.total);
  if (workspace_bytes < B.total)
    return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, B.total);
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(GDN_ERR_INVALID_ARGUMENT, "workspace is not %zu-byte aligned", kAlign);

  char *ws = static_cast<char *>(workspace);
  const bool o_bf16 = P.o_bf16;
  float *rev_o = reinterpret_cast<float *>(ws + B.off_rev);
  float *fwd_o = o_bf16 ? reinterpret_cast<float *>(ws + B.off_fwd) : static_cast<float *>(o);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  // both scans write fp32; the combine kernel writes o in its own type
  P.o_bf16 = 0;
  gdn::Args a{q, k, v, g, beta, nullptr, nullptr, fwd_o, ws, st};
  gdn::Plan R = P;
  R.flags |= GDN_FLAG_REVERSE;
  hipError_t e = enqueue(P, a);
  if (e == hipSuccess) {
    a.o = rev_o;
    e = enqueue(R, a);
  }
  if (e == hipSuccess) e = gdn::launch_combine(fwd_o, rev_o, o, o_bf16, size_t(P.B) * P.T * P.H * P.dv, st);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error[0] = '\0';
  return GDN_OK;
}

// ---- the workspace of gdn_fwd_no_alloc ----
// One fixed array per device in the library's code object, allocated when the
// code object is loaded on that device and held until the process ends.  Its
// device address comes from hipGetSymbolAddress, once per device: the name
// `scratch` in host code is only a host-side stand-in.  Nothing in it needs to
// start at zero (every kernel writes what it later reads), and calls that
// overlap on one device race on it.
static __device__ __align__(256) unsigned char scratch[GDN_NO_ALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, which must be the device
// of `hip_stream`.
gdn_status_t scratch_address(void *hip_stream, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  if (hip_stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(hip_stream), &sdev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (int(sdev) != dev)
      return fail(GDN_ERR_INVALID_ARGUMENT, "the stream belongs to device %d, the current device is %d", int(sdev),
                  dev);
  }
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(GDN_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" {

int32_t gdn_chunk_len(void) { return gdn::kChunk; }

int32_t gdn_version(void) { return GDN_ABI_VERSION; }

gdn_status_t gdn_workspace_bytes(const gdn_problem_t *p, size_t *bytes) {
  if (!bytes) return fail(GDN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  gdn::Plan P;
  gdn_status_t s = make_plan(p, &P);
  if (s == GDN_OK) *bytes = P.total;
  return s;
}

gdn_status_t gdn_workspace_layout(const gdn_problem_t *p, gdn_workspace_layout_t *layout) {
  if (!layout) return fail(GDN_ERR_INVALID_ARGUMENT, "layout is NULL");
  gdn::Plan P;
  gdn_status_t s = make_plan(p, &P);
  if (s != GDN_OK) return s;
  std::memset(layout, 0, sizeof(*layout));
  layout->beta = P.mfma ? 0 : P.off_beta;
  layout->rq = P.mfma ? 0 : P.off_rq;
  layout->rk = P.mfma ? 0 : P.off_rk;
  layout->gcum = P.mfma ? 0 : P.off_gcum;
  layout->rec = P.mfma ? P.off_rec : 0;
  layout->rec_bytes = P.mfma ? gdn::mfma_record_bytes() : 0;
  layout->carry = P.mfma ? P.off_carry : 0;
  layout->range_cap = P.mfma ? P.range_cap : 0;
  layout->first_range = P.mfma ? std::min(P.N, std::min(gdn::kFirstRange, P.range_cap)) : 0;
  layout->total = P.total;
  layout->mfma = P.mfma ? 1 : 0;
  return GDN_OK;
}

gdn_status_t gdn_fwd(const gdn_problem_t *p, const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const float *state_in, float *state_out, void *o, void *workspace,
                     size_t workspace_bytes, void *hip_stream) {
  return run(p, q, k, v, g, beta, state_in, state_out, o, workspace, workspace_bytes, hip_stream, false);
}

gdn_status_t gdn_chunk_step(const gdn_problem_t *p, const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *state_in, float *state_out, void *o,
                            void *workspace, size_t workspace_bytes, void *hip_stream) {
  return run(p, q, k, v, g, beta, state_in, state_out, o, workspace, workspace_bytes, hip_stream, true);
}

gdn_status_t gdn_fwd_no_alloc(const gdn_problem_t *p, const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const float *state_in, float *state_out, void *o,
                              void *hip_stream) {
  constexpr size_t kBytes = GDN_NO_ALLOC_SCRATCH_BYTES;
  gdn::Plan P;
  gdn_status_t s = make_plan(p, &P, kBytes);  // size checks before any HIP call
  if (s != GDN_OK) return s;
  void *ws = nullptr;
  s = scratch_address(hip_stream, &ws);
  if (s != GDN_OK) return s;
  return run(p, q, k, v, g, beta, state_in, state_out, o, ws, kBytes, hip_stream, false, kBytes);
}

// ---- the layer around the scan ----
namespace {

struct LayerPlan {
  gdn_problem_t scan;  // the inner scan: bf16 q, k, v and o, d = 112
  int M = 0, H = 0, HD = 0;
  bool bidir = false, y_bf16 = false;
  size_t off_q = 0, off_k = 0, off_v = 0, off_beta = 0, off_g = 0, off_o = 0, off_scan = 0, total = 0;
};

gdn_status_t make_layer_plan(const gdn_layer_t *L, LayerPlan *lp) {
  if (!L) return fail(GDN_ERR_INVALID_ARGUMENT, "layer descriptor is NULL");
  if (L->batch < 1 || L->seq_len < 0 || L->num_heads < 1 || L->frame_tokens < 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "bad layer shape: batch=%d seq_len=%d heads=%d frame_tokens=%d",
                L->batch, L->seq_len, L->num_heads, L->frame_tokens);
  if (L->y_dtype != GDN_F32 && L->y_dtype != GDN_BF16)
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown y dtype %d", L->y_dtype);
  if (L->flags & ~uint32_t(GDN_LAYER_BIDIRECTIONAL))
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown layer flag bits 0x%x", L->flags & ~uint32_t(GDN_LAYER_BIDIRECTIONAL));
  LayerPlan P;
  P.H = L->num_heads;
  P.HD = P.H * gdn::kMfmaDim;
  P.bidir = L->flags & GDN_LAYER_BIDIRECTIONAL;
  P.y_bf16 = L->y_dtype == GDN_BF16;
  const long long M = (long long)L->batch * L->seq_len;
  // token and column indices of the projection kernels are 32-bit
  if (M > (1LL << 30) || P.HD > 65536)
    return fail(GDN_ERR_UNSUPPORTED, "layer too large (tokens %lld, heads %d)", M, P.H);
  P.M = int(M);
  P.scan = gdn_problem_t{L->batch, L->seq_len, L->num_heads, gdn::kMfmaDim, gdn::kMfmaDim, GDN_BF16, GDN_BF16, 0u};
  size_t scan_bytes = 0;
  BidirPlan Bp;
  gdn::Plan Sp;
  gdn_status_t s = P.bidir ? make_bidir_plan(&P.scan, &Bp) : make_plan(&P.scan, &Sp);
  if (s != GDN_OK) return s;
  scan_bytes = P.bidir ? Bp.total : Sp.total;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t rows = size_t(M) * P.HD * 2, scal = size_t(M) * P.H * 4;
  P.off_q = take(rows);
  P.off_k = take(rows);
  P.off_v = take(rows);
  P.off_beta = take(scal);
  P.off_g = take(scal);
  P.off_o = take(rows);
  P.off_scan = take(scan_bytes);
  P.total = M == 0 ? 0 : off;
  *lp = P;
  return GDN_OK;
}

}  // namespace

gdn_status_t gdn_layer_workspace_bytes(const gdn_layer_t *L, size_t *bytes) {
  if (!bytes) return fail(GDN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  LayerPlan P;
  gdn_status_t s = make_layer_plan(L, &P);
  if (s == GDN_OK) *bytes = P.total;
  return s;
}

gdn_status_t gdn_in_proj(const gdn_layer_t *L, const void *x, const void *w_in, void *q, void *k, void *v,
                         float *beta, float *g, void *hip_stream) {
  LayerPlan P;
  gdn_status_t s = make_layer_plan(L, &P);
  if (s != GDN_OK) return s;
  if (P.M == 0) return GDN_OK;
  const struct {
    const void *ptr;
    const char *name;
  } need[] = {{x, "x"}, {w_in, "w_in"}, {q, "q"}, {k, "k"}, {v, "v"}, {beta, "beta"}, {g, "g"}};
  for (const auto &n : need) {
    if (!n.ptr) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is NULL", n.name);
    if (!aligned16(n.ptr)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n.name);
  }
  gdn::Args a{};
  a.stream = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = gdn::proj::launch_in_proj(
      static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w_in), P.M, P.H, L->seq_len, L->frame_tokens,
      static_cast<uint16_t *>(q), static_cast<uint16_t *>(k), static_cast<uint16_t *>(v), beta, g, a.stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error[0] = '\0';
  return GDN_OK;
}

gdn_status_t gdn_out_proj(const gdn_layer_t *L, const void *o, const void *w_out, void *y, void *hip_stream) {
  LayerPlan P;
  gdn_status_t s = make_layer_plan(L, &P);
  if (s != GDN_OK) return s;
  if (P.M == 0) return GDN_OK;
  const struct {
    const void *ptr;
    const char *name;
  } need[] = {{o, "o"}, {w_out, "w_out"}, {y, "y"}};
  for (const auto &n : need) {
    if (!n.ptr) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is NULL", n.name);
    if (!aligned16(n.ptr)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n.name);
  }
  gdn::Args a{};
  a.stream = static_cast<hipStream_t>(hip_stream);
  const hipError_t e = gdn::proj::launch_out_proj(static_cast<const uint16_t *>(o),
                                                  static_cast<const uint16_t *>(w_out), P.M, P.HD, y, P.y_bf16,
                                                  a.stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_error[0] = '\0';
  return GDN_OK;
}

gdn_status_t gdn_layer_fwd(const gdn_layer_t *L, const void *x, const void *w_in, const void *w_out,
                           const float *state_in, float *state_out, void *y, void *workspace, size_t workspace_bytes,
                           void *hip_stream) {
  LayerPlan P;
  gdn_status_t s = make_layer_plan(L, &P);
  if (s != GDN_OK) return s;
  if (P.bidir && (state_in || state_out))
    return fail(GDN_ERR_INVALID_ARGUMENT, "the bidirectional layer takes no state_in / state_out");
  if (P.M == 0) {  // no tokens: the state passes through
    if (P.bidir) return GDN_OK;
    return run(&P.scan, nullptr, nullptr, nullptr, nullptr, nullptr, state_in, state_out, nullptr, nullptr, 0,
               hip_stream, false);
  }
  const struct {
    const void *ptr;
    const char *name;
  } need[] = {{x, "x"}, {w_in, "w_in"}, {w_out, "w_out"}, {y, "y"}};
  for (const auto &n : need) {
    if (!n.ptr) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is NULL", n.name);
    if (!aligned16(n.ptr)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n.name);
  }
  if (state_in && !aligned16(state_in)) return fail(GDN_ERR_INVALID_ARGUMENT, "state_in is not 16-byte aligned");
  if (state_out && !aligned16(state_out))
    return fail(GDN_ERR_INVALID_ARGUMENT, "state_out is not 16-byte aligned");
  if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", P.total);
  if (workspace_bytes < P.total)
    return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes, P.total);
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(GDN_ERR_INVALID_ARGUMENT, "workspace is not %zu-byte aligned", kAlign);
  char *ws = static_cast<char *>(workspace);
  void *q = ws + P.off_q, *k = ws + P.off_k, *v = ws + P.off_v, *o = ws + P.off_o;
  float *beta = reinterpret_cast<float *>(ws + P.off_beta), *g = reinterpret_cast<float *>(ws + P.off_g);
  if ((s = gdn_in_proj(L, x, w_in, q, k, v, beta, g, hip_stream)) != GDN_OK) return s;
  const size_t scan_ws = P.total - P.off_scan;
  s = P.bidir ? run_bidir(&P.scan, q, k, v, g, beta, o, ws + P.off_scan, scan_ws, hip_stream)
              : run(&P.scan, q, k, v, g, beta, state_in, state_out, o, ws + P.off_scan, scan_ws, hip_stream, false);
  if (s != GDN_OK) return s;
  return gdn_out_proj(L, o, w_out, y, hip_stream);
}

gdn_status_t gdn_bidir_workspace_bytes(const gdn_problem_t *p, size_t *bytes) {
  if (!bytes) return fail(GDN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  BidirPlan B;
  gdn_status_t s = make_bidir_plan(p, &B);
  if (s == GDN_OK) *bytes = B.total;
  return s;
}

gdn_status_t gdn_bidir_fwd(const gdn_problem_t *p, const void *q, const void *k, const void *v, const float *g,
                           const float *beta, void *o, void *workspace, size_t workspace_bytes, void *hip_stream) {
  return run_bidir(p, q, k, v, g, beta, o, workspace, workspace_bytes, hip_stream);
}

const char *gdn_status_string(gdn_status_t s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    case GDN_ERR_INTERNAL: return "GDN_ERR_INTERNAL";
  }
  return "GDN_ERR_UNKNOWN";
}

const char *gdn_last_error(void) { return g_last_error; }

// ---- streaming attention block (include/sanawm_attn.h) ----
static gdn_status_t attn_plan(const attn_problem_t *p, gdn::AttnPlan &P) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "problem descriptor is NULL");
  if (p->batch < 1 || p->num_heads < 1 || p->frame_tokens < 1 || p->frames_per_block < 1 || p->cached_blocks < 0 ||
      p->sink_frames < 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "bad stream geometry: batch=%d heads=%d frame_tokens=%d "
                "frames_per_block=%d cached_blocks=%d sink_frames=%d", p->batch, p->num_heads, p->frame_tokens,
                p->frames_per_block, p->cached_blocks, p->sink_frames);
  if (p->o_dtype != GDN_F32 && p->o_dtype != GDN_BF16)
    return fail(GDN_ERR_INVALID_ARGUMENT, "unknown output dtype %d", p->o_dtype);
  if (p->head_dim != gdn::kMfmaDim)
    return fail(GDN_ERR_UNSUPPORTED, "the attention block takes head_dim %d (got %d)", gdn::kMfmaDim, p->head_dim);
  const long long lb = (long long)p->frame_tokens * p->frames_per_block;
  const long long ls = (long long)p->frame_tokens * p->sink_frames;
  const long long keys = ls + (long long)(p->cached_blocks + 1) * lb;
  const long long ls_pad = (ls + 63) / 64 * 64, lb_pad = (lb + 63) / 64 * 64;
  const long long slice = 224 * (keys + ls_pad + (long long)(p->cached_blocks + 1) * lb_pad);
  const long long rowbytes = (long long)p->num_heads * p->head_dim * 4;
  // buffer offsets inside the kernels are 32-bit: per (b, h) cache slice, per-batch q and o
  if (slice >= (1LL << 31) || lb * rowbytes >= (1LL << 31) || (long long)p->batch * p->num_heads > (1 << 24))
    return fail(GDN_ERR_UNSUPPORTED, "attention block too large (block tokens %lld, cached keys %lld)", lb, keys);
  P.B = p->batch;
  P.H = p->num_heads;
  P.ft = p->frame_tokens;
  P.fpb = p->frames_per_block;
  P.C = p->cached_blocks;
  P.S = p->sink_frames;
  P.Lb = int(lb);
  P.Ls = int(ls);
  P.total_keys = int(keys);
  P.Ls_pad = int(ls_pad);
  P.Lb_pad = int(lb_pad);
  P.vt0 = size_t(keys) * 224;
  P.bh_bytes = align_up(size_t(slice));
  P.o_bf16 = p->o_dtype == GDN_BF16;
  return GDN_OK;
}

gdn_status_t attn_cache_bytes(const attn_problem_t *p, size_t *bytes) {
  if (!bytes) return fail(GDN_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = 0;
  gdn::AttnPlan P;
  const gdn_status_t st = attn_plan(p, P);
  if (st != GDN_OK) return st;
  size_t total;
  if (!mul_ok(size_t(P.B) * size_t(P.H), P.bh_bytes, &total)) return fail(GDN_ERR_UNSUPPORTED, "cache too large");
  *bytes = total;
  return GDN_OK;
}

gdn_status_t attn_block_fwd(const attn_problem_t *p, int32_t block, const void *q, const void *k, const void *v,
                            void *cache, size_t cache_bytes, void *o, void *hip_stream) {
  gdn::AttnPlan P;
  gdn_status_t st = attn_plan(p, P);
  if (st != GDN_OK) return st;
  if (block < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "block index %d is negative", block);
  if ((long long)block * P.Lb >= (1LL << 31))
    return fail(GDN_ERR_UNSUPPORTED, "block index %d too large", block);
  const struct {
    const void *ptr;
    const char *name;
  } need[] = {{q, "q"}, {k, "k"}, {v, "v"}, {o, "o"}, {cache, "cache"}};
  for (const auto &n : need) {
    if (!n.ptr) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is NULL", n.name);
    if (reinterpret_cast<uintptr_t>(n.ptr) % 16) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", n.name);
  }
  if (reinterpret_cast<uintptr_t>(cache) % kAlign)
    return fail(GDN_ERR_INVALID_ARGUMENT, "cache is not %zu-byte aligned", kAlign);
  size_t need_bytes = 0;
  if ((st = attn_cache_bytes(p, &need_bytes)) != GDN_OK) return st;
  if (cache_bytes < need_bytes)
    return fail(GDN_ERR_WORKSPACE, "cache too small: %zu < %zu bytes", cache_bytes, need_bytes);
  const hipError_t e = gdn::attn::launch_attn(P, block, q, k, v, cache, o, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return GDN_OK;
}

}  // extern "C"
