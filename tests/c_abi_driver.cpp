// A plain C++ user of libsanawm_gdn: device memory from hipMalloc, no torch.
// It runs gdn_fwd, and the same sequence as gdn_chunk_step calls with the state
// carried between them, on inputs read from a file, and writes the outputs for
// tests/test_gpu_c_abi.py to check.
//
//   c_abi_driver IN OUT
//
// IN : int32 B, T, H, D, chunk_tokens; then bf16 q, k, v [B,T,H,D];
//      fp32 g, beta [B,T,H]; fp32 state_in [B,H,D,D]
// OUT: fp32 o [B,T,H,D] and state [B,H,D,D] of gdn_fwd, then o and state of the
//      chunk_step rollout (calls of chunk_tokens tokens)
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "sanawm_gdn.h"

namespace {

void die(const char *what) {
  std::fprintf(stderr, "c_abi_driver: %s\n", what);
  std::exit(1);
}
void hip_ok(hipError_t e, const char *what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "c_abi_driver: %s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}
void gdn_ok(gdn_status_t s, const char *what) {
  if (s != GDN_OK) {
    std::fprintf(stderr, "c_abi_driver: %s: %s: %s\n", what, gdn_status_string(s), gdn_last_error());
    std::exit(1);
  }
}
template <typename T>
void read_n(FILE *f, std::vector<T> &v, size_t n) {
  v.resize(n);
  if (std::fread(v.data(), sizeof(T), n, f) != n) die("short input file");
}
template <typename T>
T *to_device(const std::vector<T> &h) {
  void *d = nullptr;
  hip_ok(hipMalloc(&d, h.size() * sizeof(T) + 16), "hipMalloc");
  hip_ok(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy in");
  return static_cast<T *>(d);
}
template <typename T>
void write_back(FILE *f, const T *d, size_t n) {
  std::vector<T> h(n);
  hip_ok(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost), "hipMemcpy out");
  if (std::fwrite(h.data(), sizeof(T), n, f) != n) die("short write");
}

}  // namespace

int main(int argc, char **argv) {
  if (argc != 3) die("usage: c_abi_driver IN OUT");
  FILE *in = std::fopen(argv[1], "rb");
  if (!in) die("cannot open the input file");
  int32_t hdr[5];
  if (std::fread(hdr, sizeof(int32_t), 5, in) != 5) die("short header");
  const int B = hdr[0], T = hdr[1], H = hdr[2], D = hdr[3], Tc = hdr[4];
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || Tc <= 0 || T % Tc) die("bad header");
  const size_t nx = size_t(B) * T * H * D, ns = size_t(B) * T * H, nst = size_t(B) * H * D * D;
  std::vector<uint16_t> q, k, v;
  std::vector<float> g, beta, s0;
  read_n(in, q, nx);
  read_n(in, k, nx);
  read_n(in, v, nx);
  read_n(in, g, ns);
  read_n(in, beta, ns);
  read_n(in, s0, nst);
  std::fclose(in);

  uint16_t *dq = to_device(q), *dk = to_device(k), *dv = to_device(v);
  float *dg = to_device(g), *db = to_device(beta), *ds0 = to_device(s0);
  float *o = nullptr, *st = nullptr;
  hip_ok(hipMalloc(reinterpret_cast<void **>(&o), nx * sizeof(float)), "hipMalloc o");
  hip_ok(hipMalloc(reinterpret_cast<void **>(&st), nst * sizeof(float)), "hipMalloc state");
  hipStream_t stream;
  hip_ok(hipStreamCreate(&stream), "hipStreamCreate");

  // one pass
  gdn_problem_t p{B, T, H, D, D, GDN_BF16, GDN_F32, 0u};
  size_t ws_bytes = 0;
  gdn_ok(gdn_workspace_bytes(&p, &ws_bytes), "gdn_workspace_bytes");
  void *ws = nullptr;
  hip_ok(hipMalloc(&ws, ws_bytes ? ws_bytes : 1), "hipMalloc workspace");
  gdn_ok(gdn_fwd(&p, dq, dk, dv, dg, db, ds0, st, o, ws, ws_bytes, stream), "gdn_fwd");
  hip_ok(hipStreamSynchronize(stream), "sync");
  FILE *out = std::fopen(argv[2], "wb");
  if (!out) die("cannot open the output file");
  write_back(out, o, nx);
  write_back(out, st, nst);

  // the same sequence as streaming calls of Tc tokens, the state carried in place
  // (B = 1: a call's tokens are a contiguous slice of every array)
  if (B != 1) die("the rollout takes B = 1");
  gdn_problem_t pc{1, Tc, H, D, D, GDN_BF16, GDN_F32, 0u};
  size_t wsc_bytes = 0;
  gdn_ok(gdn_workspace_bytes(&pc, &wsc_bytes), "gdn_workspace_bytes (call)");
  void *wsc = nullptr;
  hip_ok(hipMalloc(&wsc, wsc_bytes ? wsc_bytes : 1), "hipMalloc call workspace");
  hip_ok(hipMemcpy(st, ds0, nst * sizeof(float), hipMemcpyDeviceToDevice), "state copy");
  for (int t0 = 0; t0 < T; t0 += Tc) {
    const size_t x0 = size_t(t0) * H * D, s0_ = size_t(t0) * H;
    gdn_ok(gdn_chunk_step(&pc, dq + x0, dk + x0, dv + x0, dg + s0_, db + s0_, st, st, o + x0, wsc, wsc_bytes,
                          stream),
           "gdn_chunk_step");
  }
  hip_ok(hipStreamSynchronize(stream), "sync");
  write_back(out, o, nx);
  write_back(out, st, nst);
  std::fclose(out);
  std::printf("c_abi_driver: ok (B=%d T=%d H=%d D=%d, %d calls)\n", B, T, H, D, T / Tc);
  return 0;
}
