// The send path through the C ABI with nothing but the HIP runtime: device
// buffers from hipMalloc, a zero-filled workspace, the default stream, no
// PyTorch.  Reads a case file, runs counts + layout in one launch, the bf16
// permute, the weighted combine and the fp8 permute, checks that an invalid call is refused
// before anything is enqueued, and writes what the calls produced for the
// caller to compare with the CPU oracle.
//
//   epdc_c_check CASE OUT
//   CASE: int64 T, K, P, E_local, H; int64 topk_idx[T*K]; float w[T*K];
//         uint16 x[T*H] (bf16 bits)
//   OUT:  int64 N; int32 send_counts[P]; int32 token_row[T*K];
//         int32 send_token_idx[N]; uint16 send_x[N*H]; uint16 out[T*H];
//         uint8 send_q[N*H]; float send_scale[N*H/128]   (H a multiple of 128)
// It then captures the send path into a HIP graph and checks three replays
// against the eager results.  Exit status 0 on success; 1 usage or file,
// 2 HIP, 3 library status, 4 ABI version, 5 an invalid call was accepted,
// 6 a graph replay differed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "epdc.h"

#define HIP_CHECK(x)                                                            \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));             \
      return 2;                                                                 \
    }                                                                           \
  } while (0)
#define EP_CHECK(x)                                                             \
  do {                                                                          \
    int s_ = (x);                                                               \
    if (s_ != EP_OK) {                                                          \
      std::fprintf(stderr, "%s: %s\n", #x, ep_status_string(s_));              \
      return 3;                                                                 \
    }                                                                           \
  } while (0)

template <typename V>
static bool read_all(std::FILE* f, std::vector<V>& v) {
  return std::fread(v.data(), sizeof(V), v.size(), f) == v.size();
}
template <typename V>
static bool write_all(std::FILE* f, const V* p, size_t n) {
  return std::fwrite(p, sizeof(V), n, f) == n;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s CASE OUT\n", argv[0]);
    return 1;
  }
  if (ep_abi_version() != EPDC_ABI_VERSION) return 4;
  std::FILE* f = std::fopen(argv[1], "rb");
  if (!f) return 1;
  int64_t h[5];
  if (std::fread(h, sizeof(int64_t), 5, f) != 5) return 1;
  const int64_t T = h[0];
  const int K = int(h[1]), P = int(h[2]), El = int(h[3]), H = int(h[4]);
  if (T < 1 || K < 1 || P < 1 || El < 1 || H < 128 || H % 128 != 0) return 1;
  const int64_t TK = T * K, cap = T * (K < P ? K : P);
  std::vector<int64_t> idx(TK);
  std::vector<float> w(TK);
  std::vector<uint16_t> x(size_t(T) * H);
  if (!read_all(f, idx) || !read_all(f, w) || !read_all(f, x)) return 1;
  std::fclose(f);

  int64_t* d_idx;
  float *d_w, *d_sw;
  uint16_t *d_x, *d_sx, *d_out;
  uint8_t* d_q;
  float* d_qs;
  int32_t *d_dest, *d_sc, *d_tpe, *d_diag, *d_sti, *d_srk, *d_sidx, *d_trow;
  uint8_t* d_iir;
  void* d_ws;
  const size_t ws = ep_dispatch_layout_workspace_bytes(T, P, El);
  HIP_CHECK(hipMalloc(&d_idx, TK * sizeof(int64_t)));
  HIP_CHECK(hipMalloc(&d_w, TK * sizeof(float)));
  HIP_CHECK(hipMalloc(&d_x, size_t(T) * H * 2));
  HIP_CHECK(hipMalloc(&d_dest, TK * 4));
  HIP_CHECK(hipMalloc(&d_iir, size_t(T) * P));
  HIP_CHECK(hipMalloc(&d_sc, size_t(P) * 4));
  HIP_CHECK(hipMalloc(&d_tpe, size_t(P) * El * 4));
  HIP_CHECK(hipMalloc(&d_diag, 4));
  HIP_CHECK(hipMalloc(&d_sti, cap * 4));
  HIP_CHECK(hipMalloc(&d_srk, cap * 4));
  HIP_CHECK(hipMalloc(&d_sidx, cap * K * 4));
  HIP_CHECK(hipMalloc(&d_sw, cap * K * 4));
  HIP_CHECK(hipMalloc(&d_trow, TK * 4));
  HIP_CHECK(hipMalloc(&d_sx, size_t(cap) * H * 2));
  HIP_CHECK(hipMalloc(&d_out, size_t(T) * H * 2));
  HIP_CHECK(hipMalloc(&d_q, size_t(cap) * H));
  HIP_CHECK(hipMalloc(&d_qs, size_t(cap) * (H / 128) * 4));
  HIP_CHECK(hipMalloc(&d_ws, ws));
  HIP_CHECK(hipMemset(d_ws, 0, ws));
  HIP_CHECK(hipMemcpy(d_idx, idx.data(), TK * sizeof(int64_t), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_w, w.data(), TK * sizeof(float), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_x, x.data(), size_t(T) * H * 2, hipMemcpyHostToDevice));

  EP_CHECK(ep_dispatch_layout(d_idx, d_w, T, K, P, El, cap, d_dest, d_iir, d_sc, d_tpe, d_diag,
                              d_sti, d_srk, d_sidx, d_sw, d_trow, d_ws, ws, nullptr));
  EP_CHECK(ep_dispatch_permute(d_x, T, H, d_trow, K, cap, EP_DTYPE_BF16, d_sx, nullptr,
                               nullptr));
  EP_CHECK(ep_combine(d_sx, cap, d_trow, d_w, T, K, H, nullptr, nullptr, d_out, nullptr));
  EP_CHECK(ep_dispatch_permute(d_x, T, H, d_trow, K, cap, EP_DTYPE_FP8_E4M3, d_q, d_qs, nullptr));
  // refused on the host, before anything is enqueued: no output buffer
  if (ep_combine(d_sx, cap, d_trow, d_w, T, K, H, nullptr, nullptr, nullptr, nullptr) !=
      EP_ERR_INVALID_ARG)
    return 5;
  HIP_CHECK(hipDeviceSynchronize());

  std::vector<int32_t> sc(P), trow(TK), sti(cap);
  std::vector<uint16_t> sx(size_t(cap) * H), out(size_t(T) * H);
  std::vector<uint8_t> q(size_t(cap) * H);
  std::vector<float> qs(size_t(cap) * (H / 128));
  HIP_CHECK(hipMemcpy(sc.data(), d_sc, size_t(P) * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(trow.data(), d_trow, TK * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(sti.data(), d_sti, cap * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(sx.data(), d_sx, size_t(cap) * H * 2, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(out.data(), d_out, size_t(T) * H * 2, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(q.data(), d_q, q.size(), hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(qs.data(), d_qs, qs.size() * 4, hipMemcpyDeviceToHost));
  int64_t N = 0;
  for (int p = 0; p < P; ++p) N += sc[p];
  if (N > cap) return 3;

  // The same send path captured into a HIP graph on a stream of its own and
  // replayed three times; its outputs are overwritten between the replays
  // (outside the capture), and each replay must give the eager results again.
  {
    hipStream_t cs;
    hipGraph_t graph;
    hipGraphExec_t exec;
    HIP_CHECK(hipStreamCreate(&cs));
    HIP_CHECK(hipStreamBeginCapture(cs, hipStreamCaptureModeGlobal));
    int st1 = ep_dispatch_layout(d_idx, d_w, T, K, P, El, cap, d_dest, d_iir, d_sc, d_tpe, d_diag,
                                 d_sti, d_srk, d_sidx, d_sw, d_trow, d_ws, ws, cs);
    int st2 = ep_dispatch_permute(d_x, T, H, d_trow, K, cap, EP_DTYPE_BF16, d_sx, nullptr, cs);
    int st3 = ep_combine(d_sx, cap, d_trow, d_w, T, K, H, nullptr, nullptr, d_out, cs);
    HIP_CHECK(hipStreamEndCapture(cs, &graph));
    if (st1 != EP_OK || st2 != EP_OK || st3 != EP_OK) return 3;
    HIP_CHECK(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
    std::vector<int32_t> trow2(TK);
    std::vector<uint16_t> sx2(size_t(N) * H), out2(size_t(T) * H);
    for (int rep = 0; rep < 3; ++rep) {
      HIP_CHECK(hipMemset(d_trow, 0xFF, TK * 4));
      HIP_CHECK(hipMemset(d_sx, 0xFF, size_t(cap) * H * 2));
      HIP_CHECK(hipMemset(d_out, 0xFF, size_t(T) * H * 2));
      HIP_CHECK(hipDeviceSynchronize());
      HIP_CHECK(hipGraphLaunch(exec, cs));
      HIP_CHECK(hipStreamSynchronize(cs));
      HIP_CHECK(hipMemcpy(trow2.data(), d_trow, TK * 4, hipMemcpyDeviceToHost));
      HIP_CHECK(hipMemcpy(sx2.data(), d_sx, size_t(N) * H * 2, hipMemcpyDeviceToHost));
      HIP_CHECK(hipMemcpy(out2.data(), d_out, size_t(T) * H * 2, hipMemcpyDeviceToHost));
      if (trow2 != trow || !std::equal(sx2.begin(), sx2.end(), sx.begin()) || out2 != out)
        return 6;
    }
    HIP_CHECK(hipGraphExecDestroy(exec));
    HIP_CHECK(hipGraphDestroy(graph));
    HIP_CHECK(hipStreamDestroy(cs));
  }

  // The one-launch layout on the library's own scratch: the same outputs as
  // the workspace call; then neither the workspace nor that scratch reports
  // a bounded wait that gave up.
  {
    int32_t *d_trow2, *d_sti2, *d_sc2, *d_flags;
    HIP_CHECK(hipMalloc(&d_trow2, TK * 4));
    HIP_CHECK(hipMalloc(&d_sti2, cap * 4));
    HIP_CHECK(hipMalloc(&d_sc2, size_t(P) * 4));
    HIP_CHECK(hipMalloc(&d_flags, 8));
    EP_CHECK(ep_dispatch_layout_noalloc(d_idx, d_w, T, K, P, El, cap, d_dest, d_iir, d_sc2,
                                        nullptr, nullptr, d_sti2, d_srk, d_sidx, d_sw, d_trow2,
                                        nullptr));
    EP_CHECK(ep_workspace_status(d_ws, ws, d_flags, nullptr));
    EP_CHECK(ep_workspace_status(nullptr, 0, d_flags + 1, nullptr));
    HIP_CHECK(hipDeviceSynchronize());
    std::vector<int32_t> trow3(TK), sti3(static_cast<size_t>(N)), sc3(P), flags(2);
    HIP_CHECK(hipMemcpy(trow3.data(), d_trow2, TK * 4, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(sti3.data(), d_sti2, size_t(N) * 4, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(sc3.data(), d_sc2, size_t(P) * 4, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(flags.data(), d_flags, 8, hipMemcpyDeviceToHost));
    if (trow3 != trow || sc3 != sc || !std::equal(sti3.begin(), sti3.end(), sti.begin()))
      return 7;
    if (flags[0] != 0 || flags[1] != 0) return 8;
    for (void* q : {(void*)d_trow2, (void*)d_sti2, (void*)d_sc2, (void*)d_flags})
      HIP_CHECK(hipFree(q));
  }

  std::FILE* g = std::fopen(argv[2], "wb");
  if (!g) return 1;
  const bool ok = write_all(g, &N, 1) && write_all(g, sc.data(), sc.size()) &&
                  write_all(g, trow.data(), trow.size()) && write_all(g, sti.data(), size_t(N)) &&
                  write_all(g, sx.data(), size_t(N) * H) && write_all(g, out.data(), out.size()) &&
                  write_all(g, q.data(), size_t(N) * H) && write_all(g, qs.data(), size_t(N) * (H / 128));
  std::fclose(g);
  for (void* p : {(void*)d_idx, (void*)d_w, (void*)d_x, (void*)d_dest, (void*)d_iir, (void*)d_sc,
                  (void*)d_tpe, (void*)d_diag, (void*)d_sti, (void*)d_srk, (void*)d_sidx,
                  (void*)d_sw, (void*)d_trow, (void*)d_sx, (void*)d_out, (void*)d_q, (void*)d_qs,
                  d_ws})
    HIP_CHECK(hipFree(p));
  return ok ? 0 : 1;
}
