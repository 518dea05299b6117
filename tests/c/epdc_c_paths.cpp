// The rest of the C ABI with nothing but the HIP runtime (no PyTorch): the
// two-call send layout (counts, one host copy of them, the layout at its
// exact size), the counts and layouts of every chunk in one launch, the
// expert-batched layouts in bf16 and in fp8 with UE8M0 scales stored
// column-major, and the regroup by local expert of every destination segment
// of the send rows at once.  Writes what the calls produced for the caller to
// compare with the CPU oracle.
//
//   epdc_c_paths CASE OUT
//   CASE: int64 T, K, P, E_local, H, C, first_expert, E_batched, max_tokens,
//         align; int64 topk_idx[T*K]; float w[T*K]; uint16 x[T*H] (bf16
//         bits; H a multiple of 512)
//   OUT, in this order:
//     two-call layout  int32 send_counts[P], tokens_per_expert[P*E_local];
//                      int64 N; int32 send_token_idx[N], send_rank[N],
//                      send_idx[N*K]; float send_w[N*K]; int32 token_row[T*K]
//     chunked layout   int64 cap; int32 send_counts[C*P], send_token_idx[C*cap],
//                      send_rank[C*cap], send_idx[C*cap*K]; float
//                      send_w[C*cap*K]; int32 token_row[T*K]  (chunk c's rows
//                      from row c*cap; the arrays start filled with 0xFF bytes)
//     batched bf16     int32 tokens_per_expert[Eb], token_row[T*K];
//                      uint16 b_x[Eb*M*H]
//     batched fp8      int32 tokens_per_expert[Eb], token_row[T*K];
//                      uint8 b_q[Eb*M*H]; int32 b_scale[Eb*(H/512)*M]
//     regroup          int64 R; int32 tokens_per_expert[P*E_local],
//                      offsets[P*E_local+1], perm_src[R]; float perm_w[R];
//                      uint16 perm_x[R*H]; int32 row_map[N*K]
// Exit status 0 on success; 1 usage or file, 2 HIP, 3 library status,
// 4 ABI version.
#include <hip/hip_runtime.h>

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

namespace {

// Device buffers of one run, freed together.
struct Pool {
  std::vector<void*> held;
  ~Pool() {
    for (void* p : held) (void)hipFree(p);
  }
  // `bytes` of device memory (at least one byte), filled with `fill`.
  template <typename V>
  hipError_t get(V** p, size_t bytes, int fill = 0) {
    void* q = nullptr;
    hipError_t e = hipMalloc(&q, bytes ? bytes : 1);
    if (e != hipSuccess) return e;
    held.push_back(q);
    *p = static_cast<V*>(q);
    return hipMemset(q, fill, bytes ? bytes : 1);
  }
};

template <typename V>
bool read_all(std::FILE* f, std::vector<V>& v) {
  return std::fread(v.data(), sizeof(V), v.size(), f) == v.size();
}

// Copies n elements back from the device and appends them to the output.
template <typename V>
hipError_t dump(std::FILE* g, const V* d, size_t n, bool& ok) {
  if (n == 0) return hipSuccess;
  std::vector<V> h(n);
  hipError_t e = hipMemcpy(h.data(), d, n * sizeof(V), hipMemcpyDeviceToHost);
  if (e == hipSuccess) ok = ok && std::fwrite(h.data(), sizeof(V), n, g) == n;
  return e;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s CASE OUT\n", argv[0]);
    return 1;
  }
  if (ep_abi_version() != EPDC_ABI_VERSION) return 4;
  std::FILE* f = std::fopen(argv[1], "rb");
  if (!f) return 1;
  int64_t h[10];
  if (std::fread(h, sizeof(int64_t), 10, f) != 10) return 1;
  const int64_t T = h[0];
  const int K = int(h[1]), P = int(h[2]), El = int(h[3]), H = int(h[4]), C = int(h[5]);
  const int first = int(h[6]), Eb = int(h[7]), align = int(h[9]);
  const int64_t M = h[8];
  if (T < 1 || K < 1 || P < 1 || El < 1 || H < 512 || H % 512 != 0 || C < 1 || Eb < 1 ||
      M < 1 || align < 1)
    return 1;
  const int64_t TK = T * K;
  std::vector<int64_t> idx(TK);
  std::vector<float> w(TK);
  std::vector<uint16_t> x(size_t(T) * H);
  if (!read_all(f, idx) || !read_all(f, w) || !read_all(f, x)) return 1;
  std::fclose(f);
  std::FILE* g = std::fopen(argv[2], "wb");
  if (!g) return 1;
  bool ok = true;

  Pool pool;
  int64_t* d_idx;
  float* d_w;
  uint16_t* d_x;
  HIP_CHECK(pool.get(&d_idx, TK * 8));
  HIP_CHECK(pool.get(&d_w, TK * 4));
  HIP_CHECK(pool.get(&d_x, size_t(T) * H * 2));
  HIP_CHECK(hipMemcpy(d_idx, idx.data(), TK * 8, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_w, w.data(), TK * 4, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_x, x.data(), size_t(T) * H * 2, hipMemcpyHostToDevice));

  // 1. counts, their sum on the host, then the send layout at exactly N rows
  int32_t *d_dest, *d_sc, *d_tpe, *d_diag;
  uint8_t* d_iir;
  void *d_wsc, *d_wsl;
  const size_t wsc = ep_counts_workspace_bytes(T, P, El, 1);
  const size_t wsl = ep_layout_workspace_bytes(T, P);
  HIP_CHECK(pool.get(&d_dest, TK * 4));
  HIP_CHECK(pool.get(&d_iir, size_t(T) * P));
  HIP_CHECK(pool.get(&d_sc, size_t(P) * 4));
  HIP_CHECK(pool.get(&d_tpe, size_t(P) * El * 4));
  HIP_CHECK(pool.get(&d_diag, 4));
  HIP_CHECK(pool.get(&d_wsc, wsc));
  HIP_CHECK(pool.get(&d_wsl, wsl));
  EP_CHECK(ep_compute_send_counts(d_idx, T, K, P, El, 1, d_dest, d_iir, d_sc, d_tpe, d_diag,
                                  d_wsc, wsc, nullptr));
  std::vector<int32_t> sc(P);
  HIP_CHECK(hipMemcpy(sc.data(), d_sc, size_t(P) * 4, hipMemcpyDeviceToHost));
  int64_t N = 0;
  for (int p = 0; p < P; ++p) N += sc[p];
  int32_t *d_sti, *d_srk, *d_sidx, *d_trow;
  float* d_sw;
  HIP_CHECK(pool.get(&d_sti, size_t(N) * 4));
  HIP_CHECK(pool.get(&d_srk, size_t(N) * 4));
  HIP_CHECK(pool.get(&d_sidx, size_t(N) * K * 4));
  HIP_CHECK(pool.get(&d_sw, size_t(N) * K * 4));
  HIP_CHECK(pool.get(&d_trow, TK * 4));
  EP_CHECK(ep_build_send_layout(d_idx, d_w, d_dest, d_sc, T, K, P, El, N, d_sti, d_srk, d_sidx,
                                d_sw, d_trow, d_wsl, wsl, nullptr));
  HIP_CHECK(dump(g, d_sc, size_t(P), ok));
  HIP_CHECK(dump(g, d_tpe, size_t(P) * El, ok));
  ok = ok && std::fwrite(&N, 8, 1, g) == 1;
  HIP_CHECK(dump(g, d_sti, size_t(N), ok));
  HIP_CHECK(dump(g, d_srk, size_t(N), ok));
  HIP_CHECK(dump(g, d_sidx, size_t(N) * K, ok));
  HIP_CHECK(dump(g, d_sw, size_t(N) * K, ok));
  HIP_CHECK(dump(g, d_trow, size_t(TK), ok));

  // 2. every chunk's counts and layout in one launch, worst-case capacities
  {
    const int64_t last = T - (C - 1) * (T / C);          // the largest chunk
    const int64_t cap = last * (K < P ? K : P);
    const size_t ws = ep_dispatch_layout_chunked_workspace_bytes(T, P, C);
    int32_t *c_sc, *c_sti, *c_srk, *c_sidx, *c_trow;
    float* c_sw;
    void* c_ws;
    HIP_CHECK(pool.get(&c_sc, size_t(C) * P * 4));
    HIP_CHECK(pool.get(&c_sti, size_t(C * cap) * 4, 0xFF));
    HIP_CHECK(pool.get(&c_srk, size_t(C * cap) * 4, 0xFF));
    HIP_CHECK(pool.get(&c_sidx, size_t(C * cap) * K * 4, 0xFF));
    HIP_CHECK(pool.get(&c_sw, size_t(C * cap) * K * 4, 0xFF));
    HIP_CHECK(pool.get(&c_trow, TK * 4, 0xFF));
    HIP_CHECK(pool.get(&c_ws, ws));
    EP_CHECK(ep_dispatch_layout_chunked(d_idx, d_w, T, K, P, El, C, cap, d_dest, d_iir, c_sc,
                                        d_diag, c_sti, c_srk, c_sidx, c_sw, c_trow, c_ws, ws,
                                        nullptr));
    ok = ok && std::fwrite(&cap, 8, 1, g) == 1;
    HIP_CHECK(dump(g, c_sc, size_t(C) * P, ok));
    HIP_CHECK(dump(g, c_sti, size_t(C * cap), ok));
    HIP_CHECK(dump(g, c_srk, size_t(C * cap), ok));
    HIP_CHECK(dump(g, c_sidx, size_t(C * cap) * K, ok));
    HIP_CHECK(dump(g, c_sw, size_t(C * cap) * K, ok));
    HIP_CHECK(dump(g, c_trow, size_t(TK), ok));
  }

  // 3. and 4. the expert-batched layouts, one workspace for both calls (each
  //    call leaves it ready for the next)
  {
    const size_t ws = ep_batched_workspace_bytes(T, Eb, M);
    const size_t rows = size_t(Eb) * M;
    const int units = H / 512;
    int32_t *b_tpe, *b_trow, *q_tpe, *q_trow, *q_scale;
    uint16_t* b_x;
    uint8_t* q_x;
    void* b_ws;
    HIP_CHECK(pool.get(&b_tpe, size_t(Eb) * 4));
    HIP_CHECK(pool.get(&b_trow, TK * 4));
    HIP_CHECK(pool.get(&b_x, rows * H * 2, 0x5A));          // every byte is written
    HIP_CHECK(pool.get(&q_tpe, size_t(Eb) * 4));
    HIP_CHECK(pool.get(&q_trow, TK * 4));
    HIP_CHECK(pool.get(&q_x, rows * H, 0x5A));
    HIP_CHECK(pool.get(&q_scale, rows * units * 4, 0x5A));
    HIP_CHECK(pool.get(&b_ws, ws));
    EP_CHECK(ep_batched_prepare(d_x, d_idx, T, K, H, first, Eb, M, b_x, b_tpe, b_trow, b_ws, ws,
                                nullptr));
    EP_CHECK(ep_batched_prepare_fp8(d_x, d_idx, T, K, H, first, Eb, M, EP_SCALE_UE8M0, 1, q_x,
                                    q_scale, q_tpe, q_trow, b_ws, ws, nullptr));
    HIP_CHECK(dump(g, b_tpe, size_t(Eb), ok));
    HIP_CHECK(dump(g, b_trow, size_t(TK), ok));
    HIP_CHECK(dump(g, b_x, rows * H, ok));
    HIP_CHECK(dump(g, q_tpe, size_t(Eb), ok));
    HIP_CHECK(dump(g, q_trow, size_t(TK), ok));
    HIP_CHECK(dump(g, q_x, rows * H, ok));
    HIP_CHECK(dump(g, q_scale, rows * units, ok));
  }

  // 5. the send rows (bf16, N exactly), then all P destination segments
  //    regrouped by local expert: bins (destination, local expert)
  {
    const int bins = P * El;
    const int64_t cap = N * (K < El ? K : El) + int64_t(bins) * (align - 1);
    const size_t ws = ep_regroup_workspace_bytes(N, bins);
    uint16_t *r_x, *p_x;
    int32_t *p_src, *p_tpe, *p_off, *p_map;
    float* p_w;
    void* r_ws;
    HIP_CHECK(pool.get(&r_x, size_t(N) * H * 2));
    HIP_CHECK(pool.get(&p_x, size_t(cap) * H * 2));
    HIP_CHECK(pool.get(&p_src, size_t(cap) * 4));
    HIP_CHECK(pool.get(&p_w, size_t(cap) * 4));
    HIP_CHECK(pool.get(&p_tpe, size_t(bins) * 4));
    HIP_CHECK(pool.get(&p_off, size_t(bins + 1) * 4));
    HIP_CHECK(pool.get(&p_map, size_t(N) * K * 4));
    HIP_CHECK(pool.get(&r_ws, ws));
    EP_CHECK(ep_dispatch_permute(d_x, T, H, d_trow, K, N, EP_DTYPE_BF16, r_x, nullptr, nullptr));
    EP_CHECK(ep_regroup_by_expert(r_x, d_sidx, d_sw, d_srk, P, N, K, H, El, align, cap, p_x,
                                  p_src, p_w, p_tpe, p_off, p_map, r_ws, ws, nullptr));
    std::vector<int32_t> off(size_t(bins) + 1);
    HIP_CHECK(hipMemcpy(off.data(), p_off, off.size() * 4, hipMemcpyDeviceToHost));
    const int64_t R = off[bins] < cap ? off[bins] : cap;
    ok = ok && std::fwrite(&R, 8, 1, g) == 1;
    HIP_CHECK(dump(g, p_tpe, size_t(bins), ok));
    HIP_CHECK(dump(g, p_off, size_t(bins) + 1, ok));
    HIP_CHECK(dump(g, p_src, size_t(R), ok));
    HIP_CHECK(dump(g, p_w, size_t(R), ok));
    HIP_CHECK(dump(g, p_x, size_t(R) * H, ok));
    HIP_CHECK(dump(g, p_map, size_t(N) * K, ok));
  }
  HIP_CHECK(hipDeviceSynchronize());
  std::fclose(g);
  return ok ? 0 : 1;
}
