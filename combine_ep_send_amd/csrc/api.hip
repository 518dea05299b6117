// C ABI of libepdc.so: argument validation on the host, then launches.
// Nothing here allocates, frees or synchronizes.
#include <stdint.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "../../include/epdc.h"
#include "epdc_launch.h"

namespace {

using namespace epdc;

constexpr int64_t kMaxTokens = int64_t(1) << 30;   // scan values are 30-bit
constexpr int64_t kMaxExperts = 8192;              // LDS expert histogram

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int launch_status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_LAUNCH; }

// Words per whole-row access of rows of K 32-bit entries: 4 when K % 4 == 0
// and every base is 16-byte aligned, 2 when K is even and every base is
// 8-byte aligned, else 1.
int row_words(int K, std::initializer_list<const void*> bases) {
  bool a16 = true, a8 = true;
  for (const void* b : bases) {
    a16 = a16 && aligned(b, 16);
    a8 = a8 && aligned(b, 8);
  }
  return (K % 4 == 0 && a16) ? 4 : ((K % 2 == 0 && a8) ? 2 : 1);
}

// A pointer is acceptable when the array it addresses is empty or the
// pointer is non-null and aligned to `a` bytes.
bool arr_ok(const void* p, int64_t count, uintptr_t a) {
  return count == 0 || (p != nullptr && aligned(p, a));
}

int check_routing(int64_t T, int K, int P, int El) {
  if (T < 0 || K < 1 || P < 1 || El < 1) return EP_ERR_INVALID_ARG;
  if (T >= kMaxTokens || K > EPDC_MAX_TOPK) return EP_ERR_UNSUPPORTED;
  if (int64_t(P) * El > kMaxExperts) return EP_ERR_UNSUPPORTED;
  if (T * K > INT32_MAX) return EP_ERR_UNSUPPORTED;
  return EP_OK;
}

int check_hidden(int H, bool fp8) {
  if (H <= 0 || (H % 8) != 0) return EP_ERR_INVALID_ARG;
  if (fp8 && (H % EPDC_FP8_GROUP) != 0) return EP_ERR_INVALID_ARG;
  return EP_OK;
}

// Control header, published rows, per-group prefixes and bin totals of the
// fused launch, laid out as ep_*_workspace_bytes sizes them.
void set_fused_workspace(FusedArgs& a, void* ws, int64_t bins, int64_t row_words,
                         int64_t groups) {
  const int64_t gcap = a.tiles < kMaxFusedGroups ? a.tiles : kMaxFusedGroups;
  a.ctrl = static_cast<uint32_t*>(ws);
  a.rows = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kWsHeaderBytes);
  a.pref = a.rows + gcap * row_words;
  a.tots = a.pref + gcap * bins;
  a.two_pass = fused_two_pass(groups, bins, a.waves);
}

// Compute units of the current device (cached per device id; callers on
// several host threads may race to fill an entry, all with the same value).
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kMaxFusedGroups;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 1;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Shape of a fused launch over T rows: tiles, tiles per workgroup (at most
// one workgroup per compute unit, each a contiguous run of tiles), and
// whether its LDS share stays within kSmemLimit.
constexpr size_t kSmemLimit = 64 * 1024;
struct FusedShape {
  int waves;
  int64_t tiles, per, groups;
  bool fits;
};
// The library's own scratch on the current device (defined below).
int library_scratch(void** out, hipStream_t stream);

FusedShape fused_shape(int64_t T, int bins, int E, int most) {
  FusedShape f{};
  f.waves = fused_waves(T, most);
  f.tiles = fused_tiles(T, most);
  int64_t gmax = device_cus();
  if (gmax > kMaxFusedGroups) gmax = kMaxFusedGroups;
  f.per = (f.tiles + gmax - 1) / gmax;
  f.groups = (f.tiles + f.per - 1) / f.per;
  f.fits = fused_smem_bytes(bins, E, int(f.per), f.waves) <= kSmemLimit;
  return f;
}


}  // namespace

extern "C" {

int ep_abi_version(void) { return EPDC_ABI_VERSION; }

const char* ep_status_string(int status) {
  switch (status) {
    case EP_OK: return "ok";
    case EP_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size or misaligned pointer)";
    case EP_ERR_UNSUPPORTED: return "argument outside the supported limits";
    case EP_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case EP_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int ep_workspace_status(void* workspace, size_t workspace_bytes, int32_t* flags,
                        hipStream_t stream) {
  if (!flags || !aligned(flags, 4)) return EP_ERR_INVALID_ARG;
  if (!workspace) {                       // the library's own scratch on this device
    const int st = library_scratch(&workspace, stream);
    if (st != EP_OK) return st;
  } else if (!aligned(workspace, 256) || workspace_bytes < kWsHeaderBytes) {
    return EP_ERR_WORKSPACE;
  }
  return launch_status(launch_workspace_status(static_cast<uint32_t*>(workspace), flags, stream));
}

size_t ep_counts_workspace_bytes(int64_t num_tokens, int num_ranks, int num_local_experts,
                                 int num_chunks) {
  if (num_tokens < 0 || num_ranks < 1 || num_local_experts < 1 || num_chunks < 1) return 0;
  if (num_tokens >= kMaxTokens || int64_t(num_ranks) * num_local_experts > kMaxExperts) return 0;
  return count_ws_bytes(num_ranks, num_ranks * num_local_experts, num_chunks);
}

size_t ep_layout_workspace_bytes(int64_t num_tokens, int num_bins) {
  if (num_tokens < 0 || num_tokens >= kMaxTokens || num_bins < 1) return 0;
  return kWsHeaderBytes + scan_status_bytes(num_tokens, num_bins);
}

size_t ep_batched_workspace_bytes(int64_t num_tokens, int num_local_experts,
                                  int64_t max_num_tokens) {
  if (num_tokens < 0 || num_tokens >= kMaxTokens || num_local_experts < 1 || max_num_tokens < 0)
    return 0;
  return kWsHeaderBytes + scan_status_bytes(num_tokens, num_local_experts);
}

int ep_compute_send_counts(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                           int num_ranks, int num_local_experts, int num_chunks, int32_t* dest,
                           uint8_t* is_in_rank, int32_t* send_counts, int32_t* tokens_per_expert,
                           int32_t* diag, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  int st = check_routing(num_tokens, num_topk, num_ranks, num_local_experts);
  if (st != EP_OK) return st;
  if (num_ranks > EPDC_MAX_BINS) return EP_ERR_UNSUPPORTED;
  if (num_chunks < 1) return EP_ERR_INVALID_ARG;
  const int64_t TK = num_tokens * num_topk;
  if (!arr_ok(topk_idx, TK, 8) || !arr_ok(dest, TK, 4) ||
      !arr_ok(is_in_rank, num_tokens * num_ranks, 4) || !arr_ok(send_counts, 1, 4) ||
      (tokens_per_expert && !aligned(tokens_per_expert, 4)) || (diag && !aligned(diag, 4)))
    return EP_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256) ||
      workspace_bytes < ep_counts_workspace_bytes(num_tokens, num_ranks, num_local_experts,
                                                  num_chunks))
    return EP_ERR_WORKSPACE;
  CountArgs a{};
  a.topk_idx = topk_idx;
  a.T = num_tokens;
  a.K = num_topk;
  a.P = num_ranks;
  a.E_local = num_local_experts;
  a.E = num_ranks * num_local_experts;
  a.C = num_chunks;
  a.chunk = num_tokens / num_chunks;
  a.dest = dest;
  a.is_in_rank = is_in_rank;
  a.send_counts = send_counts;
  a.tokens_per_expert = tokens_per_expert;
  a.diag = diag;
  a.ctrl = static_cast<uint32_t*>(workspace);
  a.accum = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kWsHeaderBytes);
  return launch_status(launch_counts(a, stream));
}

int ep_build_send_layout(const int64_t* topk_idx, const float* topk_weights, const int32_t* dest,
                         const int32_t* send_counts, int64_t num_tokens, int num_topk,
                         int num_ranks, int num_local_experts, int64_t num_send_capacity,
                         int32_t* send_token_idx, int32_t* send_rank, int32_t* send_idx,
                         float* send_w, int32_t* token_row, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  int st = check_routing(num_tokens, num_topk, num_ranks, num_local_experts);
  if (st != EP_OK) return st;
  if (num_ranks > EPDC_MAX_BINS) return EP_ERR_UNSUPPORTED;
  if (num_send_capacity < 0) return EP_ERR_INVALID_ARG;
  if (num_send_capacity > INT32_MAX || num_send_capacity * num_topk > INT32_MAX)
    return EP_ERR_UNSUPPORTED;
  const int64_t TK = num_tokens * num_topk;
  const int64_t cap = num_send_capacity;
  if (!arr_ok(topk_idx, TK, 8) || !arr_ok(topk_weights, TK, 4) || !arr_ok(dest, TK, 4) ||
      !arr_ok(send_counts, 1, 4) || !arr_ok(token_row, TK, 4) ||
      !arr_ok(send_token_idx, cap, 4) || !arr_ok(send_rank, cap, 4) ||
      !arr_ok(send_idx, cap, 4) || !arr_ok(send_w, cap, 4))
    return EP_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256) ||
      workspace_bytes < ep_layout_workspace_bytes(num_tokens, num_ranks))
    return EP_ERR_WORKSPACE;
  ScanArgs a{};
  a.topk_idx = topk_idx;
  a.T = num_tokens;
  a.K = num_topk;
  a.bins = num_ranks;
  a.ctrl = static_cast<uint32_t*>(workspace);
  a.status = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kWsHeaderBytes);
  a.token_row = token_row;
  a.topk_weights = topk_weights;
  a.dest = dest;
  a.send_counts = send_counts;
  a.E_local = num_local_experts;
  a.capacity = num_send_capacity;
  a.send_token_idx = send_token_idx;
  a.send_rank = send_rank;
  a.send_idx = send_idx;
  a.send_w = send_w;
  a.vec_rows = (num_topk % 4) == 0 && aligned(send_idx, 16) && aligned(send_w, 16);
  return launch_status(launch_send_layout(a, stream));
}

size_t ep_dispatch_layout_workspace_bytes(int64_t num_tokens, int num_ranks,
                                          int num_local_experts) {
  if (num_tokens < 0 || num_ranks < 1 || num_local_experts < 1) return 0;
  if (num_tokens >= kMaxTokens || int64_t(num_ranks) * num_local_experts > kMaxExperts) return 0;
  const int64_t nh = int64_t(num_ranks) + int64_t(num_ranks) * num_local_experts + 1;
  return fused_ws_bytes(num_tokens, num_ranks, nh, kSendMaxWaves);
}

}  // extern "C"

namespace {

// The scratch of ep_dispatch_layout_noalloc: one copy on every GPU the
// library runs on, held until the process ends.  Host code never uses this
// name as an address (it is a host-side stand-in): the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[EPDC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch.  The first call on a
// device looks it up and clears the control header on `stream` (a kernel,
// not a memset, so that it can sit in a captured graph); later calls find
// the header as the previous call left it, ready for the next.
int library_scratch(void** out, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EP_ERR_LAUNCH;
  ScratchSlot& slot = g_scratch[dev];
  bool first = false;
  std::call_once(slot.once, [&] {
    slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
    first = true;
  });
  if (slot.err != hipSuccess || slot.ptr == nullptr) return EP_ERR_LAUNCH;
  if (first && launch_clear_header(static_cast<uint32_t*>(slot.ptr), stream) != hipSuccess)
    return EP_ERR_LAUNCH;
  *out = slot.ptr;
  return EP_OK;
}

// ep_dispatch_layout, with the workspace given or (workspace == nullptr and
// use_scratch) the library's own scratch; every argument is validated
// before anything is enqueued.
int dispatch_layout_impl(const int64_t* topk_idx, const float* topk_weights, int64_t num_tokens,
                         int num_topk, int num_ranks, int num_local_experts,
                         int64_t num_send_capacity, int32_t* dest, uint8_t* is_in_rank,
                         int32_t* send_counts, int32_t* tokens_per_expert, int32_t* diag,
                         int32_t* send_token_idx, int32_t* send_rank, int32_t* send_idx,
                         float* send_w, int32_t* token_row, void* workspace,
                         size_t workspace_bytes, bool use_scratch, hipStream_t stream) {
  int st = check_routing(num_tokens, num_topk, num_ranks, num_local_experts);
  if (st != EP_OK) return st;
  if (num_ranks > EPDC_MAX_BINS) return EP_ERR_UNSUPPORTED;
  if (num_send_capacity < 0) return EP_ERR_INVALID_ARG;
  if (num_send_capacity > INT32_MAX || num_send_capacity * num_topk > INT32_MAX)
    return EP_ERR_UNSUPPORTED;
  const int64_t TK = num_tokens * num_topk;
  const int64_t cap = num_send_capacity;
  if (!arr_ok(topk_idx, TK, 8) || !arr_ok(topk_weights, TK, 4) || !arr_ok(dest, TK, 4) ||
      !arr_ok(is_in_rank, num_tokens * num_ranks, 4) || !arr_ok(send_counts, 1, 4) ||
      !arr_ok(token_row, TK, 4) || !arr_ok(send_token_idx, cap, 4) ||
      !arr_ok(send_rank, cap, 4) || !arr_ok(send_idx, cap, 4) || !arr_ok(send_w, cap, 4) ||
      (tokens_per_expert && !aligned(tokens_per_expert, 4)) || (diag && !aligned(diag, 4)))
    return EP_ERR_INVALID_ARG;
  const size_t need = ep_dispatch_layout_workspace_bytes(num_tokens, num_ranks, num_local_experts);
  if (use_scratch) {
    if (need > EPDC_NOALLOC_SCRATCH_BYTES) return EP_ERR_WORKSPACE;
  } else if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) {
    return EP_ERR_WORKSPACE;
  }
  const int E = num_ranks * num_local_experts;
  const FusedShape sh = fused_shape(num_tokens, num_ranks, E, kSendMaxWaves);
  if (!sh.fits) return EP_ERR_UNSUPPORTED;
  if (use_scratch) {
    st = library_scratch(&workspace, stream);
    if (st != EP_OK) return st;
  }

  FusedArgs a{};
  a.topk_idx = topk_idx;
  a.topk_weights = topk_weights;
  a.T = num_tokens;
  a.K = num_topk;
  a.P = num_ranks;
  a.E_local = num_local_experts;
  a.E = E;
  a.capacity = cap;
  a.dest = dest;
  a.is_in_rank = is_in_rank;
  a.send_counts = send_counts;
  a.tokens_per_expert = tokens_per_expert;
  a.diag = diag;
  a.send_token_idx = send_token_idx;
  a.send_rank = send_rank;
  a.send_idx = send_idx;
  a.send_w = send_w;
  a.token_row = token_row;
  a.rows_w = row_words(num_topk, {send_idx, send_w});
  a.in_w = aligned(topk_idx, 16) ? row_words(num_topk, {topk_weights}) : 1;
  a.out_w = row_words(num_topk, {dest, token_row});
  a.iir_w = num_ranks % 16 == 0 && aligned(is_in_rank, 16) ? 4
            : num_ranks % 8 == 0 && aligned(is_in_rank, 8) ? 2 : 1;
  a.ndest = num_ranks;
  a.C = 1;
  a.chunk = num_tokens;
  a.hist_e = E;
  a.tiles = sh.tiles;
  a.tiles_per_group = int(sh.per);
  a.waves = sh.waves;
  set_fused_workspace(a, workspace, num_ranks, int64_t(num_ranks) + E + 1, sh.groups);
  return launch_status(launch_dispatch_layout(a, unsigned(sh.groups), stream));
}

}  // namespace

extern "C" {

int ep_dispatch_layout(const int64_t* topk_idx, const float* topk_weights, int64_t num_tokens,
                       int num_topk, int num_ranks, int num_local_experts,
                       int64_t num_send_capacity, int32_t* dest, uint8_t* is_in_rank,
                       int32_t* send_counts, int32_t* tokens_per_expert, int32_t* diag,
                       int32_t* send_token_idx, int32_t* send_rank, int32_t* send_idx,
                       float* send_w, int32_t* token_row, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return dispatch_layout_impl(topk_idx, topk_weights, num_tokens, num_topk, num_ranks,
                              num_local_experts, num_send_capacity, dest, is_in_rank, send_counts,
                              tokens_per_expert, diag, send_token_idx, send_rank, send_idx, send_w,
                              token_row, workspace, workspace_bytes, false, stream);
}

int ep_dispatch_layout_noalloc(const int64_t* topk_idx, const float* topk_weights,
                               int64_t num_tokens, int num_topk, int num_ranks,
                               int num_local_experts, int64_t num_send_capacity, int32_t* dest,
                               uint8_t* is_in_rank, int32_t* send_counts,
                               int32_t* tokens_per_expert, int32_t* diag,
                               int32_t* send_token_idx, int32_t* send_rank, int32_t* send_idx,
                               float* send_w, int32_t* token_row, hipStream_t stream) {
  return dispatch_layout_impl(topk_idx, topk_weights, num_tokens, num_topk, num_ranks,
                              num_local_experts, num_send_capacity, dest, is_in_rank, send_counts,
                              tokens_per_expert, diag, send_token_idx, send_rank, send_idx, send_w,
                              token_row, nullptr, 0, true, stream);
}

size_t ep_dispatch_layout_chunked_workspace_bytes(int64_t num_tokens, int num_ranks,
                                                  int num_chunks) {
  if (num_tokens < 0 || num_tokens >= kMaxTokens || num_ranks < 1 || num_chunks < 1) return 0;
  const int64_t bins = int64_t(num_ranks) * num_chunks;
  if (bins > EPDC_MAX_BINS) return 0;
  return fused_ws_bytes(num_tokens, bins, bins + 1, kSendMaxWaves);
}

int ep_dispatch_layout_chunked(const int64_t* topk_idx, const float* topk_weights,
                               int64_t num_tokens, int num_topk, int num_ranks,
                               int num_local_experts, int num_chunks, int64_t chunk_capacity,
                               int32_t* dest, uint8_t* is_in_rank, int32_t* send_counts,
                               int32_t* diag, int32_t* send_token_idx, int32_t* send_rank,
                               int32_t* send_idx, float* send_w, int32_t* token_row,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_routing(num_tokens, num_topk, num_ranks, num_local_experts);
  if (st != EP_OK) return st;
  if (num_chunks < 1 || chunk_capacity < 0) return EP_ERR_INVALID_ARG;
  const int64_t bins64 = int64_t(num_ranks) * num_chunks;
  if (bins64 > EPDC_MAX_BINS) return EP_ERR_UNSUPPORTED;
  // every row index of the C chunks' arrays, end to end, fits int32
  const int64_t rows = chunk_capacity * num_chunks;
  if (rows > INT32_MAX || rows * num_topk > INT32_MAX) return EP_ERR_UNSUPPORTED;
  const int64_t TK = num_tokens * num_topk;
  if (!arr_ok(topk_idx, TK, 8) || !arr_ok(topk_weights, TK, 4) || !arr_ok(dest, TK, 4) ||
      !arr_ok(is_in_rank, num_tokens * num_ranks, 4) || !arr_ok(send_counts, 1, 4) ||
      !arr_ok(token_row, TK, 4) || !arr_ok(send_token_idx, rows, 4) ||
      !arr_ok(send_rank, rows, 4) || !arr_ok(send_idx, rows, 4) || !arr_ok(send_w, rows, 4) ||
      (diag && !aligned(diag, 4)))
    return EP_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256) ||
      workspace_bytes <
          ep_dispatch_layout_chunked_workspace_bytes(num_tokens, num_ranks, num_chunks))
    return EP_ERR_WORKSPACE;
  const int bins = int(bins64);
  const FusedShape sh = fused_shape(num_tokens, bins, 0, kSendMaxWaves);
  if (!sh.fits) return EP_ERR_UNSUPPORTED;

  FusedArgs a{};
  a.topk_idx = topk_idx;
  a.topk_weights = topk_weights;
  a.T = num_tokens;
  a.K = num_topk;
  a.P = bins;
  a.E_local = num_local_experts;
  a.E = num_ranks * num_local_experts;
  a.capacity = chunk_capacity;
  a.dest = dest;
  a.is_in_rank = is_in_rank;
  a.send_counts = send_counts;
  a.tokens_per_expert = nullptr;
  a.diag = diag;
  a.send_token_idx = send_token_idx;
  a.send_rank = send_rank;
  a.send_idx = send_idx;
  a.send_w = send_w;
  a.token_row = token_row;
  // rows are K words apart, so every row (chunk c's from row c*capacity on)
  // is as aligned as the arrays' bases for the whole-row forms
  a.rows_w = row_words(num_topk, {send_idx, send_w});
  a.in_w = aligned(topk_idx, 16) ? row_words(num_topk, {topk_weights}) : 1;
  a.out_w = row_words(num_topk, {dest, token_row});
  a.iir_w = num_ranks % 16 == 0 && aligned(is_in_rank, 16) ? 4
            : num_ranks % 8 == 0 && aligned(is_in_rank, 8) ? 2 : 1;
  a.ndest = num_ranks;
  a.C = num_chunks;
  a.chunk = num_tokens / num_chunks;
  a.hist_e = 0;
  a.tiles = sh.tiles;
  a.tiles_per_group = int(sh.per);
  a.waves = sh.waves;
  set_fused_workspace(a, workspace, bins, int64_t(bins) + 1, sh.groups);
  // Chunk-local single pass: a workgroup reads the rows of the groups one or
  // two chunks span, for those chunks' bins, instead of the two-pass scan
  // over every bin.  Taken while a chunk's share is within the single pass's
  // load budget (up to 8 loads per thread).
  const int64_t span = (sh.groups + num_chunks - 1) / num_chunks + 1;
  if (num_chunks > 1 && span * num_ranks <= int64_t(8) * 64 * sh.waves) {
    a.chunk_local = true;
    a.two_pass = false;
  }
  return launch_status(launch_dispatch_layout(a, unsigned(sh.groups), stream));
}

size_t ep_regroup_workspace_bytes(int64_t num_rows, int num_bins) {
  if (num_rows < 0 || num_rows >= kMaxTokens || num_bins < 1) return 0;
  return fused_ws_bytes(num_rows, num_bins, int64_t(num_bins) + 1, kRegroupMaxWaves);
}

int ep_regroup_by_expert(const void* recv_x, const int32_t* recv_idx, const float* recv_w,
                         const int32_t* row_group, int num_groups, int64_t num_rows,
                         int num_topk, int hidden, int num_local_experts, int align,
                         int64_t capacity, void* perm_x, int32_t* perm_src, float* perm_w,
                         int32_t* tokens_per_expert, int32_t* expert_offsets, int32_t* row_map,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (num_rows < 0 || num_topk < 1 || num_local_experts < 1 || align < 1 || capacity < 0 ||
      num_groups < 1 || (num_groups > 1 && !row_group && num_rows > 0))
    return EP_ERR_INVALID_ARG;
  const int64_t bins64 = int64_t(num_groups) * num_local_experts;
  if (num_rows >= kMaxTokens || num_topk > EPDC_MAX_TOPK || bins64 > EPDC_MAX_BINS ||
      num_rows * num_topk > INT32_MAX)
    return EP_ERR_UNSUPPORTED;
  const int bins = int(bins64);
  // Every regrouped row index, padding included, must fit int32: the rows
  // number at most R*min(K, E_local) (one per distinct local id of a row)
  // plus fewer than `align` padding rows per bin.
  const int64_t most_rows = num_rows * (num_topk < num_local_experts ? num_topk : num_local_experts) +
                            bins64 * (int64_t(align) - 1);
  if (capacity > INT32_MAX || most_rows > INT32_MAX) return EP_ERR_UNSUPPORTED;
  int st = check_hidden(hidden, false);
  if (st != EP_OK) return st;
  const int64_t RK = num_rows * num_topk;
  if (!arr_ok(recv_x, num_rows, 16) || !arr_ok(recv_idx, RK, 4) ||
      (recv_w && !aligned(recv_w, 4)) || !arr_ok(perm_x, capacity, 16) ||
      !arr_ok(perm_src, capacity, 4) || (perm_w && !aligned(perm_w, 4)) ||
      !arr_ok(tokens_per_expert, 1, 4) || !arr_ok(expert_offsets, 1, 4) ||
      !arr_ok(row_map, RK, 4) || (row_group && !aligned(row_group, 4)))
    return EP_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256) ||
      workspace_bytes < ep_regroup_workspace_bytes(num_rows, bins))
    return EP_ERR_WORKSPACE;
  const FusedShape sh = fused_shape(num_rows, bins, 0, kRegroupMaxWaves);
  if (!sh.fits) return EP_ERR_UNSUPPORTED;

  // 1. one launch: counts per local expert, aligned offsets, row_map, the
  //    source row and weight of every regrouped row, padding rows included
  FusedArgs a{};
  a.topk_weights = recv_w;
  a.T = num_rows;
  a.K = num_topk;
  a.P = bins;
  a.E_local = num_local_experts;
  a.E = 0;
  a.row_group = num_groups > 1 ? row_group : nullptr;
  a.capacity = capacity;
  a.ndest = bins;
  a.C = 1;
  a.chunk = num_rows;
  a.hist_e = 0;
  a.send_counts = tokens_per_expert;
  a.send_token_idx = perm_src;
  a.token_row = row_map;
  a.out_w = row_words(num_topk, {row_map});
  a.tiles = sh.tiles;
  a.tiles_per_group = int(sh.per);
  a.waves = sh.waves;
  set_fused_workspace(a, workspace, bins, int64_t(bins) + 1, sh.groups);
  a.ids32 = recv_idx;
  a.align = align;
  a.offsets = expert_offsets;
  a.perm_w = perm_w;
  if (launch_regroup_layout(a, unsigned(sh.groups), stream) != hipSuccess) return EP_ERR_LAUNCH;

  // 2. every regrouped row in address order: its source row, or zeros
  GatherArgs r{};
  r.x = recv_x;
  r.R = num_rows;
  r.H = hidden;
  r.perm_src = perm_src;
  r.offsets = expert_offsets;
  r.bins = bins;
  r.capacity = capacity;
  r.out = perm_x;
  return launch_status(launch_regroup_gather(r, stream));
}

int ep_dispatch_permute(const void* x, int64_t num_tokens, int hidden, const int32_t* token_row,
                        int num_topk, int64_t num_send_capacity, int out_dtype, void* send_x,
                        float* send_scale, hipStream_t stream) {
  if (num_tokens < 0 || num_topk < 1 || num_send_capacity < 0) return EP_ERR_INVALID_ARG;
  if (num_tokens >= kMaxTokens || num_topk > EPDC_MAX_TOPK) return EP_ERR_UNSUPPORTED;
  if (num_send_capacity > INT32_MAX) return EP_ERR_UNSUPPORTED;
  const bool fp8 = out_dtype == EP_DTYPE_FP8_E4M3;
  if (!fp8 && out_dtype != EP_DTYPE_BF16) return EP_ERR_INVALID_ARG;
  int st = check_hidden(hidden, fp8);
  if (st != EP_OK) return st;
  const int64_t cap = num_send_capacity;
  if (!arr_ok(x, num_tokens, 16) || !arr_ok(token_row, num_tokens, 4) ||
      !arr_ok(send_x, cap, 16) || (fp8 && !arr_ok(send_scale, cap, 4)))
    return EP_ERR_INVALID_ARG;
  RowArgs a{};
  a.x = x;
  a.T = num_tokens;
  a.H = hidden;
  a.token_row = token_row;
  a.K = num_topk;
  a.capacity = num_send_capacity;
  a.out = send_x;
  a.out_scale = fp8 ? send_scale : nullptr;
  a.scale_fmt = kScaleF32;
  a.scale_block_rows = 0;
  a.capped = true;
  return launch_status(fp8 ? launch_permute_fp8(a, stream) : launch_permute_bf16(a, stream));
}

int ep_batched_prepare(const void* x, const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                       int hidden, int first_expert, int num_local_experts,
                       int64_t max_num_tokens, void* b_x, int32_t* tokens_per_expert,
                       int32_t* token_row, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (num_tokens < 0 || num_topk < 1 || num_local_experts < 1 || max_num_tokens < 0 ||
      first_expert < 0)
    return EP_ERR_INVALID_ARG;
  if (num_tokens >= kMaxTokens || num_topk > EPDC_MAX_TOPK ||
      num_local_experts > EPDC_MAX_BINS || num_tokens * num_topk > INT32_MAX)
    return EP_ERR_UNSUPPORTED;
  if (max_num_tokens > INT32_MAX / num_local_experts) return EP_ERR_UNSUPPORTED;  // E_local*max
  int st = check_hidden(hidden, false);
  if (st != EP_OK) return st;
  if (!arr_ok(x, num_tokens, 16) || !arr_ok(topk_idx, num_tokens, 8) ||
      !arr_ok(token_row, num_tokens, 4) || !arr_ok(b_x, max_num_tokens, 16) ||
      !arr_ok(tokens_per_expert, 1, 4))
    return EP_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256) ||
      workspace_bytes < ep_batched_workspace_bytes(num_tokens, num_local_experts, max_num_tokens))
    return EP_ERR_WORKSPACE;

  // 1. scan: counts, slots and token_row; 2. zeros past each count;
  // 3. the token-major permute writes the data rows (token_row = e*max+slot).
  ScanArgs a{};
  a.topk_idx = topk_idx;
  a.T = num_tokens;
  a.K = num_topk;
  a.bins = num_local_experts;
  a.ctrl = static_cast<uint32_t*>(workspace);
  a.status = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kWsHeaderBytes);
  a.token_row = token_row;
  a.first_expert = first_expert;
  a.max_tokens = max_num_tokens;
  a.tokens_per_expert = tokens_per_expert;
  if (launch_batched_scan(a, stream) != hipSuccess) return EP_ERR_LAUNCH;

  PadArgs z{};
  z.tokens_per_expert = tokens_per_expert;
  z.E_local = num_local_experts;
  z.max_tokens = max_num_tokens;
  z.row_pieces = hidden >> 3;
  z.b_x = b_x;
  if (launch_zero_pad(z, stream) != hipSuccess) return EP_ERR_LAUNCH;

  RowArgs r{};
  r.x = x;
  r.T = num_tokens;
  r.H = hidden;
  r.token_row = token_row;
  r.K = num_topk;
  r.capacity = int64_t(num_local_experts) * max_num_tokens;
  r.out = b_x;
  r.out_scale = nullptr;
  r.sparse = true;
  return launch_status(launch_permute_bf16(r, stream));
}

int ep_batched_prepare_fp8(const void* x, const int64_t* topk_idx, int64_t num_tokens,
                           int num_topk, int hidden, int first_expert, int num_local_experts,
                           int64_t max_num_tokens, int scale_fmt, int scale_col_major,
                           void* b_q, void* b_scale, int32_t* tokens_per_expert,
                           int32_t* token_row, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (num_tokens < 0 || num_topk < 1 || num_local_experts < 1 || max_num_tokens < 0 ||
      first_expert < 0)
    return EP_ERR_INVALID_ARG;
  if (scale_fmt != EP_SCALE_F32 && scale_fmt != EP_SCALE_POW2 && scale_fmt != EP_SCALE_UE8M0)
    return EP_ERR_INVALID_ARG;
  if (scale_col_major != 0 && scale_col_major != 1) return EP_ERR_INVALID_ARG;
  if (num_tokens >= kMaxTokens || num_topk > EPDC_MAX_TOPK ||
      num_local_experts > EPDC_MAX_BINS || num_tokens * num_topk > INT32_MAX)
    return EP_ERR_UNSUPPORTED;
  if (max_num_tokens > INT32_MAX / num_local_experts) return EP_ERR_UNSUPPORTED;  // E_local*max
  int st = check_hidden(hidden, true);
  if (st != EP_OK) return st;
  const bool ue8m0 = scale_fmt == EP_SCALE_UE8M0;
  if (ue8m0 && hidden % (4 * EPDC_FP8_GROUP) != 0) return EP_ERR_INVALID_ARG;
  const int units = ue8m0 ? hidden / (4 * EPDC_FP8_GROUP) : hidden / EPDC_FP8_GROUP;
  if (!arr_ok(x, num_tokens, 16) || !arr_ok(topk_idx, num_tokens, 8) ||
      !arr_ok(token_row, num_tokens, 4) || !arr_ok(b_q, max_num_tokens, 16) ||
      !arr_ok(b_scale, max_num_tokens, 4) || !arr_ok(tokens_per_expert, 1, 4))
    return EP_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, 256) ||
      workspace_bytes < ep_batched_workspace_bytes(num_tokens, num_local_experts, max_num_tokens))
    return EP_ERR_WORKSPACE;

  // 1. scan: counts, slots and token_row; 2. zero codes and scales past each
  // count; 3. the token-major fp8 permute writes the data rows and scales.
  ScanArgs a{};
  a.topk_idx = topk_idx;
  a.T = num_tokens;
  a.K = num_topk;
  a.bins = num_local_experts;
  a.ctrl = static_cast<uint32_t*>(workspace);
  a.status = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + kWsHeaderBytes);
  a.token_row = token_row;
  a.first_expert = first_expert;
  a.max_tokens = max_num_tokens;
  a.tokens_per_expert = tokens_per_expert;
  if (launch_batched_scan(a, stream) != hipSuccess) return EP_ERR_LAUNCH;

  PadArgs z{};
  z.tokens_per_expert = tokens_per_expert;
  z.E_local = num_local_experts;
  z.max_tokens = max_num_tokens;
  z.row_pieces = hidden >> 4;
  z.b_x = b_q;
  if (launch_zero_pad(z, stream) != hipSuccess) return EP_ERR_LAUNCH;
  ScalePadArgs zs{};
  zs.tokens_per_expert = tokens_per_expert;
  zs.E_local = num_local_experts;
  zs.max_tokens = max_num_tokens;
  zs.units = units;
  zs.col_major = scale_col_major != 0;
  zs.scale = static_cast<uint32_t*>(b_scale);
  if (launch_scale_pad(zs, stream) != hipSuccess) return EP_ERR_LAUNCH;

  RowArgs r{};
  r.x = x;
  r.T = num_tokens;
  r.H = hidden;
  r.token_row = token_row;
  r.K = num_topk;
  r.capacity = int64_t(num_local_experts) * max_num_tokens;
  r.out = b_q;
  r.out_scale = b_scale;
  r.sparse = true;
  r.scale_fmt = scale_fmt == EP_SCALE_UE8M0 ? kScaleUe8m0
                : scale_fmt == EP_SCALE_POW2 ? kScalePow2 : kScaleF32;
  r.scale_block_rows = scale_col_major ? max_num_tokens : 0;
  return launch_status(launch_permute_fp8(r, stream));
}

int ep_combine(const void* y, int64_t num_rows, const int32_t* token_row,
               const float* topk_weights, int64_t num_tokens, int num_topk, int hidden,
               const void* bias0, const void* bias1, void* out, hipStream_t stream) {
  if (num_tokens < 0 || num_topk < 1 || num_rows < 0) return EP_ERR_INVALID_ARG;
  if (num_tokens >= kMaxTokens || num_topk > EPDC_MAX_TOPK) return EP_ERR_UNSUPPORTED;
  int st = check_hidden(hidden, false);
  if (st != EP_OK) return st;
  if (!arr_ok(y, num_rows, 16) || !arr_ok(token_row, num_tokens, 4) ||
      (topk_weights && !aligned(topk_weights, 4)) || !arr_ok(out, num_tokens, 16) ||
      (bias0 && !aligned(bias0, 16)) || (bias1 && !aligned(bias1, 16)))
    return EP_ERR_INVALID_ARG;
  CombineArgs a{};
  a.y = y;
  a.R = num_rows;
  a.token_row = token_row;
  a.w = topk_weights;
  a.bias0 = bias0;
  a.bias1 = bias1;
  a.T = num_tokens;
  a.K = num_topk;
  a.H = hidden;
  a.out = out;
  return launch_status(launch_combine(a, stream));
}

}  // extern "C"
