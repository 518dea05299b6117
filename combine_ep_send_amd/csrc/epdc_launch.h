// Internal launchers: each enqueues the kernels of one entry point on a
// stream, after the C-ABI layer has validated every argument.  They return
// the hipError_t of the launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace epdc {

// Scan workspace: a 256-byte header of uint32 control words followed by one
// 64-bit status word per (tile, bin).
constexpr size_t kWsHeaderBytes = 256;
enum : int { kCtrlTicket = 0, kCtrlDone = 1, kCtrlEpoch = 2, kCtrlError = 3 };
constexpr uint32_t kErrLookbackGaveUp = 1u;   // a bounded wait (lookback or barrier) gave up
// Copy a workspace's error word [kCtrlError] to flags[0] and clear it.
hipError_t launch_workspace_status(uint32_t* ctrl, int32_t* flags, hipStream_t s);
// Zero a workspace's 256-byte control header.
hipError_t launch_clear_header(uint32_t* ctrl, hipStream_t s);

// The layout scans work on tiles of 256 tokens (one workgroup each).
inline int64_t num_tiles(int64_t T) { return (T + 255) / 256; }
inline size_t scan_status_bytes(int64_t T, int bins) {
  int64_t tiles = num_tiles(T) > 0 ? num_tiles(T) : 1;
  return size_t(tiles) * size_t(bins) * 8u;
}

struct CountArgs {
  const int64_t* topk_idx;
  int64_t T;
  int K, P, E_local, E, C;
  int64_t chunk;                 // T / C
  int32_t* dest;
  uint8_t* is_in_rank;
  int32_t* send_counts;
  int32_t* tokens_per_expert;    // may be null
  int32_t* diag;                 // may be null
  uint32_t* ctrl;                // workspace header: [0] finished workgroups
  int32_t* accum;                // [C, P + E + 1] accumulators, zero between calls
};
// Count workspace: 256-byte header, then one accumulator per (chunk, bin).
inline size_t count_ws_bytes(int P, int E, int C) {
  return kWsHeaderBytes + size_t(C) * size_t(P + E + 1) * 4u;
}
hipError_t launch_counts(const CountArgs& a, hipStream_t s);

struct ScanArgs {
  // common
  const int64_t* topk_idx;
  int64_t T;
  int K;
  int bins;                      // P (send layout) or E_local (batched)
  uint32_t* ctrl;                // workspace header
  uint64_t* status;              // [tiles, bins]
  int32_t* token_row;
  // send layout
  const float* topk_weights;
  const int32_t* dest;
  const int32_t* send_counts;
  int E_local;
  int64_t capacity;
  int32_t* send_token_idx;
  int32_t* send_rank;
  int32_t* send_idx;
  float* send_w;
  bool vec_rows;                 // K % 4 == 0 and send_idx/send_w 16-byte aligned
  // batched layout
  int64_t first_expert;
  int64_t max_tokens;
  int32_t* tokens_per_expert;    // [E_local]
};
hipError_t launch_send_layout(const ScanArgs& a, hipStream_t s);
hipError_t launch_batched_scan(const ScanArgs& a, hipStream_t s);

struct FusedArgs {
  const int64_t* topk_idx;
  const float* topk_weights;
  int64_t T;
  int K;
  int P;
  int E_local;
  int E;
  int64_t capacity;
  int32_t* dest;
  uint8_t* is_in_rank;
  int32_t* send_counts;          // [P]
  int32_t* tokens_per_expert;    // [E] or null
  int32_t* diag;                 // [1] or null
  int32_t* send_token_idx;
  int32_t* send_rank;
  int32_t* send_idx;
  float* send_w;
  int32_t* token_row;
  // Words per load or store of a whole row, where K (P for is_in_rank) and
  // the pointers allow it: 4 (16 bytes), 2 (8 bytes) or 1.
  int rows_w;                    // send_idx / send_w rows
  int in_w;                      // topk_weights rows (topk_idx in 16-byte pairs when >= 2)
  int out_w;                     // dest / token_row rows
  int iir_w;                     // is_in_rank rows (bytes: 16, 8 or 4 per store)
  uint32_t* ctrl;                // workspace header: [0] arrivals, [2] the count at launch
  uint32_t* rows;                // [groups, P + E + 1] published totals
  uint32_t* pref;                // [groups, P] per-group exclusive prefixes (two-pass scan)
  uint32_t* tots;                // [P] bin totals (two-pass scan)
  bool two_pass;                 // scan the rows bin by bin, with a second barrier
  bool chunk_local;              // chunks: read only the rows of the own chunks' groups and bins
  // Chunks (send mode): the bins are (chunk, destination), chunk-major, with
  // P = C * ndest bins; chunk c = tokens [c*chunk, (c+1)*chunk), the last
  // chunk ending at T.  Rows are numbered within their chunk (capacity =
  // rows per chunk) and chunk c's rows are written from row c*capacity.
  int ndest;                     // destinations (P when C == 1)
  int C;                         // chunks (>= 1)
  int64_t chunk;                 // tokens per chunk, T / C
  int hist_e;                    // expert words in each published row (E, or 0)
  int64_t tiles;                 // tiles of waves*64 tokens (>= 1)
  int tiles_per_group;
  int waves;                     // waves per workgroup: 1, 2 or 4 (one token per thread)
  // regroup by local expert (P = E_local bins, E = 0)
  const int32_t* ids32;          // [R,K] local expert ids, -1 = not local
  const int32_t* row_group;      // [R] receive buffer of each row, or null (P = groups*E_local)
  int align;                     // segment alignment (>= 1)
  int32_t* offsets;              // [P+1] aligned segment starts
  float* perm_w;                 // [cap] weight of each row's slot, or null
};
// Workgroups of the fused counts + layout launch: at most one per compute
// unit and at most kMaxFusedGroups, so that all of them are resident at once.
constexpr int kMaxFusedGroups = 256;
// Bins one workgroup scans in the two-pass form (at most).
constexpr int kMaxTwoPassBins = 8;
// Tiles of the fused launch: one token per thread of a workgroup of 1 to
// `most` waves (a power of two), chosen so that about 64 tiles cover the
// input (small inputs then spread over more compute units; large ones keep
// big tiles).  The send layouts take at most 4 waves, the regroup (whose
// received rows outnumber the tokens by K) up to 16: measured on the
// expert-major regroup of 117k rows, 16-wave tiles took its launch from 690
// to 677 us, while 8- or 16-wave tiles made the headline's send layout
// slower (26 and 37 against 21.5 us).
constexpr int kSendMaxWaves = 4;
constexpr int kRegroupMaxWaves = 16;
inline int fused_waves(int64_t T, int most) {
  const int64_t w = (T + 64 * 64 - 1) / (64 * 64);
  int v = 1;
  while (v < w && v < most) v <<= 1;
  return v;
}
inline int64_t fused_tiles(int64_t T, int most) {
  const int64_t tile = int64_t(fused_waves(T, most)) * 64;
  const int64_t t = (T + tile - 1) / tile;
  return t > 0 ? t : 1;
}
// Workspace of the fused launch over T rows: header, rows, prefixes, totals.
inline size_t fused_ws_bytes(int64_t T, int64_t bins, int64_t row_words, int most) {
  const int64_t tiles = fused_tiles(T, most);
  const int64_t g = tiles < kMaxFusedGroups ? tiles : kMaxFusedGroups;
  return kWsHeaderBytes + size_t(g) * size_t(row_words) * 4u + size_t(g) * size_t(bins) * 4u +
         size_t(bins) * 4u;
}
// Whether a launch of `groups` workgroups of `waves` waves over `bins` bins
// takes the two-pass scan (the single pass would need more than 8 loads per
// thread, and no workgroup has more than kMaxTwoPassBins bins to scan).
inline bool fused_two_pass(int64_t groups, int64_t bins, int waves) {
  return groups * bins > 8 * 64 * int64_t(waves) &&
         (bins + groups - 1) / groups <= kMaxTwoPassBins;
}
size_t fused_smem_bytes(int P, int E, int tiles_per_group, int waves);
hipError_t launch_dispatch_layout(const FusedArgs& a, unsigned groups, hipStream_t s);
hipError_t launch_regroup_layout(const FusedArgs& a, unsigned groups, hipStream_t s);

struct GatherArgs {
  const void* x;                 // [R, H] bf16 received rows
  int64_t R;
  int H;
  const int32_t* perm_src;       // [cap] source row of each regrouped row, -1 = padding
  const int32_t* offsets;        // [bins+1] aligned segment starts; offsets[bins] rows in use
  int bins;
  int64_t capacity;              // rows of out
  void* out;                     // [cap, H] bf16
};
hipError_t launch_regroup_gather(const GatherArgs& a, hipStream_t s);

// fp8 scale formats: fl32(amax/448); the smallest power of two at or above
// it; that power as a UE8M0 byte, four packed per 32-bit word.
enum : int { kScaleF32 = 0, kScalePow2 = 1, kScaleUe8m0 = 2 };

struct RowArgs {
  const void* x;
  int64_t T;
  int H;
  const int32_t* token_row;
  int K;
  int64_t capacity;              // rows of the destination buffer
  void* out;
  void* out_scale;               // fp8 scales (float or packed uint32) or null
  bool sparse;                   // many tokens have no destination (fp8: look up rows first)
  bool capped;                   // several rows per token: cap the occupancy (dense permutes)
  int scale_fmt;                 // kScale*
  int64_t scale_block_rows;      // > 0: scales column-major per block of this many rows
};
hipError_t launch_permute_bf16(const RowArgs& a, hipStream_t s);
hipError_t launch_permute_fp8(const RowArgs& a, hipStream_t s);

struct PadArgs {
  const int32_t* tokens_per_expert;  // [E_local] counts from the batched scan
  int E_local;
  int64_t max_tokens;
  int64_t row_pieces;                // 16-byte pieces per row
  void* b_x;                         // [E_local, max_tokens, row] rows
};
hipError_t launch_zero_pad(const PadArgs& a, hipStream_t s);

// Zero scales of the padding slots of an expert-batched fp8 buffer: per
// expert, max_tokens rows of `units` 32-bit scale words, row-major or
// column-major ([units, max_tokens]).
struct ScalePadArgs {
  const int32_t* tokens_per_expert;
  int E_local;
  int64_t max_tokens;
  int units;
  bool col_major;
  uint32_t* scale;
};
hipError_t launch_scale_pad(const ScalePadArgs& a, hipStream_t s);

// Largest workgroup of the combine (one 16-byte piece per thread).
constexpr int kMaxRowBlock = 1024;
// Workgroup of the bf16 permute (one 16-byte piece per thread).
constexpr int kPermuteBlock = 128;
// Workgroup of the regroup's gather (one 4 KiB window of the output).
constexpr int kGatherBlock = 256;
// Largest workgroup of the combine for sparse slots (several pieces per thread).
constexpr int kSparseMaxBlock = 512;

struct CombineArgs {
  const void* y;
  int64_t R;
  const int32_t* token_row;
  const float* w;                // null: unweighted, each distinct row once
  const void* bias0;             // [T,H] bf16 or null
  const void* bias1;             // [T,H] bf16 or null
  int64_t T;
  int K;
  int H;
  void* out;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace epdc
