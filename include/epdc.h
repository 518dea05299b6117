/*
 * epdc.h - MoE token dispatch and combine on one MI355X (gfx950).
 *
 * C ABI of libepdc.so.  The library computes, on one GPU's share of the work,
 * what an expert-parallel dispatcher does before and after its all-to-all:
 * routing counts, a stable destination-major send layout (or the
 * expert-batched layout), the permuted hidden rows (bf16, or fp8 e4m3 with
 * per-128-channel scales) and the weighted per-token combine.  The P
 * "destinations" are contiguous segments of one device buffer; nothing here
 * talks to another GPU.
 *
 * Sources (page title, then the section the call follows):
 *  - axolotl API docs, "integrations.expert_parallel.torch_dispatch":
 *    module overview, compute_send_counts, build_send_layout, dispatch,
 *    combine, chunk_bounds, dispatch_chunked_forward, to_host.
 *  - NeMo AutoModel API docs, "nemo_automodel.components.moe.uccl_ep.buffer":
 *    Buffer.get_dispatch_layout, Buffer.dispatch, Buffer.combine,
 *    Buffer.low_latency_dispatch (fp8 rows + scales per 128 channels: float,
 *    power-of-two, or packed UE8M0).
 *  - vLLM API docs, "vllm.model_executor.layers.fused_moe.prepare_finalize":
 *    BatchedPrepareAndFinalize.prepare / finalize.
 *  - NeMo AutoModel API docs,
 *    "nemo_automodel.components.moe.megatron.token_dispatcher":
 *    TokenDispatcherConfig.moe_router_dtype (fp32 weighted averaging).
 *
 * Conventions shared by every call:
 *  - Tensor pointers are DEVICE pointers to row-major, contiguous arrays.
 *    The caller owns every buffer; the library allocates nothing, frees
 *    nothing, keeps no state between calls and never synchronizes.  Each call
 *    only validates its arguments on the host and enqueues kernels on
 *    `stream`.
 *  - Shapes use T = num_tokens, K = num_topk, P = num_ranks,
 *    E_local = num_local_experts, E = P * E_local, H = hidden.
 *    Destination p owns the experts [p*E_local, (p+1)*E_local).
 *  - Expert ids are int64 in [-1, E); -1 means "unrouted".  Routed ids of one
 *    token are expected to be distinct (a router's top-k).  Ids outside
 *    [-1, E) are treated as unrouted and counted in `diag`.
 *  - Every index and count written is int32; membership flags are uint8 0/1.
 *  - Errors: a negative ep_status_t is returned BEFORE anything is enqueued
 *    when an argument is invalid (null pointer, bad size, misaligned
 *    pointer, workspace too small); EP_ERR_LAUNCH if the runtime rejects a
 *    launch.  Conditions only the device can see (capacity overflow, bad
 *    ids) never fault: rows past a capacity are not written, their slots get
 *    token_row = -1, and the true counts are still reported.
 *  - Alignment: hidden-row buffers (x, send_x, y, out, b_x) 16 bytes;
 *    topk_idx 8 bytes; all other arrays 4 bytes; workspaces 256 bytes.
 *    A pointer to an empty array (e.g. every [T,..] array when T = 0) may
 *    be NULL.
 *  - Limits: 1 <= K <= 16; T < 2^30; P and E_local <= 1024; E <= 8192;
 *    H a positive multiple of 8 (of 128 for fp8); every row index fits int32.
 *  - Workspaces: each serves one family of calls, whose control words it
 *    keeps: ep_compute_send_counts; the scans (ep_build_send_layout,
 *    ep_batched_prepare, ep_batched_prepare_fp8); or the one-launch layouts
 *    (ep_dispatch_layout, ep_dispatch_layout_chunked, ep_regroup_by_expert).  Zero it once, size it for
 *    the largest call, and do not hand it to a call of another family or to
 *    two calls that may run at the same time.  The ep_*_workspace_bytes
 *    functions return 0 for negative or zero sizes and for T >= 2^30 or
 *    E > 8192, which the calls reject before they look at a workspace.
 */
#ifndef EPDC_H
#define EPDC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = -1,   /* null pointer, bad size or misalignment */
    EP_ERR_UNSUPPORTED = -2,   /* outside the documented limits */
    EP_ERR_WORKSPACE = -3,     /* workspace missing or too small */
    EP_ERR_LAUNCH = -4         /* the HIP runtime rejected a kernel launch */
} ep_status_t;

typedef enum {
    EP_DTYPE_BF16 = 0,         /* rows copied bit for bit */
    EP_DTYPE_FP8_E4M3 = 1      /* OCP e4m3 (float8_e4m3fn) + fp32 scales */
} ep_dtype_t;

typedef enum {
    EP_SCALE_F32 = 0,          /* fp32 scale = amax / 448 */
    EP_SCALE_POW2 = 1,         /* fp32 scale, rounded up to a power of two */
    EP_SCALE_UE8M0 = 2         /* that power as a UE8M0 byte, 4 per int32 */
} ep_scale_fmt_t;

#define EPDC_ABI_VERSION 6
#define EPDC_MAX_TOPK 16
#define EPDC_MAX_BINS 1024
#define EPDC_FP8_GROUP 128
/* Bytes of the library's own scratch per GPU (ep_dispatch_layout_noalloc). */
#define EPDC_NOALLOC_SCRATCH_BYTES (4u << 20)

/* Version of this ABI (EPDC_ABI_VERSION). */
int ep_abi_version(void);

/* Static, human-readable text for a status code. */
const char* ep_status_string(int status);

/* Bits of the error word that ep_workspace_status reports. */
#define EP_WS_WAIT_GAVE_UP 1   /* a bounded wait inside a call gave up */

/*
 * Errors a workspace has collected since the last query, copied to `flags`
 * and cleared.
 * axolotl "torch_dispatch", module overview (hang safety): there, every
 * rank derives its split sizes from the same routing, so that no rank waits
 * for data that never comes.  On one GPU the only waits are between the
 * workgroups of one launch (the grid barrier of ep_dispatch_layout and
 * ep_regroup_by_expert, the lookback of ep_build_send_layout,
 * ep_batched_prepare and ep_batched_prepare_fp8), and each is bounded: a
 * wait that outlasts its limit gives up, sets EP_WS_WAIT_GAVE_UP in the
 * workspace header (word 3) and the call carries on, so every kernel
 * finishes but that call's outputs are undefined.  This call makes such a
 * give-up visible to the caller.
 *
 *   workspace        any workspace the calls above were given (at least its
 *                    256-byte header, 256-byte aligned), or NULL for the
 *                    library's own scratch on the current device (the one
 *                    ep_dispatch_layout_noalloc uses)
 *   flags            [1] int32 out, DEVICE memory: the error word (0 = no
 *                    wait gave up) as it stood when this call's kernel ran
 * Like the other calls it only enqueues a kernel on `stream` (run it on the
 * stream of the calls it is meant to cover) and never synchronizes; read
 * `flags` after the stream has finished.  The word is cleared in the same
 * atomic step, so each query reports what happened since the previous one.
 * Returns EP_ERR_INVALID_ARG for a null or misaligned `flags` and
 * EP_ERR_WORKSPACE for a missing, misaligned or too small workspace.
 */
int ep_workspace_status(void* workspace, size_t workspace_bytes, int32_t* flags,
                        hipStream_t stream);

/*
 * Bytes of workspace ep_compute_send_counts needs: a 256-byte header (uint32
 * word [0] counts finished workgroups) followed by one int32 accumulator per
 * (chunk, bin), P + E + 1 bins per chunk.  Zero-filled once before first use;
 * every call clears what it used, leaving it ready for the next call; calls
 * that may overlap in time must use different workspaces.
 */
size_t ep_counts_workspace_bytes(int64_t num_tokens, int num_ranks,
                                 int num_local_experts, int num_chunks);

/*
 * Bytes of workspace ep_build_send_layout needs for T tokens and P
 * destinations (its scan bins).  The workspace holds the cross-workgroup
 * scan state: a 256-byte header (uint32 words: [0] tile ticket, [1] finished
 * tiles, [2] call epoch, [3] error flags: bit 0 = a lookback wait gave up)
 * followed by one 64-bit status word per (bin, tile of 256 tokens).
 * It must be zero-filled once before its first use; every call leaves it
 * ready for the next call.  Calls that may overlap in time (different
 * streams) must use different workspaces.
 */
size_t ep_layout_workspace_bytes(int64_t num_tokens, int num_bins);

/*
 * Bytes of workspace ep_batched_prepare needs: the scan state above with
 * E_local bins (max_num_tokens does not change it).  Same zero-once /
 * no-overlap rules.
 */
size_t ep_batched_workspace_bytes(int64_t num_tokens, int num_local_experts,
                                  int64_t max_num_tokens);

/*
 * Routing decode and histograms.
 * axolotl "torch_dispatch": compute_send_counts; NeMo "uccl_ep.buffer":
 * Buffer.get_dispatch_layout (num_tokens_per_rank, num_tokens_per_expert,
 * is_token_in_rank); axolotl chunk_bounds for the per-chunk split.
 *
 *   topk_idx           [T,K] int64 in   global expert ids, -1 = unrouted
 *   num_chunks         C >= 1           chunk c = [c*(T/C), (c+1)*(T/C)),
 *                                       the last chunk ends at T
 *   dest               [T,K] int32 out  owning destination id / E_local, or -1
 *   is_in_rank         [T,P] uint8 out  1 iff some slot of t is owned by p
 *   send_counts        [C,P] int32 out  sum of is_in_rank over chunk c
 *   tokens_per_expert  [C,E] int32 out  routed slots naming e in chunk c
 *                                       (may be NULL)
 *   diag               [1]   int32 out  ids outside [-1, E) (may be NULL)
 *   workspace          ep_counts_workspace_bytes(T, P, E_local, C) bytes
 * All outputs are fully overwritten (integer sums, so the result does not
 * depend on the order in which workgroups add their histograms).
 */
int ep_compute_send_counts(const int64_t* topk_idx, int64_t num_tokens,
                           int num_topk, int num_ranks, int num_local_experts,
                           int num_chunks, int32_t* dest, uint8_t* is_in_rank,
                           int32_t* send_counts, int32_t* tokens_per_expert,
                           int32_t* diag, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Stable destination-major send layout.
 * axolotl "torch_dispatch": build_send_layout and the module overview (each
 * token is sent once to every destination owning one of its experts, with a
 * K-wide table of local expert ids, -1 on slots owned elsewhere, and fp32
 * weights, 0 on those slots).
 *
 * Rows are ordered by destination, then by ascending token.  With
 * seg[p] = send_counts[0] + ... + send_counts[p-1], the pair (t, p) takes row
 * n = seg[p] + #{t' < t : is_in_rank[t', p]}, and the call writes
 *   send_token_idx[n] = t, send_rank[n] = p,
 *   send_idx[n,k] = topk_idx[t,k] - p*E_local where dest[t,k] == p, else -1,
 *   send_w[n,k]   = topk_weights[t,k]           where dest[t,k] == p, else 0,
 *   token_row[t,k] = n where dest[t,k] == p (row of slot k's owner), -1 for
 *   unrouted slots.
 *
 *   topk_idx, topk_weights  [T,K] int64 / fp32 in
 *   dest                    [T,K] int32 in   from ep_compute_send_counts
 *   send_counts             [P]   int32 in   counts of these T tokens (one
 *                                            chunk's row of the [C,P] array)
 *   num_send_capacity       rows available in the four send arrays; the exact
 *                           N = sum(send_counts) (a host copy of the counts)
 *                           or a bound such as T*min(K,P) that needs no sync.
 *                           Rows >= capacity are not written.  Rows in
 *                           [N, capacity) are left untouched.
 *   send_token_idx, send_rank [cap] int32 out; send_idx [cap,K] int32 out;
 *   send_w [cap,K] fp32 out; token_row [T,K] int32 out
 *   workspace               ep_layout_workspace_bytes(T, P) bytes (see there)
 * The membership flags (is_in_rank) are implied by dest and are not read.
 */
int ep_build_send_layout(const int64_t* topk_idx, const float* topk_weights,
                         const int32_t* dest, const int32_t* send_counts,
                         int64_t num_tokens, int num_topk, int num_ranks,
                         int num_local_experts, int64_t num_send_capacity,
                         int32_t* send_token_idx, int32_t* send_rank,
                         int32_t* send_idx, float* send_w, int32_t* token_row,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Bytes of workspace ep_dispatch_layout needs: a 256-byte header (uint32
 * words: [0] barrier arrivals, counted on over all calls, [2] the count at
 * the end of the last call, [3] error flags: bit 0 = a barrier wait gave
 * up) followed by G rows of P + E + 1 uint32 (one per
 * workgroup), G rows of P uint32 (per-workgroup prefixes) and P uint32
 * (totals), G = min(ceil(T/tile), 256) with tiles of 64 tokens for T <= 4096,
 * 128 for T <= 8192, 256 above.  Zero-filled once before first use;
 * every call leaves it ready for the next; calls that may overlap in time
 * must use different workspaces.
 */
size_t ep_dispatch_layout_workspace_bytes(int64_t num_tokens, int num_ranks,
                                          int num_local_experts);

/*
 * Counts and send layout in one launch: the outputs of
 * ep_compute_send_counts (one chunk) and of ep_build_send_layout, bit for
 * bit the same, without the host seeing the counts in between.
 * axolotl "torch_dispatch": compute_send_counts + build_send_layout (the
 * module overview's send layout); NeMo "uccl_ep.buffer":
 * Buffer.get_dispatch_layout.
 *
 *   topk_idx, topk_weights      [T,K] int64 / fp32 in
 *   num_send_capacity           rows the send arrays hold; pairs past it are
 *                               not written and their slots get token_row -1
 *                               (T*min(K,P) always suffices)
 *   dest, is_in_rank, send_counts [P], tokens_per_expert [E] (may be NULL),
 *   diag (may be NULL)          as ep_compute_send_counts with C = 1
 *   send_token_idx, send_rank, send_idx, send_w, token_row
 *                               as ep_build_send_layout
 *   workspace                   ep_dispatch_layout_workspace_bytes(T, P, E_local)
 * The launch uses at most one workgroup per compute unit and one grid-wide
 * barrier; the workgroups must be able to run at the same time, which holds
 * unless other work keeps the device full for the barrier's whole time-out,
 * after which the call gives up, sets EP_WS_WAIT_GAVE_UP in the workspace
 * header (ep_workspace_status reports it) and its outputs are undefined.
 * Returns
 * EP_ERR_UNSUPPORTED when a workgroup's LDS share (P, E and the tiles per
 * workgroup) would exceed 64 KiB; the two separate calls cover those sizes.
 */
int ep_dispatch_layout(const int64_t* topk_idx, const float* topk_weights,
                       int64_t num_tokens, int num_topk, int num_ranks,
                       int num_local_experts, int64_t num_send_capacity,
                       int32_t* dest, uint8_t* is_in_rank, int32_t* send_counts,
                       int32_t* tokens_per_expert, int32_t* diag,
                       int32_t* send_token_idx, int32_t* send_rank,
                       int32_t* send_idx, float* send_w, int32_t* token_row,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * ep_dispatch_layout for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same outputs
 * bit for bit.  Its workspace is the library's own scratch, a static device
 * array of EPDC_NOALLOC_SCRATCH_BYTES on each GPU, held until the process
 * ends; the first call on a GPU looks up its address and clears its control
 * header (one small kernel on `stream`).  No call allocates or frees memory.
 * Calls whose workspace would need more (ep_dispatch_layout_workspace_bytes
 * above the limit; at P = 32 and E = 256 the need is about 82 KiB) return
 * EP_ERR_WORKSPACE.  Every call on one GPU shares that GPU's scratch, so
 * calls that may overlap in time on one GPU (other streams, other host
 * threads) race and must not be made; ep_workspace_status(NULL, ...)
 * reports its error word.
 */
int ep_dispatch_layout_noalloc(const int64_t* topk_idx, const float* topk_weights,
                               int64_t num_tokens, int num_topk, int num_ranks,
                               int num_local_experts, int64_t num_send_capacity,
                               int32_t* dest, uint8_t* is_in_rank, int32_t* send_counts,
                               int32_t* tokens_per_expert, int32_t* diag,
                               int32_t* send_token_idx, int32_t* send_rank,
                               int32_t* send_idx, float* send_w, int32_t* token_row,
                               hipStream_t stream);

/*
 * Bytes of workspace ep_dispatch_layout_chunked needs: as
 * ep_dispatch_layout's with C*P bins and no expert totals (G rows of
 * C*P + 1 uint32, G rows of C*P uint32 and C*P uint32 after the 256-byte
 * header).  0 for invalid sizes or C*P > 1024.
 */
size_t ep_dispatch_layout_chunked_workspace_bytes(int64_t num_tokens, int num_ranks,
                                                  int num_chunks);

/*
 * The counts of every chunk and the send layouts of all chunks in one
 * launch (the no-sync path of a chunked dispatch).
 * axolotl "torch_dispatch": chunk_bounds, dispatch_chunked_forward (the
 * split counts of every chunk from one count pass; each chunk dispatched
 * on its own), compute_send_counts, build_send_layout.
 *
 * Chunk c is tokens [c*(T/C), (c+1)*(T/C)), the last chunk ending at T.
 * The outputs are those of ep_compute_send_counts with C chunks (without
 * tokens_per_expert) and, for every chunk, those of ep_build_send_layout
 * on that chunk's tokens with capacity chunk_capacity, laid end to end:
 *   dest [T,K], is_in_rank [T,P]   as ep_compute_send_counts
 *   send_counts [C,P]              per chunk and destination
 *   send_token_idx, send_rank      [C*chunk_capacity] int32: chunk c's rows
 *   send_idx, send_w               [C*chunk_capacity, K]: from row
 *                                  c*chunk_capacity on, numbered within the
 *                                  chunk; send_token_idx counts from the
 *                                  chunk's first token
 *   token_row [T,K]                the slot's row within its chunk, -1 for
 *                                  unrouted slots and rows past the capacity
 *   diag                           as ep_compute_send_counts (may be NULL)
 * chunk_capacity >= (tokens of the largest chunk) * min(K, P) always
 * suffices.  Limits: C*P <= 1024 bins, C*chunk_capacity*K fits int32; the
 * one-launch rules of ep_dispatch_layout (grid barrier, time-out,
 * EP_ERR_UNSUPPORTED when the LDS share would pass 64 KiB) apply.
 */
int ep_dispatch_layout_chunked(const int64_t* topk_idx, const float* topk_weights,
                               int64_t num_tokens, int num_topk, int num_ranks,
                               int num_local_experts, int num_chunks, int64_t chunk_capacity,
                               int32_t* dest, uint8_t* is_in_rank, int32_t* send_counts,
                               int32_t* diag, int32_t* send_token_idx, int32_t* send_rank,
                               int32_t* send_idx, float* send_w, int32_t* token_row,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of workspace ep_regroup_by_expert needs for R received rows and
 * num_bins = num_groups * E_local bins: a 256-byte header (as
 * ep_dispatch_layout's), G rows of num_bins + 1 uint32, G rows of num_bins
 * uint32 and num_bins uint32, G = min(256, ceil(R / tile)) with tiles of
 * 64 * w rows, w the smallest power of two up to 16 with 64 * 64 * w >= R.
 * Same zero-once / no-overlap rules.
 */
size_t ep_regroup_workspace_bytes(int64_t num_rows, int num_bins);

/*
 * Receive side: the received rows regrouped so that each local expert's rows
 * are contiguous, each expert's segment padded to a multiple of `align`.
 * NeMo "token_dispatcher": MoEFlexTokenDispatcher.dispatch_postprocess,
 * _DeepepManager.get_permuted_hidden_states_by_experts,
 * TokenDispatcherConfig.moe_router_expert_pad_multiple; NeMo
 * "uccl_ep.buffer": Buffer.dispatch expert_alignment.
 *
 * The rows may be several receive buffers laid end to end (on one GPU: the
 * P destination segments of a send buffer): row_group[r] in
 * [0, num_groups) names the buffer of row r, and the bins are (group, local
 * expert), group-major; with num_groups == 1 row_group may be NULL.  For
 * every bin in order, each row r of its group whose recv_idx names its
 * expert (in ascending r) takes the next row of the bin's segment; the
 * segment then gets zero rows up to a multiple of align.  So the result is
 * the regroups of the buffers one after the other.  The inverse (expert
 * outputs back to the received rows) is ep_combine with token_row = row_map
 * and the received weights (or none).
 *
 *   recv_x        [R,H] bf16 in
 *   recv_idx      [R,K] int32 in   local expert ids, -1 = not local;
 *                                  values outside [-1, E_local) are ignored
 *   recv_w        [R,K] fp32 in, or NULL (then perm_w may be NULL too)
 *   row_group     [R] int32 in, or NULL when num_groups == 1
 *   align         >= 1
 *   capacity      rows perm_x / perm_src / perm_w hold; rows past it are
 *                 not written and their slots get row_map -1
 *                 (R*min(K,E_local) + bins*(align-1) always suffices)
 *   perm_x        [capacity,H] bf16 out   rows past offsets[bins] untouched
 *   perm_src      [capacity] int32 out    source row, -1 on padding
 *   perm_w        [capacity] fp32 out     the slot's weight, 0 on padding
 *                                         (may be NULL)
 *   tokens_per_expert [bins] int32 out    rows per bin, without padding
 *   expert_offsets    [bins+1] int32 out  aligned segment starts; the last
 *                                         entry is the total row count
 *   row_map       [R,K] int32 out  regrouped row of each local slot, else -1
 *   workspace     ep_regroup_workspace_bytes(R, bins) bytes
 * One launch with a grid barrier (as ep_dispatch_layout: same time-out and
 * EP_ERR_UNSUPPORTED rule) for the counts, offsets, row_map, perm_src and
 * perm_w (padding included), then one launch that writes the rows of perm_x
 * in address order (each its source row, or zeros).
 */
int ep_regroup_by_expert(const void* recv_x, const int32_t* recv_idx,
                         const float* recv_w, const int32_t* row_group,
                         int num_groups, int64_t num_rows, int num_topk,
                         int hidden, int num_local_experts, int align,
                         int64_t capacity, void* perm_x, int32_t* perm_src,
                         float* perm_w, int32_t* tokens_per_expert,
                         int32_t* expert_offsets, int32_t* row_map,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Row permute into the send buffer (optionally quantizing to fp8).
 * axolotl "torch_dispatch": dispatch (row n of the send buffer is hidden row
 * send_token_idx[n]); NeMo "uccl_ep.buffer": Buffer.dispatch /
 * low_latency_dispatch for the fp8 form ([.., H] float8_e4m3fn plus
 * [.., H/128] float scales).
 *
 * Works token by token: hidden row t is read once and stored to every
 * distinct row token_row[t,k] >= 0 (which must be < capacity; others are
 * skipped).  That is exactly send_x[n] = x[send_token_idx[n]] for every
 * written row.
 *
 *   x           [T,H] bf16 in
 *   token_row   [T,K] int32 in   from ep_build_send_layout
 *   out_dtype   EP_DTYPE_BF16: send_x [cap,H] bf16, bit-exact copies;
 *               EP_DTYPE_FP8_E4M3: send_x [cap,H] uint8 e4m3 codes and
 *               send_scale [cap,H/128] fp32.  Per row and group g of 128
 *               channels: amax = max |x|, scale = fp32(amax / 448),
 *               code = e4m3(fp32(x / scale)) rounded to nearest, ties to
 *               even, saturating at +-448, sign kept; amax == 0 gives
 *               scale 0 and codes 0x00.  Non-finite inputs: NaN elements
 *               do not count toward amax and give the NaN code 0x7F; a
 *               group holding an infinity gets an infinite scale (finite
 *               elements then give zeros, infinite ones 0x7F).
 *   send_scale  NULL for bf16.
 */
int ep_dispatch_permute(const void* x, int64_t num_tokens, int hidden,
                        const int32_t* token_row, int num_topk,
                        int64_t num_send_capacity, int out_dtype, void* send_x,
                        float* send_scale, hipStream_t stream);

/*
 * Expert-batched layout [E_local, max_num_tokens, H].
 * vLLM "fused_moe.prepare_finalize": BatchedPrepareAndFinalize.prepare (the
 * buffer is zero-filled; the tokens that name local expert e in any slot take
 * slots 0, 1, ... in ascending token order; tokens_per_expert holds the
 * counts).
 *
 *   x                  [T,H] bf16 in
 *   topk_idx           [T,K] int64 in
 *   first_expert       global id of local expert 0 (rank * E_local)
 *   b_x                [E_local, max_num_tokens, H] bf16 out; every row past
 *                      an expert's count is written with zeros
 *   tokens_per_expert  [E_local] int32 out  true counts (may exceed max;
 *                      slots >= max_num_tokens are then dropped)
 *   token_row          [T,K] int32 out  e*max_num_tokens + slot for local
 *                      slots, -1 otherwise (and for dropped slots)
 *   workspace          ep_batched_workspace_bytes(T, E_local, max) bytes
 */
int ep_batched_prepare(const void* x, const int64_t* topk_idx,
                       int64_t num_tokens, int num_topk, int hidden,
                       int first_expert, int num_local_experts,
                       int64_t max_num_tokens, void* b_x,
                       int32_t* tokens_per_expert, int32_t* token_row,
                       void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * Expert-batched layout with fp8 rows: [E_local, max_num_tokens, H] e4m3
 * codes plus one scale per 128 channels.
 * NeMo "uccl_ep.buffer": Buffer.low_latency_dispatch with use_fp8 (rows
 * [E_local, max, H] float8_e4m3fn; scales [E_local, max, H/128] float, or
 * with use_ue8m0 packed [E_local, max, H/512] int; round_scale makes the
 * scales powers of two; the last two dimensions of the scales may be stored
 * column-major); vLLM "fused_moe.prepare_finalize":
 * BatchedPrepareAndFinalize.prepare, quantized branch (zeroed buffers, the
 * rows of each expert quantized per token with groups of 128 channels).
 *
 * The slots, counts and token_row are those of ep_batched_prepare; slot s of
 * expert e holds the quantized row of its token.  Per row and group g of 128
 * channels: amax = max |x|, s = fp32(amax / 448), and
 *   EP_SCALE_F32    scale = s, stored as fp32 [E_local, max, H/128];
 *   EP_SCALE_POW2   scale = the smallest power of two >= s, stored as fp32;
 *   EP_SCALE_UE8M0  the same power 2^e stored as the byte max(e + 127, 0)
 *                   (so scales below 2^-127 become 2^-127), four bytes per
 *                   int32 (groups 4j..4j+3 of word j, 4j in the low byte):
 *                   [E_local, max, H/512] int32; H must be a multiple of 512.
 * code = e4m3(fp32(x / scale)) with scale the stored value (2^(byte-127) for
 * UE8M0), rounded to nearest, ties to even, saturating at +-448, sign kept;
 * amax == 0 gives codes 0x00 and scale 0 (byte 0).  Non-finite inputs as in
 * ep_dispatch_permute; an infinite scale is stored as such (UE8M0 byte 0xFF).
 * Every padding slot (past an expert's count) gets zero codes and zero
 * scale words, each byte written once.
 *
 *   x                  [T,H] bf16 in
 *   topk_idx           [T,K] int64 in
 *   first_expert       global id of local expert 0
 *   scale_fmt          EP_SCALE_F32, EP_SCALE_POW2 or EP_SCALE_UE8M0
 *   scale_col_major    0: b_scale row-major [E_local, max, units];
 *                      1: each expert's block stored as [units, max], i.e.
 *                      word u of slot s of expert e at (e*units + u)*max + s
 *                      (units = H/128, or H/512 for UE8M0)
 *   b_q                [E_local, max_num_tokens, H] uint8 out (16-byte aligned)
 *   b_scale            the scale words described above, out
 *   tokens_per_expert  [E_local] int32 out  true counts (may exceed max)
 *   token_row          [T,K] int32 out  e*max_num_tokens + slot, or -1
 *   workspace          ep_batched_workspace_bytes(T, E_local, max) bytes
 */
int ep_batched_prepare_fp8(const void* x, const int64_t* topk_idx,
                           int64_t num_tokens, int num_topk, int hidden,
                           int first_expert, int num_local_experts,
                           int64_t max_num_tokens, int scale_fmt,
                           int scale_col_major, void* b_q, void* b_scale,
                           int32_t* tokens_per_expert, int32_t* token_row,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Combine back onto the source tokens, weighted or as per-destination
 * partial sums, with optional biases.
 * axolotl "torch_dispatch": module overview and combine (the local kernel
 * weights and sums over its slots; combine sums the per-destination partial
 * outputs); NeMo "uccl_ep.buffer": Buffer.combine (topk_weights optional,
 * bias: one tensor or a pair) / low_latency_combine; vLLM
 * BatchedPrepareAndFinalize.finalize; NeMo token_dispatcher
 * TokenDispatcherConfig.moe_router_dtype (fp32 for the weighted average).
 *
 * With topk_weights:
 *   out[t,:] = bf16( sum_{k=0..K-1, r = token_row[t,k] >= 0} w[t,k] * y[r,:]
 *                    + bias0[t,:] + bias1[t,:] )
 * each product rounded to fp32, then added to the running fp32 sum (starting
 * at +0.0) in ascending k.  Without (topk_weights == NULL): each distinct row
 * of token t is added once, in the order of its first slot.  The biases that
 * are given are added after the expert terms, bias0 first; the sum is rounded
 * once to bf16, to nearest with ties to even (past the largest bf16: an
 * infinity; a NaN stays a quiet NaN, sign and payload unspecified).  Rows
 * r >= num_rows are skipped.  Tokens with no row give +0 (plus the biases).
 *
 *   y             [num_rows, H] bf16 in   expert outputs (send rows, or the
 *                                         batched buffer viewed as rows)
 *   token_row     [T,K] int32 in
 *   topk_weights  [T,K] fp32 in, or NULL for the unweighted partial sums
 *   bias0, bias1  [T,H] bf16 in, or NULL (16-byte aligned)
 *   out           [T,H] bf16 out
 * The launch shape follows from num_rows, with the same results either way:
 * when num_rows < 2T, or num_rows > K*T (a padded buffer such as the
 * expert-batched one, whose tokens read only their local experts' rows), a
 * workgroup walks a token's rows one after another with several 16-byte
 * pieces per thread; otherwise it loads all of a token's rows at once, one
 * piece per thread.
 */
int ep_combine(const void* y, int64_t num_rows, const int32_t* token_row,
               const float* topk_weights, int64_t num_tokens, int num_topk,
               int hidden, const void* bias0, const void* bias1, void* out,
               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* EPDC_H */
