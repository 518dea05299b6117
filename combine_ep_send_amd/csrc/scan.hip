// Routing histograms and the stable counting-sort scatters that build the
// send layout and the expert-batched layout (gfx950, wave64).
//
// Counts (axolotl "torch_dispatch": compute_send_counts; NeMo
// "uccl_ep.buffer": Buffer.get_dispatch_layout): one thread per token decodes
// its K slots; destination membership is counted per wave with one ballot per
// destination bin and a popcount, experts with LDS atomics; each workgroup
// then adds its LDS histogram to the global counts with one atomic per bin.
//
// Layouts (axolotl build_send_layout; vLLM BatchedPrepareAndFinalize.prepare):
// a single-pass scan with decoupled lookback.  Workgroups take tiles of 256
// tokens from an atomic ticket (so every tile a workgroup waits on belongs to
// a workgroup that is already running), rank their tokens inside each bin with
// ballots, publish the tile's per-bin aggregate, then walk back over earlier
// tiles' status words until an inclusive prefix is found.  The status words
// carry the call's epoch, so the workspace never needs clearing between calls.
#include "epdc_device.h"
#include "epdc_launch.h"

namespace epdc {

namespace {

constexpr uint32_t kSpinLimit = 1u << 22;   // sleeps per lookback step (~0.1 s)

__global__ __launch_bounds__(kBlock) void zero3_kernel(int32_t* a, int64_t na, int32_t* b,
                                                       int64_t nb, int32_t* c, int64_t nc) {
  const int64_t i0 = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  const int64_t step = int64_t(gridDim.x) * kBlock;
  for (int64_t i = i0; i < na; i += step) a[i] = 0;
  for (int64_t i = i0; i < nb; i += step) b[i] = 0;
  for (int64_t i = i0; i < nc; i += step) c[i] = 0;
}

// ---------------------------------------------------------------------------
// Counts.  Grid (tiles per chunk, C); the block of chunk c covers tokens
// [c*chunk + bx*256, ...) clipped to the chunk, so no block spans chunks.
// ---------------------------------------------------------------------------
template <int KMAX>
__global__ __launch_bounds__(kBlock) void counts_kernel(CountArgs a) {
  extern __shared__ int32_t s_hist[];  // [P] destinations, [E] experts, [1] bad ids
  const int c = blockIdx.y;
  const int64_t cs = int64_t(c) * a.chunk;
  const int64_t ce = (c == a.C - 1) ? a.T : cs + a.chunk;
  const int64_t t0 = cs + int64_t(blockIdx.x) * kTile;
  if (t0 >= ce) return;  // the whole workgroup is past its chunk

  const bool want_e = a.tokens_per_expert != nullptr;
  const int n_hist = a.P + (want_e ? a.E : 0) + 1;
  for (int i = threadIdx.x; i < n_hist; i += kBlock) s_hist[i] = 0;
  __syncthreads();

  const int lane = lane_id();
  const int64_t t = t0 + threadIdx.x;
  const bool valid = t < ce;
  int d[KMAX];
  int e[KMAX];
  int bad = 0;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    d[k] = -1;
    e[k] = -1;
    if (valid && k < a.K) {
      const int64_t v = a.topk_idx[t * a.K + k];
      if (v >= 0 && v < a.E) {
        e[k] = int(v);
        d[k] = int(v / a.E_local);
      } else if (v != -1) {
        ++bad;
      }
    }
  }
  if (valid) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < a.K) a.dest[t * a.K + k] = d[k];
  }

  // Destination membership, 64 bins at a time.
  for (int w0 = 0; w0 < a.P; w0 += kWave) {
    uint64_t m = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (d[k] >= w0 && d[k] < w0 + kWave) m |= uint64_t(1) << (d[k] - w0);
    const int nwin = min(kWave, a.P - w0);
    if (valid) {
      uint8_t* row = a.is_in_rank + t * a.P + w0;
      if ((a.P & 3) == 0) {
        for (int j = 0; j < nwin; j += 4) {
          const uint32_t word = uint32_t((m >> j) & 1u) | (uint32_t((m >> (j + 1)) & 1u) << 8) |
                                (uint32_t((m >> (j + 2)) & 1u) << 16) |
                                (uint32_t((m >> (j + 3)) & 1u) << 24);
          *reinterpret_cast<uint32_t*>(row + j) = word;
        }
      } else {
        for (int j = 0; j < nwin; ++j) row[j] = uint8_t((m >> j) & 1u);
      }
    }
    for (int j = 0; j < nwin; ++j) {
      const uint64_t b = ballot((m >> j) & 1u);
      if (b != 0 && lane == 0) atomicAdd(&s_hist[w0 + j], int(__popcll(b)));
    }
  }
  if (want_e) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (e[k] >= 0) atomicAdd(&s_hist[a.P + e[k]], 1);
  }
  if (bad) atomicAdd(&s_hist[n_hist - 1], bad);
  __syncthreads();

  for (int i = threadIdx.x; i < n_hist; i += kBlock) {
    const int v = s_hist[i];
    if (v == 0) continue;
    if (i < a.P)
      atomicAdd(&a.send_counts[int64_t(c) * a.P + i], v);
    else if (i < n_hist - 1)
      atomicAdd(&a.tokens_per_expert[int64_t(c) * a.E + (i - a.P)], v);
    else if (a.diag)
      atomicAdd(a.diag, v);
  }
}

// ---------------------------------------------------------------------------
// Single-pass scan + stable scatter (send layout or batched layout).
// ---------------------------------------------------------------------------
enum { kModeSend = 0, kModeBatched = 1 };

template <int MODE, int KMAX>
__global__ __launch_bounds__(kBlock) void scan_kernel(ScanArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nb = a.bins;
  uint64_t* s_bal = reinterpret_cast<uint64_t*>(smem);                        // [4][nb]
  int32_t* s_woff = reinterpret_cast<int32_t*>(s_bal + kWavesPerBlock * nb);  // [4][nb]
  int32_t* s_cnt = s_woff + kWavesPerBlock * nb;                              // [nb]
  int32_t* s_excl = s_cnt + nb;                                               // [nb]
  int32_t* s_seg = s_excl + nb;                                               // [nb]
  __shared__ uint32_t s_tile, s_epoch;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  if (tid == 0) {
    s_tile = fetch_add(&a.ctrl[kCtrlTicket], 1u);
    s_epoch = ld_relaxed(&a.ctrl[kCtrlEpoch]);
  }
  __syncthreads();
  const uint32_t tile = s_tile;
  const uint32_t epoch = s_epoch;
  const int64_t t = int64_t(tile) * kTile + tid;
  const bool valid = t < a.T;

  // Bin of every slot: owning destination, or local expert index.
  int bin[KMAX];
  int64_t ids[KMAX];
  float wts[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    bin[k] = -1;
    ids[k] = -1;
    wts[k] = 0.0f;
    if (valid && k < a.K) {
      const int64_t v = a.topk_idx[t * a.K + k];
      ids[k] = v;
      if (MODE == kModeSend) {
        const int dd = a.dest[t * a.K + k];
        bin[k] = (dd >= 0 && dd < nb) ? dd : -1;
        wts[k] = a.topk_weights[t * a.K + k];
      } else {
        const int64_t le = v - a.first_expert;
        bin[k] = (v >= 0 && le >= 0 && le < nb) ? int(le) : -1;
      }
    }
  }

  // Per-wave ballot of every bin; lane j keeps the ballot of bin w0 + j.
  for (int w0 = 0; w0 < nb; w0 += kWave) {
    uint64_t m = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (bin[k] >= w0 && bin[k] < w0 + kWave) m |= uint64_t(1) << (bin[k] - w0);
    const int nwin = min(kWave, nb - w0);
    uint64_t mine = 0;
    for (int j = 0; j < nwin; ++j) {
      const uint64_t b = ballot((m >> j) & 1u);
      if (lane == j) mine = b;
    }
    if (lane < nwin) s_bal[wave * nb + w0 + lane] = mine;
  }
  __syncthreads();

  // Tile count per bin, exclusive offsets of the waves, and publication of
  // the tile's aggregate (tile 0 publishes its inclusive prefix directly).
  for (int b = tid; b < nb; b += kBlock) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      s_woff[w * nb + b] = run;
      run += int(__popcll(s_bal[w * nb + b]));
    }
    s_cnt[b] = run;
    st_release(&a.status[size_t(tile) * nb + b],
               pack_status(epoch, tile == 0 ? kFlagPrefix : kFlagAggregate, uint32_t(run)));
  }

  // Segment starts of the send layout: exclusive scan of send_counts.
  if (MODE == kModeSend && wave == 0) {
    int carry = 0;
    for (int b0 = 0; b0 < nb; b0 += kWave) {
      const int b = b0 + lane;
      const int v = (b < nb) ? a.send_counts[b] : 0;
      int incl = v;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int u = __shfl_up(incl, off);
        if (lane >= off) incl += u;
      }
      if (b < nb) s_seg[b] = carry + incl - v;
      carry += __shfl(incl, kWave - 1);
    }
  }

  // Decoupled lookback: one thread per bin sums earlier tiles' aggregates
  // until it meets an inclusive prefix, then publishes its own prefix.
  for (int b = tid; b < nb; b += kBlock) {
    uint32_t excl = 0;
    if (tile > 0) {
      int64_t j = int64_t(tile) - 1;
      uint32_t spins = 0;
      while (true) {
        const uint64_t w = ld_acquire(&a.status[size_t(j) * nb + b]);
        const uint32_t f = status_flag(w);
        if (status_epoch(w) != epoch || f == kFlagNone) {
          if (++spins > kSpinLimit) {
            fetch_or(&a.ctrl[kCtrlError], kErrLookbackGaveUp);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        spins = 0;
        excl += status_value(w);
        if (f == kFlagPrefix || j == 0) break;
        --j;
      }
      st_release(&a.status[size_t(tile) * nb + b],
                 pack_status(epoch, kFlagPrefix, excl + uint32_t(s_cnt[b])));
    }
    s_excl[b] = int(excl);
  }
  __syncthreads();

  // Stable scatter: a lane's rank inside bin b is the popcount of the lower
  // lanes in its wave's ballot, plus the earlier waves and tiles.
  const uint64_t lt = lanemask_lt();
  int32_t rowk[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    rowk[k] = -1;
    if (bin[k] >= 0) {
      const int b = bin[k];
      const int64_t rank = int64_t(s_excl[b]) + s_woff[wave * nb + b] +
                           __popcll(s_bal[wave * nb + b] & lt);
      if (MODE == kModeSend) {
        const int64_t n = s_seg[b] + rank;
        if (n < a.capacity) rowk[k] = int32_t(n);
      } else {
        if (rank < a.max_tokens) rowk[k] = int32_t(int64_t(b) * a.max_tokens + rank);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (rowk[k] < 0) continue;
    bool first = true;
#pragma unroll
    for (int j = 0; j < k; ++j)
      if (bin[j] == bin[k]) first = false;
    if (!first) continue;
    const int32_t n = rowk[k];
    const int b = bin[k];
    if (MODE == kModeSend) {
      a.send_token_idx[n] = int32_t(t);
      a.send_rank[n] = b;
      const int64_t ob = int64_t(b) * a.E_local;
#pragma unroll
      for (int kk = 0; kk < KMAX; ++kk) {
        if (kk < a.K) {
          const bool own = bin[kk] == b;
          a.send_idx[int64_t(n) * a.K + kk] = own ? int32_t(ids[kk] - ob) : -1;
          a.send_w[int64_t(n) * a.K + kk] = own ? wts[kk] : 0.0f;
        }
      }
    } else {
      a.slot_token[n] = int32_t(t);
    }
  }
  if (valid) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < a.K) a.token_row[t * a.K + k] = rowk[k];
  }

  // The last tile holds the totals of the batched layout.
  if (MODE == kModeBatched && tile == gridDim.x - 1) {
    for (int b = tid; b < nb; b += kBlock) a.tokens_per_expert[b] = s_excl[b] + s_cnt[b];
  }

  // The workgroup that finishes last rearms the workspace for the next call.
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = fetch_add(&a.ctrl[kCtrlDone], 1u);
    if (prev == gridDim.x - 1) {
      st_relaxed(&a.ctrl[kCtrlTicket], 0u);
      st_relaxed(&a.ctrl[kCtrlDone], 0u);
      st_relaxed(&a.ctrl[kCtrlEpoch], epoch + 1u);
    }
  }
}

inline size_t scan_smem_bytes(int bins) {
  return size_t(bins) * (kWavesPerBlock * 8 + kWavesPerBlock * 4 + 3 * 4);
}

template <int MODE>
hipError_t launch_scan(const ScanArgs& a, hipStream_t s, unsigned grid) {
  const size_t smem = scan_smem_bytes(a.bins);
  if (a.K <= 4)
    scan_kernel<MODE, 4><<<grid, kBlock, smem, s>>>(a);
  else if (a.K <= 8)
    scan_kernel<MODE, 8><<<grid, kBlock, smem, s>>>(a);
  else
    scan_kernel<MODE, 16><<<grid, kBlock, smem, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_counts(const CountArgs& a, hipStream_t s) {
  const int64_t n_sc = int64_t(a.C) * a.P;
  const int64_t n_te = a.tokens_per_expert ? int64_t(a.C) * a.E : 0;
  const int64_t n_dg = a.diag ? 1 : 0;
  const int64_t most = n_sc > n_te ? n_sc : n_te;
  unsigned zgrid = unsigned((most + kBlock - 1) / kBlock);
  if (zgrid < 1) zgrid = 1;
  if (zgrid > 1024) zgrid = 1024;
  zero3_kernel<<<zgrid, kBlock, 0, s>>>(a.send_counts, n_sc, a.tokens_per_expert, n_te, a.diag,
                                       n_dg);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.T == 0) return err;

  const int64_t longest = a.T - int64_t(a.C - 1) * a.chunk;  // the last chunk
  const unsigned gx = unsigned((longest + kTile - 1) / kTile);
  const dim3 grid(gx, unsigned(a.C));
  const size_t smem = size_t(a.P + (a.tokens_per_expert ? a.E : 0) + 1) * 4;
  if (a.K <= 4)
    counts_kernel<4><<<grid, kBlock, smem, s>>>(a);
  else if (a.K <= 8)
    counts_kernel<8><<<grid, kBlock, smem, s>>>(a);
  else
    counts_kernel<16><<<grid, kBlock, smem, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_send_layout(const ScanArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return launch_scan<kModeSend>(a, s, unsigned(num_tiles(a.T)));
}

hipError_t launch_batched_scan(const ScanArgs& a, hipStream_t s) {
  // At least one workgroup, so that an empty batch still reports zero counts.
  const int64_t tiles = num_tiles(a.T) > 0 ? num_tiles(a.T) : 1;
  return launch_scan<kModeBatched>(a, s, unsigned(tiles));
}

}  // namespace epdc
