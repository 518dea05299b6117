// Routing histograms and the stable counting-sort scatters that build the
// send layout and the expert-batched layout (gfx950, wave64).
//
// Counts (axolotl "torch_dispatch": compute_send_counts; NeMo
// "uccl_ep.buffer": Buffer.get_dispatch_layout): one thread per token decodes
// its K slots; destination membership is counted per wave with one ballot per
// destination bin and a popcount, experts with LDS atomics.  Each workgroup
// adds its non-zero LDS bins into accumulators in the workspace; the
// workgroup that finishes last copies them out and clears them, so the call
// is one launch and leaves the workspace zeroed for the next call.
//
// Layouts (axolotl build_send_layout; vLLM BatchedPrepareAndFinalize.prepare):
// a single-pass scan with decoupled lookback over tiles of 256 tokens, one
// workgroup of 4 waves per tile.  Tiles are taken from an atomic ticket, so
// every tile a workgroup waits on belongs to one that is already running.
// Each wave ranks its tokens inside each bin with a ballot and a popcount; the
// workgroup publishes the tile's per-bin aggregate, looks back over earlier
// tiles (64 at a time, one lane per tile), publishes its inclusive prefix,
// then writes each token's send rows (token-major: a thread loops over the
// destinations of its own token).  Status words carry the call's epoch, so the workspace never needs
// clearing between calls.  The code is kept compact on purpose: a fully
// unrolled lookback grows the kernel past the instruction cache, and then
// instruction fetch, not memory, sets its duration.
#include "epdc_device.h"
#include "epdc_launch.h"

namespace epdc {

namespace {

// Polls per lookback window before the wait gives up (each an agent-scope
// load of the window plus a short sleep: on the order of a second).
constexpr uint32_t kSpinLimit = 1u << 22;
constexpr int kLookGroup = 8;               // bins whose lookback loads a wave overlaps

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ---------------------------------------------------------------------------
// Counts.  Grid (tiles per chunk, C); the workgroup of chunk c covers tokens
// [c*chunk + bx*256, ...) clipped to the chunk, so none spans two chunks.
// ---------------------------------------------------------------------------
template <int KMAX>
__global__ __launch_bounds__(kBlock) void counts_kernel(CountArgs a) {
  extern __shared__ int32_t s_hist[];  // [P] destinations, [E] experts, [1] bad ids
  __shared__ bool s_last;
  const int c = blockIdx.y;
  const int64_t cs = int64_t(c) * a.chunk;
  const int64_t ce = (c == a.C - 1) ? a.T : cs + a.chunk;
  const int64_t t0 = cs + int64_t(blockIdx.x) * kBlock;
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
        d[k] = e[k] / a.E_local;
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
    const uint64_t col = wave_bin_ballots(m);
    if (lane < nwin && col != 0) atomicAdd(&s_hist[w0 + lane], int(__popcll(col)));
  }
  if (want_e) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (e[k] >= 0) atomicAdd(&s_hist[a.P + e[k]], 1);
  }
  if (bad) atomicAdd(&s_hist[n_hist - 1], bad);
  __syncthreads();

  int32_t* acc = a.accum + int64_t(c) * n_hist;
  for (int i = threadIdx.x; i < n_hist; i += kBlock) {
    const int v = s_hist[i];
    if (v != 0) atomicAdd(&acc[i], v);
  }
  // Wait until this thread's adds are performed, then count the workgroup
  // done.  The accumulators are only touched by device-scope atomics, so no
  // cache writeback is needed to publish them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = fetch_add_relaxed(&a.ctrl[0], 1u) == gridDim.x * gridDim.y - 1;
  __syncthreads();
  if (!s_last) return;

  // Last workgroup: copy the accumulators out and clear them for the next call.
  uint32_t* accu = reinterpret_cast<uint32_t*>(a.accum);
  for (int64_t i = threadIdx.x; i < int64_t(a.C) * n_hist; i += kBlock) {
    const int cc = int(i / n_hist);
    const int bin = int(i - int64_t(cc) * n_hist);
    const int v = int(ld_relaxed(accu + i));
    if (bin < a.P)
      a.send_counts[int64_t(cc) * a.P + bin] = v;
    else if (bin < n_hist - 1)
      a.tokens_per_expert[int64_t(cc) * a.E + (bin - a.P)] = v;
  }
  if (a.diag && threadIdx.x == 0) {
    uint32_t sum = 0;
    for (int cc = 0; cc < a.C; ++cc) sum += ld_relaxed(accu + int64_t(cc) * n_hist + n_hist - 1);
    a.diag[0] = int(sum);
  }
  __syncthreads();
  for (int64_t i = threadIdx.x; i < int64_t(a.C) * n_hist; i += kBlock) st_relaxed(accu + i, 0u);
  if (threadIdx.x == 0) st_relaxed(&a.ctrl[0], 0u);
}

// ---------------------------------------------------------------------------
// Single-pass scan + stable scatter (send layout or batched layout).  One
// workgroup of 4 waves per tile of 256 tokens, one token per thread.
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
    s_tile = fetch_add_relaxed(&a.ctrl[kCtrlTicket], 1u);
    s_epoch = ld_relaxed(&a.ctrl[kCtrlEpoch]);
  }
  __syncthreads();
  const uint32_t tile = s_tile;
  const uint32_t epoch = s_epoch;
  const uint32_t tiles = gridDim.x;
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

  // Ballot of every bin per wave; lane j keeps the ballot of bin w0 + j.
  for (int w0 = 0; w0 < nb; w0 += kWave) {
    uint64_t m = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (bin[k] >= w0 && bin[k] < w0 + kWave) m |= uint64_t(1) << (bin[k] - w0);
    const int nwin = min(kWave, nb - w0);
    const uint64_t mine = wave_bin_ballots(m);
    if (lane < nwin) s_bal[wave * nb + w0 + lane] = mine;
  }
  // Segment starts of the send layout: exclusive scan of send_counts.
  if (MODE == kModeSend && wave == kWavesPerBlock - 1) {
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
  __syncthreads();

  // Tile count per bin and the waves' exclusive offsets; publish the tile's
  // aggregate (tile 0 publishes its inclusive prefix directly).
  for (int b = tid; b < nb; b += kBlock) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      s_woff[w * nb + b] = run;
      run += int(__popcll(s_bal[w * nb + b]));
    }
    s_cnt[b] = run;
    st_status(&a.status[size_t(b) * tiles + tile],
              pack_status(epoch, tile == 0 ? kFlagPrefix : kFlagAggregate, uint32_t(run)));
  }
  __syncthreads();

  // Decoupled lookback; the waves share the bins (wave w takes bins w, w+4,
  // ...), kLookGroup at a time.  For one bin, lane j reads the status word of
  // tile (base - j), so 64 predecessors arrive in one coalesced load; the
  // window adds aggregates up to the nearest inclusive prefix or moves 64
  // tiles further back.
  for (int g0 = wave; g0 < nb; g0 += kWavesPerBlock * kLookGroup) {
    uint32_t excl[kLookGroup];
    int64_t base[kLookGroup];
    bool done[kLookGroup];
#pragma unroll
    for (int g = 0; g < kLookGroup; ++g) {
      done[g] = g0 + kWavesPerBlock * g >= nb || tile == 0;
      excl[g] = 0;
      base[g] = int64_t(tile) - 1;
    }
    uint32_t spins = 0;
    while (true) {
      uint64_t w[kLookGroup];
#pragma unroll
      for (int g = 0; g < kLookGroup; ++g) {
        const int64_t j = base[g] - lane;
        w[g] = pack_status(epoch, kFlagPrefix, 0u);
        if (!done[g] && j >= 0)
          w[g] = ld_status(&a.status[size_t(g0 + kWavesPerBlock * g) * tiles + size_t(j)]);
      }
      bool pending = false, waiting = false;
#pragma unroll
      for (int g = 0; g < kLookGroup; ++g) {
        if (done[g]) continue;
        const uint32_t f = status_epoch(w[g]) == epoch ? status_flag(w[g]) : kFlagNone;
        const uint64_t pm = ballot(f == kFlagPrefix);
        const uint64_t xm = ballot(f == kFlagNone);
        const int fp = pm ? int(__builtin_ctzll(pm)) : kWave;          // nearest prefix
        const uint64_t upto = fp >= kWave - 1 ? ~uint64_t(0) : ((uint64_t(2) << fp) - 1);
        if (xm & upto) {                       // a tile in the window has not published
          pending = waiting = true;
          continue;
        }
        excl[g] += wave_sum(lane <= fp ? status_value(w[g]) : 0u);
        if (pm) {
          done[g] = true;
        } else {
          base[g] -= kWave;
          pending = true;
        }
      }
      if (!pending) break;
      if (waiting) {
        if (++spins > kSpinLimit) {
          if (lane == 0) fetch_or(&a.ctrl[kCtrlError], kErrLookbackGaveUp);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
#pragma unroll
    for (int g = 0; g < kLookGroup; ++g) {
      const int b = g0 + kWavesPerBlock * g;
      if (b < nb && lane == 0) {
        if (tile > 0)
          st_status(&a.status[size_t(b) * tiles + tile],
                    pack_status(epoch, kFlagPrefix, excl[g] + uint32_t(s_cnt[b])));
        s_excl[b] = int(excl[g]);
      }
    }
  }
  __syncthreads();

  // Row of every routed slot: segment start + earlier tiles + earlier waves
  // + lower lanes of this wave that share the bin.
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
  if (valid) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < a.K) a.token_row[t * a.K + k] = rowk[k];
  }

  // Send layout, token-major: each thread writes the send row of every
  // destination its token reaches (the first slot of each destination).
  if (MODE == kModeSend) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      bool first = bin[k] >= 0 && rowk[k] >= 0;
#pragma unroll
      for (int j = 0; j < k; ++j)
        if (bin[j] == bin[k]) first = false;
      if (!first) continue;
      const int b = bin[k];
      const int32_t n = rowk[k];
      a.send_token_idx[n] = int32_t(t);
      a.send_rank[n] = b;
      const int64_t ob = int64_t(b) * a.E_local;
      int32_t* irow = a.send_idx + int64_t(n) * a.K;
      float* wrow = a.send_w + int64_t(n) * a.K;
#pragma unroll
      for (int kk = 0; kk < KMAX; kk += 4) {
        if (kk >= a.K) break;
        int32_t iv[4];
        float wv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool own = bin[kk + q] == b;
          iv[q] = own ? int32_t(ids[kk + q] - ob) : -1;
          wv[q] = own ? wts[kk + q] : 0.0f;
        }
        if (a.vec_rows) {
          *reinterpret_cast<u32x4*>(irow + kk) =
              u32x4{uint32_t(iv[0]), uint32_t(iv[1]), uint32_t(iv[2]), uint32_t(iv[3])};
          *reinterpret_cast<u32x4*>(wrow + kk) =
              u32x4{__float_as_uint(wv[0]), __float_as_uint(wv[1]), __float_as_uint(wv[2]),
                    __float_as_uint(wv[3])};
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (kk + q < a.K) {
              irow[kk + q] = iv[q];
              wrow[kk + q] = wv[q];
            }
          }
        }
      }
    }
  }

  // The last tile holds the totals of the batched layout.
  if (MODE == kModeBatched && tile == tiles - 1) {
    for (int b = tid; b < nb; b += kBlock) a.tokens_per_expert[b] = s_excl[b] + s_cnt[b];
  }

  // The workgroup that finishes last rearms the workspace for the next call
  // (the next launch sees these stores: kernel boundaries order memory).
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = fetch_add_relaxed(&a.ctrl[kCtrlDone], 1u);
    if (prev == tiles - 1) {
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
  const int64_t longest = a.T - int64_t(a.C - 1) * a.chunk;  // the last chunk
  int64_t gx = (longest + kBlock - 1) / kBlock;
  if (gx < 1) gx = 1;              // empty input: one workgroup still writes zeros
  const dim3 grid(unsigned(gx), unsigned(a.C));
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
  // At least one tile, so that an empty batch still reports zero counts.
  const int64_t tiles = num_tiles(a.T) > 0 ? num_tiles(a.T) : 1;
  return launch_scan<kModeBatched>(a, s, unsigned(tiles));
}

namespace {
// The error word of a workspace header handed to the caller and cleared in
// one atomic exchange, so a flag set by a later call is never lost.
__global__ void workspace_status_kernel(uint32_t* ctrl, int32_t* flags) {
  if (threadIdx.x == 0)
    flags[0] = int32_t(__hip_atomic_exchange(&ctrl[kCtrlError], 0u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}

// Zero the 256-byte control header of a workspace (one word per thread).
__global__ void clear_header_kernel(uint32_t* ctrl) {
  if (threadIdx.x < kWsHeaderBytes / 4) ctrl[threadIdx.x] = 0u;
}
}  // namespace

hipError_t launch_workspace_status(uint32_t* ctrl, int32_t* flags, hipStream_t s) {
  workspace_status_kernel<<<1, kWave, 0, s>>>(ctrl, flags);
  return hipGetLastError();
}

hipError_t launch_clear_header(uint32_t* ctrl, hipStream_t s) {
  clear_header_kernel<<<1, kWsHeaderBytes / 4, 0, s>>>(ctrl);
  return hipGetLastError();
}

}  // namespace epdc
