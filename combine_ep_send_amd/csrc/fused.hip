// Counts and send layout in one launch (gfx950, wave64).
//
// axolotl "torch_dispatch": compute_send_counts + build_send_layout; NeMo
// "uccl_ep.buffer": Buffer.get_dispatch_layout.  Same outputs as the two
// separate calls, computed as reduce-then-scan with one grid-wide barrier:
//
//  1. Each workgroup owns a contiguous run of tiles (one token per thread:
//     64, 128 or 256 tokens, so that small inputs still spread over many
//     compute units).  It
//     decodes them (dest, is_in_rank), counts every tile's tokens per
//     destination with per-wave ballots, histograms experts in LDS, and
//     publishes its totals per destination / expert as one row.
//  2. Barrier: every workgroup has published.  The grid is at most one
//     workgroup per compute unit, so all of them are resident together.
//  3. Each workgroup reads the rows: the destination totals give the segment
//     starts, the rows of lower workgroups its base inside each segment.  A
//     slice of the experts is summed by every workgroup.  With many groups
//     and bins the rows are instead scanned bin by bin, one slice of bins
//     per workgroup, and read back after a second barrier; with chunks, a
//     workgroup reads only the rows of the groups its chunks span.
//  4. It ranks its tokens again and writes token_row and the send rows
//     token-major.
//
// Against the two-call path this removes one launch and the tile-to-tile
// lookback chain; only the barrier's round trip remains.
//
// The same kernel regroups received rows by local expert (NeMo
// token_dispatcher: dispatch_postprocess / get_permuted_hidden_states_by_
// experts; moe_router_expert_pad_multiple; uccl Buffer.dispatch
// expert_alignment): the bins are the local expert ids themselves, each
// expert's segment starts at the exclusive scan of the counts rounded up to
// the alignment, and each row records its source row and its slot's weight.
#include "epdc_device.h"
#include "epdc_launch.h"

namespace epdc {

namespace {

// Polls before a barrier wait gives up: each is an agent-scope load plus a
// short sleep, about 1.2 s in all on MI355X (measured with every workgroup
// waiting on a target set past reach).
constexpr uint32_t kBarrierSpinLimit = 1u << 22;

// Grid-wide barrier number k (1, 2, ...) of this launch.  The arrivals word
// counts on across calls: `base` is its value when the launch began (the
// previous call's last barrier leaves it in the generation word), so
// barrier k is complete once the count reaches base + k*G.  Thread 0 of
// every workgroup adds one arrival and, unless its own arrival completed the
// barrier, polls the count itself: the completing atomic publishes the
// barrier, with no separate store to wait for.  The launch's last barrier
// hands the final count to the next call.  A wait that outlasts the spin
// limit sets an error bit instead of hanging.
__device__ __forceinline__ void grid_sync(uint32_t* ctrl, int G, uint32_t base, uint32_t k,
                                          bool last) {
  __builtin_amdgcn_s_waitcnt(0);   // this thread's stores are performed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t target = base + k * uint32_t(G);
    if (fetch_add_relaxed(&ctrl[kCtrlTicket], 1u) + 1u == target) {
      if (last) st_relaxed(&ctrl[kCtrlEpoch], target);
    } else {
      uint32_t spins = 0;
      while (int32_t(ld_relaxed(&ctrl[kCtrlTicket]) - target) < 0) {
        if (++spins > kBarrierSpinLimit) {
          fetch_or(&ctrl[kCtrlError], kErrLookbackGaveUp);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  }
  __syncthreads();
}

// Exclusive prefix sum over the workgroup's threads (thread order); `total`
// receives the sum of all.  s_scan holds one word per wave.
template <int NW>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_scan,
                                                         uint32_t& total) {
  const int lane = lane_id();
  const int wave = wave_id();
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t u = __shfl_up(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == kWave - 1) s_scan[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = s_scan[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  return before + incl - v;
}

// One tile's slots: owning destination (bin), global id and weight.
template <int KMAX>
struct TileSlots {
  int bin[KMAX];
  int64_t ids[KMAX];
  float wts[KMAX];
  int bad;
  int cidx;     // chunk of the token (send mode with chunks), else 0
  int cbase;    // its first bin, cidx * ndest
};

enum { kFusedSend = 0, kFusedRegroup = 1 };

template <int MODE, int KMAX>
__device__ __forceinline__ void decode(const FusedArgs& a, int64_t t, bool valid,
                                       TileSlots<KMAX>& s) {
  s.bad = 0;
  s.cidx = 0;
  s.cbase = 0;
  if (MODE == kFusedRegroup) {
    // received rows: K-wide local expert ids (int32); the bin is the id,
    // offset by the row's group (the receive buffer it came from) when rows
    // of several buffers are laid end to end
    const int gbase = (valid && a.row_group) ? a.row_group[t] * a.E_local : 0;
    const bool gok = !a.row_group || (gbase >= 0 && gbase < a.P);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      s.ids[k] = -1;
      s.wts[k] = 0.0f;
      s.bin[k] = -1;
      if (valid && k < a.K) {
        const int v = a.ids32[t * a.K + k];
        s.ids[k] = v;
        if (a.topk_weights) s.wts[k] = a.topk_weights[t * a.K + k];
        if (v >= 0 && v < a.E_local && gok)
          s.bin[k] = gbase + v;
        else if (v != -1)
          ++s.bad;
      }
    }
    return;
  }
  if (valid && a.in_w >= 2 && a.K == KMAX) {
    // whole rows: ids as 16-byte pairs, weights as 16- or 8-byte pieces
    const u32x4* pi = reinterpret_cast<const u32x4*>(a.topk_idx + t * KMAX);
#pragma unroll
    for (int q = 0; q < KMAX / 2; ++q) {
      const u32x4 v = pi[q];
      s.ids[2 * q] = int64_t((uint64_t(v.y) << 32) | v.x);
      s.ids[2 * q + 1] = int64_t((uint64_t(v.w) << 32) | v.z);
    }
    if (KMAX % 4 == 0 && a.in_w == 4) {
      const u32x4* pw = reinterpret_cast<const u32x4*>(a.topk_weights + t * KMAX);
#pragma unroll
      for (int q = 0; q < KMAX / 4; ++q) {
        const u32x4 v = pw[q];
        s.wts[4 * q] = __uint_as_float(v.x);
        s.wts[4 * q + 1] = __uint_as_float(v.y);
        s.wts[4 * q + 2] = __uint_as_float(v.z);
        s.wts[4 * q + 3] = __uint_as_float(v.w);
      }
    } else {
      const u32x2* pw = reinterpret_cast<const u32x2*>(a.topk_weights + t * KMAX);
#pragma unroll
      for (int q = 0; q < KMAX / 2; ++q) {
        const u32x2 v = pw[q];
        s.wts[2 * q] = __uint_as_float(v.x);
        s.wts[2 * q + 1] = __uint_as_float(v.y);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      s.ids[k] = -1;
      s.wts[k] = 0.0f;
      if (valid && k < a.K) {
        s.ids[k] = a.topk_idx[t * a.K + k];
        s.wts[k] = a.topk_weights[t * a.K + k];
      }
    }
  }
  if (a.C > 1 && valid) {       // bins (chunk, destination), chunk-major
    uint32_t c = a.chunk > 0 ? uint32_t(t) / uint32_t(a.chunk) : uint32_t(a.C - 1);
    if (c > uint32_t(a.C - 1)) c = uint32_t(a.C - 1);
    s.cidx = int(c);
    s.cbase = int(c) * a.ndest;
  }
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int64_t v = s.ids[k];
    s.bin[k] = -1;
    if (v >= 0 && v < a.E)
      s.bin[k] = s.cbase + int(v) / a.E_local;
    else if (v != -1)
      ++s.bad;
  }
}

// One token's K int32 entries: when K == KMAX, as whole-row pieces of w
// words (16 or 8 bytes; w = 4 needs K % 4 == 0, w = 2 an even K), else one
// word per slot.
template <int KMAX>
__device__ __forceinline__ void store_row(int32_t* dst, const int (&v)[KMAX], int K, int w) {
  if (KMAX % 4 == 0 && K == KMAX && w == 4) {
#pragma unroll
    for (int q = 0; q < KMAX / 4; ++q)
      reinterpret_cast<u32x4*>(dst)[q] = u32x4{uint32_t(v[4 * q]), uint32_t(v[4 * q + 1]),
                                               uint32_t(v[4 * q + 2]), uint32_t(v[4 * q + 3])};
  } else if (KMAX % 2 == 0 && K == KMAX && w >= 2) {
#pragma unroll
    for (int q = 0; q < KMAX / 2; ++q)
      reinterpret_cast<u32x2*>(dst)[q] = u32x2{uint32_t(v[2 * q]), uint32_t(v[2 * q + 1])};
  } else {
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < K) dst[k] = v[k];
  }
}

// Per-wave ballots of every destination for one tile: s_bal[wave*P + b].
template <int KMAX>
__device__ __forceinline__ void ballots(const TileSlots<KMAX>& s, int P, int wave, int lane,
                                        uint64_t* s_bal) {
  for (int w0 = 0; w0 < P; w0 += kWave) {
    uint64_t m = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (s.bin[k] >= w0 && s.bin[k] < w0 + kWave) m |= uint64_t(1) << (s.bin[k] - w0);
    const int nwin = min(kWave, P - w0);
    const uint64_t mine = wave_bin_ballots(m);
    if (lane < nwin) s_bal[wave * P + w0 + lane] = mine;
  }
}

// Chunks of the send mode: chunk c holds tokens [c*chunk, (c+1)*chunk), the
// last one the rest (all of them when chunk is 0, i.e. fewer tokens than
// chunks).  chunk_first > chunk_last marks an empty chunk.
__device__ __forceinline__ int chunk_of(const FusedArgs& a, int64_t t) {
  const int64_t c = a.chunk > 0 ? t / a.chunk : int64_t(a.C - 1);
  return int(c < a.C - 1 ? c : a.C - 1);
}
__device__ __forceinline__ int64_t chunk_first(const FusedArgs& a, int c) {
  return int64_t(c) * a.chunk;
}
__device__ __forceinline__ int64_t chunk_last(const FusedArgs& a, int c) {
  return (c == a.C - 1 ? a.T : int64_t(c + 1) * a.chunk) - 1;
}

template <int MODE, int KMAX, int NW>
__global__ __launch_bounds__(NW * kWave) void dispatch_layout_kernel(FusedArgs a) {
  constexpr int BS = NW * kWave;        // threads per workgroup = tokens per tile
  extern __shared__ __align__(16) unsigned char smem[];
  const int P = a.P;                            // bins: destinations (x chunks)
  const int nh = a.P + a.hist_e + 1;            // published row: P bins, experts, bad
  uint64_t* s_bal = reinterpret_cast<uint64_t*>(smem);                        // [4][P]
  int32_t* s_woff = reinterpret_cast<int32_t*>(s_bal + NW * P);             // [NW][P]
  int32_t* s_tcnt = s_woff + NW * P;                                         // [tpw][P]
  int32_t* s_hist = s_tcnt + a.tiles_per_group * P;                          // [nh]
  int32_t* s_tot = s_hist + nh;                                              // [P]
  int32_t* s_base = s_tot + P;                                               // [P]
  __shared__ int32_t s_bad;
  __shared__ uint32_t s_scan[NW];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int G = gridDim.x;
  const int g = blockIdx.x;
  const int64_t tile0 = int64_t(g) * a.tiles_per_group;
  int64_t tile1 = tile0 + a.tiles_per_group;
  if (tile1 > a.tiles) tile1 = a.tiles;
  const int my_tiles = tile1 > tile0 ? int(tile1 - tile0) : 0;
  const bool want_e = MODE == kFusedSend && a.tokens_per_expert != nullptr;

  // The arrival count this launch starts from is read now and first used at
  // the barrier, so its round trip overlaps the decode.
  const uint32_t base = tid == 0 ? ld_relaxed(&a.ctrl[kCtrlEpoch]) : 0u;
  if (tid == 0) s_bad = 0;
  for (int i = tid; i < nh; i += BS) s_hist[i] = 0;
  __syncthreads();

  // ---- 1. decode, count, publish ------------------------------------------
  TileSlots<KMAX> sl;
  for (int j = 0; j < my_tiles; ++j) {
    const int64_t t = (tile0 + j) * BS + tid;
    const bool valid = t < a.T;
    decode<MODE, KMAX>(a, t, valid, sl);
    if (MODE == kFusedSend && valid) {
      int dv[KMAX];                             // owning destination, or -1
#pragma unroll
      for (int k = 0; k < KMAX; ++k) dv[k] = sl.bin[k] >= 0 ? sl.bin[k] - sl.cbase : -1;
      store_row<KMAX>(a.dest + t * a.K, dv, a.K, a.out_w);
      // membership row: 16 or 8 destinations per store when the rows allow
      // it, else 4 per 32-bit store (ndest % 4 == 0) or bytes
      const int D = a.ndest;
      uint8_t* row = a.is_in_rank + t * D;
      const int step = a.iir_w == 4 ? 16 : (a.iir_w == 2 ? 8 : 4);
      for (int p0 = 0; p0 < D; p0 += step) {
        uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int d = dv[k] - p0;
          if (d >= 0 && d < step) word[d >> 2] |= 1u << (8 * (d & 3));
        }
        if (a.iir_w == 4) {
          *reinterpret_cast<u32x4*>(row + p0) = u32x4{word[0], word[1], word[2], word[3]};
        } else if (a.iir_w == 2) {
          *reinterpret_cast<u32x2*>(row + p0) = u32x2{word[0], word[1]};
        } else if ((D & 3) == 0) {
          *reinterpret_cast<uint32_t*>(row + p0) = word[0];
        } else {
          for (int q = 0; q < 4 && p0 + q < D; ++q) row[p0 + q] = uint8_t((word[0] >> (8 * q)) & 1u);
        }
      }
    }
    if (want_e) {
#pragma unroll
      for (int k = 0; k < KMAX; ++k)
        if (sl.bin[k] >= 0) atomicAdd(&s_hist[P + int(sl.ids[k])], 1);
    }
    if (sl.bad) atomicAdd(&s_hist[nh - 1], sl.bad);
    ballots<KMAX>(sl, P, wave, lane, s_bal);
    __syncthreads();
    for (int b = tid; b < P; b += BS) {
      int cnt = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) cnt += int(__popcll(s_bal[w * P + b]));
      s_tcnt[j * P + b] = cnt;
      s_hist[b] += cnt;
    }
    __syncthreads();
  }
  uint32_t* row_out = a.rows + int64_t(g) * nh;
  for (int i = tid; i < nh; i += BS) st_relaxed(row_out + i, uint32_t(s_hist[i]));

  // ---- 2. grid barrier --------------------------------------------------------
  grid_sync(a.ctrl, G, base, 1, !a.two_pass);

  // ---- 3. totals, bases, expert slice -----------------------------------------
  // experts [e0, e1) are this workgroup's slice of the expert totals
  const int per_g = (a.E + G - 1) / G;
  const int e0 = g * per_g;
  const int e1 = min(a.E, e0 + per_g);
  const int ne = want_e && e1 > e0 ? e1 - e0 : 0;
  int32_t* s_etot = s_hist;            // reuse (the row is published): [ne] expert totals
  for (int b = tid; b < P; b += BS) {
    s_tot[b] = 0;
    s_base[b] = 0;
  }
  for (int i = tid; i < ne; i += BS) s_etot[i] = 0;
  __syncthreads();
  if (a.two_pass) {
    // Many groups and bins: every workgroup reading all lower rows would
    // take G*P loads each.  Instead workgroup g scans a slice of the bins
    // over the groups (thread i holds the counts of groups [i*q, i*q + q),
    // all loads in flight together), and publishes each group's exclusive
    // prefix and the bin's total; after a second barrier every workgroup
    // reads its own prefixes and the totals (P loads each).
    constexpr int kQ = kMaxFusedGroups / BS > 0 ? kMaxFusedGroups / BS : 1;  // groups per thread
    const int q = (G + BS - 1) / BS;
    const int per_b = (P + G - 1) / G;
    const int b0 = g * per_b;
    uint32_t v[kMaxTwoPassBins][kQ];
#pragma unroll
    for (int u = 0; u < kMaxTwoPassBins; ++u) {
      const int b = b0 + u;
#pragma unroll
      for (int i = 0; i < kQ; ++i) {
        const int grp = tid * q + i;
        v[u][i] = (u < per_b && b < P && i < q && grp < G)
                      ? ld_relaxed(a.rows + int64_t(grp) * nh + b) : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < kMaxTwoPassBins; ++u) {
      const int b = b0 + u;
      if (u >= per_b || b >= P) break;             // uniform across the workgroup
      uint32_t mine = 0;
#pragma unroll
      for (int i = 0; i < kQ; ++i) mine += v[u][i];
      uint32_t total = 0;
      uint32_t ex = block_exclusive_scan<NW>(mine, s_scan, total);
#pragma unroll
      for (int i = 0; i < kQ; ++i) {
        const int grp = tid * q + i;
        if (i < q && grp < G) st_relaxed(a.pref + int64_t(grp) * P + b, ex);
        ex += v[u][i];
      }
      if (tid == 0) st_relaxed(a.tots + b, total);
    }
    // the expert slice, as in the single pass
    for (int i0 = tid; i0 < G * ne; i0 += BS * 8) {
      uint32_t vx[8];
      int ex[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * BS;
        vx[u] = 0u;
        ex[u] = 0;
        if (i < G * ne) {
          ex[u] = i % ne;
          vx[u] = ld_relaxed(a.rows + int64_t(i / ne) * nh + P + e0 + ex[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (vx[u]) atomicAdd(&s_etot[ex[u]], int(vx[u]));
    }
    grid_sync(a.ctrl, G, base, 2, true);
    for (int b = tid; b < P; b += BS) {
      s_base[b] = int(ld_relaxed(a.pref + int64_t(g) * P + b));
      s_tot[b] = int(ld_relaxed(a.tots + b));
    }
  } else if (a.chunk_local) {
    // Chunks: a chunk's rows are numbered on their own, so a workgroup needs
    // only the totals and lower-group counts of the bins of the chunks its
    // tokens fall in, and only the groups those chunks' tokens span.
    if (my_tiles > 0) {
      const int64_t t_lo = tile0 * BS;
      const int64_t t_hi = (tile1 * BS < a.T ? tile1 * BS : a.T) - 1;
      const int c_lo = chunk_of(a, t_lo), c_hi = chunk_of(a, t_hi);
      const int g_lo = int((chunk_first(a, c_lo) / BS) / a.tiles_per_group);
      const int g_hi = int((chunk_last(a, c_hi) / BS) / a.tiles_per_group);
      const int D = a.ndest;
      const int b_lo = c_lo * D;
      const int nb = (c_hi - c_lo + 1) * D;
      const int n = (g_hi - g_lo + 1) * nb;
      for (int i0 = tid; i0 < n; i0 += BS * 8) {
        uint32_t vd[8];
        int gd[8], bd[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * BS;
          vd[u] = 0u;
          gd[u] = 0;
          bd[u] = 0;
          if (i < n) {
            gd[u] = g_lo + i / nb;
            bd[u] = b_lo + i % nb;
            vd[u] = ld_relaxed(a.rows + int64_t(gd[u]) * nh + bd[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (vd[u]) {
            atomicAdd(&s_tot[bd[u]], int(vd[u]));
            if (gd[u] < g) atomicAdd(&s_base[bd[u]], int(vd[u]));
          }
        }
      }
    }
  } else {
    // (group, destination) and (group, expert of the slice) pairs, all loads
    // of a batch in flight together; groups start at different rows so the
    // same words are not all requested at once.
    const uint32_t* rows_in = a.rows;
    const int nd = G * P;
    const int nx = G * ne;
    const int n = nd > nx ? nd : nx;
    for (int i0 = tid; i0 < n; i0 += BS * 8) {
      uint32_t vd[8], vx[8];
      int gd[8], bd[8], ex[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * BS;
        vd[u] = 0u;
        vx[u] = 0u;
        gd[u] = 0;
        bd[u] = 0;
        ex[u] = 0;
        if (i < nd) {
          int grp = i / P + g;
          if (grp >= G) grp -= G;
          gd[u] = grp;
          bd[u] = i % P;
          vd[u] = ld_relaxed(rows_in + int64_t(grp) * nh + bd[u]);
        }
        if (i < nx) {
          ex[u] = i % ne;
          vx[u] = ld_relaxed(rows_in + int64_t(i / ne) * nh + P + e0 + ex[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (vd[u]) {
          atomicAdd(&s_tot[bd[u]], int(vd[u]));
          if (gd[u] < g) atomicAdd(&s_base[bd[u]], int(vd[u]));
        }
        if (vx[u]) atomicAdd(&s_etot[ex[u]], int(vx[u]));
      }
    }
  }
  if (g == 0 && a.diag) {
    for (int grp = tid; grp < G; grp += BS) {
      const uint32_t v = ld_relaxed(a.rows + int64_t(grp) * nh + nh - 1);
      if (v) atomicAdd(&s_bad, int(v));
    }
  }
  __syncthreads();
  for (int i = tid; i < ne; i += BS) a.tokens_per_expert[e0 + i] = s_etot[i];
  if (a.chunk_local) {
    // each chunk's counts come from the workgroup holding its first token;
    // workgroup 0 writes the zero counts of the chunks with no token
    for (int c = 0; c < a.C; ++c) {
      const bool empty = chunk_first(a, c) > chunk_last(a, c);
      const int owner = empty ? 0 : int((chunk_first(a, c) / BS) / a.tiles_per_group);
      if (owner != g) continue;
      for (int d = tid; d < a.ndest; d += BS)
        a.send_counts[c * a.ndest + d] = empty ? 0 : s_tot[c * a.ndest + d];
    }
    if (g == 0 && tid == 0 && a.diag) a.diag[0] = s_bad;
  } else if (g == 0) {
    for (int b = tid; b < P; b += BS) a.send_counts[b] = s_tot[b];
    if (tid == 0 && a.diag) a.diag[0] = s_bad;
  }
  // Segment starts (exclusive scan of the totals, each rounded up to the
  // alignment when regrouping) added into the bases.  With chunks the scan
  // restarts at each chunk's first bin: a chunk's rows are numbered on
  // their own.
  if (wave == 0) {
    const int span = a.C > 1 ? a.ndest : P;
    for (int r0 = 0; r0 < P; r0 += span) {
      int carry = 0;
      for (int b0 = r0; b0 < r0 + span; b0 += kWave) {
        const int b = b0 + lane;
        int v = b < r0 + span ? s_tot[b] : 0;
        if (MODE == kFusedRegroup) v = (v + a.align - 1) / a.align * a.align;
        int incl = v;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int u = __shfl_up(incl, off);
          if (lane >= off) incl += u;
        }
        if (b < r0 + span) {
          s_base[b] += carry + incl - v;
          if (MODE == kFusedRegroup) {
            s_hist[b] = carry + incl - v;     // segment start (the published row is done with)
            if (g == 0) a.offsets[b] = carry + incl - v;
          }
        }
        carry += __shfl(incl, kWave - 1);
      }
      if (MODE == kFusedRegroup && g == 0 && lane == 0) a.offsets[P] = carry;
    }
  }
  __syncthreads();
  if (MODE == kFusedRegroup) {
    // Padding rows [start + count, aligned end) of every segment get source
    // -1 and weight 0, the bins dealt to the workgroups in turn.  Every index
    // fits int32: the host bounds the rows plus their padding.
    for (int b = g; b < P; b += G) {
      const int64_t r0 = int64_t(s_hist[b]) + s_tot[b];
      int64_t r1 = int64_t(s_hist[b]) + (s_tot[b] + a.align - 1) / a.align * a.align;
      if (r1 > a.capacity) r1 = a.capacity;
      for (int64_t r = r0 + tid; r < r1; r += BS) {
        a.send_token_idx[r] = -1;
        if (a.perm_w) a.perm_w[r] = 0.0f;
      }
    }
  }

  // ---- 4. rows and scatter ------------------------------------------------------
  const uint64_t lt = lanemask_lt();
  for (int j = 0; j < my_tiles; ++j) {
    const int64_t t = (tile0 + j) * BS + tid;
    const bool valid = t < a.T;
    if (my_tiles > 1) {       // a single tile's slots are still in registers
      decode<MODE, KMAX>(a, t, valid, sl);
      ballots<KMAX>(sl, P, wave, lane, s_bal);
    }
    __syncthreads();
    for (int b = tid; b < P; b += BS) {
      int run = s_base[b];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        s_woff[w * P + b] = run;
        run += int(__popcll(s_bal[w * P + b]));
      }
    }
    __syncthreads();
    int32_t rowk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      rowk[k] = -1;
      const int b = sl.bin[k];
      if (b >= 0) {
        const int64_t n = int64_t(s_woff[wave * P + b]) + __popcll(s_bal[wave * P + b] & lt);
        if (n < a.capacity) rowk[k] = int32_t(n);
      }
    }
    if (valid) store_row<KMAX>(a.token_row + t * a.K, rowk, a.K, a.out_w);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      bool first = sl.bin[k] >= 0 && rowk[k] >= 0;
#pragma unroll
      for (int q = 0; q < k; ++q)
        if (sl.bin[q] == sl.bin[k]) first = false;
      if (!first) continue;
      const int b = sl.bin[k];
      const int32_t n = rowk[k];
      if (MODE == kFusedRegroup) {          // source row and the slot's weight
        a.send_token_idx[n] = int32_t(t);
        if (a.perm_w) a.perm_w[n] = sl.wts[k];
        continue;
      }
      // chunk c's rows start at row c * capacity; its tokens count from the
      // chunk's first token
      const int64_t row = int64_t(sl.cidx) * a.capacity + n;
      a.send_token_idx[row] = int32_t(t - int64_t(sl.cidx) * a.chunk);
      a.send_rank[row] = b - sl.cbase;
      const int64_t ob = int64_t(b - sl.cbase) * a.E_local;
      int32_t* irow = a.send_idx + row * a.K;
      float* wrow = a.send_w + row * a.K;
#pragma unroll
      for (int kk = 0; kk < KMAX; kk += 4) {
        if (kk >= a.K) break;
        int32_t iv[4];
        float wv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool own = kk + q < KMAX && sl.bin[kk + q] == b;
          iv[q] = own ? int32_t(sl.ids[kk + q] - ob) : -1;
          wv[q] = own ? sl.wts[kk + q] : 0.0f;
        }
        if (KMAX % 4 == 0 && a.rows_w == 4) {
          *reinterpret_cast<u32x4*>(irow + kk) =
              u32x4{uint32_t(iv[0]), uint32_t(iv[1]), uint32_t(iv[2]), uint32_t(iv[3])};
          *reinterpret_cast<u32x4*>(wrow + kk) =
              u32x4{__float_as_uint(wv[0]), __float_as_uint(wv[1]), __float_as_uint(wv[2]),
                    __float_as_uint(wv[3])};
        } else if (KMAX % 2 == 0 && a.K == KMAX && a.rows_w >= 2) {
          *reinterpret_cast<u32x2*>(irow + kk) = u32x2{uint32_t(iv[0]), uint32_t(iv[1])};
          *reinterpret_cast<u32x2*>(wrow + kk) = u32x2{__float_as_uint(wv[0]), __float_as_uint(wv[1])};
          if (kk + 2 < KMAX) {
            *reinterpret_cast<u32x2*>(irow + kk + 2) = u32x2{uint32_t(iv[2]), uint32_t(iv[3])};
            *reinterpret_cast<u32x2*>(wrow + kk + 2) =
                u32x2{__float_as_uint(wv[2]), __float_as_uint(wv[3])};
          }
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
    __syncthreads();
    for (int b = tid; b < P; b += BS) s_base[b] += s_tcnt[j * P + b];
  }
}

}  // namespace

size_t fused_smem_bytes(int P, int E, int tiles_per_group, int waves) {
  return size_t(P) * (size_t(waves) * 8 + size_t(waves) * 4 + 2 * 4) +
         size_t(tiles_per_group) * P * 4 + size_t(P + E + 1) * 4;
}

template <int MODE, int NW>
void launch_fused_nw(const FusedArgs& a, unsigned groups, size_t smem, hipStream_t s) {
  // K = 2 and 6 have instances of their own, so that every even K up to 8
  // reads and writes whole rows (K == KMAX) without per-slot guards.
  if (a.K <= 2)
    dispatch_layout_kernel<MODE, 2, NW><<<groups, NW * kWave, smem, s>>>(a);
  else if (a.K <= 4)
    dispatch_layout_kernel<MODE, 4, NW><<<groups, NW * kWave, smem, s>>>(a);
  else if (a.K <= 6)
    dispatch_layout_kernel<MODE, 6, NW><<<groups, NW * kWave, smem, s>>>(a);
  else if (a.K <= 8)
    dispatch_layout_kernel<MODE, 8, NW><<<groups, NW * kWave, smem, s>>>(a);
  else
    dispatch_layout_kernel<MODE, 16, NW><<<groups, NW * kWave, smem, s>>>(a);
}

template <int MODE>
hipError_t launch_fused(const FusedArgs& a, unsigned groups, hipStream_t s) {
  const size_t smem = fused_smem_bytes(a.P, a.hist_e, a.tiles_per_group, a.waves);
  if (a.waves == 1)
    launch_fused_nw<MODE, 1>(a, groups, smem, s);
  else if (a.waves == 2)
    launch_fused_nw<MODE, 2>(a, groups, smem, s);
  else if (a.waves == 4)
    launch_fused_nw<MODE, 4>(a, groups, smem, s);
  else if constexpr (MODE == kFusedRegroup) {     // the send layouts stop at 4 waves
    if (a.waves == 8)
      launch_fused_nw<MODE, 8>(a, groups, smem, s);
    else
      launch_fused_nw<MODE, 16>(a, groups, smem, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dispatch_layout(const FusedArgs& a, unsigned groups, hipStream_t s) {
  return launch_fused<kFusedSend>(a, groups, s);
}

hipError_t launch_regroup_layout(const FusedArgs& a, unsigned groups, hipStream_t s) {
  return launch_fused<kFusedRegroup>(a, groups, s);
}

}  // namespace epdc
