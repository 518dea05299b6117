// Hidden-row kernels: permute (bf16 copy or fp8 quantize-on-dispatch), the
// expert-batched fill, and the weighted combine (gfx950, wave64).
//
// Every kernel gives one wavefront one row: 64 lanes move the row in 16-byte
// pieces, so a wave covers 1 KiB per access and H = 7168 bf16 (14 KiB) is 14
// pieces per lane.  Stores of rows nobody re-reads soon are non-temporal;
// hidden-row loads are plain loads (measured faster than non-temporal ones for
// the token-major permute on gfx950), the combine's expert-output loads are
// non-temporal.  Which rows a token touches is wave-uniform, so the row
// indices and weights sit in scalar registers.
#include "epdc_device.h"
#include "epdc_launch.h"

namespace epdc {

namespace {

// Distinct destination rows of token t (wave-uniform).  Slot k is used when
// its row is valid and no earlier slot named the same row.
template <int KMAX>
__device__ __forceinline__ int token_rows(const int32_t* token_row, int64_t t, int K,
                                          int64_t cap, int32_t (&rows)[KMAX],
                                          bool (&use)[KMAX]) {
  int n = 0;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    rows[k] = -1;
    use[k] = false;
    if (k < K) {
      const int32_t r = token_row[t * K + k];
      rows[k] = r;
      bool u = r >= 0 && int64_t(r) < cap;
#pragma unroll
      for (int j = 0; j < k; ++j)
        if (use[j] && rows[j] == r) u = false;
      use[k] = u;
      n += u ? 1 : 0;
    }
  }
  return n;
}

// ---------------------------------------------------------------------------
// bf16 permute: read hidden row t once, store it to each of its send rows.
// ---------------------------------------------------------------------------
template <int KMAX, int VPL>
__global__ __launch_bounds__(kBlock) void permute_bf16_kernel(RowArgs a) {
  const int lane = lane_id();
  const int64_t t = int64_t(blockIdx.x) * kWavesPerBlock + wave_id();
  if (t >= a.T) return;
  int32_t rows[KMAX];
  bool use[KMAX];
  if (token_rows<KMAX>(a.token_row, t, a.K, a.capacity, rows, use) == 0) return;

  const int H8 = a.H >> 3;
  const u32x4* src = static_cast<const u32x4*>(a.x) + t * H8;
  u32x4* dst = static_cast<u32x4*>(a.out);
  for (int base = 0; base < H8; base += kWave * VPL) {
    u32x4 v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int j = base + i * kWave + lane;
      if (j < H8) v[i] = src[j];
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (!use[k]) continue;
      u32x4* d = dst + int64_t(rows[k]) * H8;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int j = base + i * kWave + lane;
        if (j < H8) st_stream(d + j, v[i]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp8 quantize-on-dispatch.  A lane owns 16 consecutive channels (32 bytes
// of bf16 in, 16 bytes of e4m3 out); 8 lanes form one 128-channel group and
// reduce its amax with three xor shuffles.  The row is quantized once and
// stored to every send row of the token.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return a | (b << 8) | (c << 16) | (d << 24);
}

template <int KMAX, int IT>
__global__ __launch_bounds__(kBlock) void permute_fp8_kernel(RowArgs a) {
  const int lane = lane_id();
  const int64_t t = int64_t(blockIdx.x) * kWavesPerBlock + wave_id();
  if (t >= a.T) return;
  int32_t rows[KMAX];
  bool use[KMAX];
  if (token_rows<KMAX>(a.token_row, t, a.K, a.capacity, rows, use) == 0) return;

  const int H8 = a.H >> 3;
  const int H16 = a.H >> 4;
  const int G = a.H >> 7;
  const u32x4* src = static_cast<const u32x4*>(a.x) + t * H8;
  u32x4* dq = static_cast<u32x4*>(a.out);
  for (int base = 0; base < H16; base += kWave * IT) {
    u32x4 in[IT][2];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int p = base + it * kWave + lane;
      in[it][0] = u32x4{0u, 0u, 0u, 0u};
      in[it][1] = u32x4{0u, 0u, 0u, 0u};
      if (p < H16) {
        in[it][0] = src[2 * p];
        in[it][1] = src[2 * p + 1];
      }
    }
    u32x4 q[IT];
    float sc[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const uint32_t w[8] = {in[it][0].x, in[it][0].y, in[it][0].z, in[it][0].w,
                             in[it][1].x, in[it][1].y, in[it][1].z, in[it][1].w};
      float f[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      amax = fmaxf(amax, __shfl_xor(amax, 4));
      const float scale = amax / 448.0f;
      uint32_t c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = scale > 0.0f ? e4m3_encode(f[i] / scale) : 0u;
      q[it] = u32x4{pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7]),
                    pack4(c[8], c[9], c[10], c[11]), pack4(c[12], c[13], c[14], c[15])};
      sc[it] = scale;
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (!use[k]) continue;
      u32x4* drow = dq + int64_t(rows[k]) * H16;
      float* srow = a.out_scale + int64_t(rows[k]) * G;
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int p = base + it * kWave + lane;
        if (p < H16) {
          st_stream(drow + p, q[it]);
          if ((lane & 7) == 0) srow[p >> 3] = sc[it];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Expert-batched fill: row (e, slot) of [E_local, max, H] gets hidden row
// slot_token[e, slot] while slot < count_e, zeros after.  Each output byte is
// written once, in address order across the grid.
// ---------------------------------------------------------------------------
template <int VPL>
__global__ __launch_bounds__(kBlock) void batched_fill_kernel(FillArgs a) {
  const int lane = lane_id();
  const int64_t row = int64_t(blockIdx.x) * kWavesPerBlock + wave_id();
  const int64_t nrows = int64_t(a.E_local) * a.max_tokens;
  if (row >= nrows) return;
  const int e = int(row / a.max_tokens);
  const int64_t slot = row - int64_t(e) * a.max_tokens;
  int64_t cnt = a.tokens_per_expert[e];
  if (cnt > a.max_tokens) cnt = a.max_tokens;

  const int H8 = a.H >> 3;
  u32x4* dst = static_cast<u32x4*>(a.b_x) + row * H8;
  // A slot past the count, or a map entry that is not a token of this call,
  // is written as zeros: the fill never reads outside x.
  const int64_t t = slot < cnt ? int64_t(a.slot_token[row]) : -1;
  if (t >= 0 && t < a.T) {
    const u32x4* src = static_cast<const u32x4*>(a.x) + t * H8;
    for (int base = 0; base < H8; base += kWave * VPL) {
      u32x4 v[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int j = base + i * kWave + lane;
        if (j < H8) v[i] = src[j];
      }
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int j = base + i * kWave + lane;
        if (j < H8) st_stream(dst + j, v[i]);
      }
    }
  } else {
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    for (int j = lane; j < H8; j += kWave) st_stream(dst + j, z);
  }
}

// ---------------------------------------------------------------------------
// Combine: out[t] = bf16( sum_k w[t,k] * y[token_row[t,k]] ), fp32 product
// rounded, then added in ascending k (no contraction into FMA).  All K rows
// of a chunk are loaded before the adds so the loads overlap.
// ---------------------------------------------------------------------------
template <int KMAX, int VPL>
__global__ __launch_bounds__(kBlock) void combine_kernel(CombineArgs a) {
#pragma clang fp contract(off)
  const int lane = lane_id();
  const int64_t t = int64_t(blockIdx.x) * kWavesPerBlock + wave_id();
  if (t >= a.T) return;
  int32_t rows[KMAX];
  float wk[KMAX];
  bool use[KMAX];    // slot contributes
  int from[KMAX];    // slot whose loaded row it reuses (itself if first)
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    rows[k] = 0;
    wk[k] = 0.0f;
    use[k] = false;
    from[k] = k;
    if (k < a.K) {
      const int32_t r = a.token_row[t * a.K + k];
      rows[k] = r;
      wk[k] = a.w[t * a.K + k];
      use[k] = r >= 0 && int64_t(r) < a.R;
#pragma unroll
      for (int j = k - 1; j >= 0; --j)
        if (use[j] && from[j] == j && rows[j] == r) from[k] = j;
    }
  }
  const int H8 = a.H >> 3;
  const u32x4* y = static_cast<const u32x4*>(a.y);
  u32x4* out = static_cast<u32x4*>(a.out) + t * H8;
  for (int base = 0; base < H8; base += kWave * VPL) {
    // Every distinct row of the chunk is loaded before the first add, so the
    // loads of all K slots are in flight together; a slot that repeats an
    // earlier slot's row takes the registers instead of reading HBM again.
    u32x4 v[KMAX][VPL];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        v[k][i] = u32x4{0u, 0u, 0u, 0u};
        const int j = base + i * kWave + lane;
        if (use[k] && from[k] == k && j < H8) v[k][i] = ld_stream(y + int64_t(rows[k]) * H8 + j);
      }
    }
#pragma unroll
    for (int k = 1; k < KMAX; ++k) {
      if (from[k] == k) continue;
#pragma unroll
      for (int j = 0; j < k; ++j) {
        if (from[k] == j) {
#pragma unroll
          for (int i = 0; i < VPL; ++i) v[k][i] = v[j][i];
        }
      }
    }
    float acc[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[i][q] = 0.0f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (!use[k]) continue;
      const float wt = wk[k];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const uint32_t wd[4] = {v[k][i].x, v[k][i].y, v[k][i].z, v[k][i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float p0 = wt * bf16_lo(wd[q]);
          const float p1 = wt * bf16_hi(wd[q]);
          acc[i][2 * q] = acc[i][2 * q] + p0;
          acc[i][2 * q + 1] = acc[i][2 * q + 1] + p1;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int j = base + i * kWave + lane;
      if (j < H8) {
        u32x4 o;
        o.x = f32_to_bf16_rne(acc[i][0]) | (f32_to_bf16_rne(acc[i][1]) << 16);
        o.y = f32_to_bf16_rne(acc[i][2]) | (f32_to_bf16_rne(acc[i][3]) << 16);
        o.z = f32_to_bf16_rne(acc[i][4]) | (f32_to_bf16_rne(acc[i][5]) << 16);
        o.w = f32_to_bf16_rne(acc[i][6]) | (f32_to_bf16_rne(acc[i][7]) << 16);
        st_stream(out + j, o);
      }
    }
  }
}

inline unsigned row_grid(int64_t rows) {
  return unsigned((rows + kWavesPerBlock - 1) / kWavesPerBlock);
}

// Vectors per lane for a row of H8 16-byte pieces (one chunk covers the row
// when it fits in 16 per lane).
inline int pieces_per_lane(int64_t pieces) { return int((pieces + kWave - 1) / kWave); }

template <int KMAX>
hipError_t launch_permute_bf16_k(const RowArgs& a, hipStream_t s) {
  const unsigned grid = row_grid(a.T);
  const int need = pieces_per_lane(a.H >> 3);
  if (need <= 1)
    permute_bf16_kernel<KMAX, 1><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 2)
    permute_bf16_kernel<KMAX, 2><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 4)
    permute_bf16_kernel<KMAX, 4><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 7)
    permute_bf16_kernel<KMAX, 7><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 8)
    permute_bf16_kernel<KMAX, 8><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 14)
    permute_bf16_kernel<KMAX, 14><<<grid, kBlock, 0, s>>>(a);
  else
    permute_bf16_kernel<KMAX, 16><<<grid, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

template <int KMAX>
hipError_t launch_permute_fp8_k(const RowArgs& a, hipStream_t s) {
  const unsigned grid = row_grid(a.T);
  const int need = pieces_per_lane(a.H >> 4);
  if (need <= 1)
    permute_fp8_kernel<KMAX, 1><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 2)
    permute_fp8_kernel<KMAX, 2><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 4)
    permute_fp8_kernel<KMAX, 4><<<grid, kBlock, 0, s>>>(a);
  else
    permute_fp8_kernel<KMAX, 7><<<grid, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute_bf16(const RowArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.K <= 4) return launch_permute_bf16_k<4>(a, s);
  if (a.K <= 8) return launch_permute_bf16_k<8>(a, s);
  return launch_permute_bf16_k<16>(a, s);
}

hipError_t launch_permute_fp8(const RowArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.K <= 4) return launch_permute_fp8_k<4>(a, s);
  if (a.K <= 8) return launch_permute_fp8_k<8>(a, s);
  return launch_permute_fp8_k<16>(a, s);
}

hipError_t launch_batched_fill(const FillArgs& a, hipStream_t s) {
  const int64_t nrows = int64_t(a.E_local) * a.max_tokens;
  if (nrows == 0) return hipSuccess;
  const unsigned grid = row_grid(nrows);
  const int need = pieces_per_lane(a.H >> 3);
  if (need <= 1)
    batched_fill_kernel<1><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 2)
    batched_fill_kernel<2><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 4)
    batched_fill_kernel<4><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 8)
    batched_fill_kernel<8><<<grid, kBlock, 0, s>>>(a);
  else if (need <= 14)
    batched_fill_kernel<14><<<grid, kBlock, 0, s>>>(a);
  else
    batched_fill_kernel<16><<<grid, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

// Vectors per lane per chunk for the combine: about 56 loads in flight per
// lane (K rows x VPL pieces), with the row split into equal chunks.
template <int KMAX, int VMAX>
hipError_t launch_combine_k(const CombineArgs& a, hipStream_t s) {
  const unsigned grid = row_grid(a.T);
  const int need = pieces_per_lane(a.H >> 3);
  const int chunks = (need + VMAX - 1) / VMAX;
  const int vpl = (need + chunks - 1) / chunks;
  if (vpl <= 1)
    combine_kernel<KMAX, 1><<<grid, kBlock, 0, s>>>(a);
  else if (vpl <= 2)
    combine_kernel<KMAX, (VMAX < 2 ? VMAX : 2)><<<grid, kBlock, 0, s>>>(a);
  else if (vpl <= 4)
    combine_kernel<KMAX, (VMAX < 4 ? VMAX : 4)><<<grid, kBlock, 0, s>>>(a);
  else
    combine_kernel<KMAX, VMAX><<<grid, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.K <= 2) return launch_combine_k<2, 16>(a, s);
  if (a.K <= 4) return launch_combine_k<4, 14>(a, s);
  if (a.K <= 8) return launch_combine_k<8, 7>(a, s);
  return launch_combine_k<16, 4>(a, s);
}

}  // namespace epdc
