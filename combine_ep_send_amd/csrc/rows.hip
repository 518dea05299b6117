// Hidden-row kernels: permute (bf16 copy or fp8 quantize-on-dispatch), the
// zero padding of the expert-batched layout, the rows of the regrouped
// layout, and the weighted combine (gfx950, wave64).
//
// Every kernel walks "items" = (row, chunk of the row) in address order, one
// workgroup per item, so consecutive workgroups touch consecutive pieces of
// memory and each wave retires after a handful of 16-byte accesses.  On
// MI355X this keeps far more independent accesses in flight than a
// wave-per-row loop and, with the Infinity Cache cleared, moves rows 15-20 %
// faster.  Which rows an item touches is uniform across the workgroup, so row
// indices and weights sit in scalar registers.  Hidden rows are written with
// non-temporal stores (each byte is touched once per call), except the zero
// padding, whose plain stores measured faster; the combine reads its rows
// non-temporally, the permutes with plain loads (both measured faster).
#include "epdc_device.h"
#include "epdc_launch.h"

namespace epdc {

namespace {

// Quotient of two wave-uniform non-negative values; 32-bit when it can be.
__device__ __forceinline__ int64_t udiv(int64_t a, int b) {
  if (a < (int64_t(1) << 32)) return int64_t(uint32_t(a) / uint32_t(b));
  return a / b;
}

// The K routing entries of token t, loaded together (block-uniform, so they
// come through the scalar cache): slot k < K reads its own entry, the unused
// slots up to KMAX re-read the last one and are masked afterwards.
template <int KMAX, typename V>
__device__ __forceinline__ void load_slots(const V* base, int64_t t, int K, V (&v)[KMAX]) {
  const V* p = base + t * K;
  if (K == KMAX) {             // one contiguous run: a single wide scalar load
#pragma unroll
    for (int k = 0; k < KMAX; ++k) v[k] = p[k];
  } else {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) v[k] = p[k < K ? k : K - 1];
  }
}

// Distinct destination rows of token t.  Slot k is used when it is a real
// slot, its row is valid and no earlier slot named the same row.
template <int KMAX>
__device__ __forceinline__ int token_rows(const int32_t* token_row, int64_t t, int K,
                                          int64_t cap, int32_t (&rows)[KMAX],
                                          bool (&use)[KMAX]) {
  load_slots<KMAX>(token_row, t, K, rows);
  int n = 0;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    bool u = k < K && rows[k] >= 0 && int64_t(rows[k]) < cap;
#pragma unroll
    for (int j = 0; j < k; ++j)
      if (use[j] && rows[j] == rows[k]) u = false;
    use[k] = u;
    n += u ? 1 : 0;
  }
  return n;
}

// ---------------------------------------------------------------------------
// bf16 permute, token-major: one workgroup of kPermuteBlock threads per
// (token, chunk of kPermuteBlock pieces), one 16-byte piece per thread; the
// chunk of hidden row t is read once and stored to each of its rows.  Also
// fills the data rows of the expert-batched layout (token_row then holds
// e*max + slot).
// ---------------------------------------------------------------------------
template <int KMAX, int PER>
__global__ __launch_bounds__(kPermuteBlock) void permute_bf16_kernel(RowArgs a, int nchunks,
                                                                     int64_t item0) {
  const int lane = threadIdx.x;
  const int H8 = a.H >> 3;
  const int64_t item = item0 + blockIdx.x;
  const int64_t t = udiv(item, nchunks);
  const int j0 = int(item - t * nchunks) * (kPermuteBlock * PER);
  // The row is loaded before its destinations are known, so both round
  // trips overlap; a token with no destination then wastes one load (the
  // sparse expert-batched fill too measured faster this way: its step 0.632
  // against 0.637 ms when it looked the rows up first).  The hidden row is
  // read with plain loads and the rows are stored non-temporally: on the
  // 16k-token scatter plain loads took the permute from 346 to 331 us
  // (same-box A/B over two passes), while plain stores, faster still alone,
  // left dirty lines that slowed the combine after it by as much.
  const u32x4* src = static_cast<const u32x4*>(a.x) + t * H8;
  u32x4 v[PER];
  int32_t rows[KMAX];
  bool use[KMAX];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = j0 + i * kPermuteBlock + lane;
    if (j < H8) v[i] = src[j];
  }
  token_rows<KMAX>(a.token_row, t, a.K, a.capacity, rows, use);
  u32x4* dst = static_cast<u32x4*>(a.out);
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (!use[k]) continue;
    u32x4* d = dst + int64_t(rows[k]) * H8;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = j0 + i * kPermuteBlock + lane;
      if (j < H8) st_stream(d + j, v[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// fp8 quantize-on-dispatch.  A lane owns 16 consecutive channels (32 bytes
// of bf16 in, 16 bytes of e4m3 out); 8 lanes form one 128-channel group and
// reduce its amax with three xor shuffles.  One wave per (token, chunk of
// 64*IT 16-channel pieces); the chunk is quantized once and stored to every
// row of the token.
//
// Scales: fl32(amax/448) (SFMT kScaleF32); the smallest power of two at or
// above it (kScalePow2); or that power's UE8M0 byte, exponent + 127 and at
// least 0, i.e. 2^-127 (kScaleUe8m0), with the codes divided by the byte's
// value.  UE8M0 bytes of groups 4j..4j+3 go into 32-bit word j, group 4j in
// the low byte; a chunk starts on a multiple of 64 pieces, so the four
// groups of a word always sit in lanes L, L+8, L+16, L+24 of one wave.  An
// all-zero group has codes 0x00 and scale 0 (byte 0).
//
// Scale words of row r sit at r*units + u (row-major), or, with
// scale_block_rows = M > 0, at (r/M)*M*units + u*M + r%M: each block of M
// rows (an expert's slots) stores its scales column-major.
// ---------------------------------------------------------------------------
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return a | (b << 8) | (c << 16) | (d << 24);
}

// Smallest power of two at or above s (s >= 0 and finite); 0 stays 0.  On
// the bits: a normal value with a non-zero mantissa moves to the next
// exponent; a subnormal mantissa m that is not a power of two becomes the
// next power of two above m (2^23 being the smallest normal).
__device__ __forceinline__ float pow2_ceil(float s) {
  uint32_t u = __float_as_uint(s);
  const uint32_t m = u & 0x7FFFFFu;
  if (u >= 0x00800000u) {
    if (m != 0u) u = (u & 0x7F800000u) + 0x00800000u;
  } else if ((m & (m - 1u)) != 0u) {
    u = 1u << (32 - __clz(m));
  }
  return __uint_as_float(u);
}

template <int KMAX, int IT, int SFMT, bool LOAD_FIRST>
__global__ __launch_bounds__(kWave) void permute_fp8_kernel(RowArgs a, int nchunks,
                                                            int64_t item0) {
  const int lane = threadIdx.x;
  const int H8 = a.H >> 3;
  const int H16 = a.H >> 4;
  // scale words per row: one per group, or one per four groups (UE8M0)
  const int units = SFMT == kScaleUe8m0 ? (a.H >> 9) : (a.H >> 7);
  u32x4* dq = static_cast<u32x4*>(a.out);
  const int64_t item = item0 + blockIdx.x;
  const int64_t t = udiv(item, nchunks);
  const int p0 = int(item - t * nchunks) * (kWave * IT);
  // LOAD_FIRST: the row is loaded before its destinations are known (as in
  // the bf16 permute), so both round trips overlap; the sparse
  // expert-batched fill looks the rows up first and skips tokens with none
  // (loading first made its step slower here: 0.391 against 0.385 ms).
  const u32x4* src = static_cast<const u32x4*>(a.x) + t * H8;
  int32_t rows[KMAX];
  bool use[KMAX];
  if (!LOAD_FIRST && token_rows<KMAX>(a.token_row, t, a.K, a.capacity, rows, use) == 0) return;
  u32x4 in[IT][2];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int p = p0 + it * kWave + lane;
    in[it][0] = u32x4{0u, 0u, 0u, 0u};
    in[it][1] = u32x4{0u, 0u, 0u, 0u};
    if (p < H16) {                  // plain loads, as in the bf16 permute
      in[it][0] = src[2 * p];
      in[it][1] = src[2 * p + 1];
    }
  }
  if (LOAD_FIRST) token_rows<KMAX>(a.token_row, t, a.K, a.capacity, rows, use);
  u32x4 q[IT];
  uint32_t sw[IT];   // this lane's scale word: float bits, or the packed bytes
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
    // amax on the bits: for magnitudes (sign cleared) the unsigned order of
    // the bf16 bit patterns is the numeric order, and a NaN (above 0x7F80)
    // is left out.  Float max instructions would return a NaN for a
    // signalling NaN input, which the next max then drops, losing the
    // elements before it.  Both halves of each word are maxed at once; only
    // a lane whose maximum is a NaN pattern looks again without its NaNs.
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
    uint32_t mh = max(uint32_t(m2.x), uint32_t(m2.y));
    const bool lane_nan = mh > 0x7F80u;
    if (lane_nan) {
      mh = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
        if (lo <= 0x7F80u) mh = max(mh, lo);
        if (hi <= 0x7F80u) mh = max(mh, hi);
      }
    }
    uint32_t mbits = mh << 16;               // the fp32 bit pattern
    mbits = max(mbits, uint32_t(__shfl_xor(int(mbits), 1)));
    mbits = max(mbits, uint32_t(__shfl_xor(int(mbits), 2)));
    mbits = max(mbits, uint32_t(__shfl_xor(int(mbits), 4)));
    const float amax = __uint_as_float(mbits);
    float scale = amax / 448.0f;
    if (SFMT != kScaleF32) scale = pow2_ceil(scale);
    float divisor = scale;
    if (SFMT == kScaleUe8m0) {
      const uint32_t byte = __float_as_uint(scale) >> 23;   // 0 below 2^-126
      divisor = __uint_as_float(byte ? byte << 23 : 0x00400000u);
      const uint32_t b1 = __shfl_down(byte, 8);
      const uint32_t b2 = __shfl_down(byte, 16);
      const uint32_t b3 = __shfl_down(byte, 24);
      sw[it] = pack4(byte, b1, b2, b3);
    } else {
      sw[it] = __float_as_uint(scale);
    }
    // A quotient can be NaN only where this lane holds a NaN or the group
    // an infinity (infinity / infinity); such lanes take the integer encoder
    // with its NaN rule.  Elsewhere every quotient is finite and below 464
    // in magnitude: scale >= fl32(amax / 448) is off amax/448 by at most
    // 2^-24 relative when normal, and by less than 0.4 % when an fp32
    // subnormal (amax >= 2^-133, the least bf16 value).  There the hardware
    // conversion to OCP e4m3 (v_cvt_pk_fp8_f32: nearest, ties to even, sign
    // kept, codes of two values per instruction) gives the saturating
    // encoder's codes; it turns magnitudes from 464 up into NaN, which such
    // quotients never reach.  A power-of-two divisor of at least 2^-127
    // (every UE8M0 one) is applied as a multiplication by its reciprocal, a
    // float exactly, so both round the same real quotient once; smaller
    // powers (pow2 scales of tiny groups) have no float reciprocal.
    if (!lane_nan && mbits != 0x7F800000u) {
      float qv[16];
      if (SFMT != kScaleF32 && __float_as_uint(divisor) >= 0x00400000u) {
        const float rcp = 1.0f / divisor;
#pragma unroll
        for (int i = 0; i < 16; ++i) qv[i] = f[i] * rcp;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) qv[i] = f[i] / divisor;
      }
      uint32_t wq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(qv[4 * j], qv[4 * j + 1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(qv[4 * j + 2], qv[4 * j + 3], wd, true);
        wq[j] = amax > 0.0f ? uint32_t(wd) : 0u;
      }
      q[it] = u32x4{wq[0], wq[1], wq[2], wq[3]};
    } else {
      uint32_t c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        c[i] = amax > 0.0f ? e4m3_encode(f[i] / divisor) : (f[i] != f[i] ? 0x7Fu : 0u);
      q[it] = u32x4{pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7]),
                    pack4(c[8], c[9], c[10], c[11]), pack4(c[12], c[13], c[14], c[15])};
    }
  }
  const int shift = SFMT == kScaleUe8m0 ? 5 : 3;      // pieces per scale word: 32 or 8
  uint32_t* sbase = static_cast<uint32_t*>(a.out_scale);
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (!use[k]) continue;
    const int64_t r = rows[k];
    u32x4* drow = dq + r * H16;
    int64_t s0 = r * units, ustride = 1;
    if (a.scale_block_rows > 0) {
      const int64_t M = a.scale_block_rows;
      const int64_t blk = udiv(r, int(M));
      s0 = blk * M * units + (r - blk * M);
      ustride = M;
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int p = p0 + it * kWave + lane;
      if (p < H16) {
        st_stream(drow + p, q[it]);
        if ((p & ((1 << shift) - 1)) == 0) sbase[s0 + int64_t(p >> shift) * ustride] = sw[it];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Zero padding of the expert-batched layout: expert e's region of
// [E_local, max, H] holds its count of data rows, then zeros.  Grid (pieces
// of the region / 256, E_local); each thread stores one 16-byte zero when its
// piece lies past the count.  The data rows are written by the permute, so
// every byte of the buffer is written exactly once.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void zero_pad_kernel(PadArgs a) {
  const int e = blockIdx.y;
  int64_t cnt = a.tokens_per_expert[e];
  if (cnt > a.max_tokens) cnt = a.max_tokens;
  const int64_t per_row = a.row_pieces;
  const int64_t region = a.max_tokens * per_row;
  u32x4* base = static_cast<u32x4*>(a.b_x) + int64_t(e) * region;
  for (int64_t v = int64_t(blockIdx.x) * kBlock + threadIdx.x; v < region;
       v += int64_t(gridDim.x) * kBlock) {
    if (v >= cnt * per_row) base[v] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Zero scale words of the padding slots.  Row-major, expert e's padding is
// one run [cnt*units, max*units); column-major it is one run [u*max + cnt,
// (u+1)*max) per scale word u.  Grid (chunks of the longest run, E_local);
// each workgroup stores its chunk of every run of its expert.
__global__ __launch_bounds__(kBlock) void scale_pad_kernel(ScalePadArgs a) {
  const int e = blockIdx.y;
  int64_t cnt = a.tokens_per_expert[e];
  if (cnt > a.max_tokens) cnt = a.max_tokens;
  const int64_t M = a.max_tokens;
  uint32_t* base = a.scale + int64_t(e) * M * a.units;
  const int runs = a.col_major ? a.units : 1;
  const int64_t len = a.col_major ? M - cnt : (M - cnt) * a.units;
  const int64_t v = int64_t(blockIdx.x) * kBlock + threadIdx.x;
  if (v >= len) return;
  for (int u = 0; u < runs; ++u) {
    const int64_t start = a.col_major ? int64_t(u) * M + cnt : cnt * a.units;
    base[start + v] = 0u;
  }
}

// ---------------------------------------------------------------------------
// Rows of the regrouped layout, gathered: the rows in use (expert_offsets[
// bins] of them, at most the capacity) are written as one flat run of
// 16-byte pieces, one workgroup of kGatherBlock threads per 4 KiB window; a
// piece of row n holds the same piece of received row perm_src[n], or zero
// where the source is -1 (a padding row).  Rows past the ones in use are left
// as they are.  The stores stream as a sequential fill would, while the
// reads are gathered (a received row that several experts share is read
// once per expert).  Against scattering each received row to its experts
// (one read, scattered writes) and zeroing the padding in a kernel of its
// own, the expert-major step measured 1.975-1.983 ms against 2.005-2.011.
// Windows of 4 KiB beat 2 KiB ones (a sequential fill in 2 KiB blocks runs
// at 5.5 TB/s on 2 KiB boundaries, 6.6 TB/s 1 KiB past them, in 4 KiB blocks
// at 6.5-6.6 TB/s wherever they start): the gather took 638-645 us against
// 664 us for 2 KiB windows placed 1 KiB past a boundary, 676 us for a
// workgroup per (row, 2 KiB chunk); 8 and 16 KiB windows were no faster.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGatherBlock) void regroup_gather_kernel(GatherArgs a, int64_t item0) {
  const int H8 = a.H >> 3;
  const int64_t p = (item0 + blockIdx.x) * kGatherBlock + int(threadIdx.x);
  int64_t rows = a.offsets[a.bins];
  if (rows > a.capacity) rows = a.capacity;
  if (p >= rows * H8) return;
  const int64_t n = udiv(p, H8);
  const int j = int(p - n * H8);
  const int32_t src = a.perm_src[n];
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (src >= 0 && int64_t(src) < a.R) v = static_cast<const u32x4*>(a.x)[int64_t(src) * H8 + j];
  st_stream(static_cast<u32x4*>(a.out) + p, v);
}

// ---------------------------------------------------------------------------
// Combine.  Weighted: out[t] = bf16( sum_k w[t,k] * y[token_row[t,k]] ), the
// fp32 product rounded, then added in ascending k (no contraction into FMA).
// Unweighted (no weights given): each distinct row of t, i.e. each
// destination's partial output, is added once, in the order of its first
// slot.  Then up to two bias rows [T,H] are added, and the sum is rounded
// once to bf16.  One workgroup per (token, chunk of blockDim.x pieces), one
// 16-byte piece per thread: all distinct rows' loads are issued before the
// first add, and a slot that repeats an earlier slot's row reuses its
// registers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void add_row(float (&acc)[8], const u32x4& v) {
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] = acc[2 * q] + bf16_lo(wd[q]);
    acc[2 * q + 1] = acc[2 * q + 1] + bf16_hi(wd[q]);
  }
}

template <int KMAX, bool WEIGHTED>
__global__ __launch_bounds__(kMaxRowBlock) void combine_kernel(CombineArgs a, int nchunks,
                                                               int64_t item0) {
#pragma clang fp contract(off)
  const int H8 = a.H >> 3;
  const int64_t item = item0 + blockIdx.x;
  const int64_t t = udiv(item, nchunks);
  const int j = int(item - t * nchunks) * int(blockDim.x) + int(threadIdx.x);
  int32_t rows[KMAX];
  float wk[KMAX];
  load_slots<KMAX>(a.token_row, t, a.K, rows);
  if (WEIGHTED) load_slots<KMAX>(a.w, t, a.K, wk);
  bool use[KMAX];    // slot contributes
  int from[KMAX];    // slot whose loaded row it reuses (itself if first)
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    use[k] = k < a.K && rows[k] >= 0 && int64_t(rows[k]) < a.R;
    from[k] = k;
#pragma unroll
    for (int q = k - 1; q >= 0; --q)
      if (use[q] && from[q] == q && rows[q] == rows[k]) from[k] = q;
  }
  if (j >= H8) return;
  const u32x4* y = static_cast<const u32x4*>(a.y);
  u32x4 v[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    v[k] = u32x4{0u, 0u, 0u, 0u};
    if (use[k] && from[k] == k) v[k] = ld_stream(y + int64_t(rows[k]) * H8 + j);
  }
  u32x4 b0 = u32x4{0u, 0u, 0u, 0u}, b1 = u32x4{0u, 0u, 0u, 0u};
  if (a.bias0) b0 = ld_stream(static_cast<const u32x4*>(a.bias0) + t * H8 + j);
  if (a.bias1) b1 = ld_stream(static_cast<const u32x4*>(a.bias1) + t * H8 + j);
  if (WEIGHTED) {
#pragma unroll
    for (int k = 1; k < KMAX; ++k) {
#pragma unroll
      for (int q = 0; q < k; ++q)
        if (from[k] == q) v[k] = v[q];
    }
  }
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (!use[k]) continue;
    if (WEIGHTED) {
      const float wt = wk[k];
      const uint32_t wd[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float p0 = wt * bf16_lo(wd[q]);
        const float p1 = wt * bf16_hi(wd[q]);
        acc[2 * q] = acc[2 * q] + p0;
        acc[2 * q + 1] = acc[2 * q + 1] + p1;
      }
    } else if (from[k] == k) {
      add_row(acc, v[k]);
    }
  }
  if (a.bias0) add_row(acc, b0);
  if (a.bias1) add_row(acc, b1);
  u32x4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  st_stream(static_cast<u32x4*>(a.out) + t * H8 + j, o);
}

// ---------------------------------------------------------------------------
// Combine for sparse slots (most tokens name one or two rows, e.g. expert
// outputs restored onto received rows): the same sums in the same order, but
// a thread owns PER pieces, blockDim.x apart, and each valid slot's row is
// loaded and added in turn, so every wave keeps PER loads in flight.
// ---------------------------------------------------------------------------
template <int KMAX, bool WEIGHTED, int PER>
__global__ __launch_bounds__(kSparseMaxBlock) void combine_sparse_kernel(CombineArgs a,
                                                                         int nchunks,
                                                                         int64_t item0) {
#pragma clang fp contract(off)
  const int H8 = a.H >> 3;
  const int BS = int(blockDim.x);
  const int64_t item = item0 + blockIdx.x;
  const int64_t t = udiv(item, nchunks);
  const int j0 = int(item - t * nchunks) * (BS * PER) + int(threadIdx.x);
  int32_t rows[KMAX];
  float wk[KMAX];
  load_slots<KMAX>(a.token_row, t, a.K, rows);
  if (WEIGHTED) load_slots<KMAX>(a.w, t, a.K, wk);
  bool use[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    use[k] = k < a.K && rows[k] >= 0 && int64_t(rows[k]) < a.R;
    if (!WEIGHTED) {         // unweighted: each distinct row once
#pragma unroll
      for (int q = 0; q < k; ++q)
        if (use[q] && rows[q] == rows[k]) use[k] = false;
    }
  }
  const u32x4* y = static_cast<const u32x4*>(a.y);
  float acc[PER][8];
#pragma unroll
  for (int i = 0; i < PER; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[i][q] = 0.0f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (!use[k]) continue;
    u32x4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = j0 + i * BS;
      v[i] = u32x4{0u, 0u, 0u, 0u};
      if (j < H8) v[i] = ld_stream(y + int64_t(rows[k]) * H8 + j);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (WEIGHTED) {
        const float wt = wk[k];
        const uint32_t wd[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float p0 = wt * bf16_lo(wd[q]);
          const float p1 = wt * bf16_hi(wd[q]);
          acc[i][2 * q] = acc[i][2 * q] + p0;
          acc[i][2 * q + 1] = acc[i][2 * q + 1] + p1;
        }
      } else {
        add_row(acc[i], v[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = j0 + i * BS;
    if (j >= H8) continue;
    if (a.bias0) add_row(acc[i], ld_stream(static_cast<const u32x4*>(a.bias0) + t * H8 + j));
    if (a.bias1) add_row(acc[i], ld_stream(static_cast<const u32x4*>(a.bias1) + t * H8 + j));
    u32x4 o;
    o.x = pack_bf16x2(acc[i][0], acc[i][1]);
    o.y = pack_bf16x2(acc[i][2], acc[i][3]);
    o.z = pack_bf16x2(acc[i][4], acc[i][5]);
    o.w = pack_bf16x2(acc[i][6], acc[i][7]);
    st_stream(static_cast<u32x4*>(a.out) + t * H8 + j, o);
  }
}

// ---- launch shapes -----------------------------------------------------------

// A launch may span at most 2^32-1 work-items per grid dimension, so the
// largest grid in workgroups depends on the workgroup size.
constexpr int64_t max_blocks(int threads) { return int64_t(UINT32_MAX) / threads; }

// Occupancy caps of the dense (token-major) permutes.  An unused dynamic LDS
// allocation limits how many workgroups share a compute unit (160 KiB of LDS
// each on gfx950): 18 KiB per 128-thread bf16 workgroup leaves room for 8 of
// them, 10 KiB per one-wave fp8 workgroup for 16, i.e. 16 waves per CU in
// both.  With fewer rows in flight the scattered row stores stream better:
// on the 16k-token scatter the bf16 permute measured 329 us against 351 us
// at full occupancy, the fp8 permute 109 against 113 us on an 8k-token
// chunk (caps of 7, 9 or more workgroups were slower).  Only the send
// layout's permutes (about 7 rows per token) are capped: a copy of about one
// row per row read measured slower capped (903 against 728 us on the
// expert-major regroup), and the sparse expert-batched fills write about
// one row per token.
constexpr unsigned kPermuteLdsCap = 18 * 1024;
constexpr unsigned kFp8PermuteLdsCap = 10 * 1024;

// One workgroup of `threads` per item; grids beyond the work-item limit go
// out as several launches, each told its first item.
template <typename Launch>
void for_each_launch(int64_t items, int threads, Launch launch) {
  const int64_t most = max_blocks(threads);
  for (int64_t i0 = 0; i0 < items; i0 += most)
    launch(i0, unsigned(items - i0 < most ? items - i0 : most));
}

// Split a row of `pieces` per-lane-sized units into the fewest chunks of at
// most `most` units per lane, as evenly as possible.
struct Split {
  int nchunks;
  int per;
};
inline Split split_row(int64_t units, int most) {
  const int64_t per_lane = (units + kWave - 1) / kWave;
  const int64_t n = (per_lane + most - 1) / most;
  return Split{int(n), int((per_lane + n - 1) / n)};
}

template <int KMAX>
void launch_permute_bf16_k(const RowArgs& a, hipStream_t s) {
  // One piece per thread, two waves per workgroup: a 7168-channel row is
  // seven chunks of 2 KiB.  Of the shapes measured on the cache-cleared
  // 16k-token scatter (1-7 pieces per lane, 1-4 waves per workgroup) this
  // one moved the rows fastest: short-lived waves keep the stores streaming,
  // while larger chunks at full occupancy put so many rows in flight that
  // the stores slow down.
  const int nchunks = int(((a.H >> 3) + kPermuteBlock - 1) / kPermuteBlock);
  for_each_launch(a.T * nchunks, kPermuteBlock, [&](int64_t i0, unsigned g) {
    permute_bf16_kernel<KMAX, 1><<<g, kPermuteBlock, a.capped ? kPermuteLdsCap : 0u, s>>>(
        a, nchunks, i0);
  });
}

template <int KMAX, int IT, int SFMT>
void launch_permute_fp8_p(const RowArgs& a, Split sp, hipStream_t s) {
  for_each_launch(a.T * sp.nchunks, kWave, [&](int64_t i0, unsigned g) {
    if (a.sparse)
      permute_fp8_kernel<KMAX, IT, SFMT, false><<<g, kWave, 0, s>>>(a, sp.nchunks, i0);
    else
      permute_fp8_kernel<KMAX, IT, SFMT, true><<<g, kWave, a.capped ? kFp8PermuteLdsCap : 0u, s>>>(
          a, sp.nchunks, i0);
  });
}

template <int KMAX>
void launch_permute_fp8_k(const RowArgs& a, hipStream_t s) {
  // One 16-channel piece per lane, one wave per 1024 channels (7 per 7168-
  // channel row): the fastest of the shapes measured (1-7 pieces per lane,
  // 1-7 waves per workgroup) on the cache-cleared 8k-token chunk.
  const Split sp = split_row(a.H >> 4, 1);
  if (a.scale_fmt == kScaleUe8m0)
    launch_permute_fp8_p<KMAX, 1, kScaleUe8m0>(a, sp, s);
  else if (a.scale_fmt == kScalePow2)
    launch_permute_fp8_p<KMAX, 1, kScalePow2>(a, sp, s);
  else
    launch_permute_fp8_p<KMAX, 1, kScaleF32>(a, sp, s);
}

template <int KMAX>
void launch_combine_k(const CombineArgs& a, hipStream_t s) {
  const int64_t H8 = a.H >> 3;
  // The sparse form keeps more bytes in flight when tokens read one or two
  // rows: fewer than two rows per token, or more rows than the K*T slots can
  // name (a padded buffer such as the expert-batched one, where a token reads
  // only its local experts' rows: 50 against 93 us on the 8k-token batched
  // combine).  Tokens that read many rows are faster in the dense form (312
  // against 360 us on the 16k-token send layout).  A workgroup of up to
  // kSparseMaxBlock threads covers the row with up to 7 pieces per thread:
  // at 7168 channels 512 threads with 2 pieces each took the expert-major
  // restore from 583-604 to 558-566 us and the batched combine from 50 to
  // 45.6 us, against 128 threads with 7 pieces (256 threads: no gain; 1024
  // threads with one piece each: 806 us).
  if (a.R < 2 * a.T || a.R > int64_t(a.K) * a.T) {
    const int64_t w = (H8 + kWave - 1) / kWave * kWave;
    const int threads = int(w < kSparseMaxBlock ? w : kSparseMaxBlock);
    const int per = int((H8 + threads - 1) / threads) < 7 ? int((H8 + threads - 1) / threads) : 7;
    const int64_t nch = (H8 + int64_t(threads) * per - 1) / (int64_t(threads) * per);
    for_each_launch(a.T * nch, threads, [&](int64_t i0, unsigned g) {
#define EPDC_SPARSE(P)                                                                \
  if (a.w)                                                                            \
    combine_sparse_kernel<KMAX, true, P><<<g, threads, 0, s>>>(a, int(nch), i0);     \
  else                                                                                \
    combine_sparse_kernel<KMAX, false, P><<<g, threads, 0, s>>>(a, int(nch), i0);
      switch (per) {
        case 1: EPDC_SPARSE(1) break;
        case 2: EPDC_SPARSE(2) break;
        case 3: EPDC_SPARSE(3) break;
        case 4: EPDC_SPARSE(4) break;
        case 5: EPDC_SPARSE(5) break;
        case 6: EPDC_SPARSE(6) break;
        default: EPDC_SPARSE(7) break;
      }
#undef EPDC_SPARSE
    });
    return;
  }
  // One piece per thread; a workgroup covers the whole row when it has at
  // most kMaxRowBlock pieces (rounded up to whole waves), else equal chunks.
  const int64_t nch = (H8 + kMaxRowBlock - 1) / kMaxRowBlock;
  const int64_t per_chunk = (H8 + nch - 1) / nch;
  const int threads = int((per_chunk + kWave - 1) / kWave) * kWave;
  for_each_launch(a.T * nch, threads, [&](int64_t i0, unsigned g) {
    if (a.w)
      combine_kernel<KMAX, true><<<g, threads, 0, s>>>(a, int(nch), i0);
    else
      combine_kernel<KMAX, false><<<g, threads, 0, s>>>(a, int(nch), i0);
  });
}

}  // namespace

hipError_t launch_permute_bf16(const RowArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.K <= 2)
    launch_permute_bf16_k<2>(a, s);
  else if (a.K <= 4)
    launch_permute_bf16_k<4>(a, s);
  else if (a.K == 6)
    launch_permute_bf16_k<6>(a, s);
  else if (a.K <= 8)
    launch_permute_bf16_k<8>(a, s);
  else
    launch_permute_bf16_k<16>(a, s);
  return hipGetLastError();
}

hipError_t launch_permute_fp8(const RowArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.K <= 2)
    launch_permute_fp8_k<2>(a, s);
  else if (a.K <= 4)
    launch_permute_fp8_k<4>(a, s);
  else if (a.K == 6)
    launch_permute_fp8_k<6>(a, s);
  else if (a.K <= 8)
    launch_permute_fp8_k<8>(a, s);
  else
    launch_permute_fp8_k<16>(a, s);
  return hipGetLastError();
}

hipError_t launch_zero_pad(const PadArgs& a, hipStream_t s) {
  const int64_t region = a.max_tokens * a.row_pieces;
  if (region == 0 || a.E_local == 0) return hipSuccess;
  const int64_t gx = (region + kBlock - 1) / kBlock;
  const dim3 grid{unsigned(gx < max_blocks(kBlock) ? gx : max_blocks(kBlock)), unsigned(a.E_local),
                  1u};
  zero_pad_kernel<<<grid, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_scale_pad(const ScalePadArgs& a, hipStream_t s) {
  const int64_t longest = a.col_major ? a.max_tokens : a.max_tokens * a.units;
  if (longest == 0 || a.E_local == 0) return hipSuccess;
  const int64_t gx = (longest + kBlock - 1) / kBlock;
  if (gx > max_blocks(kBlock)) return hipErrorInvalidValue;
  const dim3 grid{unsigned(gx), unsigned(a.E_local), 1u};
  scale_pad_kernel<<<grid, kBlock, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_regroup_gather(const GatherArgs& a, hipStream_t s) {
  if (a.capacity == 0) return hipSuccess;
  // Grid over the capacity's pieces: the row count is known only on the device.
  const int64_t windows = (a.capacity * (a.H >> 3) + kGatherBlock - 1) / kGatherBlock;
  for_each_launch(windows, kGatherBlock, [&](int64_t i0, unsigned g) {
    regroup_gather_kernel<<<g, kGatherBlock, 0, s>>>(a, i0);
  });
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.K <= 2)
    launch_combine_k<2>(a, s);
  else if (a.K <= 4)
    launch_combine_k<4>(a, s);
  else if (a.K == 6)
    launch_combine_k<6>(a, s);
  else if (a.K <= 8)
    launch_combine_k<8>(a, s);
  else
    launch_combine_k<16>(a, s);
  return hipGetLastError();
}

}  // namespace epdc
