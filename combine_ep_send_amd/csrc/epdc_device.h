// Device-side helpers shared by the epdc kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace epdc {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 256;               // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kTile = kBlock;             // tokens per scan tile (one per thread)

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Wave index as a value the compiler knows is uniform across the wave.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (uint64_t(1) << lane_id()) - 1;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Per-bin ballots of a wave, all 64 at once: lane i holds a mask m whose bit
// j says "lane i belongs to bin j"; lane j receives the ballot of bin j (bit
// i set when lane i's mask has bit j).  That is the transpose of a 64x64
// bit matrix, done in six exchange steps: at step s the lanes i and i^s swap
// the s-by-s blocks that lie off the diagonal.  It replaces 64 ballots.
__device__ __forceinline__ uint64_t wave_bin_ballots(uint64_t m) {
  const int lane = int(threadIdx.x) & (kWave - 1);
  constexpr uint64_t kBlockMask[6] = {0x00000000FFFFFFFFull, 0x0000FFFF0000FFFFull,
                                      0x00FF00FF00FF00FFull, 0x0F0F0F0F0F0F0F0Full,
                                      0x3333333333333333ull, 0x5555555555555555ull};
#pragma unroll
  for (int st = 0; st < 6; ++st) {
    const int s = 32 >> st;
    const uint64_t mask = kBlockMask[st];
    const uint64_t p = __shfl_xor(m, s);
    // the lower lane takes the partner's low block into its high half, the
    // upper lane the partner's high block into its low half
    const uint64_t t_lo = (((m >> s) ^ p) & mask) << s;
    const uint64_t t_hi = ((p >> s) ^ m) & mask;
    m ^= (lane & s) ? t_hi : t_lo;
  }
  return m;
}

// ---- agent-scope atomics (visible across all XCDs of the device) ----------
__device__ __forceinline__ uint64_t ld_acquire(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
// Scan status words: the value travels inside the word, so relaxed ordering
// is enough; agent scope keeps the access coherent across XCDs.
__device__ __forceinline__ uint64_t ld_status(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_status(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t fetch_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
// Ticket and completion counters order nothing but themselves: relaxed, so
// they do not write back or invalidate the L2 the way acq_rel would.
__device__ __forceinline__ uint32_t fetch_add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fetch_or(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- 16-byte streaming loads/stores ----------------------------------------
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) {
  return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ void st_stream(u32x4* p, u32x4 v) {
  __builtin_nontemporal_store(v, p);
}

// ---- bf16 <-> fp32 ---------------------------------------------------------
// A bf16 value is the upper half of a binary32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 values rounded to bf16 and packed, the first in the low half, by
// the hardware conversion (v_cvt_pk_bf16_f32): to nearest with ties to even
// (subnormals kept, a value past the largest bf16 becomes an infinity), and
// a NaN stays a quiet NaN (its sign and leading payload bits).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// ---- OCP e4m3 (float8_e4m3fn) encode ----------------------------------------
// Nearest code with ties to even, saturating at 448 (0x7E; infinities too),
// sign kept.  e4m3_encode_finite takes a non-NaN value; e4m3_encode also
// maps any NaN to the NaN code 0x7F.
// Normal range (|v| >= 2^-6): round the binary32 mantissa from 23 to 3 bits
// on the raw bits (a carry moves into the exponent) and rebias 127 -> 7.
// Below 2^-6 the codes are the uniform grid m * 2^-9, m = 0..8, so the code
// is rint(|v| * 2^9) (the scaling is exact; rint rounds ties to even).
__device__ __forceinline__ uint32_t e4m3_encode_finite(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {                    // |v| >= 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {              // |v| < 2^-6
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;   // exp32:mant3
    code = r - (120u << 3);                  // exponent bias 127 -> 7
  }
  return code | sign;
}
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  return (__float_as_uint(v) & 0x7FFFFFFFu) > 0x7F800000u ? 0x7Fu : e4m3_encode_finite(v);
}

// ---- packed scan status words ------------------------------------------------
// [63:32] call epoch, [31:30] flag, [29:0] value.
constexpr uint32_t kFlagNone = 0, kFlagAggregate = 1, kFlagPrefix = 2;
__device__ __forceinline__ uint64_t pack_status(uint32_t epoch, uint32_t flag, uint32_t value) {
  return (uint64_t(epoch) << 32) | (uint64_t(flag) << 30) | uint64_t(value & 0x3FFFFFFFu);
}
__device__ __forceinline__ uint32_t status_epoch(uint64_t w) { return uint32_t(w >> 32); }
__device__ __forceinline__ uint32_t status_flag(uint64_t w) { return uint32_t(w >> 30) & 3u; }
__device__ __forceinline__ uint32_t status_value(uint64_t w) { return uint32_t(w) & 0x3FFFFFFFu; }

}  // namespace epdc
