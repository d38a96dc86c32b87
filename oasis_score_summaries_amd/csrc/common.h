// Internal helpers shared by the gfx950 kernels of liboasis (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace oasis {

constexpr int kHeadDim = 128;
constexpr int kMaxBlocks = 32768;   // NB limit (top-K keeps one register slice per thread)
constexpr int kMaxTopK = 1024;
constexpr int kMaxRows = 128;       // G * Q limit of the score kernel (8 row tiles of 16)
constexpr int kMaxGroup = 16;       // query heads per KV head in the attention kernel
constexpr int kMaxTableStride = 4096;
// Waves per workgroup of the scoring and attention-gather kernels (one value for
// both, so that the fused kernel of the overlapped step can hold either role).
#ifndef OASIS_WAVES_PER_WG
#define OASIS_WAVES_PER_WG 4
#endif
constexpr int kWavesPerWG = OASIS_WAVES_PER_WG;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- sequence geometry (identical on host and device) ----------------------------
// Blocks hold 1 << bshift tokens (bshift 3..6: 8 to 64 tokens; 16 is the default).
constexpr int kMinBlockShift = 3;
constexpr int kMaxBlockShift = 6;
__host__ __device__ inline int clamp_len(int len, int max_blocks, int bshift) {
  const int cap = max_blocks << bshift;
  return len < 0 ? 0 : (len > cap ? cap : len);
}
// Blocks that hold at least one token.
__host__ __device__ inline int num_blocks(int len, int bshift) {
  return (len + (1 << bshift) - 1) >> bshift;
}
// First block overlapping the last `window` tokens; earlier blocks are scoring candidates.
__host__ __device__ inline int first_window_block(int len, int window, int bshift) {
  const int x = len - window;
  return x > 0 ? x >> bshift : 0;
}

// ---- workgroup placement ---------------------------------------------------------
// The dispatcher deals workgroups to the eight XCDs in turn (workgroup i to XCD
// i % 8), each XCD with its own L2.  Item i of a role with gx items per head and nh
// heads maps to (x, head): head-major in the plain order, or, with `by_xcd` and nh a
// multiple of 8 (and the role's first workgroup index too), with every item of a
// head on one XCD, so that the head's queries are fetched into one L2 instead of
// eight.  Measured for the kernels that place both their scoring and their
// attention this way: 2 % faster steps at 80 query rows per KV head (20 KB of
// queries per head), 0.5 % slower at 20 rows and 32 x 8 heads, 14 % slower at 20
// rows and 4 x 8 heads of 8192 blocks; the host asks for it from 64 query rows on.
// The overlapped step's first launch places only its attention splits (and the merge)
// by XCD, always: 1 % faster at 20 rows and 8 x 8 heads.
__device__ inline void xcd_item(int i, int gx, int nh, bool by_xcd, int& x, int& head) {
  if (by_xcd && (nh & 7) == 0) {
    const int j = i >> 3;
    head = (j / gx) * 8 + (i & 7);
    x = j % gx;
    return;
  }
  x = i % gx;
  head = i / gx;
}
__host__ inline bool place_by_xcd(int query_rows) { return query_rows >= 64; }

// ---- hand-offs between workgroups of one launch -----------------------------------
// Producers write their data with device-scope stores (written through to where every
// XCD reads them), then store a flag word of their own (1 = "my stores are issued");
// no producer waits, and no two producers write one word (an arrival counter shared
// by many producers serializes their atomics).  A consumer wave polls the flags of its
// producers, one per lane, then reads the data with device-scope loads.  As nothing
// orders a producer's data before its flag, the data carry their own validity: zero
// means "not written yet", and a consumer reads again until every word it needs is
// non-zero.  Consumers write zeros back over what they read (flags and data), so that
// every region is zero again when the launch ends.  All waits are bounded by the
// constant-rate clock (100 MHz): past kSpinTicks the consumer raises a bit in the
// status word and goes on, so no launch can hang.
constexpr uint64_t kSpinTicks = 1000000;  // 10 ms
constexpr uint32_t kStatusScoreWait = 1u;
constexpr int kDevScopeAux = 0x10;  // buffer-instruction cache policy: device scope (sc1)

__device__ inline uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void raise_status(uint32_t* status, uint32_t bit) {
  (void)__hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// One wave waits until flags[0 .. n) are all non-zero (lane i polls flags i, i + 64,
// ...; n <= 256), then clears them.  False (and the status bit raised) on time-out.
// Every lane of the wave must call it.
__device__ inline bool wait_flags(uint32_t* flags, int n, uint32_t* status, uint32_t bit) {
  const int lane = threadIdx.x & 63;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  bool ok = true;
  for (;;) {
    bool mine = true;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = c * 64 + lane;
      if (i < n && ld_dev(flags + i) == 0u) mine = false;
    }
    if (__ballot(!mine) == 0ull) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
      if (lane == 0) raise_status(status, bit);
      ok = false;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  if (ok) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = c * 64 + lane;
      if (i < n) st_dev(flags + i, 0u);
    }
  }
  return ok;
}
// Reads a device-scope word until it is non-zero (bounded as above; on time-out the
// zero is returned and the status bit raised).
__device__ inline uint32_t ld_dev_nonzero(const uint32_t* p, uint32_t* status, uint32_t bit) {
  uint32_t w = ld_dev(p);
  if (w != 0u) return w;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while ((w = ld_dev(p)) == 0u) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
      raise_status(status, bit);
      return 0u;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return w;
}
// The hand-off region of step_kernel (inside the caller's workspace).
struct Handoff {
  uint32_t* flag_score;  // [B*H, score_waves]: one flag per scoring wave
  uint32_t* status;      // stays 0 unless a wait timed out
  uint32_t* mbox;        // [B*H, NB]: order keys of the candidate scores (never 0)
  float* scores;         // [B*H, NB]: the scores output, written by the selection workgroups
  int score_waves;       // scoring waves per (sequence, KV head), <= 256
};

// ---- bf16 bit helpers -------------------------------------------------------------
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Keep the lanes of a packed bf16 pair whose sign bit is set (x < 0), zero the others.
__device__ inline uint32_t bf16x2_neg_part(uint32_t w) {
  const uint32_t lo = (w & 0x00008000u) ? (w & 0x0000ffffu) : 0u;
  const uint32_t hi = (w & 0x80000000u) ? (w & 0xffff0000u) : 0u;
  return lo | hi;
}
// Keep the lanes whose sign bit is clear (x >= 0), zero the others.
__device__ inline uint32_t bf16x2_pos_part(uint32_t w) {
  const uint32_t lo = (w & 0x00008000u) ? 0u : (w & 0x0000ffffu);
  const uint32_t hi = (w & 0x80000000u) ? 0u : (w & 0xffff0000u);
  return lo | hi;
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Order-preserving map of a non-NaN fp32 value to uint32 (-0.0 maps like +0.0).
__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// The float of an order key (-0.0 comes back as +0.0).
__device__ inline float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---- wave64 cross-lane primitives on DPP (no LDS traffic) ---------------------------
// DPP controls: row_shr:n = 0x110 + n, quad_perm [1,0,3,2] = 0xb1, [2,3,0,1] = 0x4e,
// row_half_mirror = 0x141, row_mirror = 0x140.  Lanes without a source keep `old` (0).
template <int CTRL>
__device__ inline int dpp_i32(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active).
__device__ inline int wave_scan_incl(int x) {
  x += dpp_i32<0x111>(x);
  x += dpp_i32<0x112>(x);
  x += dpp_i32<0x114>(x);
  x += dpp_i32<0x118>(x);  // inclusive within each row of 16 lanes
  const int t0 = __builtin_amdgcn_readlane(x, 15);
  const int t1 = __builtin_amdgcn_readlane(x, 31);
  const int t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// Max / min of a uint32 over the 64 lanes of a wave; the result is wave-uniform.
__device__ inline uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0xb1>(x));
  x = max(x, dpp_u32<0x4e>(x));
  x = max(x, dpp_u32<0x141>(x));
  x = max(x, dpp_u32<0x140>(x));  // every lane holds its row's max
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48));
  return max(a, b);
}
__device__ inline uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u32<0xb1>(x));
  x = min(x, dpp_u32<0x4e>(x));
  x = min(x, dpp_u32<0x141>(x));
  x = min(x, dpp_u32<0x140>(x));
  const uint32_t a = min((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16));
  const uint32_t b = min((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48));
  return min(a, b);
}

// Max and sum of a float over the 64 lanes of a wave; the result is wave-uniform.
template <int CTRL>
__device__ inline float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ inline float wave_max_f32(float x) {
  x = fmaxf(x, dpp_f32<0xb1>(x));
  x = fmaxf(x, dpp_f32<0x4e>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  const float a = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16)));
  const float b = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)),
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48)));
  return fmaxf(a, b);
}
__device__ inline float wave_sum_f32(float x) {
  x += dpp_f32<0xb1>(x);
  x += dpp_f32<0x4e>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0)) +
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32)) +
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return a + b;
}

// Exclusive rank of this lane among the lanes whose flag is set, and their count.
__device__ inline int wave_flag_rank(bool flag, int* count) {
  const uint64_t m = __ballot(flag);
  *count = __popcll(m);
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---- wave64 / workgroup scans -----------------------------------------------------
__device__ inline int wave_inclusive_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Exclusive prefix sum over the threads of a workgroup (in thread order).
// `scratch` needs blockDim.x / 64 + 1 ints of LDS.  Returns the prefix, stores
// the total in *total.  Must be reached by every thread of the workgroup.
__device__ inline int block_exclusive_scan(int x, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  const int inc = wave_inclusive_scan(x);
  if (lane == 63 || threadIdx.x == blockDim.x - 1) scratch[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[nw] = run;
  }
  __syncthreads();
  const int r = scratch[wave] + inc - x;
  *total = scratch[nw];
  __syncthreads();
  return r;
}

}  // namespace oasis
