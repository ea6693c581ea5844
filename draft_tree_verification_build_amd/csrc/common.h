// Device helpers shared by the gfx950 kernels of the draft-tree step.
//
// Every kernel here runs with 256-thread workgroups (4 wave64s). Logit rows are read as
// 16-byte vectors (8 bf16 or 4 fp32 values); element e of load i of thread t in a chunk
// sits at index  chunk_base + i * 256 * VEC + t * VEC + e, so a (load, thread, element)
// triple orders like the vocabulary index, which tie-breaking relies on.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dtv {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kLoads = 4;                 // 16-byte loads per thread per chunk

// ---------------------------------------------------------------- values and keys

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Order-preserving unsigned key of a finite float: larger value <=> larger key, -0 == +0.
// Key 0 is never produced by a finite value and marks an empty element.
__device__ __forceinline__ uint32_t f32_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;                       // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------- reductions

// Wave-wide reductions (all 64 lanes active; every lane receives the result, the same bits
// in every lane). Inside each row of 16 lanes, four DPP moves pair lane i with i^1, i^2
// (quad permutations), then 7-i (half mirror: quads within 8) and 15-i (mirror: 8-lane
// halves), so each row ends uniform; the four row values are then read from lanes 0, 16,
// 32 and 48 and combined in a fixed order. No step goes through shared memory.
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_move(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "4- or 8-byte values");
  if constexpr (sizeof(T) == 4) {
    const int r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(T, r);
  } else {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xFFFFFFFFull), CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(T, (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) |
                                     static_cast<uint32_t>(lo));
  }
}

// dpp_move with a row mask: lanes of rows outside ROWMASK, and lanes whose source lies
// outside their row, receive 0.
template <int CTRL, int ROWMASK, typename T>
__device__ __forceinline__ T dpp_move_or0(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "4- or 8-byte values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xF, true));
  } else {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xFFFFFFFFull), CTRL, ROWMASK, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), CTRL, ROWMASK, 0xF, true);
    return __builtin_bit_cast(T, (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) |
                                     static_cast<uint32_t>(lo));
  }
}

template <typename T>
__device__ __forceinline__ T read_lane(T v, int lane) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "4- or 8-byte values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
  } else {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(u & 0xFFFFFFFFull), lane);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), lane);
    return __builtin_bit_cast(T, (static_cast<unsigned long long>(static_cast<uint32_t>(hi)) << 32) |
                                     static_cast<uint32_t>(lo));
  }
}

template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp_move<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_move<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_move<0x141>(v));   // row_half_mirror
  v = op(v, dpp_move<0x140>(v));   // row_mirror
  return op(op(read_lane(v, 0), read_lane(v, 16)), op(read_lane(v, 32), read_lane(v, 48)));
}

// The same over the two halves of the wave separately: lo receives the result over lanes
// 0..31, hi over lanes 32..63 (both wave-uniform, the same bits in every lane).
template <typename T, typename Op>
__device__ __forceinline__ void half_wave_reduce(T v, Op op, T& lo, T& hi) {
  v = op(v, dpp_move<0xB1>(v));
  v = op(v, dpp_move<0x4E>(v));
  v = op(v, dpp_move<0x141>(v));
  v = op(v, dpp_move<0x140>(v));
  lo = op(read_lane(v, 0), read_lane(v, 16));
  hi = op(read_lane(v, 32), read_lane(v, 48));
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), in registers: shifts
// of 1, 2, 4 and 8 inside each 16-lane row (row_shr), then row 0's total goes to row 1 and
// row 2's to row 3 (row_bcast:15), and rows 0-1's total to rows 2 and 3 (row_bcast:31).
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  v = v + dpp_move_or0<0x111, 0xF>(v);
  v = v + dpp_move_or0<0x112, 0xF>(v);
  v = v + dpp_move_or0<0x114, 0xF>(v);
  v = v + dpp_move_or0<0x118, 0xF>(v);
  v = v + dpp_move_or0<0x142, 0xA>(v);
  v = v + dpp_move_or0<0x143, 0xC>(v);
  return v;
}

// The value of the next lower lane (0 in lane 0): wave_shr:1.
template <typename T>
__device__ __forceinline__ T wave_shift_up1(T v) {
  return dpp_move_or0<0x138, 0xF>(v);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  return wave_reduce(v, [](T a, T b) { return b > a ? b : a; });
}

template <typename T>
__device__ __forceinline__ T wave_min(T v) {
  return wave_reduce(v, [](T a, T b) { return b < a ? b : a; });
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_reduce(v, [](T a, T b) { return a + b; });
}

// Order-preserving 64-bit key of a double: larger value, larger key; -0 and +0 share one.
__device__ __forceinline__ unsigned long long dkey(double d) {
  unsigned long long u = static_cast<unsigned long long>(__double_as_longlong(d));
  if ((u << 1) == 0) u = 0;
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Block-wide reductions over NW waves (kBlock threads by default); `red` is a __shared__
// scratch of at least NW entries of T. Every thread returns the result. Contains two
// __syncthreads().
template <typename T, int NW = kWaves>
__device__ __forceinline__ T block_max(T v, T* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  T r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = red[i] > r ? red[i] : r;
  __syncthreads();
  return r;
}

template <typename T, int NW = kWaves>
__device__ __forceinline__ T block_min(T v, T* red) {
  v = wave_min(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  T r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = red[i] < r ? red[i] : r;
  __syncthreads();
  return r;
}

template <typename T, int NW = kWaves>
__device__ __forceinline__ T block_sum(T v, T* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  T r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r += red[i];
  __syncthreads();
  return r;
}

// Exclusive prefix sum over the block (NW waves) in thread order (wave scans, then wave
// offsets). `wsum` is shared scratch of at least NW entries; *total receives the block sum.
template <typename T, int NW = kWaves>
__device__ __forceinline__ T block_exclusive_scan(T v, T* wsum, T* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const T inc = wave_inclusive_scan(v);
  const T exc = wave_shift_up1(inc);
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  T before = T(0), tot = T(0);
#pragma unroll
  for (int q = 0; q < NW; ++q) {
    if (q < w) before += wsum[q];
    tot += wsum[q];
  }
  __syncthreads();
  *total = tot;
  return before + exc;
}

// ---------------------------------------------------------------- cross-workgroup signalling
//
// The eight XCDs of an MI355X each have their own L2, so data one workgroup hands to
// another must not sit dirty in one XCD's L2. An agent-scope fence makes ordinary stores
// visible by writing back the whole L2, which costs microseconds per call; instead, every
// value that crosses workgroups here is written with st_cc (a relaxed agent-scope atomic
// store: a store the hardware keeps coherent across XCDs) and read with ld_cc (its load
// counterpart). Before a workgroup signals (ticket or barrier), every wave waits for its
// outstanding memory operations to complete (drain), so the data is in place before the
// signalling atomic is performed.

template <typename T>
__device__ __forceinline__ void st_cc(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T ld_cc(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Agent-scope acquire: after it, this workgroup's loads see everything made visible before
// the observed signal (the L1/L2 copies this CU might still hold are invalidated).
__device__ __forceinline__ void acquire_cc() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Wait until this wave's memory operations have completed (no compiler reordering across).
__device__ __forceinline__ void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ unsigned atomic_add_cc(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true in every thread of the workgroup that arrives last (count reaches n).
// The counter is reset to 0 by that workgroup so the next launch can reuse it. Data the
// arriving workgroups produced must have been written with st_cc and is read with ld_cc.
__device__ __forceinline__ bool last_arrival(unsigned* counter, unsigned n, int* flag_lds) {
  drain();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomic_add_cc(counter, 1u);
    const int last = (prev == n - 1) ? 1 : 0;
    if (last) {
      st_cc(counter, 0u);
      acquire_cc();
    }
    *flag_lds = last;
  }
  __syncthreads();
  return *flag_lds != 0;
}

// ---------------------------------------------------------------- error codes in workspaces
// The first 256 bytes of every workspace hold: int err; unsigned bar[2]; unsigned exit_count.
struct WsHeader {
  int err;
  unsigned bar[2];
  unsigned exit_count;
  unsigned pad[60];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

// kErrBadRow: a node's row lies outside its logit table (row < 0 or row >= R), or a drafted
// token outside the vocabulary where a kernel would read the logit at that token.
enum : int { kErrNone = 0, kErrCapacity = 1, kErrTimeout = 2, kErrBadTree = 3, kErrBadRow = 4 };

}  // namespace dtv
