// Device helpers shared by the forward and backward block-sparse attention
// kernels: bf16 fragment types, direct global->LDS loads, vector-memory
// waits, the fence-free barrier, the LDS swizzles of the K / V^T ring images,
// the block-bitmap walk and the cross-half merges.  Internal to libfva.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fva_attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Key slot order inside one 32-key half of the VT layout: slot s holds key
// 16*c + 8*(j/4) + 4*g + j%4 with c = s/16, g = (s%16)/8, j = s%8.  This is
// the key order in which a 32x32x16 bf16 matrix-core instruction's B-operand
// lanes receive P^T when P^T comes straight from the S^T accumulators, so the
// matching A operand (V^T) is one contiguous 16-byte load per lane.
__device__ __forceinline__ int vt_slot_key(int s) {
  const int c = s >> 4, g = (s >> 3) & 1, j = s & 7;
  return 16 * c + 8 * (j >> 2) + 4 * g + (j & 3);
}

constexpr int kXcds = 8;    // MI355X: 8 XCDs, workgroups dealt round-robin

// Work-list position of the k-th row an XCD takes: the list is cut into
// chunks of `chunk` rows dealt round-robin to the XCDs, so the workgroups of
// one XCD (one L2) walk contiguous query blocks of the same head.
__device__ __forceinline__ int64_t xcd_item(int x, int64_t k, int chunk) {
  return ((k / chunk) * kXcds + x) * chunk + k % chunk;
}

// Direct global->LDS load of 16 bytes per lane from the wave-uniform base
// plus the lane's 32-bit byte offset; lane i's bytes land at LDS address
// lds_addr + 16*i (lds_addr wave-uniform).
// Written as inline assembly on purpose: the compiler cannot tell which ring
// stage a direct load writes, so for the builtin it makes every later LDS
// read wait for all direct loads in flight, which would drain the prefetch
// pipeline each step.  Ordering is kept by hand instead: each wave waits on
// its own vector-memory count (wait_vm) and a workgroup barrier publishes
// the stage before any wave reads it.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds_addr) : "memory", "m0");
}

// dma16 for call sites where the compiler cannot prove the (wave-uniform)
// LDS address scalar, e.g. a ring index modulo 3: readfirstlane states it.
__device__ __forceinline__ void dma16u(const void* base, uint32_t off, uint32_t lds_addr) {
  dma16(base, off, __builtin_amdgcn_readfirstlane(lds_addr));
}

// LDS byte address of a shared-memory object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt with only the vector-memory count limited to n (other counters
// left free).  gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt_hi[15:14].
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence __syncthreads() implies: the
// fence would drain every outstanding vector load, including the direct
// loads of the steps still in flight.  The empty asm statements keep the
// compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Combine lane l with lane l^32 without an LDS round trip: v_permlane32_swap
// of x with itself leaves x[l%32] in one result and x[l%32 + 32] in the other.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-uniform reads of read-only metadata through the scalar cache.
template <typename T>
__device__ __forceinline__ T sload(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

// XOR swizzles of the LDS images (16-byte chunk index within a row).  They
// keep every group of 8 and of 16 consecutive lanes of a ds_read_b128 on
// distinct 16-byte bank slots.  K rows are D*2 bytes (KCH chunks); V^T rows
// are 64 bytes (4 chunks).
template <int D>
__device__ __forceinline__ int kswz(int row) {
  return D == 128 ? (row & 15) : ((row & 6) | ((row ^ (row >> 3)) & 1));
}
__device__ __forceinline__ int vswz(int d) {
  return (((d >> 1) ^ (d >> 2)) & 1) | ((((d >> 2) ^ (d >> 3)) & 1) << 1);
}

// Word w (blocks 64w..64w+63) of a block bitmap held one 64-bit word per
// lane, read out as a wave-uniform value.
__device__ __forceinline__ uint64_t lane_word(uint32_t lo, uint32_t hi, int w) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, w) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)lo, w);
}

// Steps of a walk over such a bitmap: two 32-position halves per set bit,
// summed over the wave (wave-uniform result).
__device__ __forceinline__ int union_steps(uint32_t lo, uint32_t hi) {
  int c = __popc(lo) + __popc(hi);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
  return 2 * __builtin_amdgcn_readfirstlane(c);
}

// Ascending walk over the set bits of such a bitmap; the state is
// wave-uniform, so the walk is scalar arithmetic with no memory access.
struct BitWalk {
  uint64_t bits = 0;  // unvisited bits of word w
  int w = -1;
  __device__ __forceinline__ bool next(uint32_t lo, uint32_t hi, int nw, int* J) {
    while (bits == 0) {
      if (++w >= nw) return false;
      bits = lane_word(lo, hi, w);
    }
    *J = 64 * w + __builtin_ctzll(bits);
    bits &= bits - 1;
    return true;
  }
  // The next set bit when the caller knows one is left (no end test).
  __device__ __forceinline__ int next_known(uint32_t lo, uint32_t hi) {
    while (bits == 0) bits = lane_word(lo, hi, ++w);
    const int J = 64 * w + __builtin_ctzll(bits);
    bits &= bits - 1;
    return J;
  }
};

}  // namespace fva_attn
