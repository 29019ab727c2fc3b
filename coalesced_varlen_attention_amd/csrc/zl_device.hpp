// Device-side building blocks for gfx950 (CDNA4): bf16 MFMA tiles, transposed LDS reads,
// lane-half exchange and bf16 rounding.
//
// Lane layouts used throughout (wave of 64 lanes, l = lane, i = element):
//   v_mfma_f32_32x32x16_bf16  A[m][k]: m = l%32, k = 8*(l/32) + i (i < 8)
//                             B[k][n]: n = l%32, k = 8*(l/32) + i
//                             C[m][n]: n = l%32, m = 8*(i/4) + 4*(l/32) + i%4 (i < 16)
//   ds_read_b64_tr_b16        within each group of 16 lanes, lane r supplies the address of
//                             4 consecutive 16-bit values (row r of a 16x4 matrix S); lane i
//                             receives S[4k + i/4][i%4] for k = 0..3. Pointing the 16 lanes at
//                             a 4-row x 16-column block (lane r -> row r/4, columns 4*(r%4)..)
//                             hands lane i the 4 rows of column i: a transposed load.
//   v_permlane32_swap         swaps the upper half of one register with the lower half of
//                             another; applied to (x, x) it yields both halves' values in
//                             every lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zl_internal.h"

namespace zl {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define ZL_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposed read of four 16-bit values from LDS (see the layout note above).
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ZL_LDS i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}
// The same at an LDS address.
__device__ __forceinline__ bf16x4 lds_read_tr(uint32_t a) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ZL_LDS i16x4*)a);
  return __builtin_bit_cast(bf16x4, r);
}
__device__ __forceinline__ bf16x4 lds_read_tr(ZL_LDS const char* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ZL_LDS i16x4*)p);
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Round-to-nearest-even conversion of 8 floats to bf16.
__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

// max / sum of a value over lane l and lane l^32.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS tiles of bf16 rows (d elements each) are stored with a row stride of d + 8 elements and
// logical row r at physical row lds_row(r). The LDS has 64 banks of 4 bytes. The stride puts
// consecutive physical rows 16 bytes apart modulo 256, so 16 lanes reading the same 16-byte
// column of 16 rows hit distinct banks; the row permutation (within each group of 16 rows,
// r -> 4*(r%4) + r/4) puts the 4 consecutive logical rows of a transposed read 4 physical
// rows apart, so 32 lanes reading 4 rows x 64 bytes hit distinct banks as well. Both the
// 16-byte operand reads and the transposed reads are then free of bank conflicts, and every
// read address stays affine in the loop indices.
template <int D>
struct LdsTile {
  static constexpr int kLd = D + 8;  // row stride in elements
};
__device__ __forceinline__ int lds_row(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// A pointer that every lane of the wave holds, moved to scalar registers (the compiler cannot
// always prove that a value loaded from memory is the same in every lane).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
  const uint64_t v = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// Direct global -> LDS load of 16 bytes per lane: lane l reads base + off (off per lane) and
// its bytes land at lds_base + 16 l (base and lds_base are the same for the whole wave).
// Issued as inline assembly so that the compiler does not order later LDS reads of other
// buffers behind it; completion is awaited explicitly (dma_wait) before the workgroup barrier
// that publishes the buffer.
__device__ __forceinline__ void lds_dma16(uint32_t lds_base, const char* base, uint32_t off) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_base);
  // An LDS DMA right after a SALU write of M0 needs one wait state (s_nop 0).
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory");
}

// The same with 4 bytes per lane: lane l's bytes land at lds_base + 4 l.
__device__ __forceinline__ void lds_dma4(uint32_t lds_base, const char* base, uint32_t off) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(off), "s"(base)
               : "memory");
}

__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector memory operations of this wave are outstanding (they complete in
// issue order): the loads issued before the last N have landed.
template <int N>
__device__ __forceinline__ void dma_wait_all_but() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Device-coherent 16-byte store and loads (sc1: written through to, and read from, the point
// of coherence of all XCDs, past the per-XCD L2 and per-CU L1). For data one workgroup hands
// to another within a launch without fences, which would write back and invalidate a whole
// L2. The stores are complete once vmcnt reaches 0 (store_dev_wait). A store of more than
// 8 bytes reads its data registers after issue, and the compiler does not see inside inline
// assembly to keep the next write of those registers away: the s_nop after the store gives
// the required wait states.
__device__ __forceinline__ void store_dev16(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 4" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_dev_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Eight device-coherent 16-byte loads at p + 8 k floats (k < 8), one wait for all.
__device__ __forceinline__ void load_dev16x8(const float* p, f32x4 (&x)[8]) {
  asm volatile(
      "global_load_dwordx4 %0, %8, off sc1\n\t"
      "global_load_dwordx4 %1, %8, off offset:32 sc1\n\t"
      "global_load_dwordx4 %2, %8, off offset:64 sc1\n\t"
      "global_load_dwordx4 %3, %8, off offset:96 sc1\n\t"
      "global_load_dwordx4 %4, %8, off offset:128 sc1\n\t"
      "global_load_dwordx4 %5, %8, off offset:160 sc1\n\t"
      "global_load_dwordx4 %6, %8, off offset:192 sc1\n\t"
      "global_load_dwordx4 %7, %8, off offset:224 sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
      : "v"(p)
      : "memory");
}
// Sixteen device-coherent 16-byte loads at p + 8 k floats (k < 16), one wait for all.
__device__ __forceinline__ void load_dev16x16(const float* p, f32x4 (&x)[16]) {
  asm volatile(
      "global_load_dwordx4 %0, %16, off sc1\n\t"
      "global_load_dwordx4 %1, %16, off offset:32 sc1\n\t"
      "global_load_dwordx4 %2, %16, off offset:64 sc1\n\t"
      "global_load_dwordx4 %3, %16, off offset:96 sc1\n\t"
      "global_load_dwordx4 %4, %16, off offset:128 sc1\n\t"
      "global_load_dwordx4 %5, %16, off offset:160 sc1\n\t"
      "global_load_dwordx4 %6, %16, off offset:192 sc1\n\t"
      "global_load_dwordx4 %7, %16, off offset:224 sc1\n\t"
      "global_load_dwordx4 %8, %16, off offset:256 sc1\n\t"
      "global_load_dwordx4 %9, %16, off offset:288 sc1\n\t"
      "global_load_dwordx4 %10, %16, off offset:320 sc1\n\t"
      "global_load_dwordx4 %11, %16, off offset:352 sc1\n\t"
      "global_load_dwordx4 %12, %16, off offset:384 sc1\n\t"
      "global_load_dwordx4 %13, %16, off offset:416 sc1\n\t"
      "global_load_dwordx4 %14, %16, off offset:448 sc1\n\t"
      "global_load_dwordx4 %15, %16, off offset:480 sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]),
        "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]), "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]),
        "=&v"(x[15])
      : "v"(p)
      : "memory");
}

// Copies a queue set's bounds (kernel arguments) into LDS, where take_item reads them: held in
// scalar registers they would stay live through every item. Called by the thread that calls
// take_item, which alone reads the copy, so no barrier is needed.
__device__ __forceinline__ void stage_bounds(const Queues& q, ZL_LDS int32_t* lds) {
#pragma unroll
  for (int k = 0; k <= kQueues; ++k) lds[k] = q.bounds[k];
}

// Next work item for a workgroup, called by one thread; returns -1 once every queue is drained.
// The workgroup's queue state lives in LDS, so that nothing holds registers for it during an
// item: `bounds` is the copy of the queue bounds and `state` packs the queues known to be
// drained (bits 0-7; counters only grow, so a drained queue stays drained), the queue to try
// first (bits 8-10) and whether the static first item was taken (bit 11); the kernel sets
// `state` to its home queue (home << 8) before the first call.
//   * The first call takes the workgroup's static item, item blockIdx.x / kQueues of its home
//     queue (the launch set that queue's counter to home_count, past those items).
//   * Later calls pop the current queue (home, or the queue the last item was stolen from).
//   * When it is drained, the counters of all other queues are read at once (one round trip),
//     and only queues that still hold items are popped, nearest to home first. A workgroup
//     that finds every queue drained leaves after two round trips instead of one atomic per
//     queue.
// Every call ends after at most kQueues + 1 atomics. With `visits` (the scheduler check), the
// item taken is also counted there.
__device__ __forceinline__ int take_item(const Queues& q, const ZL_LDS int32_t* bounds, ZL_LDS int32_t* state,
                                         int32_t* visits) {
  constexpr uint32_t kAll = (1u << kQueues) - 1;
  const uint32_t st = (uint32_t)*state;
  uint32_t empty = st & kAll;
  int cur = (int)(st >> 8) & (kQueues - 1);
  const int home = (int)(blockIdx.x % kQueues);
  int idx = -1;
  if (!(st & (1u << 11))) {
    const int j = bounds[home] + (int)(blockIdx.x / kQueues);
    if (j < bounds[home + 1]) idx = j;
    else empty |= 1u << home;
  }
  if (idx < 0 && !(empty >> cur & 1)) {
    const int j = bounds[cur] + atomicAdd(&q.counters[cur * kCounterStride], 1);
    if (j < bounds[cur + 1]) idx = j;
    else empty |= 1u << cur;
  }
  if (idx < 0 && empty != kAll) {
    int c[kQueues];
#pragma unroll
    for (int k = 0; k < kQueues; ++k)
      c[k] = __hip_atomic_load(&q.counters[k * kCounterStride], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int k = 0; k < kQueues; ++k)
      if (bounds[k] + c[k] >= bounds[k + 1]) empty |= 1u << k;
    for (int i = 1; i < kQueues && idx < 0; ++i) {
      const int k = (home + i) & (kQueues - 1);
      if (empty >> k & 1) continue;
      const int j = bounds[k] + atomicAdd(&q.counters[k * kCounterStride], 1);
      if (j < bounds[k + 1]) {
        idx = j;
        cur = k;
      } else {
        empty |= 1u << k;
      }
    }
  }
  *state = (int32_t)(empty | (uint32_t)cur << 8 | 1u << 11);
  if (idx >= 0 && visits) atomicAdd(visits + idx, 1);
  return idx;
}

}  // namespace zl
