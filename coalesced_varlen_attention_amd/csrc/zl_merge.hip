// Exact merge of ring partial results (Zellige page §II-B: ring attention accumulates the
// output block by block; the merge of normalised partials by their log-sum-exps is exact):
//   LSE = M + ln sum_b exp(LSE_b - M),  O = sum_b exp(LSE_b - LSE) O_b,  M = max_b LSE_b.
// Parts with LSE_b = -inf weigh 0; if all are -inf the row gets O = 0, LSE = -inf.
// Two forms: one contiguous run of rows (merge_kernel), and every group of a plan, whose
// head subsets scatter to strided O rows (plan_merge_kernel).
// HBM-bound: one pass over the partials, D/4 lanes per row with 16-byte nontemporal loads, every
// part's load of a row in flight before the first is used, one workgroup per pass of rows (a
// grid-stride loop only beyond kMergeMaxGrid workgroups). On the ring shard's slab (8 parts x
// 378,000 rows x 128) this streams 6.3 TB/s, against 5.0 TB/s with cached loads and a grid of
// 16 workgroups per compute unit.
#include "zl_device.hpp"
#include "zl_internal.h"

namespace zl {
namespace {

// Merge of one row: `row` indexes part 0's slab rows, parts are `stride` rows apart; lane
// `sub` of the row's D/4 lanes handles 4 columns. NP > 0: exactly NP parts, fully unrolled, so
// every part's LSE and 16-byte O load is issued before the first one is used (the row's bytes
// are in flight at once); NP == 0: any n_parts, in batches of 8 with the running form of the
// same merge. Weights are exp2 of log2(e)-scaled differences, each part's LSE read once.
template <int D, int NP>
__device__ __forceinline__ void merge_row(int32_t n_parts, int64_t stride, int64_t row, int sub,
                                          const float* __restrict__ o_part, const float* __restrict__ lse_part,
                                          float* __restrict__ o_out, float* __restrict__ lse_out) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.69314718055994531f;
  constexpr int kB = NP > 0 ? NP : 8;  // parts per batch
  // Running state over batches (NP > 0: one batch): reference m (the largest LSE so far, natural
  // log), sum of the weights exp(LSE_b - m), and the weighted sum of O. The reference stays in
  // natural-log units, so that LSE = m + ln 2 log2(sum) returns a lone part's LSE unchanged.
  float m = -INFINITY, tot = 0.f;
  f32x4 acc = f32x4{};
  for (int b0 = 0; b0 < n_parts; b0 += kB) {
    float l[kB];
    f32x4 x[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b)
      l[b] = (NP > 0 || b0 + b < n_parts) ? lse_part[(int64_t)(b0 + b) * stride + row] : -INFINITY;
#pragma unroll
    for (int b = 0; b < kB; ++b)
      if (NP > 0 || b0 + b < n_parts)  // streamed once: nontemporal loads keep it out of the caches
        x[b] = __builtin_nontemporal_load((const f32x4*)(o_part + ((int64_t)(b0 + b) * stride + row) * D + 4 * sub));
    float mb = m;
#pragma unroll
    for (int b = 0; b < kB; ++b) mb = fmaxf(mb, l[b]);
    if (mb == -INFINITY) continue;  // no keys so far: nothing to add
    const float r = __builtin_amdgcn_exp2f((m - mb) * kLog2e);  // rescale of earlier batches (0 if none)
    tot *= r;
    acc *= r;
#pragma unroll
    for (int b = 0; b < kB; ++b) {
      if (l[b] == -INFINITY) continue;  // a part with no keys: weight 0, its O is not used
      const float w = __builtin_amdgcn_exp2f((l[b] - mb) * kLog2e);
      tot += w;
      acc += w * x[b];
    }
    m = mb;
  }
  float out_lse = -INFINITY;
  if (m != -INFINITY) {
    acc *= 1.0f / tot;
    out_lse = m + kLn2 * __builtin_amdgcn_logf(tot);
  }
  *(f32x4*)(o_out + 4 * sub) = acc;
  if (sub == 0) *lse_out = out_lse;
}

template <int D, int NP>
__global__ __launch_bounds__(256) void merge_kernel(int32_t n_parts, int64_t n_rows, const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, float* __restrict__ o,
                                                    float* __restrict__ lse) {
  constexpr int kLanes = D / 4;             // lanes per row
  constexpr int kRows = merge_rows(D);      // rows per workgroup pass
  const int sub = threadIdx.x % kLanes;
  for (int64_t row = (int64_t)blockIdx.x * kRows + threadIdx.x / kLanes; row < n_rows;
       row += (int64_t)gridDim.x * kRows)
    merge_row<D, NP>(n_parts, n_rows, row, sub, o_part, lse_part, o + row * D, lse + row);
}

// Every group of a plan in one launch. Merge block vb belongs to the last group whose block0
// is <= vb; its rows are the group's slab rows (token-major over the group's heads), each
// written to its O/LSE row o_row + (r / n_sub) * nh + r % n_sub.
template <int D>
__global__ __launch_bounds__(256) void plan_merge_kernel(const GroupDev* __restrict__ groups, int32_t n_groups,
                                                         int64_t n_blocks, const float* __restrict__ o_part,
                                                         const float* __restrict__ lse_part, float* __restrict__ o,
                                                         float* __restrict__ lse) {
  constexpr int kLanes = D / 4;
  constexpr int kRows = merge_rows(D);
  const int sub = threadIdx.x % kLanes;
  for (int64_t vb = blockIdx.x; vb < n_blocks; vb += gridDim.x) {
    int lo = 0, hi = n_groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (groups[mid].block0 <= vb) lo = mid; else hi = mid - 1;
    }
    const GroupDev g = groups[lo];
    const int64_t r = (vb - g.block0) * kRows + threadIdx.x / kLanes;
    if (r >= g.n_rows) continue;
    const int64_t out = g.o_row + (r / g.n_sub) * g.nh + r % g.n_sub;
    float* orow = o + out * D;
    const int64_t prow = g.part_row + r;
    switch (g.n_parts) {  // the common ring degrees fully unrolled
      case 2: merge_row<D, 2>(2, g.n_rows, prow, sub, o_part, lse_part, orow, lse + out); break;
      case 4: merge_row<D, 4>(4, g.n_rows, prow, sub, o_part, lse_part, orow, lse + out); break;
      case 8: merge_row<D, 8>(8, g.n_rows, prow, sub, o_part, lse_part, orow, lse + out); break;
      default: merge_row<D, 0>(g.n_parts, g.n_rows, prow, sub, o_part, lse_part, orow, lse + out); break;
    }
  }
}

template <int D, int NP>
void launch_merge_np(int32_t n_parts, int64_t n_rows, const float* o_part, const float* lse_part, float* o,
                     float* lse, int grid, hipStream_t s) {
  hipLaunchKernelGGL((merge_kernel<D, NP>), dim3(grid), dim3(256), 0, s, n_parts, n_rows, o_part, lse_part, o, lse);
}

template <int D>
void launch_merge_d(int32_t n_parts, int64_t n_rows, const float* o_part, const float* lse_part, float* o, float* lse,
                    int grid, hipStream_t s) {
  switch (n_parts) {
    case 1: launch_merge_np<D, 1>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s); break;
    case 2: launch_merge_np<D, 2>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s); break;
    case 3: launch_merge_np<D, 3>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s); break;
    case 4: launch_merge_np<D, 4>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s); break;
    case 5: launch_merge_np<D, 5>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s); break;
    case 6: launch_merge_np<D, 6>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s); break;
    case 7: launch_merge_np<D, 7>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s); break;
    case 8: launch_merge_np<D, 8>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s); break;
    default: launch_merge_np<D, 0>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s); break;
  }
}

}  // namespace

int launch_plan_merge(int d, const GroupDev* groups, int32_t n_groups, int64_t n_blocks, const float* o_part,
                      const float* lse_part, float* o, float* lse, int grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (d == 64)
    hipLaunchKernelGGL(plan_merge_kernel<64>, dim3(grid), dim3(256), 0, s, groups, n_groups, n_blocks, o_part,
                       lse_part, o, lse);
  else
    hipLaunchKernelGGL(plan_merge_kernel<128>, dim3(grid), dim3(256), 0, s, groups, n_groups, n_blocks, o_part,
                       lse_part, o, lse);
  return hipPeekAtLastError() == hipSuccess ? 0 : 1;
}

int launch_merge(int d, int32_t n_parts, int64_t n_rows, const float* o_part, const float* lse_part, float* o,
                 float* lse, int grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (d == 64)
    launch_merge_d<64>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s);
  else
    launch_merge_d<128>(n_parts, n_rows, o_part, lse_part, o, lse, grid, s);
  return hipPeekAtLastError() == hipSuccess ? 0 : 1;
}

}  // namespace zl
