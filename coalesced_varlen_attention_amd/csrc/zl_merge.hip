// Exact merge of ring partial results (Zellige page §II-B: ring attention accumulates the
// output block by block; the merge of normalised partials by their log-sum-exps is exact):
//   LSE = M + ln sum_b exp(LSE_b - M),  O = sum_b exp(LSE_b - LSE) O_b,  M = max_b LSE_b.
// Parts with LSE_b = -inf weigh 0; if all are -inf the row gets O = 0, LSE = -inf.
// Two forms: one contiguous run of rows (merge_kernel), and every group of a plan, whose
// head subsets scatter to strided O rows (plan_merge_kernel).
// HBM-bound: one pass over the partials, D/4 lanes per row with 16-byte loads.
#include "zl_device.hpp"
#include "zl_internal.h"

namespace zl {
namespace {

// Merge of one row: `row` indexes part 0's slab rows, parts are `stride` rows apart; lane
// `sub` of the row's D/4 lanes handles 4 columns.
template <int D>
__device__ __forceinline__ void merge_row(int32_t n_parts, int64_t stride, int64_t row, int sub,
                                          const float* __restrict__ o_part, const float* __restrict__ lse_part,
                                          float* __restrict__ o_out, float* __restrict__ lse_out) {
  float m = -INFINITY;
  for (int b = 0; b < n_parts; ++b) m = fmaxf(m, lse_part[(int64_t)b * stride + row]);
  f32x4 acc = f32x4{};
  float out_lse = -INFINITY;
  if (m != -INFINITY) {
    float tot = 0.f;
    for (int b = 0; b < n_parts; ++b) {
      const float lb = lse_part[(int64_t)b * stride + row];
      if (lb != -INFINITY) tot += expf(lb - m);
    }
    out_lse = m + logf(tot);
    for (int b = 0; b < n_parts; ++b) {
      const float lb = lse_part[(int64_t)b * stride + row];
      if (lb == -INFINITY) continue;
      const float w = expf(lb - out_lse);
      const f32x4 x = *(const f32x4*)(o_part + ((int64_t)b * stride + row) * D + 4 * sub);
      acc += w * x;
    }
  }
  *(f32x4*)(o_out + 4 * sub) = acc;
  if (sub == 0) *lse_out = out_lse;
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(int32_t n_parts, int64_t n_rows, const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, float* __restrict__ o,
                                                    float* __restrict__ lse) {
  constexpr int kLanes = D / 4;             // lanes per row
  constexpr int kRows = merge_rows(D);      // rows per workgroup pass
  const int sub = threadIdx.x % kLanes;
  for (int64_t row = (int64_t)blockIdx.x * kRows + threadIdx.x / kLanes; row < n_rows;
       row += (int64_t)gridDim.x * kRows)
    merge_row<D>(n_parts, n_rows, row, sub, o_part, lse_part, o + row * D, lse + row);
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
    merge_row<D>(g.n_parts, g.n_rows, g.part_row + r, sub, o_part, lse_part, o + out * D, lse + out);
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
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(256), 0, s, n_parts, n_rows, o_part, lse_part, o, lse);
  else
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(256), 0, s, n_parts, n_rows, o_part, lse_part, o, lse);
  return hipPeekAtLastError() == hipSuccess ? 0 : 1;
}

}  // namespace zl
