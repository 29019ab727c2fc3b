// Exact merge of ring partial results (Zellige page §II-B: ring attention accumulates the
// output block by block; the merge of normalised partials by their log-sum-exps is exact):
//   LSE = M + ln sum_b exp(LSE_b - M),  O = sum_b exp(LSE_b - LSE) O_b,  M = max_b LSE_b.
// Parts with LSE_b = -inf weigh 0; if all are -inf the row gets O = 0, LSE = -inf.
// HBM-bound: one pass over the partials, D/4 lanes per row with 16-byte loads.
#include "zl_device.hpp"
#include "zl_internal.h"

namespace zl {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(int32_t n_parts, int64_t n_rows, const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, float* __restrict__ o,
                                                    float* __restrict__ lse) {
  constexpr int kLanes = D / 4;             // lanes per row
  constexpr int kRows = 256 / kLanes;       // rows per workgroup pass
  const int sub = threadIdx.x % kLanes;
  for (int64_t row = (int64_t)blockIdx.x * kRows + threadIdx.x / kLanes; row < n_rows;
       row += (int64_t)gridDim.x * kRows) {
    float m = -INFINITY;
    for (int b = 0; b < n_parts; ++b) m = fmaxf(m, lse_part[(int64_t)b * n_rows + row]);
    f32x4 acc = f32x4{};
    float out_lse = -INFINITY;
    if (m != -INFINITY) {
      float tot = 0.f;
      for (int b = 0; b < n_parts; ++b) {
        const float lb = lse_part[(int64_t)b * n_rows + row];
        if (lb != -INFINITY) tot += expf(lb - m);
      }
      out_lse = m + logf(tot);
      for (int b = 0; b < n_parts; ++b) {
        const float lb = lse_part[(int64_t)b * n_rows + row];
        if (lb == -INFINITY) continue;
        const float w = expf(lb - out_lse);
        const f32x4 x = *(const f32x4*)(o_part + ((int64_t)b * n_rows + row) * D + 4 * sub);
        acc += w * x;
      }
    }
    *(f32x4*)(o + row * D + 4 * sub) = acc;
    if (sub == 0) lse[row] = out_lse;
  }
}

}  // namespace

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
