// Forward kernel: persistent, per-XCD cost-ordered queues of (segment, head, 128 query rows)
// items.
//
// Computes, per item, softmax attention of 128 query rows against the segment's key rows
// (dense bidirectional attention of one sequence, Zellige page §II-A; segments never read
// another sequence's keys, §IV-D), with an online softmax over blocks of 64 keys, and
// writes either the final O and LSE at the query rows or, for a ring part, the normalised
// partial O and its LSE to the partial slab (§II-B ring accumulation).
//
// Shape of one workgroup: 4 waves x 32 query rows. Each wave keeps its 32 query rows in
// registers as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so every lane owns
// one query row of the score tile: the running max and sum are per-lane values that only
// combine with the partner lane l^32. The exponentiated scores, rounded to bf16, are already
// in the B-operand layout of O^T = V^T P^T; V^T comes from a natural [key][d] LDS tile
// through transposed LDS reads. K and V blocks are double-buffered in LDS and the next
// block's global loads are in flight while the current block is computed.
#include "zl_device.hpp"
#include "zl_internal.h"

namespace zl {
namespace {

template <int D>
struct FwdCfg {
  static constexpr int kThreads = 256;
  static constexpr int kBk = 64;                              // keys per block
  static constexpr int kLd = LdsTile<D>::kLd;                 // K and V row stride in LDS (elements)
  static constexpr int kSteps = D / 16;                       // k-steps over d for S^T
  static constexpr int kCb = D / 32;                          // 32-wide column blocks of O^T
  static constexpr int kChunks = kBk * D / 8 / kThreads;      // 16-byte chunks per thread per block
  static constexpr int kRowChunks = D / 8;                    // 16-byte chunks per row
};

// Global -> registers for one block of 64 key rows of K and V (16-byte chunks, rows clamped
// to the last valid key), and registers -> LDS.
template <int D>
__device__ __forceinline__ void fwd_load_block(u32x4 (&kreg)[FwdCfg<D>::kChunks], u32x4 (&vreg)[FwdCfg<D>::kChunks],
                                               const bf16* kbase, const bf16* vbase, int64_t rs, int j, int n_kv,
                                               int tid) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int c = 0; c < C::kChunks; ++c) {
    const int chunk = tid + c * C::kThreads;
    const int r = chunk / C::kRowChunks;
    const int col = (chunk % C::kRowChunks) * 8;
    const int key = min(j * C::kBk + r, n_kv - 1);
    kreg[c] = *(const u32x4*)(kbase + (int64_t)key * rs + col);
    vreg[c] = *(const u32x4*)(vbase + (int64_t)key * rs + col);
  }
}

template <int D>
__device__ __forceinline__ void fwd_store_block(const u32x4 (&kreg)[FwdCfg<D>::kChunks],
                                                const u32x4 (&vreg)[FwdCfg<D>::kChunks], bf16* k_lds, bf16* v_lds,
                                                int tid) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int c = 0; c < C::kChunks; ++c) {
    const int chunk = tid + c * C::kThreads;
    const int r = chunk / C::kRowChunks;
    const int col = (chunk % C::kRowChunks) * 8;
    *(u32x4*)&k_lds[lds_row(r) * C::kLd + col] = kreg[c];
    *(u32x4*)&v_lds[lds_row(r) * C::kLd + col] = vreg[c];
  }
}

__global__ void zero_counters_kernel(int32_t* counters) { counters[threadIdx.x * kCounterStride] = 0; }

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const FwdParams p) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 k_lds[2][C::kBk * C::kLd];
  __shared__ __attribute__((aligned(16))) bf16 v_lds[2][C::kBk * C::kLd];
  __shared__ int32_t s_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int r_in = (lane & 15) >> 2;                        // transposed-read row within 4
  const int c_in = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // transposed-read column within 32
  const int prow_b = lds_row(l32);                           // physical row of this lane's operand row
  const int prow_t = lds_row(4 * hi + r_in);                 // physical row of its transposed reads
  const bf16* __restrict__ gq = (const bf16*)p.q;
  const bf16* __restrict__ gk = (const bf16*)p.k;
  const bf16* __restrict__ gv = (const bf16*)p.v;

  const int home = blockIdx.x % kQueues;
  int drained = 0;
  for (;;) {
    if (tid == 0) s_item = take_item(p.queue, home, drained);
    __syncthreads();
    const int item = s_item;
    if (item < 0) break;
    const Tile tile = p.queue.items[item];
    const SegDev sg = p.segs[tile.seg];
    const int nh = sg.nh;
    const int h = tile.head;
    const int64_t rs = (int64_t)nh * D;  // elements between consecutive tokens

    // This lane's query row (clamped to the last valid row; results of clamped rows are dropped).
    const int qi = wave * 32 + l32;
    const bool q_valid = qi < tile.nrows;
    const int qtok = tile.row0 + (q_valid ? qi : tile.nrows - 1);
    bf16x8 qreg[C::kSteps];
    {
      const bf16* qp = gq + (sg.q_row0 + (int64_t)qtok * nh + h) * D + 8 * hi;
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) qreg[s] = *(const bf16x8*)(qp + 16 * s);
    }

    const int n_kv = sg.kv_end - sg.kv_begin;
    const int n_blk = (n_kv + C::kBk - 1) / C::kBk;
    const bf16* kbase = gk + (sg.kv_row0 + (int64_t)sg.kv_begin * nh + h) * D;
    const bf16* vbase = gv + (sg.kv_row0 + (int64_t)sg.kv_begin * nh + h) * D;

    u32x4 kreg[C::kChunks], vreg[C::kChunks];
    f32x16 oacc[C::kCb];
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb) oacc[cb] = f32x16{};
    float m_run = -INFINITY;  // running max of scaled scores, log2 units
    float l_run = 0.f;        // this lane's share of the running sum

    fwd_load_block<D>(kreg, vreg, kbase, vbase, rs, 0, n_kv, tid);
    fwd_store_block<D>(kreg, vreg, k_lds[0], v_lds[0], tid);
    __syncthreads();

    for (int j = 0; j < n_blk; ++j) {
      const int buf = j & 1;
      if (j + 1 < n_blk) fwd_load_block<D>(kreg, vreg, kbase, vbase, rs, j + 1, n_kv, tid);

      // S^T[key][q] for the block's 64 keys, as two 32x32 tiles.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        const bf16* kr = &k_lds[buf][(kb * 32 + prow_b) * C::kLd + 8 * hi];
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) sacc[kb] = mfma32(*(const bf16x8*)(kr + 16 * s), qreg[s], sacc[kb]);
      }
      // Keys past the end of the segment (last block only) get -inf.
      const int valid = n_kv - j * C::kBk;
      if (valid < C::kBk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
            if (key >= valid) sacc[kb][i] = -INFINITY;
          }
      }
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = half_max(mx) * p.scale_log2;
      // Lazy rescaling: the exponent reference m_run only moves when the block max exceeds it
      // by more than kSlack (log2 units), so exponentials stay below 2^kSlack and the O and l
      // rescale runs only when some lane of the wave needs it. The result is the same quantity;
      // only the reference of the running sums changes.
      constexpr float kSlack = 8.0f;
      const bool need = mx > m_run + kSlack;
      if (__any(need)) {
        const float m_new = need ? mx : m_run;
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb) oacc[cb] *= alpha;
      }

      bf16x8 pb[4];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          f32x8 e;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            e[u] = fast_exp2(fmaf(sacc[kb][8 * hs + u], p.scale_log2, -m_run));
            lsum += e[u];
          }
          pb[kb * 2 + hs] = to_bf16x8(e);
        }
      l_run += lsum;

      // O^T[c][q] += V^T[c][key] P^T[key][q], 16 keys per step. The k order of P^T in this
      // lane is keys {16hs + 4hi + 0..3, 16hs + 8 + 4hi + 0..3} of each 32-key half; the two
      // transposed reads fetch V rows in that same order (logical rows +8 are physical rows +2).
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int row = (ks >> 1) * 32 + 16 * (ks & 1) + prow_t;
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb) {
          const bf16* vp = &v_lds[buf][row * C::kLd + cb * 32 + c_in];
          const bf16x8 a = cat(lds_read_tr(vp), lds_read_tr(vp + 2 * C::kLd));
          oacc[cb] = mfma32(a, pb[ks], oacc[cb]);
        }
      }

      if (j + 1 < n_blk) fwd_store_block<D>(kreg, vreg, k_lds[buf ^ 1], v_lds[buf ^ 1], tid);
      __syncthreads();
    }

    // Epilogue: O = O_acc / l, LSE = ln(2) * (m + log2 l), natural log.
    const float l_tot = half_sum(l_run);
    if (q_valid) {
      const float inv = 1.0f / l_tot;
      float* orow;
      int64_t lrow;
      float* lse_out;
      if (sg.part < 0) {
        lrow = sg.q_row0 + (int64_t)qtok * nh + h;
        orow = p.o + lrow * D;
        lse_out = p.lse;
      } else {
        lrow = sg.part_row0 + (int64_t)(qtok - sg.q_begin) * nh + h;
        orow = p.o_part + lrow * D;
        lse_out = p.lse_part;
      }
#pragma unroll
      for (int cb = 0; cb < C::kCb; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = cb * 32 + 8 * g + 4 * hi;
          f32x4 val = {oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv, oacc[cb][4 * g + 2] * inv,
                       oacc[cb][4 * g + 3] * inv};
          *(f32x4*)(orow + c) = val;
        }
      if (hi == 0) lse_out[lrow] = 0.69314718055994531f * (m_run + __log2f(l_tot));
    }
    __syncthreads();
  }
}

template <int D>
int blocks_per_cu_impl() {
  static int cached = -1;
  if (cached < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_kernel<D>, 256, 0) != hipSuccess) n = 0;
    cached = n;
  }
  return cached;
}

}  // namespace

int fwd_blocks_per_cu(int d) { return d == 64 ? blocks_per_cu_impl<64>() : blocks_per_cu_impl<128>(); }

int launch_fwd(int d, const FwdParams& p, int grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(kQueues), 0, s, p.queue.counters);
  if (d == 64)
    hipLaunchKernelGGL(fwd_kernel<64>, dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(fwd_kernel<128>, dim3(grid), dim3(256), 0, s, p);
  return hipPeekAtLastError() == hipSuccess ? 0 : 1;
}

}  // namespace zl
