// Backward kernels: the pre-pass and the persistent main kernel.
//
// Gradients of f = sum dO . O for softmax attention (the exact backward named on the Zellige
// page, §V-A), recomputing the probabilities from the forward's LSE:
//   P = exp(tau Q K^T - LSE),  dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dK = tau dS^T Q,  dQ = tau dS K,  with D_i = sum_c dO_ic O_ic.
// For a ring part the LSE and O are the merged ones, so P is the global softmax restricted
// to the part's keys and dQ sums over parts.
//
// Pre-pass: D for every covered query row, and dQ zeroed (dQ is accumulated with atomics).
// Main kernel: one item = 128 key rows of one (segment, head); 4 waves x 32 keys. Each wave
// keeps its K and V rows in registers as B operands of S = Q K^T and dP = dO V^T (lane = one
// key column), so P and dS come out of the MFMA already in the B-operand layout of
// dV^T = dO^T P and dK^T = Q^T dS; dO^T and Q^T are read from natural LDS tiles with
// transposed LDS reads. dS^T goes through LDS once more to form dQ = dS K for the 64 query
// rows of the step, which is added to global dQ with fp32 atomics. The loop over query
// blocks starts at a block that depends on the key block, so that items of one head that
// run at the same time add into different dQ rows.
#include "zl_device.hpp"
#include "zl_internal.h"

namespace zl {
namespace {

template <int D>
struct BwdCfg {
  static constexpr int kThreads = 256;
  static constexpr int kBq = kBwdRows;                    // 64 query rows per step
  static constexpr int kBk = kBwdKeys;                    // 128 keys per item
  static constexpr int kQld = D + 8;                      // Q / dO row stride in LDS
  static constexpr int kKld = D + 16;                     // K tile row stride in LDS
  static constexpr int kSld = kBq + 8;                    // dS^T row stride in LDS
  static constexpr int kSteps = D / 16;                   // k-steps over d
  static constexpr int kCb = D / 32;                      // 32-wide column blocks over d
  static constexpr int kQChunks = kBq * D / 8 / kThreads; // 16-B chunks per thread (Q or dO)
  static constexpr int kKChunks = kBk * D / 8 / kThreads; // 16-B chunks per thread (K tile)
  static constexpr int kRowChunks = D / 8;
  // dQ: waves split (column block, 32-row block) pairs of the 64 x D output.
  static constexpr int kWavesPerCb = 4 / kCb;             // 1 (D=128) or 2 (D=64)
  static constexpr int kMbPerWave = 2 / kWavesPerCb;      // 2 (D=128) or 1 (D=64)
};

// D_i = sum_c dO_ic O_ic for every covered query row; dQ rows zeroed; queue counter zeroed.
// 16 lanes per row, 16 rows per workgroup pass.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdParams p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *p.counter = 0;
  constexpr int kPer = D / 16;  // elements per lane
  const int sub = threadIdx.x & 15;
  const int rsel = threadIdx.x >> 4;
  const bf16* gdo = (const bf16*)p.d_o;
  for (int it = blockIdx.x; it < p.n_pre; it += gridDim.x) {
    const Tile t = p.pre_tiles[it];
    const SegDev sg = p.segs[t.seg];
    const int nhr = sg.head_end - sg.head_begin;
    const int rows = t.nrows * nhr;
    for (int r = rsel; r < rows; r += 16) {
      const int tok = t.row0 + r / nhr;
      const int h = sg.head_begin + r % nhr;
      const int64_t row = sg.q_row0 + (int64_t)tok * sg.nh + h;
      const int64_t e0 = row * D + sub * kPer;
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < kPer; u += 4) {
        const f32x4 o4 = *(const f32x4*)(p.o + e0 + u);
        const bf16x4 d4 = *(const bf16x4*)(gdo + e0 + u);
        acc += (float)d4[0] * o4[0] + (float)d4[1] * o4[1] + (float)d4[2] * o4[2] + (float)d4[3] * o4[3];
        *(f32x4*)(p.dq + e0 + u) = f32x4{};
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
      if (sub == 0) p.dvec[row] = acc;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_kernel(const BwdParams p) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 q_lds[C::kBq * C::kQld];
  __shared__ __attribute__((aligned(16))) bf16 do_lds[C::kBq * C::kQld];
  __shared__ __attribute__((aligned(16))) bf16 k_lds[C::kBk * C::kKld];
  __shared__ __attribute__((aligned(16))) bf16 st_lds[C::kBk * C::kSld];
  __shared__ __attribute__((aligned(16))) float lse_lds[C::kBq];
  __shared__ __attribute__((aligned(16))) float dd_lds[C::kBq];
  __shared__ int32_t s_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int r_in = (lane & 15) >> 2;                         // transposed-read row within 4
  const int c_in = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);   // transposed-read column within 32
  const bf16* __restrict__ gq = (const bf16*)p.q;
  const bf16* __restrict__ gk = (const bf16*)p.k;
  const bf16* __restrict__ gv = (const bf16*)p.v;
  const bf16* __restrict__ gdo = (const bf16*)p.d_o;

  for (;;) {
    if (tid == 0) s_item = atomicAdd(p.counter, 1);
    __syncthreads();
    const int item = s_item;
    if (item >= p.n_tiles) break;
    const Tile tile = p.tiles[item];
    const SegDev sg = p.segs[tile.seg];
    const int nh = sg.nh;
    const int h = tile.head;
    const int64_t rs = (int64_t)nh * D;
    const int nk = tile.nrows;

    // This wave's 32 keys in registers (B operands, lane = key column); clamped past the end.
    const int key_local = wave * 32 + l32;
    const bool k_valid = key_local < nk;
    const int ktok = tile.row0 + min(key_local, nk - 1);
    bf16x8 kreg[C::kSteps], vreg[C::kSteps];
    {
      const int64_t off = (sg.kv_row0 + (int64_t)ktok * nh + h) * D + 8 * hi;
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) {
        kreg[s] = *(const bf16x8*)(gk + off + 16 * s);
        vreg[s] = *(const bf16x8*)(gv + off + 16 * s);
      }
    }
    // The item's K tile in LDS, then K^T operands for dQ: lane = output column c, k = key.
    {
      const bf16* kb = gk + (sg.kv_row0 + (int64_t)tile.row0 * nh + h) * D;
#pragma unroll
      for (int c = 0; c < C::kKChunks; ++c) {
        const int chunk = tid + c * C::kThreads;
        const int r = chunk / C::kRowChunks;
        const int col = (chunk % C::kRowChunks) * 8;
        const int key = min(r, nk - 1);
        *(u32x4*)&k_lds[r * C::kKld + col] = *(const u32x4*)(kb + (int64_t)key * rs + col);
      }
    }
    __syncthreads();
    const int dq_cb = wave / C::kWavesPerCb;                   // this wave's dQ column block
    const int dq_mb0 = (wave % C::kWavesPerCb) * C::kMbPerWave; // and first 32-row block
    bf16x8 ktreg[C::kBk / 16];
#pragma unroll
    for (int ks = 0; ks < C::kBk / 16; ++ks) {
      const bf16* kp = &k_lds[(16 * ks + 8 * hi + r_in) * C::kKld + dq_cb * 32 + c_in];
      ktreg[ks] = cat(lds_read_tr(kp), lds_read_tr(kp + 4 * C::kKld));
    }

    f32x16 dk_acc[C::kCb], dv_acc[C::kCb];
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb) {
      dk_acc[cb] = f32x16{};
      dv_acc[cb] = f32x16{};
    }

    const int n_q = sg.q_end - sg.q_begin;
    const int nqb = (n_q + C::kBq - 1) / C::kBq;
    const int start = (tile.row0 / C::kBk + 3 * h) % nqb;
    const bf16* qbase = gq + (sg.q_row0 + (int64_t)sg.q_begin * nh + h) * D;
    const bf16* dobase = gdo + (sg.q_row0 + (int64_t)sg.q_begin * nh + h) * D;
    const int64_t rowbase = sg.q_row0 + (int64_t)sg.q_begin * nh + h;  // query-side row of local token 0

    u32x4 qpre[C::kQChunks], dopre[C::kQChunks];
    float lpre = 0.f;
    auto prefetch = [&](int qb) {
      const int q0 = qb * C::kBq;
      const int nrow = min(C::kBq, n_q - q0);
#pragma unroll
      for (int c = 0; c < C::kQChunks; ++c) {
        const int chunk = tid + c * C::kThreads;
        const int r = chunk / C::kRowChunks;
        const int col = (chunk % C::kRowChunks) * 8;
        const int64_t off = (int64_t)(q0 + min(r, nrow - 1)) * rs + col;
        qpre[c] = *(const u32x4*)(qbase + off);
        dopre[c] = *(const u32x4*)(dobase + off);
      }
      if (tid < 2 * C::kBq) {
        const int r = tid & (C::kBq - 1);
        const int64_t row = rowbase + (int64_t)(q0 + min(r, nrow - 1)) * nh;
        if (tid < C::kBq)
          lpre = r < nrow ? p.lse[row] * 1.4426950408889634f : INFINITY;  // invalid rows: P = 0
        else
          lpre = r < nrow ? p.dvec[row] : 0.f;
      }
    };

    prefetch(start);
    for (int it = 0; it < nqb; ++it) {
      const int qb = (start + it) % nqb;
      const int q0 = qb * C::kBq;
      const int nrow = min(C::kBq, n_q - q0);
      // Stage this step's Q, dO, LSE (log2 units) and D in LDS.
#pragma unroll
      for (int c = 0; c < C::kQChunks; ++c) {
        const int chunk = tid + c * C::kThreads;
        const int r = chunk / C::kRowChunks;
        const int col = (chunk % C::kRowChunks) * 8;
        *(u32x4*)&q_lds[r * C::kQld + col] = qpre[c];
        *(u32x4*)&do_lds[r * C::kQld + col] = dopre[c];
      }
      if (tid < C::kBq)
        lse_lds[tid] = lpre;
      else if (tid < 2 * C::kBq)
        dd_lds[tid - C::kBq] = lpre;
      __syncthreads();
      if (it + 1 < nqb) prefetch((start + it + 1) % nqb);

      // S = Q K^T and dP = dO V^T: two 32-row blocks, lane = this wave's key column.
      f32x16 sacc[2], dpacc[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        sacc[mb] = f32x16{};
        dpacc[mb] = f32x16{};
        const bf16* qa = &q_lds[(mb * 32 + l32) * C::kQld + 8 * hi];
        const bf16* da = &do_lds[(mb * 32 + l32) * C::kQld + 8 * hi];
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) {
          sacc[mb] = mfma32(*(const bf16x8*)(qa + 16 * s), kreg[s], sacc[mb]);
          dpacc[mb] = mfma32(*(const bf16x8*)(da + 16 * s), vreg[s], dpacc[mb]);
        }
      }
      // P = exp2(S tau log2e - LSE log2e), dS = P (dP - D); rows 8(i/4) + 4hi + i%4.
      bf16x8 pb[4], dsb[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 pv, dsv;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 L = *(const f32x4*)&lse_lds[mb * 32 + 8 * g + 4 * hi];
          const f32x4 Dd = *(const f32x4*)&dd_lds[mb * 32 + 8 * g + 4 * hi];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 4 * g + u;
            const float pe = k_valid ? fast_exp2(fmaf(sacc[mb][i], p.scale_log2, -L[u])) : 0.f;
            pv[i] = pe;
            dsv[i] = pe * (dpacc[mb][i] - Dd[u]);
          }
        }
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          f32x8 a, b;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            a[u] = pv[8 * hs + u];
            b[u] = dsv[8 * hs + u];
          }
          pb[mb * 2 + hs] = to_bf16x8(a);
          dsb[mb * 2 + hs] = to_bf16x8(b);
        }
        // dS^T to LDS for dQ: row = key, 4 consecutive query rows per store.
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x = {dsv[4 * g], dsv[4 * g + 1], dsv[4 * g + 2], dsv[4 * g + 3]};
          *(bf16x4*)&st_lds[key_local * C::kSld + mb * 32 + 8 * g + 4 * hi] = to_bf16x4(x);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS, 16 query rows per step, in the k order of P's rows.
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int row = (ks >> 1) * 32 + 16 * (ks & 1) + 4 * hi + r_in;
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb) {
          const bf16* dp_ = &do_lds[row * C::kQld + cb * 32 + c_in];
          const bf16* qp_ = &q_lds[row * C::kQld + cb * 32 + c_in];
          const bf16x8 a_do = cat(lds_read_tr(dp_), lds_read_tr(dp_ + 8 * C::kQld));
          const bf16x8 a_q = cat(lds_read_tr(qp_), lds_read_tr(qp_ + 8 * C::kQld));
          dv_acc[cb] = mfma32(a_do, pb[ks], dv_acc[cb]);
          dk_acc[cb] = mfma32(a_q, dsb[ks], dk_acc[cb]);
        }
      }
      __syncthreads();
      // dQ[q][c] = sum over the item's 128 keys of dS[q][key] K[key][c], then atomics.
#pragma unroll
      for (int m = 0; m < C::kMbPerWave; ++m) {
        const int mb = dq_mb0 + m;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::kBk / 16; ++ks) {
          const bf16* sp = &st_lds[(16 * ks + 8 * hi + r_in) * C::kSld + mb * 32 + c_in];
          acc = mfma32(cat(lds_read_tr(sp), lds_read_tr(sp + 4 * C::kSld)), ktreg[ks], acc);
        }
        const int c = dq_cb * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = mb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
          if (qr < nrow) unsafeAtomicAdd(p.dq + (rowbase + (int64_t)(q0 + qr) * nh) * D + c, acc[i] * p.scale);
        }
      }
    }

    // dK = tau dK^T, dV = dV^T, written once: lane = key, 4 consecutive columns per store.
    if (k_valid) {
      const int64_t row = sg.kv_row0 + (int64_t)ktok * nh + h;
      float* dkr = p.dk + row * D;
      float* dvr = p.dv + row * D;
#pragma unroll
      for (int cb = 0; cb < C::kCb; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = cb * 32 + 8 * g + 4 * hi;
          *(f32x4*)(dkr + c) = f32x4{dk_acc[cb][4 * g] * p.scale, dk_acc[cb][4 * g + 1] * p.scale,
                                     dk_acc[cb][4 * g + 2] * p.scale, dk_acc[cb][4 * g + 3] * p.scale};
          *(f32x4*)(dvr + c) = f32x4{dv_acc[cb][4 * g], dv_acc[cb][4 * g + 1], dv_acc[cb][4 * g + 2],
                                     dv_acc[cb][4 * g + 3]};
        }
    }
    __syncthreads();
  }
}

template <int D>
int blocks_per_cu_impl() {
  static int cached = -1;
  if (cached < 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, bwd_kernel<D>, 256, 0) != hipSuccess) n = 0;
    cached = n;
  }
  return cached;
}

}  // namespace

int bwd_blocks_per_cu(int d) { return d == 64 ? blocks_per_cu_impl<64>() : blocks_per_cu_impl<128>(); }

int launch_bwd(int d, const BwdParams& p, int grid_pre, int grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (d == 64) {
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(grid_pre), dim3(256), 0, s, p);
    hipLaunchKernelGGL(bwd_kernel<64>, dim3(grid), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(grid_pre), dim3(256), 0, s, p);
    hipLaunchKernelGGL(bwd_kernel<128>, dim3(grid), dim3(256), 0, s, p);
  }
  return hipPeekAtLastError() == hipSuccess ? 0 : 1;
}

}  // namespace zl
