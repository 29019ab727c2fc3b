// Backward kernels: pre-pass, dK/dV (key-major) and dQ (query-major).
//
// Gradients of f = sum dO . O for softmax attention (the exact backward named on the Zellige
// page, §V-A), recomputing the probabilities from the forward's LSE:
//   P = exp(tau Q K^T - LSE),  dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dK = tau dS^T Q,  dQ = tau dS K,  with D_i = sum_c dO_ic O_ic.
// For a ring part the LSE and O are the merged ones, so P is the global softmax restricted
// to the part's keys; dQ sums over every part of the group.
//
// Pre-pass: D and LSE log2(e) for every covered query row, stored head-major (row
//   q_row0 + h * Lq + t of the sequence) so that the key-major kernel reads the 64 rows of a
//   step as one contiguous 256-byte run; both queue counters zeroed.
// dK/dV kernel: one item = 128 key rows of one (segment, head); 4 waves x 32 keys. Each wave
//   keeps its K and V rows in registers as B operands of S = Q K^T and dP = dO V^T (lane = one
//   key column), so P and dS come out of the MFMA already in the B-operand layout of
//   dV^T = dO^T P and dK^T = Q^T dS; dO^T and Q^T are read from natural LDS tiles with
//   transposed LDS reads. dK and dV accumulate in registers and are written once.
// dQ kernel: one item = 128 query rows of one (segment or ring group, head); 4 waves x 32
//   query rows, the forward's shape: S^T = K Q^T and dP^T = V dO^T with Q and dO in registers
//   (lane = one query row, whose LSE and D are then per-lane scalars), and
//   dQ^T += K^T dS^T with K^T from transposed LDS reads. dQ is written once: no atomics.
//   Computing dQ in its own query-major pass costs S and dP a second time, but fp32 atomics
//   into dQ from every key block were measured to cost more than the whole key-major pass.
#include "zl_device.hpp"
#include "zl_internal.h"

namespace zl {
namespace {

// ---------------------------------------------------------------------------------------------
// Pre-pass: D_i = sum_c dO_ic O_ic and LSE_i log2(e) for every covered query row (16 lanes per
// row), written head-major.

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdParams p) {
  if (blockIdx.x == 0 && threadIdx.x < kQueues) {
    p.kvq.counters[threadIdx.x * kCounterStride] = 0;
    p.dqq.counters[threadIdx.x * kCounterStride] = 0;
  }
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
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
      if (sub == 0) {
        const int64_t hm = sg.q_row0 + (int64_t)h * sg.lq + tok;
        p.dvec[hm] = acc;
        p.lse2[hm] = p.lse[row] * 1.4426950408889634f;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dK/dV kernel.

template <int D>
struct KvCfg {
  static constexpr int kThreads = 256;
  static constexpr int kBq = kBwdRows;                    // 64 query rows per step
  static constexpr int kQld = LdsTile<D>::kLd;            // Q / dO row stride in LDS
  static constexpr int kSteps = D / 16;                   // k-steps over d
  static constexpr int kCb = D / 32;                      // 32-wide column blocks over d
  static constexpr int kQChunks = kBq * D / 8 / kThreads; // 16-B chunks per thread (Q or dO)
  static constexpr int kRowChunks = D / 8;
};

template <int D>
__device__ __forceinline__ void kv_prefetch(u32x4 (&qpre)[KvCfg<D>::kQChunks], u32x4 (&dopre)[KvCfg<D>::kQChunks],
                                            float& lpre, const bf16* qbase, const bf16* dobase, int64_t rs,
                                            int64_t hmbase, int q0, int nrow, const float* lse2,
                                            const float* dvec, int tid) {
  using C = KvCfg<D>;
#pragma unroll
  for (int c = 0; c < C::kQChunks; ++c) {
    const int chunk = tid + c * C::kThreads;
    const int r = chunk / C::kRowChunks;
    const int col = (chunk % C::kRowChunks) * 8;
    const int64_t off = (int64_t)(q0 + min(r, nrow - 1)) * rs + col;
    qpre[c] = *(const u32x4*)(qbase + off);
    dopre[c] = *(const u32x4*)(dobase + off);
  }
  if (tid < 2 * C::kBq) {  // head-major rows: 64 consecutive floats per array
    const int r = tid & (C::kBq - 1);
    const int64_t hm = hmbase + q0 + min(r, nrow - 1);
    if (tid < C::kBq)
      lpre = r < nrow ? lse2[hm] : INFINITY;  // rows past the end: P = 0
    else
      lpre = r < nrow ? dvec[hm] : 0.f;
  }
}

// P = exp2(S tau log2e - LSE log2e) and dS = P (dP - D) for one 32-row half of a step, rounded
// to bf16 in the two B-operand halves (rows 8(i/4) + 4hi + i%4; lse and dd point at row 4hi).
__device__ __forceinline__ void bwd_p_ds(const f32x16& sacc, const f32x16& dpacc, const float* lse,
                                         const float* dd, bool k_valid, float scale_log2, bf16x8 (&pb)[2],
                                         bf16x8 (&dsb)[2]) {
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    f32x8 a, b;
#pragma unroll
    for (int g2 = 0; g2 < 2; ++g2) {
      const int g = 2 * hs + g2;
      const f32x4 L = *(const f32x4*)&lse[8 * g];
      const f32x4 Dd = *(const f32x4*)&dd[8 * g];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 4 * g + u;
        const float pe = k_valid ? fast_exp2(fmaf(sacc[i], scale_log2, -L[u])) : 0.f;
        a[4 * g2 + u] = pe;
        b[4 * g2 + u] = pe * (dpacc[i] - Dd[u]);
      }
    }
    pb[hs] = to_bf16x8(a);
    dsb[hs] = to_bf16x8(b);
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(const BwdParams p) {
  using C = KvCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 q_lds[C::kBq * C::kQld];
  __shared__ __attribute__((aligned(16))) bf16 do_lds[C::kBq * C::kQld];
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
  const int prow_b = lds_row(l32);                             // physical row of this lane's operand row
  const int prow_t = lds_row(4 * hi + r_in);                   // physical row of its transposed reads
  const bf16* __restrict__ gq = (const bf16*)p.q;
  const bf16* __restrict__ gk = (const bf16*)p.k;
  const bf16* __restrict__ gv = (const bf16*)p.v;
  const bf16* __restrict__ gdo = (const bf16*)p.d_o;

  const int home = blockIdx.x % kQueues;
  int drained = 0;
  for (;;) {
    if (tid == 0) s_item = take_item(p.kvq, home, drained);
    __syncthreads();
    const int item = s_item;
    if (item < 0) break;
    const Tile tile = p.kvq.items[item];
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

    f32x16 dk_acc[C::kCb], dv_acc[C::kCb];
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb) {
      dk_acc[cb] = f32x16{};
      dv_acc[cb] = f32x16{};
    }

    const int n_q = sg.q_end - sg.q_begin;
    const int nqb = (n_q + C::kBq - 1) / C::kBq;
    const bf16* qbase = gq + (sg.q_row0 + (int64_t)sg.q_begin * nh + h) * D;
    const bf16* dobase = gdo + (sg.q_row0 + (int64_t)sg.q_begin * nh + h) * D;
    const int64_t hmbase = sg.q_row0 + (int64_t)h * sg.lq + sg.q_begin;  // head-major row of local token 0

    u32x4 qpre[C::kQChunks], dopre[C::kQChunks];
    float lpre = 0.f;
    kv_prefetch<D>(qpre, dopre, lpre, qbase, dobase, rs, hmbase, 0, min(C::kBq, n_q), p.lse2, p.dvec, tid);
    for (int qb = 0; qb < nqb; ++qb) {
      // Stage this step's Q, dO, LSE (log2 units) and D in LDS.
#pragma unroll
      for (int c = 0; c < C::kQChunks; ++c) {
        const int chunk = tid + c * C::kThreads;
        const int r = chunk / C::kRowChunks;
        const int col = (chunk % C::kRowChunks) * 8;
        *(u32x4*)&q_lds[lds_row(r) * C::kQld + col] = qpre[c];
        *(u32x4*)&do_lds[lds_row(r) * C::kQld + col] = dopre[c];
      }
      if (tid < C::kBq)
        lse_lds[tid] = lpre;
      else if (tid < 2 * C::kBq)
        dd_lds[tid - C::kBq] = lpre;
      __syncthreads();
      if (qb + 1 < nqb) {
        const int q0n = (qb + 1) * C::kBq;
        kv_prefetch<D>(qpre, dopre, lpre, qbase, dobase, rs, hmbase, q0n, min(C::kBq, n_q - q0n), p.lse2,
                       p.dvec, tid);
      }

      // One step = two 32-row halves mb of the 64 query rows. For each half: S = Q K^T and
      // dP = dO V^T (lane = this wave's key column; rows 8(i/4) + 4hi + i%4), then
      // P = exp2(S tau log2e - LSE log2e), dS = P (dP - D), then dV^T += dO^T P and
      // dK^T += Q^T dS with dO^T and Q^T from transposed reads (k order of P's rows; logical
      // rows +8 are physical rows +2). The step is software-pipelined in four phases so that
      // each wave keeps the matrix cores busy while it runs the exponentials of the other
      // half and waits on LDS:
      //   A: S, dP of half 0              | LDS: Q, dO operands of half 1
      //   B: S, dP of half 1              | P, dS of half 0; LDS: transposed operands of half 0
      //   C: dV, dK of half 0             | P, dS of half 1; LDS: transposed operands of half 1
      //   D: dV, dK of half 1
      constexpr int kS = C::kSteps;   // MFMAs per S (or dP) of one half
      constexpr int kT = 2 * C::kCb;  // MFMAs per dV (or dK) of one half
      bf16x8 qop0[kS], dop0[kS];
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        qop0[s] = *(const bf16x8*)&q_lds[prow_b * C::kQld + 8 * hi + 16 * s];
        dop0[s] = *(const bf16x8*)&do_lds[prow_b * C::kQld + 8 * hi + 16 * s];
      }
      // Phase A.
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s0 = f32x16{}, dp0 = f32x16{};
      bf16x8 qop1[kS], dop1[kS];
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        s0 = mfma32(qop0[s], kreg[s], s0);
        dp0 = mfma32(dop0[s], vreg[s], dp0);
        qop1[s] = *(const bf16x8*)&q_lds[(32 + prow_b) * C::kQld + 8 * hi + 16 * s];
        dop1[s] = *(const bf16x8*)&do_lds[(32 + prow_b) * C::kQld + 8 * hi + 16 * s];
      }
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads
      }
      __builtin_amdgcn_sched_barrier(0);
      // Phase B.
      f32x16 s1 = f32x16{}, dp1 = f32x16{};
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        s1 = mfma32(qop1[s], kreg[s], s1);
        dp1 = mfma32(dop1[s], vreg[s], dp1);
      }
      bf16x8 pb[2], dsb[2];
      bwd_p_ds(s0, dp0, &lse_lds[4 * hi], &dd_lds[4 * hi], k_valid, p.scale_log2, pb, dsb);
      bf16x8 tdo[kT / 2][2], tq[kT / 2][2];
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb) {
          const int row = 16 * hs + prow_t;
          const bf16* dp_ = &do_lds[row * C::kQld + cb * 32 + c_in];
          const bf16* qp_ = &q_lds[row * C::kQld + cb * 32 + c_in];
          tdo[cb][hs] = cat(lds_read_tr(dp_), lds_read_tr(dp_ + 2 * C::kQld));
          tq[cb][hs] = cat(lds_read_tr(qp_), lds_read_tr(qp_ + 2 * C::kQld));
        }
#pragma unroll
      for (int s = 0; s < 2 * kS; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // 6 VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // 3 LDS reads
      }
      __builtin_amdgcn_sched_barrier(0);
      // Phase C.
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb) {
          dv_acc[cb] = mfma32(tdo[cb][hs], pb[hs], dv_acc[cb]);
          dk_acc[cb] = mfma32(tq[cb][hs], dsb[hs], dk_acc[cb]);
        }
      bf16x8 pb1[2], dsb1[2];
      bwd_p_ds(s1, dp1, &lse_lds[32 + 4 * hi], &dd_lds[32 + 4 * hi], k_valid, p.scale_log2, pb1, dsb1);
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb) {
          const int row = 32 + 16 * hs + prow_t;
          const bf16* dp_ = &do_lds[row * C::kQld + cb * 32 + c_in];
          const bf16* qp_ = &q_lds[row * C::kQld + cb * 32 + c_in];
          tdo[cb][hs] = cat(lds_read_tr(dp_), lds_read_tr(dp_ + 2 * C::kQld));
          tq[cb][hs] = cat(lds_read_tr(qp_), lds_read_tr(qp_ + 2 * C::kQld));
        }
#pragma unroll
      for (int s = 0; s < 2 * kT; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // 6 VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // 3 LDS reads
      }
      __builtin_amdgcn_sched_barrier(0);
      // Phase D.
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb) {
          dv_acc[cb] = mfma32(tdo[cb][hs], pb1[hs], dv_acc[cb]);
          dk_acc[cb] = mfma32(tq[cb][hs], dsb1[hs], dk_acc[cb]);
        }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
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
  }
}

// ---------------------------------------------------------------------------------------------
// dQ kernel.

template <int D>
struct DqCfg {
  static constexpr int kThreads = 256;
  static constexpr int kBk = 64;                          // keys per block
  static constexpr int kKld = LdsTile<D>::kLd;            // K row stride (natural and transposed reads)
  static constexpr int kVld = LdsTile<D>::kLd;            // V row stride (natural reads)
  static constexpr int kSteps = D / 16;
  static constexpr int kCb = D / 32;
  static constexpr int kChunks = kBk * D / 8 / kThreads;
  static constexpr int kRowChunks = D / 8;
};

template <int D>
__device__ __forceinline__ void dq_load_block(u32x4 (&kreg)[DqCfg<D>::kChunks], u32x4 (&vreg)[DqCfg<D>::kChunks],
                                              const bf16* kbase, const bf16* vbase, int64_t rs, int key0, int n_kv,
                                              int tid) {
  using C = DqCfg<D>;
#pragma unroll
  for (int c = 0; c < C::kChunks; ++c) {
    const int chunk = tid + c * C::kThreads;
    const int r = chunk / C::kRowChunks;
    const int col = (chunk % C::kRowChunks) * 8;
    const int key = min(key0 + r, n_kv - 1);
    kreg[c] = *(const u32x4*)(kbase + (int64_t)key * rs + col);
    vreg[c] = *(const u32x4*)(vbase + (int64_t)key * rs + col);
  }
}

template <int D>
__device__ __forceinline__ void dq_store_block(const u32x4 (&kreg)[DqCfg<D>::kChunks],
                                               const u32x4 (&vreg)[DqCfg<D>::kChunks], bf16* k_lds, bf16* v_lds,
                                               int tid) {
  using C = DqCfg<D>;
#pragma unroll
  for (int c = 0; c < C::kChunks; ++c) {
    const int chunk = tid + c * C::kThreads;
    const int r = chunk / C::kRowChunks;
    const int col = (chunk % C::kRowChunks) * 8;
    *(u32x4*)&k_lds[lds_row(r) * C::kKld + col] = kreg[c];
    *(u32x4*)&v_lds[lds_row(r) * C::kVld + col] = vreg[c];
  }
}

// Block j of a key-range chain: the range it lies in and its first key within the range.
__device__ __forceinline__ void chain_block(const int32_t* ranges, int off, int len, int j, int bk, int* kv0,
                                            int* n_kv, int* key0) {
  for (int r = 0; r < len; ++r) {
    const int b = ranges[2 * (off + r)], e = ranges[2 * (off + r) + 1];
    const int nb = (e - b + bk - 1) / bk;
    if (j < nb || r == len - 1) {
      *kv0 = b;
      *n_kv = e - b;
      *key0 = j * bk;
      return;
    }
    j -= nb;
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void dq_kernel(const BwdParams p) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(16))) bf16 k_lds[2][C::kBk * C::kKld];
  __shared__ __attribute__((aligned(16))) bf16 v_lds[2][C::kBk * C::kVld];
  __shared__ int32_t s_item;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int r_in = (lane & 15) >> 2;
  const int c_in = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int prow_b = lds_row(l32);
  const int prow_t = lds_row(4 * hi + r_in);
  const bf16* __restrict__ gq = (const bf16*)p.q;
  const bf16* __restrict__ gk = (const bf16*)p.k;
  const bf16* __restrict__ gv = (const bf16*)p.v;
  const bf16* __restrict__ gdo = (const bf16*)p.d_o;

  const int home = blockIdx.x % kQueues;
  int drained = 0;
  for (;;) {
    if (tid == 0) s_item = take_item(p.dqq, home, drained);
    __syncthreads();
    const int item = s_item;
    if (item < 0) break;
    const Tile tile = p.dqq.items[item];
    const SegDev sg = p.segs[tile.seg];
    const int nh = sg.nh;
    const int h = tile.head;
    const int64_t rs = (int64_t)nh * D;

    // This lane's query row (clamped; results of clamped rows are dropped), with its Q and dO
    // as B operands (k = d) and its LSE (log2 units) and D as scalars.
    const int qi = wave * 32 + l32;
    const bool q_valid = qi < tile.nrows;
    const int qtok = tile.row0 + (q_valid ? qi : tile.nrows - 1);
    const int64_t qrow = sg.q_row0 + (int64_t)qtok * nh + h;
    bf16x8 qreg[C::kSteps], doreg[C::kSteps];
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      qreg[s] = *(const bf16x8*)(gq + qrow * D + 8 * hi + 16 * s);
      doreg[s] = *(const bf16x8*)(gdo + qrow * D + 8 * hi + 16 * s);
    }
    const int64_t hm = sg.q_row0 + (int64_t)h * sg.lq + qtok;
    const float lse2 = p.lse2[hm];
    const float dd = p.dvec[hm];

    int n_blk = 0;
    for (int r = 0; r < sg.chain_len; ++r) {
      const int len = p.kv_ranges[2 * (sg.chain_off + r) + 1] - p.kv_ranges[2 * (sg.chain_off + r)];
      n_blk += (len + C::kBk - 1) / C::kBk;
    }
    const bf16* kseq = gk + (sg.kv_row0 + h) * D;
    const bf16* vseq = gv + (sg.kv_row0 + h) * D;

    f32x16 acc[C::kCb];
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb) acc[cb] = f32x16{};

    u32x4 kreg[C::kChunks], vreg[C::kChunks];
    int kv0, n_kv, key0;
    chain_block(p.kv_ranges, sg.chain_off, sg.chain_len, 0, C::kBk, &kv0, &n_kv, &key0);
    dq_load_block<D>(kreg, vreg, kseq + (int64_t)kv0 * rs, vseq + (int64_t)kv0 * rs, rs, key0, n_kv, tid);
    dq_store_block<D>(kreg, vreg, k_lds[0], v_lds[0], tid);
    __syncthreads();

    for (int j = 0; j < n_blk; ++j) {
      const int buf = j & 1;
      const int valid = n_kv - key0;  // keys of this block inside its range
      if (j + 1 < n_blk) {
        chain_block(p.kv_ranges, sg.chain_off, sg.chain_len, j + 1, C::kBk, &kv0, &n_kv, &key0);
        dq_load_block<D>(kreg, vreg, kseq + (int64_t)kv0 * rs, vseq + (int64_t)kv0 * rs, rs, key0, n_kv, tid);
      }

      // Per 32-key half kb: S^T = K Q^T and dP^T = V dO^T, then
      // dS^T = P^T (dP^T - D) with P^T = exp2(S^T tau log2e - LSE log2e) (keys past the range: 0),
      // then dQ^T[c][q] += K^T[c][key] dS^T[key][q] in the k order of dS^T's rows.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
        const bf16* kr = &k_lds[buf][(kb * 32 + prow_b) * C::kKld + 8 * hi];
        const bf16* vr = &v_lds[buf][(kb * 32 + prow_b) * C::kVld + 8 * hi];
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) {
          sacc = mfma32(*(const bf16x8*)(kr + 16 * s), qreg[s], sacc);
          dpacc = mfma32(*(const bf16x8*)(vr + 16 * s), doreg[s], dpacc);
        }
        bf16x8 dsb[2];
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          f32x8 x;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int i = 8 * hs + u;
            const int key = kb * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
            const float pe = key < valid ? fast_exp2(fmaf(sacc[i], p.scale_log2, -lse2)) : 0.f;
            x[u] = pe * (dpacc[i] - dd);
          }
          dsb[hs] = to_bf16x8(x);
        }
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const int row = kb * 32 + 16 * hs + prow_t;
#pragma unroll
          for (int cb = 0; cb < C::kCb; ++cb) {
            const bf16* kp = &k_lds[buf][row * C::kKld + cb * 32 + c_in];
            acc[cb] = mfma32(cat(lds_read_tr(kp), lds_read_tr(kp + 2 * C::kKld)), dsb[hs], acc[cb]);
          }
        }
      }
      if (j + 1 < n_blk) dq_store_block<D>(kreg, vreg, k_lds[buf ^ 1], v_lds[buf ^ 1], tid);
      __syncthreads();
    }

    if (q_valid) {
      float* out = p.dq + qrow * D;
#pragma unroll
      for (int cb = 0; cb < C::kCb; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = cb * 32 + 8 * g + 4 * hi;
          *(f32x4*)(out + c) = f32x4{acc[cb][4 * g] * p.scale, acc[cb][4 * g + 1] * p.scale,
                                     acc[cb][4 * g + 2] * p.scale, acc[cb][4 * g + 3] * p.scale};
        }
    }
  }
}

template <typename K>
int occupancy(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess) n = 0;
  return n;
}

}  // namespace

int bwd_blocks_per_cu(int d) {
  static int c64 = -1, c128 = -1;
  int& c = d == 64 ? c64 : c128;
  if (c < 0) c = d == 64 ? occupancy(dkdv_kernel<64>) : occupancy(dkdv_kernel<128>);
  return c;
}

int dq_blocks_per_cu(int d) {
  static int c64 = -1, c128 = -1;
  int& c = d == 64 ? c64 : c128;
  if (c < 0) c = d == 64 ? occupancy(dq_kernel<64>) : occupancy(dq_kernel<128>);
  return c;
}

int launch_bwd(int d, const BwdParams& p, int grid_pre, int grid, int grid_dq, unsigned stages, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (d == 64) {
    if (stages & ZL_BWD_PRE) hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(grid_pre), dim3(256), 0, s, p);
    if (stages & ZL_BWD_DKDV) hipLaunchKernelGGL(dkdv_kernel<64>, dim3(grid), dim3(256), 0, s, p);
    if (stages & ZL_BWD_DQ) hipLaunchKernelGGL(dq_kernel<64>, dim3(grid_dq), dim3(256), 0, s, p);
  } else {
    if (stages & ZL_BWD_PRE) hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(grid_pre), dim3(256), 0, s, p);
    if (stages & ZL_BWD_DKDV) hipLaunchKernelGGL(dkdv_kernel<128>, dim3(grid), dim3(256), 0, s, p);
    if (stages & ZL_BWD_DQ) hipLaunchKernelGGL(dq_kernel<128>, dim3(grid_dq), dim3(256), 0, s, p);
  }
  return hipPeekAtLastError() == hipSuccess ? 0 : 1;
}

}  // namespace zl
