// Backward kernels: pre-pass, dK/dV (key-major) and dQ (query-major).
//
// Gradients of f = sum dO . O for softmax attention (the exact backward named on the Zellige
// page, §V-A), recomputing the probabilities from the forward's LSE:
//   P = exp(tau Q K^T - LSE),  dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dK = tau dS^T Q,  dQ = tau dS K,  with D_i = sum_c dO_ic O_ic.
// For a ring part the LSE and O are the merged ones, so P is the global softmax restricted
// to the part's keys; dQ sums over every part of the group.
//
// Pre-pass: -D and -LSE / tau for every covered query row, stored head-major (row
//   q_row0 + h * Lq + t of the sequence) so that the key-major kernel loads the 64 rows of a
//   step as one contiguous 256-byte run; both queues' counters set past the static first
//   items of their launches and the split-item counters zeroed; the sentinel rows (-inf, 0) that stand in for rows past a segment's end written.
// dK/dV kernel: one item = 128 key rows of one (segment, head); 4 waves x 32 keys. Each wave
//   keeps its K and V rows in registers as B operands of S = Q K^T and dP = dO V^T (lane = one
//   key column), so P and dS come out of the MFMA already in the B-operand layout of
//   dV^T = dO^T P and dK^T = Q^T dS; dO^T and Q^T are read from the same LDS tiles with
//   transposed LDS reads. The 64-row Q and dO tiles of a step, and its rows' -LSE / tau and
//   -D (the initial values of the S and dP accumulators), reach LDS by direct global-to-LDS
//   loads into a ring of three stages, issued two steps ahead, so a step costs one barrier and
//   waits only for loads issued a step earlier. dK and dV accumulate in registers and are
//   written once.
// dQ kernel: one item = 32 W query rows of one (segment or ring group, head), W = 8 (256 rows,
//   one workgroup per CU) for deep queues, else 4 (128 rows, two per CU); W waves x 32 query
//   rows, the forward's shape per wave: S^T = K Q^T and dP^T = V dO^T with Q and dO in registers
//   (lane = one query row, whose LSE and D are then per-lane scalars), and
//   dQ^T += K^T dS^T with K^T from transposed LDS reads. K and V blocks reach LDS by direct
//   global-to-LDS loads in the key-major kernel's layout, one block ahead, walking the chain
//   of the segment's key ranges (all parts of a ring group). dQ is written once: no atomics.
// Split items (short queues): an item of either kernel may cover only a run of the blocks it
//   loops over (query blocks for dK/dV, key blocks for dQ). Each piece stores its partial
//   gradient rows to the workspace with device-coherent stores and counts itself done; the
//   last piece to finish adds all pieces' partials in piece order and writes the rows, so the
//   result does not depend on which piece finished last.
//   Computing dQ in its own query-major pass costs S and dP a second time, but fp32 atomics
//   into dQ from every key block were measured to cost more than the whole key-major pass.
#include "zl_device.hpp"
#include "zl_internal.h"

namespace zl {
namespace {

// ---------------------------------------------------------------------------------------------
// Pre-pass: -D_i = -sum_c dO_ic O_ic and -LSE_i / tau for every covered query row (16 lanes per
// row, 8 rows in flight per lane group), written head-major.

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdParams p) {
  if (blockIdx.x == 0 && threadIdx.x < kQueues) {  // past the static first items of each launch
    p.kvq.counters[threadIdx.x * kCounterStride] = home_count(p.kv_grid, threadIdx.x);
    p.dqq.counters[threadIdx.x * kCounterStride] = home_count(p.dq_grid, threadIdx.x);
  }
  if (blockIdx.x == 0 && threadIdx.x < 2 * kBwdRows) p.sentinel[threadIdx.x] = threadIdx.x < kBwdRows ? -INFINITY : 0.f;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < p.n_dq_split; j += gridDim.x * blockDim.x)
    p.dq_split_cnt[j] = 0;  // pieces finished per split dQ item
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < p.n_kv_split; j += gridDim.x * blockDim.x)
    p.kv_split_cnt[j] = 0;  // pieces finished per split dK/dV item
  if (p.kv_visits) {      // scheduler check: visits per item of both queues
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < p.n_kv_visits; j += gridDim.x * blockDim.x)
      p.kv_visits[j] = 0;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < p.n_dq_visits; j += gridDim.x * blockDim.x)
      p.dq_visits[j] = 0;
  }
  const float neg_inv_tau = -1.0f / p.scale;
  constexpr int kPer = D / 16;  // elements per lane
  constexpr int kPreUnroll = kPreRows / 16;
  const int sub = threadIdx.x & 15;
  const int rsel = threadIdx.x >> 4;
  const bf16* gdo = (const bf16*)p.d_o;
  for (int it = blockIdx.x; it < p.n_pre; it += gridDim.x) {
    const Tile t = p.pre_tiles[it];
    const SegDev sg = p.segs[t.seg];
    const int nhr = sg.head_end - sg.head_begin;
    const int rows = t.nrows * nhr;
    // kPreUnroll rows per 16-lane group per pass, every row's loads issued before the first
    // sum (a short pack is a few passes of dependent loads). Rows past the tile's end repeat
    // its last row's loads and store nothing.
    for (int r0 = rsel; r0 < rows; r0 += kPreUnroll * 16) {
      f32x4 o4[kPreUnroll][kPer / 4];
      bf16x4 d4[kPreUnroll][kPer / 4];
      float lse[kPreUnroll];
      int64_t hm[kPreUnroll];
#pragma unroll
      for (int j = 0; j < kPreUnroll; ++j) {
        const int r = min(r0 + 16 * j, rows - 1);
        const int tok = t.row0 + r / nhr;
        const int h = sg.head_begin + r % nhr;
        const int64_t row = sg.q_row0 + (int64_t)tok * sg.nh + h;
        const int64_t e0 = row * D + sub * kPer;
#pragma unroll
        for (int u = 0; u < kPer / 4; ++u) {
          o4[j][u] = *(const f32x4*)(p.o + e0 + 4 * u);
          d4[j][u] = *(const bf16x4*)(gdo + e0 + 4 * u);
        }
        lse[j] = p.lse[row];
        hm[j] = sg.q_row0 + (int64_t)h * sg.lq + tok;
      }
#pragma unroll
      for (int j = 0; j < kPreUnroll; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < kPer / 4; ++u)
          acc += (float)d4[j][u][0] * o4[j][u][0] + (float)d4[j][u][1] * o4[j][u][1] +
                 (float)d4[j][u][2] * o4[j][u][2] + (float)d4[j][u][3] * o4[j][u][3];
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
        if (sub == 0 && r0 + 16 * j < rows) {
          p.dneg[hm[j]] = -acc;
          p.lsec[hm[j]] = lse[j] * neg_inv_tau;
        }
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
  static constexpr int kSteps = D / 16;                   // k-steps over d
  static constexpr int kCb = D / 32;                      // 32-wide column blocks over d
  static constexpr int kRowChunks = D / 8;                // 16-byte chunks per row
  // Q and dO tiles of kBq rows: rows in 1 KB groups with a 16-byte gap; 16-byte chunk c of
  // row r at position c ^ x(r) (x below). With 64 banks of 4 bytes this keeps both read kinds
  // free of bank conflicts: 16 consecutive rows read at one chunk (16-byte operand reads) fall
  // on 16 distinct 16-byte bank groups, and 4 consecutive rows x 64 bytes (transposed reads)
  // on 4 distinct 64-byte groups. Every group is one 1 KB global-to-LDS load of one wave.
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kGroupRows = 1024 / kRowBytes;     // 4 (d = 128) or 8 (d = 64)
  static constexpr int kPitch = 1024 + 16;
  static constexpr int kTileBytes = kBq / kGroupRows * kPitch;
  static constexpr int kDma = kBq / kGroupRows / 4;       // loads per thread per tile
  static constexpr int kStageBytes = 2 * kTileBytes + 2 * kBq * 4;  // Q, dO, -LSE/tau, -D
  static constexpr int kStages = 3;
  static constexpr int kDmaPerStep = 2 * kDma;            // tile loads per wave per step (+1 rows
                                                          // load on waves 0 and 1)
  static constexpr int kSub = kSteps / 4;                 // k-steps per operand base
  static constexpr int kAhead = 3;                        // MFMAs between an operand read and its use
};

// Chunk swizzle of row r (r % 8 matters only).
template <int D>
__device__ __forceinline__ int qt_x(int r) {
  if (D == 128) return 4 * (r & 3);
  const int w = r & 7;
  return 4 * ((w >> 1) & 1) + 2 * ((w >> 2) & 1);
}

// Byte offset of row r within a tile.
template <int D>
__device__ __forceinline__ int qt_row(int r) {
  using C = KvCfg<D>;
  return (r / C::kGroupRows) * C::kPitch + (r % C::kGroupRows) * C::kRowBytes;
}

// Per-item state of the key-major kernel's Q / dO loads.
struct KvDma {
  const char* qbase;    // row of local query 0 of the segment (Q)
  const char* dobase;   // ... (dO)
  int64_t rs_bytes;     // bytes between consecutive query tokens of Q
  int64_t rs_do;        // ... of dO (differs from Q's in the QKV-packed layout)
  uint32_t lane_off;    // this lane's byte offset within a full step (row in group, chunk), Q
  uint32_t lane_off_do; // ... dO
  int lane_row;         // this lane's row within its load group
  int lane_col;         // this lane's byte column
  int n_q;
};

// Global -> LDS loads of the Q and dO rows of step qb into one stage; rows past the end of
// the segment read its last row (their probabilities are forced to 0 through LSE = +inf).
template <int D>
__device__ __forceinline__ void kv_dma(const KvDma& dm, uint32_t stage, int qb, int wave) {
  using C = KvCfg<D>;
  const int q0 = qb * C::kBq;
  if (q0 + C::kBq <= dm.n_q) {
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) {
      const int grp = i * 4 + wave;
      const int64_t r = q0 + grp * C::kGroupRows;
      lds_dma16(stage + grp * C::kPitch, dm.qbase + r * dm.rs_bytes, dm.lane_off);
      lds_dma16(stage + C::kTileBytes + grp * C::kPitch, dm.dobase + r * dm.rs_do, dm.lane_off_do);
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) {
      const int grp = i * 4 + wave;
      const int row = min(grp * C::kGroupRows + dm.lane_row, dm.n_q - 1 - q0);
      lds_dma16(stage + grp * C::kPitch, dm.qbase + (int64_t)q0 * dm.rs_bytes,
                (uint32_t)row * (uint32_t)dm.rs_bytes + dm.lane_col);
      lds_dma16(stage + C::kTileBytes + grp * C::kPitch, dm.dobase + (int64_t)q0 * dm.rs_do,
                (uint32_t)row * (uint32_t)dm.rs_do + dm.lane_col);
    }
  }
}

// Row values of step qb into a stage (after its Q and dO tiles): wave 0 loads the 64 rows'
// -LSE / tau, wave 1 their -D, one direct global-to-LDS load each. Rows past the segment's end
// read the sentinel (-inf: P = 0; 0), so every value is the initial value of the S or dP
// accumulator of its row. Offsets are bytes from the array (the sentinel lies after both).
__device__ __forceinline__ void kv_dma_rows(uint32_t rows_lds, const BwdParams& p, int64_t hmbase, int qb, int n_q,
                                            int wave, int lane) {
  if (wave >= 2) return;
  const char* base = wave == 0 ? (const char*)p.lsec : (const char*)p.dneg;
  const int q = qb * kBwdRows + lane;
  const uint32_t off = q < n_q ? (uint32_t)((hmbase + q) * 4)
                               : (uint32_t)((const char*)(p.sentinel + wave * kBwdRows) - base);
  lds_dma4(rows_lds + wave * kBwdRows * 4, base, off);
}

// acc += a b with the accumulator in AGPRs (inline assembly pins the register class: the dK and
// dV accumulators are only ever read by MFMAs, so they need no arch VGPRs). The compiler does not
// see into the assembly, so it keeps neither of the MFMA's hazards: a vector write of a or b needs
// two wait states before the MFMA reads it (the s_nop 1), and readers of acc outside MFMAs must
// wait for it (kv_acc_settle).
__device__ __forceinline__ void mfma32_acc(bf16x8 a, bf16x8 b, f32x16& acc) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void kv_acc_settle() { asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory"); }

// Operand reads of the key-major kernel (offsets in bytes within a stage's tile).
template <int D>
__device__ __forceinline__ bf16x8 kv_row_op(ZL_LDS const char* tile, const int (&rbase)[4], int mb, int st) {
  using C = KvCfg<D>;
  constexpr int kHalf = 32 / C::kGroupRows * C::kPitch;
  return *(ZL_LDS const bf16x8*)(tile + mb * kHalf + rbase[st / C::kSub] + 32 * (st % C::kSub));
}

template <int D>
__device__ __forceinline__ bf16x8 kv_tr_op(ZL_LDS const char* tile, const int (&tbase)[KvCfg<D>::kCb], int mb, int hs,
                                           int cb) {
  using C = KvCfg<D>;
  const int r0 = 32 * mb + 16 * hs;
  return cat(lds_read_tr(tile + r0 / C::kGroupRows * C::kPitch + tbase[cb]),
             lds_read_tr(tile + (r0 + 8) / C::kGroupRows * C::kPitch + tbase[cb]));
}

// The step's row initialisers of half mb in accumulator order: element i of a lane is row
// 8(i/4) + 4hi + i%4.
__device__ __forceinline__ f32x16 kv_rowinit(ZL_LDS const float* vals, int mb, int hi) {
  f32x16 r;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 x = *(ZL_LDS const f32x4*)&vals[32 * mb + 8 * g + 4 * hi];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[4 * g + u] = x[u];
  }
  return r;
}

// Operand m of a phase: the row reads of scores half mb, or the transposed reads of gradients
// half mb (used for a phase's first kAhead operands).
template <int D, bool kGrads>
__device__ __forceinline__ bf16x8 kv_first_op(ZL_LDS const char* qt, ZL_LDS const char* dot, const int (&rbase)[4],
                                              const int (&tbase)[KvCfg<D>::kCb], int mb, int m) {
  if (kGrads) return kv_tr_op<D>(m & 1 ? qt : dot, tbase, mb, (m >> 1) / KvCfg<D>::kCb, (m >> 1) % KvCfg<D>::kCb);
  return kv_row_op<D>(m & 1 ? dot : qt, rbase, mb, m >> 1);
}

// S' = Q K^T - LSE / tau and dP' = dO V^T - D of one 32-row half (16 MFMAs, alternating; sacc
// and dpacc hold the row initialisers on entry), operands kAhead (three) MFMAs ahead: the first
// kAhead come in `first`, and the last kAhead slots read the next phase's first kAhead into
// `next` (the scores of half 1 after half 0, the gradients of half 0 after half 1), so that no
// phase starts on an LDS wait. With kValu, the P = exp2(S' tau log2e) and dS = P dP' of the
// other half (element m per MFMA, rounded per 8) in the slots.
template <int D, bool kValu>
__device__ __forceinline__ void kv_scores(ZL_LDS const char* qt, ZL_LDS const char* dot, const int (&rbase)[4],
                                          const int (&tbase)[KvCfg<D>::kCb], int mb,
                                          const bf16x8 (&kreg)[KvCfg<D>::kSteps],
                                          const bf16x8 (&vreg)[KvCfg<D>::kSteps], f32x16& sacc, f32x16& dpacc,
                                          const f32x16& s_o, const f32x16& dp_o, float scale_log2, bf16x8 (&pb)[2],
                                          bf16x8 (&dsb)[2], const bf16x8 (&first)[KvCfg<D>::kAhead],
                                          bf16x8 (&next)[KvCfg<D>::kAhead]) {
  using C = KvCfg<D>;
  constexpr int kM = 2 * C::kSteps;
  constexpr int A = C::kAhead;
  bf16x8 op[kM];
#pragma unroll
  for (int j = 0; j < A; ++j) op[j] = first[j];
  f32x8 pe, ds;
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    if (m + A < kM) op[m + A] = kv_row_op<D>((m + A) & 1 ? dot : qt, rbase, mb, (m + A) >> 1);
    else if (mb == 0) next[m + A - kM] = kv_first_op<D, false>(qt, dot, rbase, tbase, 1, m + A - kM);
    else next[m + A - kM] = kv_first_op<D, true>(qt, dot, rbase, tbase, 0, m + A - kM);
    if (m & 1)
      dpacc = mfma32(op[m], vreg[m >> 1], dpacc);
    else
      sacc = mfma32(op[m], kreg[m >> 1], sacc);
    if (kValu) {
#pragma unroll
      for (int u = 0; u < 16 / kM; ++u) {
        const int e = m * (16 / kM) + u;
        const float pv = fast_exp2(s_o[e] * scale_log2);
        pe[e % 8] = pv;
        ds[e % 8] = pv * dp_o[e];
        if (e % 8 == 7) {
          pb[e / 8] = to_bf16x8(pe);
          dsb[e / 8] = to_bf16x8(ds);
        }
      }
    }
  }
}

// dV^T += dO^T P and dK^T += Q^T dS of one half (16 MFMAs, alternating), transposed operands
// kAhead MFMAs ahead; with kValu, the P / dS of the other half in the slots.
// (Half 0's last kAhead slots read half 1's first kAhead operands into `next`; half 1 has none.)
template <int D, bool kValu>
__device__ __forceinline__ void kv_grads(ZL_LDS const char* qt, ZL_LDS const char* dot,
                                         const int (&tbase)[KvCfg<D>::kCb], int mb, const bf16x8 (&pb)[2],
                                         const bf16x8 (&dsb)[2], f32x16 (&dv_acc)[KvCfg<D>::kCb],
                                         f32x16 (&dk_acc)[KvCfg<D>::kCb], const f32x16& s_o, const f32x16& dp_o,
                                         float scale_log2, bf16x8 (&pb_o)[2], bf16x8 (&dsb_o)[2],
                                         const bf16x8 (&first)[KvCfg<D>::kAhead], bf16x8 (&next)[KvCfg<D>::kAhead]) {
  using C = KvCfg<D>;
  constexpr int kM = 4 * C::kCb;  // (hs, cb) x {dV, dK}
  constexpr int A = C::kAhead;
  bf16x8 op[kM];
#pragma unroll
  for (int j = 0; j < A; ++j) op[j] = first[j];
  f32x8 pe, ds;
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    if (m + A < kM)
      op[m + A] = kv_tr_op<D>((m + A) & 1 ? qt : dot, tbase, mb, ((m + A) >> 1) / C::kCb, ((m + A) >> 1) % C::kCb);
    else if (mb == 0)
      next[m + A - kM] = kv_tr_op<D>((m + A - kM) & 1 ? qt : dot, tbase, 1, ((m + A - kM) >> 1) / C::kCb,
                                     ((m + A - kM) >> 1) % C::kCb);
    const int hs = (m >> 1) / C::kCb, cb = (m >> 1) % C::kCb;
    if (m & 1)
      mfma32_acc(op[m], dsb[hs], dk_acc[cb]);
    else
      mfma32_acc(op[m], pb[hs], dv_acc[cb]);
    if (kValu) {
#pragma unroll
      for (int u = 0; u < 16 / kM; ++u) {
        const int e = m * (16 / kM) + u;
        const float pv = fast_exp2(s_o[e] * scale_log2);
        pe[e % 8] = pv;
        ds[e % 8] = pv * dp_o[e];
        if (e % 8 == 7) {
          pb_o[e / 8] = to_bf16x8(pe);
          dsb_o[e / 8] = to_bf16x8(ds);
        }
      }
    }
  }
}

template <int D, bool kPacked>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(const BwdParams p) {
  using C = KvCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[C::kStages * C::kStageBytes];
  __shared__ int32_t s_item;
  __shared__ int32_t s_queue_mem[kQueues + 2];  // queue state of thread 0: bounds, then take_item's state
  ZL_LDS int32_t* const s_bounds = (ZL_LDS int32_t*)s_queue_mem;
  ZL_LDS int32_t* const s_taker = s_bounds + kQueues + 1;
  __shared__ int32_t s_last;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(ZL_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bf16* __restrict__ gk = (const bf16*)p.k;
  const bf16* __restrict__ gv = (const bf16*)p.v;

  // Per-lane LDS read offsets (bytes within a tile).
  // Operand reads of row l32 (+32 per half), k-step s: rbase[s / kSub] + 32 (s % kSub).
  int rbase[4];
  {
    const int x = qt_x<D>(l32);
#pragma unroll
    for (int k = 0; k < 4; ++k) rbase[k] = qt_row<D>(l32) + 16 * hi + 32 * C::kSub * (k ^ (x / (2 * C::kSub)));
  }
  // Transposed reads: lane (r_in, c_in) of rows R + 4hi + r_in, column block cb: tbase[cb] plus
  // the offset of row R (a multiple of 8).
  int tbase[C::kCb];
  {
    const int r_in = (lane & 15) >> 2;
    const int c_in = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int r = 4 * hi + r_in;
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb)
      tbase[cb] = qt_row<D>(r) + 16 * ((4 * cb + (c_in >> 3)) ^ qt_x<D>(r)) + 2 * (c_in & 7);
  }
  const int dma_row = lane / C::kRowChunks;
  const int dma_col = 16 * ((lane % C::kRowChunks) ^ qt_x<D>(dma_row));

  const int home = blockIdx.x % kQueues;
  if (tid == 0) {
    stage_bounds(p.kvq, s_bounds);
    *s_taker = home << 8;
  }
  for (;;) {
    if (tid == 0) s_item = take_item(p.kvq, s_bounds, s_taker, p.kv_visits);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);  // the same for every lane
    if (item < 0) break;
    const Tile tile = p.kvq.items[item];
    const SegDev sg = p.segs[tile.seg];
    const int nh = sg.nh;
    const int h = tile.head;
    const int nk = tile.nrows;

    KvDma dm;
    dm.n_q = sg.q_end - sg.q_begin;
    const QkvRows qr = qkv_rows<kPacked>(sg);  // planar, or the QKV-packed layout
    const int tstr = qr.t_stride;
    const int64_t kp0 = qr.k0;
    const int voff = qr.v_off;
    dm.rs_bytes = (int64_t)tstr * D * 2;
    dm.rs_do = (int64_t)nh * D * 2;
    dm.qbase = (const char*)p.q + (qr.q0 + (int64_t)sg.q_begin * tstr + h) * D * 2;
    dm.dobase = (const char*)p.d_o + (sg.q_row0 + (int64_t)sg.q_begin * nh + h) * D * 2;
    dm.lane_row = dma_row;
    dm.lane_col = dma_col;
    dm.lane_off = (uint32_t)dma_row * (uint32_t)dm.rs_bytes + dma_col;
    dm.lane_off_do = (uint32_t)dma_row * (uint32_t)dm.rs_do + dma_col;
    // The item's query blocks [qb0, qb1): all of the segment's, or one piece's run.
    const int qb0 = tile.kv_begin, qb1 = tile.kv_end;
    const int64_t hmbase = sg.q_row0 + (int64_t)h * sg.lq + sg.q_begin;  // head-major row of local token 0

    // This wave's 32 keys in registers (B operands, lane = key column); clamped past the end.
    // Issued before the first two steps' loads, so that waiting for step 0 covers them.
    const int key_local = wave * 32 + l32;
    const bool k_valid = key_local < nk;
    const int ktok = tile.row0 + min(key_local, nk - 1);
    bf16x8 kreg[C::kSteps], vreg[C::kSteps];
    {
      const int64_t off = (kp0 + (int64_t)ktok * tstr + h) * D + 8 * hi;
      const int64_t vo = off + (int64_t)voff * D;
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) {
        kreg[s] = *(const bf16x8*)(gk + off + 16 * s);
        vreg[s] = *(const bf16x8*)(gv + vo + 16 * s);
      }
    }
    f32x16 dk_acc[C::kCb], dv_acc[C::kCb];
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb) {
      dk_acc[cb] = f32x16{};
      dv_acc[cb] = f32x16{};
    }
    // Steps 0 and 1 into stages 0 and 1, then wait for everything: the key registers must be
    // complete before the step loop in the compiler's own accounting too (the fake uses below),
    // or it would wait inside every step; waiting for step 1 as well costs once per item.
    kv_dma<D>(dm, lds0, qb0, wave_u);
    kv_dma_rows(lds0 + 2 * C::kTileBytes, p, hmbase, qb0, dm.n_q, wave_u, lane);
    if (qb0 + 1 < qb1) {
      kv_dma<D>(dm, lds0 + C::kStageBytes, qb0 + 1, wave_u);
      kv_dma_rows(lds0 + C::kStageBytes + 2 * C::kTileBytes, p, hmbase, qb0 + 1, dm.n_q, wave_u, lane);
    }
    dma_wait();
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) asm volatile("" ::"v"(kreg[s]), "v"(vreg[s]));
    __syncthreads();

    uint32_t cur = lds0, ahead = lds0 + 2 * C::kStageBytes;  // stages of steps qb and qb + 2
    for (int qb = qb0; qb < qb1; ++qb) {
      // Step qb + 2 goes to the stage step qb - 1 read (every wave passed the barrier after it).
      if (qb + 2 < qb1) {
        kv_dma<D>(dm, ahead, qb + 2, wave_u);
        kv_dma_rows(ahead + 2 * C::kTileBytes, p, hmbase, qb + 2, dm.n_q, wave_u, lane);
      }
      ZL_LDS const char* qt = (ZL_LDS const char*)cur;
      ZL_LDS const char* dot = (ZL_LDS const char*)(cur + C::kTileBytes);
      ZL_LDS const float* lse_s = (ZL_LDS const float*)(cur + 2 * C::kTileBytes);
      ZL_LDS const float* dd_s = lse_s + C::kBq;
      constexpr int kHalf = 32 / C::kGroupRows * C::kPitch;  // bytes between the two 32-row halves

      // One step = two 32-row halves mb of the 64 query rows. For each half: S = Q K^T and
      // dP = dO V^T (lane = this wave's key column; rows 8(i/4) + 4hi + i%4), then
      // P = exp2(S tau log2e - LSE log2e), dS = P (dP - D), then dV^T += dO^T P and
      // dK^T += Q^T dS with dO^T and Q^T from transposed reads (k order of P's rows). Keys past
      // the end of the item need no mask: their P and dS only reach their own dK and dV
      // columns, which are not written. The step runs in four phases, each written in issue
      // order, so that the vector work of one half runs under the MFMAs of the other:
      //   A: S, dP of half 0
      //   B: S, dP of half 1              | P, dS of half 0
      //   C: dV, dK of half 0             | P, dS of half 1
      //   D: dV, dK of half 1
      f32x16 s0, dp0, s1, dp1;
      bf16x8 pb0[2], dsb0[2], pb1[2], dsb1[2];
      // Row initialisers: half 0 first (its first MFMAs need them), half 1 under phase A.
      s0 = kv_rowinit(lse_s, 0, hi);
      dp0 = kv_rowinit(dd_s, 0, hi);
      s1 = kv_rowinit(lse_s, 1, hi);
      dp1 = kv_rowinit(dd_s, 1, hi);
      bf16x8 opa[C::kAhead], opb[C::kAhead];
#pragma unroll
      for (int j = 0; j < C::kAhead; ++j) opa[j] = kv_first_op<D, false>(qt, dot, rbase, tbase, 0, j);
      kv_scores<D, false>(qt, dot, rbase, tbase, 0, kreg, vreg, s0, dp0, s1, dp1, p.scale_log2, pb1, dsb1, opa, opb);
      __builtin_amdgcn_sched_barrier(0);
      kv_scores<D, true>(qt, dot, rbase, tbase, 1, kreg, vreg, s1, dp1, s0, dp0, p.scale_log2, pb0, dsb0, opb, opa);
      __builtin_amdgcn_sched_barrier(0);
      kv_grads<D, true>(qt, dot, tbase, 0, pb0, dsb0, dv_acc, dk_acc, s1, dp1, p.scale_log2, pb1, dsb1, opa, opb);
      __builtin_amdgcn_sched_barrier(0);
      kv_grads<D, false>(qt, dot, tbase, 1, pb1, dsb1, dv_acc, dk_acc, s1, dp1, p.scale_log2, pb0, dsb0, opb, opa);
      __builtin_amdgcn_sched_barrier(0);
      // Step qb + 1's loads (issued a step ago) have landed once only step qb + 2's are
      // outstanding.
      if (qb + 1 < qb1) {
        if (qb + 2 < qb1) {
          if (wave_u < 2)
            dma_wait_all_but<C::kDmaPerStep + 1>();
          else
            dma_wait_all_but<C::kDmaPerStep>();
        } else {
          dma_wait();
        }
        __syncthreads();
      }
      cur = cur + C::kStageBytes == lds0 + C::kStages * C::kStageBytes ? lds0 : cur + C::kStageBytes;
      ahead = ahead + C::kStageBytes == lds0 + C::kStages * C::kStageBytes ? lds0 : ahead + C::kStageBytes;
    }

    // dK = tau dK^T, dV = dV^T, written once: lane = key, 4 consecutive columns per store. A
    // piece of a split item publishes its partial tau dK and dV (device-coherent stores) and
    // counts itself done; the last piece adds every piece's partial in piece order, its own
    // included, and stores the item's rows.
    kv_acc_settle();
    float ksc = p.scale;
    bool store = true;
    if (tile.split >= 0) {
      const int n_pieces = tile.piece >> 16;
      const int64_t slot = tile.split + (tile.piece & 0xffff);
      if (k_valid) {
        float* sp = p.kv_split + (slot * kBwdKeys + key_local) * (2 * D);
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = cb * 32 + 8 * g + 4 * hi;
            store_dev16(sp + c, f32x4{dk_acc[cb][4 * g] * ksc, dk_acc[cb][4 * g + 1] * ksc,
                                      dk_acc[cb][4 * g + 2] * ksc, dk_acc[cb][4 * g + 3] * ksc});
            store_dev16(sp + D + c, f32x4{dv_acc[cb][4 * g], dv_acc[cb][4 * g + 1], dv_acc[cb][4 * g + 2],
                                          dv_acc[cb][4 * g + 3]});
          }
      }
      store_dev_wait();
      __syncthreads();
      if (tid == 0)
        s_last = __hip_atomic_fetch_add(p.kv_split_cnt + tile.split, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 n_pieces - 1;
      __syncthreads();
      store = s_last;
      if (store && k_valid) {
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb) {
          dk_acc[cb] = f32x16{};
          dv_acc[cb] = f32x16{};
        }
        for (int c = 0; c < n_pieces; ++c) {
          const float* sp = p.kv_split + (((int64_t)tile.split + c) * kBwdKeys + key_local) * (2 * D) + 4 * hi;
          // this lane's D/2 values of each row: D/8 chunks of 16 bytes, 8 floats apart; chunk k
          // holds (column block k/4, group k%4)
          f32x4 x[D / 8];
          if constexpr (D == 128)
            load_dev16x16(sp, x);
          else
            load_dev16x8(sp, x);
#pragma unroll
          for (int k = 0; k < D / 8; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) dk_acc[k / 4][4 * (k % 4) + e] += x[k][e];
          if constexpr (D == 128)
            load_dev16x16(sp + D, x);
          else
            load_dev16x8(sp + D, x);
#pragma unroll
          for (int k = 0; k < D / 8; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) dv_acc[k / 4][4 * (k % 4) + e] += x[k][e];
        }
        ksc = 1.0f;
      }
    }
    if (store && k_valid) {
      const int64_t row = kp0 + (int64_t)ktok * tstr + h;
      float* dkr = p.dk + row * D;
      float* dvr = p.dv + (row + voff) * D;
#pragma unroll
      for (int cb = 0; cb < C::kCb; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = cb * 32 + 8 * g + 4 * hi;
          *(f32x4*)(dkr + c) = f32x4{dk_acc[cb][4 * g] * ksc, dk_acc[cb][4 * g + 1] * ksc,
                                     dk_acc[cb][4 * g + 2] * ksc, dk_acc[cb][4 * g + 3] * ksc};
          *(f32x4*)(dvr + c) = f32x4{dv_acc[cb][4 * g], dv_acc[cb][4 * g + 1], dv_acc[cb][4 * g + 2],
                                     dv_acc[cb][4 * g + 3]};
        }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dQ kernel.

template <int D, int W = 8>
struct DqCfg {
  static constexpr int kWaves = W;                        // 32 query rows each
  static constexpr int kRows = 32 * W;                    // query rows per item
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBk = kBwdRows;                    // keys per block (64)
  static constexpr int kSteps = D / 16;
  static constexpr int kCb = D / 32;
  // K and V blocks use the key-major kernel's tile layout (64 rows, both read kinds free of
  // bank conflicts): K is read by rows (S^T = K Q^T) and transposed (dQ^T = K^T dS^T), V by rows.
  static constexpr int kTileBytes = KvCfg<D>::kTileBytes;
  static constexpr int kStageBytes = 2 * kTileBytes;
  static constexpr int kGroups = kBk / KvCfg<D>::kGroupRows;  // 1 KB row groups per tile
  static constexpr int kDma = kGroups / kWaves;               // K (and V) loads per thread per block
  static_assert(kDma >= 1 && kDma * kWaves == kGroups, "the waves share each block's loads evenly");
};

// Global -> LDS loads of one key block: rows [0, 64) after `kblk` / `vblk` (the block's first
// key row), rows at or past `rows` read row rows - 1.
template <int D, int W>
__device__ __forceinline__ void dq_dma(uint32_t stage, const char* kblk, const char* vblk, int64_t rs_bytes, int rows,
                                       uint32_t lane_off, int lane_row, int lane_col, int wave) {
  using L = KvCfg<D>;
  using C = DqCfg<D, W>;
  if (rows >= L::kBq) {
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) {
      const int grp = i * C::kWaves + wave;
      const int64_t off = (int64_t)grp * L::kGroupRows * rs_bytes;
      lds_dma16(stage + grp * L::kPitch, kblk + off, lane_off);
      lds_dma16(stage + L::kTileBytes + grp * L::kPitch, vblk + off, lane_off);
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) {
      const int grp = i * C::kWaves + wave;
      const int row = min(grp * L::kGroupRows + lane_row, rows - 1);
      const uint32_t off = (uint32_t)row * (uint32_t)rs_bytes + lane_col;
      lds_dma16(stage + grp * L::kPitch, kblk, off);
      lds_dma16(stage + L::kTileBytes + grp * L::kPitch, vblk, off);
    }
  }
}

// Walk over the 64-key blocks of a key-range chain (one range, or the parts of a ring group in
// order): the current range [kv0, kv0 + n_kv) and the block's first key within it. Range bounds
// are read only when the walk enters a range, so the block loop issues no other memory reads.
struct ChainWalk {
  const int32_t* ranges;  // [begin, end) pairs of the chain
  int r, kv0, n_kv, key0;

  __device__ __forceinline__ void enter(int rr) {
    r = rr;
    kv0 = __builtin_amdgcn_readfirstlane(ranges[2 * rr]);
    n_kv = __builtin_amdgcn_readfirstlane(ranges[2 * rr + 1]) - kv0;
    key0 = 0;
  }
  // The next block; the caller guarantees that one exists (ranges are never empty).
  __device__ __forceinline__ void next(int bk) {
    key0 += bk;
    if (key0 >= n_kv) enter(r + 1);
  }
};

// dS^T = exp2(S^T tau log2e - LSE log2e) (dP^T - D) of element e of a tile (lane = query row);
// `dpd` is dP^T - D (the dP^T accumulator starts at -D).
__device__ __forceinline__ float dq_ds(float s, float dpd, float scale_log2, float lse2) {
  return fast_exp2(fmaf(s, scale_log2, -lse2)) * dpd;
}

// S^T and dP^T - D of one 32-key half of a block (16 MFMAs, alternating; the dP^T chain starts
// from `negd`, this lane's -D in every element), operands two MFMAs ahead; with kValu, the dS^T
// of the other half (one element per MFMA, rounded per 8) in the slots.
template <int D, bool kValu>
__device__ __forceinline__ void dq_scores(ZL_LDS const char* kt, ZL_LDS const char* vt, const int (&rbase)[4], int kb,
                                          const bf16x8 (&qreg)[DqCfg<D>::kSteps],
                                          const bf16x8 (&doreg)[DqCfg<D>::kSteps], f32x16& sacc, f32x16& dpacc,
                                          const f32x16& s_o, const f32x16& dp_o, const f32x16& negd,
                                          float scale_log2, float lse2, bf16x8 (&dsb)[2]) {
  using C = DqCfg<D>;
  constexpr int kM = 2 * C::kSteps;
  bf16x8 op[kM];
#pragma unroll
  for (int m = 0; m < 2; ++m) op[m] = kv_row_op<D>(m & 1 ? vt : kt, rbase, kb, m >> 1);
  f32x8 x;
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    if (m + 2 < kM) op[m + 2] = kv_row_op<D>((m + 2) & 1 ? vt : kt, rbase, kb, (m + 2) >> 1);
    if (m & 1)
      dpacc = mfma32(op[m], doreg[m >> 1], m == 1 ? negd : dpacc);
    else
      sacc = mfma32(op[m], qreg[m >> 1], m == 0 ? f32x16{} : sacc);
    if (kValu) {
#pragma unroll
      for (int u = 0; u < 16 / kM; ++u) {
        const int e = m * (16 / kM) + u;
        x[e % 8] = dq_ds(s_o[e], dp_o[e], scale_log2, lse2);
        if (e % 8 == 7) dsb[e / 8] = to_bf16x8(x);
      }
    }
  }
}

// dQ^T += K^T dS^T of one half (2 x kCb MFMAs), transposed operands two MFMAs ahead; with
// kValu, the dS^T of the other half in the slots.
template <int D, bool kValu>
__device__ __forceinline__ void dq_grads(ZL_LDS const char* kt, const int (&tbase)[DqCfg<D>::kCb], int kb,
                                         const bf16x8 (&dsb)[2], f32x16 (&acc)[DqCfg<D>::kCb], const f32x16& s_o,
                                         const f32x16& dp_o, float scale_log2, float lse2, bf16x8 (&dsb_o)[2]) {
  using C = DqCfg<D>;
  constexpr int kM = 2 * C::kCb;
  bf16x8 op[kM];
#pragma unroll
  for (int m = 0; m < 2; ++m) op[m] = kv_tr_op<D>(kt, tbase, kb, m / C::kCb, m % C::kCb);
  f32x8 x;
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    if (m + 2 < kM) op[m + 2] = kv_tr_op<D>(kt, tbase, kb, (m + 2) / C::kCb, (m + 2) % C::kCb);
    acc[m % C::kCb] = mfma32(op[m], dsb[m / C::kCb], acc[m % C::kCb]);
    if (kValu) {
#pragma unroll
      for (int u = 0; u < 16 / kM; ++u) {
        const int e = m * (16 / kM) + u;
        x[e % 8] = dq_ds(s_o[e], dp_o[e], scale_log2, lse2);
        if (e % 8 == 7) dsb_o[e / 8] = to_bf16x8(x);
      }
    }
  }
}

// Keys at or past vr (lane-independent offsets 8(i/4) + i%4) get S = -inf, hence P = 0.
__device__ __forceinline__ void dq_mask(f32x16& s, int vr) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (8 * (i / 4) + (i % 4) >= vr) s[i] = -INFINITY;
}

template <int D, bool kPacked, int W>
__global__ __launch_bounds__(64 * W, 8 / W) void dq_kernel(const BwdParams p) {
  using C = DqCfg<D, W>;
  using L = KvCfg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::kStageBytes];
  __shared__ int32_t s_item;
  __shared__ int32_t s_queue_mem[kQueues + 2];  // queue state of thread 0: bounds, then take_item's state
  ZL_LDS int32_t* const s_bounds = (ZL_LDS int32_t*)s_queue_mem;
  ZL_LDS int32_t* const s_taker = s_bounds + kQueues + 1;
  __shared__ int32_t s_last;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(ZL_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bf16* __restrict__ gq = (const bf16*)p.q;
  const bf16* __restrict__ gdo = (const bf16*)p.d_o;

  // Per-lane LDS read offsets within a tile (as in the key-major kernel).
  int rbase[4];
  {
    const int x = qt_x<D>(l32);
#pragma unroll
    for (int k = 0; k < 4; ++k) rbase[k] = qt_row<D>(l32) + 16 * hi + 32 * L::kSub * (k ^ (x / (2 * L::kSub)));
  }
  int tbase[C::kCb];
  {
    const int r_in = (lane & 15) >> 2;
    const int c_in = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int r = 4 * hi + r_in;
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb)
      tbase[cb] = qt_row<D>(r) + 16 * ((4 * cb + (c_in >> 3)) ^ qt_x<D>(r)) + 2 * (c_in & 7);
  }
  const int dma_row = lane / L::kRowChunks;
  const int dma_col = 16 * ((lane % L::kRowChunks) ^ qt_x<D>(dma_row));

  const int home = blockIdx.x % kQueues;
  if (tid == 0) {
    stage_bounds(p.dqq, s_bounds);
    *s_taker = home << 8;
  }
  for (;;) {
    if (tid == 0) s_item = take_item(p.dqq, s_bounds, s_taker, p.dq_visits);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);  // the same for every lane
    if (item < 0) break;
    const Tile tile = p.dqq.items[item];
    const SegDev sg = p.segs[tile.seg];
    const int nh = sg.nh;
    const int h = tile.head;
    const QkvRows qr = qkv_rows<kPacked>(sg);  // planar, or the QKV-packed layout
    const int tstr = qr.t_stride;
    const int64_t kp0 = qr.k0;
    const int voff = qr.v_off;
    const int64_t rs_bytes = (int64_t)tstr * D * 2;
    const uint32_t lane_off = (uint32_t)dma_row * (uint32_t)rs_bytes + dma_col;
    const char* kseq = uniform_ptr((const char*)p.k + (kp0 + h) * D * 2);
    const char* vseq = uniform_ptr((const char*)p.v + (kp0 + voff + h) * D * 2);

    // The item's key blocks [kv_begin, kv_end) of the chain: all of them, or one piece's run.
    const int n_blk = tile.kv_end - tile.kv_begin;
    ChainWalk cw;
    cw.ranges = p.kv_ranges + 2 * sg.chain_off;
    cw.enter(0);
    for (int b = tile.kv_begin;;) {
      const int nb = (cw.n_kv + C::kBk - 1) / C::kBk;
      if (b < nb) {
        cw.key0 = b * C::kBk;
        break;
      }
      b -= nb;
      cw.enter(cw.r + 1);
    }
    {
      const int64_t off = (int64_t)(cw.kv0 + cw.key0) * rs_bytes;
      dq_dma<D, W>(lds0, kseq + off, vseq + off, rs_bytes, cw.n_kv - cw.key0, lane_off, dma_row, dma_col, wave_u);
    }

    // This lane's query row (clamped; results of clamped rows are dropped), with its Q and dO
    // as B operands (k = d) and its LSE (log2 units) and D as scalars.
    const int qi = wave * 32 + l32;
    const bool q_valid = qi < tile.nrows;
    const int qtok = tile.row0 + (q_valid ? qi : tile.nrows - 1);
    const int64_t qrow = sg.q_row0 + (int64_t)qtok * nh + h;                // dO (planar)
    const int64_t qprow = qr.q0 + (int64_t)qtok * tstr + h;  // Q, dQ
    bf16x8 qreg[C::kSteps], doreg[C::kSteps];
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
      qreg[s] = *(const bf16x8*)(gq + qprow * D + 8 * hi + 16 * s);
      doreg[s] = *(const bf16x8*)(gdo + qrow * D + 8 * hi + 16 * s);
    }
    const int64_t hm = sg.q_row0 + (int64_t)h * sg.lq + qtok;
    const float lse2 = -p.lsec[hm] * p.scale_log2;  // LSE log2(e)
    f32x16 negd;                                      // -D in every element
#pragma unroll
    for (int i = 0; i < 16; ++i) negd[i] = p.dneg[hm];

    f32x16 acc[C::kCb];
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb) acc[cb] = f32x16{};
    dma_wait();
    __syncthreads();

    for (int j = 0; j < n_blk; ++j) {
      const uint32_t cur = lds0 + (j & 1) * C::kStageBytes;
      const int valid = cw.n_kv - cw.key0;  // keys of this block inside its range
      if (j + 1 < n_blk) {
        cw.next(C::kBk);
        const int64_t off = (int64_t)(cw.kv0 + cw.key0) * rs_bytes;
        dq_dma<D, W>(lds0 + ((j + 1) & 1) * C::kStageBytes, kseq + off, vseq + off, rs_bytes, cw.n_kv - cw.key0,
                  lane_off, dma_row, dma_col, wave_u);
      }
      ZL_LDS const char* kt = (ZL_LDS const char*)cur;
      ZL_LDS const char* vt = (ZL_LDS const char*)(cur + C::kTileBytes);

      // Per 32-key half kb: S^T = K Q^T and dP^T = V dO^T, then
      // dS^T = P^T (dP^T - D) with P^T = exp2(S^T tau log2e - LSE log2e) (keys past the range: 0),
      // then dQ^T[c][q] += K^T[c][key] dS^T[key][q] in the k order of dS^T's rows. Four phases,
      // each in issue order, so that the vector work of one half runs under the MFMAs of the
      // other: A: S, dP of half 0 | B: S, dP of half 1 with dS of half 0 |
      // C: dQ of half 0 with dS of half 1 | D: dQ of half 1.
      f32x16 s0, dp0, s1, dp1;
      bf16x8 dsb0[2], dsb1[2];
      dq_scores<D, false>(kt, vt, rbase, 0, qreg, doreg, s0, dp0, s1, dp1, negd, p.scale_log2, lse2, dsb1);
      if (valid < C::kBk) dq_mask(s0, valid - 4 * hi);
      __builtin_amdgcn_sched_barrier(0);
      dq_scores<D, true>(kt, vt, rbase, 1, qreg, doreg, s1, dp1, s0, dp0, negd, p.scale_log2, lse2, dsb0);
      if (valid < C::kBk) dq_mask(s1, valid - 32 - 4 * hi);
      __builtin_amdgcn_sched_barrier(0);
      dq_grads<D, true>(kt, tbase, 0, dsb0, acc, s1, dp1, p.scale_log2, lse2, dsb1);
      __builtin_amdgcn_sched_barrier(0);
      dq_grads<D, false>(kt, tbase, 1, dsb1, acc, s1, dp1, p.scale_log2, lse2, dsb0);
      __builtin_amdgcn_sched_barrier(0);
      dma_wait();
      __syncthreads();
    }

    // dQ = tau dQ^T, written once: lane = query row, 4 consecutive columns per store. A piece of
    // a split item publishes its scaled partial (device-coherent stores, as the forward's
    // pieces do) and counts itself done; the last piece adds every piece's partial in piece
    // order, its own included, and stores the item's rows.
    float osc = p.scale;
    bool store = true;
    if (tile.split >= 0) {
      const int n_pieces = tile.piece >> 16;
      const int64_t slot = tile.split + (tile.piece & 0xffff);
      if (q_valid) {
        float* so = p.dq_split + (slot * C::kRows + qi) * D;
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            store_dev16(so + cb * 32 + 8 * g + 4 * hi,
                        f32x4{acc[cb][4 * g] * osc, acc[cb][4 * g + 1] * osc, acc[cb][4 * g + 2] * osc,
                              acc[cb][4 * g + 3] * osc});
      }
      store_dev_wait();
      __syncthreads();
      if (tid == 0)
        s_last = __hip_atomic_fetch_add(p.dq_split_cnt + tile.split, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 n_pieces - 1;
      __syncthreads();
      store = s_last;
      if (store && q_valid) {
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb) acc[cb] = f32x16{};
        for (int c = 0; c < n_pieces; ++c) {
          const float* so = p.dq_split + (((int64_t)tile.split + c) * C::kRows + qi) * D + 4 * hi;
          // this lane's D/2 values of the row: D/8 chunks of 16 bytes, 8 floats apart; chunk k
          // holds (column block k/4, group k%4)
          f32x4 x[D / 8];
          if constexpr (D == 128)
            load_dev16x16(so, x);
          else
            load_dev16x8(so, x);
#pragma unroll
          for (int k = 0; k < D / 8; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[k / 4][4 * (k % 4) + e] += x[k][e];
        }
        osc = 1.0f;
      }
    }
    if (store && q_valid) {
      float* out = p.dq + qprow * D;
#pragma unroll
      for (int cb = 0; cb < C::kCb; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = cb * 32 + 8 * g + 4 * hi;
          *(f32x4*)(out + c) = f32x4{acc[cb][4 * g] * osc, acc[cb][4 * g + 1] * osc, acc[cb][4 * g + 2] * osc,
                                     acc[cb][4 * g + 3] * osc};
        }
    }
  }
}

template <typename K>
int occupancy(K kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) n = 0;
  return n;
}

}  // namespace

// Resident workgroups per compute unit, queried once per kernel (function-local statics, so
// concurrent first calls are safe); 0 if the query fails.
int bwd_blocks_per_cu(int d) {
  static const int c64 = occupancy(dkdv_kernel<64, false>, 256);
  static const int c128 = occupancy(dkdv_kernel<128, false>, 256);
  return d == 64 ? c64 : c128;
}

int dq_blocks_per_cu(int d, int rows) {
  static const int c64w = occupancy(dq_kernel<64, false, 8>, DqCfg<64, 8>::kThreads);
  static const int c128w = occupancy(dq_kernel<128, false, 8>, DqCfg<128, 8>::kThreads);
  static const int c64n = occupancy(dq_kernel<64, false, 4>, DqCfg<64, 4>::kThreads);
  static const int c128n = occupancy(dq_kernel<128, false, 4>, DqCfg<128, 4>::kThreads);
  if (rows == kDqRowsWide) return d == 64 ? c64w : c128w;
  return d == 64 ? c64n : c128n;
}

template <int D, bool kPacked>
void launch_bwd_impl(const BwdParams& p, int dq_rows, int grid_pre, int grid, int grid_dq, unsigned stages,
                     hipStream_t s) {
  if (stages & ZL_BWD_PRE) hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3(grid_pre), dim3(256), 0, s, p);
  if (stages & ZL_BWD_DKDV) hipLaunchKernelGGL((dkdv_kernel<D, kPacked>), dim3(grid), dim3(256), 0, s, p);
  if (stages & ZL_BWD_DQ) {
    if (dq_rows == kDqRowsWide)
      hipLaunchKernelGGL((dq_kernel<D, kPacked, 8>), dim3(grid_dq), dim3(DqCfg<D, 8>::kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((dq_kernel<D, kPacked, 4>), dim3(grid_dq), dim3(DqCfg<D, 4>::kThreads), 0, s, p);
  }
}

int launch_bwd(int d, int dq_rows, const BwdParams& p, int grid_pre, int grid, int grid_dq, unsigned stages,
               void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (d == 64 && p.packed)
    launch_bwd_impl<64, true>(p, dq_rows, grid_pre, grid, grid_dq, stages, s);
  else if (d == 64)
    launch_bwd_impl<64, false>(p, dq_rows, grid_pre, grid, grid_dq, stages, s);
  else if (p.packed)
    launch_bwd_impl<128, true>(p, dq_rows, grid_pre, grid, grid_dq, stages, s);
  else
    launch_bwd_impl<128, false>(p, dq_rows, grid_pre, grid, grid_dq, stages, s);
  return hipPeekAtLastError() == hipSuccess ? 0 : 1;
}

}  // namespace zl
