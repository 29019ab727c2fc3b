// Forward kernel: persistent, per-XCD cost-ordered queues of (segment, head, query rows) items.
//
// Computes, per item, softmax attention of its query rows against the segment's key rows
// (dense bidirectional attention of one sequence, Zellige page §II-A; segments never read
// another sequence's keys, §IV-D), with an online softmax over blocks of 64 keys, and
// writes either the final O and LSE at the query rows or, for a ring part, the normalised
// partial O and its LSE to the partial slab (§II-B ring accumulation).
//
// Split items: an item may cover only a piece of its segment's keys. Its normalised partial
// goes to the workspace through device-coherent stores; the last piece to finish (a
// device-scope counter) merges the pieces by their log-sum-exps, read back with
// device-coherent loads, and stores the item's result as an unsplit item would.
//
// Shape of one workgroup: W waves x 32 query rows, W = 4 (narrow items of 128 rows, two
// workgroups per CU) or 8 (wide items of 256 rows, one workgroup per CU, every K/V block in LDS
// shared by twice the rows); the plan picks the size. Each wave keeps its 32 query rows in
// registers as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so every lane owns
// one query row of the score tile: the running max and sum are per-lane values that only
// combine with the partner lane l^32. The exponentiated scores, rounded to bf16, are already
// in the B-operand layout of O^T = V^T P^T; V^T comes from LDS through transposed reads.
//
// Software pipeline. On gfx950 the matrix cores and the vector ALU overlap when one wave
// interleaves both kinds of instruction; a wave in a pure softmax phase does not hide behind
// another wave's MFMAs. Step t of an item therefore runs, as two interleaved regions,
//   region 1: the MFMAs of O += P(t-1) V(t-1), with the exponentials of block t in place;
//   region 2: rounding of those exponentials to bf16 P(t), with the MFMAs of S(t+1) = K(t+1) Q^T
//             in the freed registers, the row sums of P(t) and the row max of S(t+1),
// so the vector work of one block runs under the matrix work of its neighbours and the
// registers of S and P are reused in place. K and V blocks reach LDS by direct global-to-LDS
// loads (no staging registers) issued at the start of a step for use in the next one: K(t+2)
// and V(t) into the buffers step t-1 finished reading.
//
// LDS layouts (64 banks of 4 bytes; 16 lanes per cycle for 16-byte reads, 32 lanes for the
// 8-byte transposed reads):
//   K: rows in groups of 1 KB (4 rows of d = 128, 8 of d = 64) with a 64-byte gap between
//      groups; 16-byte chunk c of row r sits at position c ^ g(r), g(r) in 0..3. The 16 rows
//      read together fall on 16 distinct bank groups, and since g only flips the two low
//      chunk bits the read address of every k-step is one of two per-lane bases plus a
//      constant.
//   V: column-block major, [d/32][64 keys][32 values]: the 4 consecutive keys x 64 bytes of a
//      transposed read are 256 contiguous bytes, and every address is affine.
// Both layouts are what a global-to-LDS load can write: each wave instruction fills 1 KB of
// contiguous LDS, lane l the 16 bytes at offset 16 l, and each lane picks its source chunk.
#include "zl_device.hpp"
#include "zl_internal.h"

namespace zl {
namespace {

template <int D, int W = 4>
struct FwdCfg {
  static constexpr int kWaves = W;
  static constexpr int kRows = 32 * W;                    // query rows per item
  static constexpr int kBk = 64;                          // keys per block
  static constexpr int kKb = kBk / 32;                    // 32x32 S^T tiles per block
  static constexpr int kKs = kBk / 16;                    // 16-key steps of O^T += V^T P^T
  static constexpr int kSteps = D / 16;                   // k-steps over d for S^T
  static constexpr int kCb = D / 32;                      // 32-wide column blocks of O^T
  static constexpr int kRowBytes = 2 * D;                 // one K or V row in bf16
  static constexpr int kRowChunks = D / 8;                // 16-byte chunks per row
  static constexpr int kGroupRows = 1024 / kRowBytes;     // K rows per 1 KB group
  static constexpr int kGroupPitch = 1024 + 64;           // bytes between K row groups
  static constexpr int kKBytes = kBk / kGroupRows * kGroupPitch;
  static constexpr int kKbStride = 32 / kGroupRows * kGroupPitch;  // bytes between 32-row K tiles
  static constexpr int kVBytes = kBk * kRowBytes;
  static constexpr int kVCbStride = kBk * 64;             // bytes between V column blocks
  static constexpr int kKDma = kBk / kGroupRows / W;      // K loads per thread per block
  static constexpr int kVDma = kVBytes / 1024 / W;        // V loads per thread per block
  static_assert(kKDma >= 1 && kVDma >= 1, "every wave loads part of each block");
  static constexpr float kSlack = 8.0f;                   // lazy-rescale slack, log2 units
  static constexpr int kAhead = 2;                        // MFMAs between an operand read and its use
};

// Per-lane constants and per-item pointers shared by the pipeline steps.
template <int D>
struct FwdCtx {
  const bf16* kbase;  // key row (kv_begin, head h)
  const bf16* vbase;
  int64_t rs;         // elements between consecutive tokens
  int n_kv, n_blk;
  int koff0, koff1;   // K read bases for even / odd k-steps (bytes)
  int voff;           // V transposed-read base (bytes)
  int64_t blk_bytes;                    // bytes between consecutive key blocks
  uint32_t row_bytes;                   // bytes between consecutive key rows (tokens)
  uint32_t koff_dma;                    // this lane's byte offset of K load 0 in a full block
  uint32_t voff_dma;                    // ... of V load 0
  int64_t k_dma_step;                   // bytes between the rows of consecutive K loads
  int dma_krow, dma_kcol;               // this lane's row within its K load group, byte column
  int dma_vrow, dma_vcol;               // this lane's key within the block, byte column (load 0)
  int wave;
  float scale_log2;
};

template <int D>
struct FwdState {
  f32x16 oacc[FwdCfg<D>::kCb];
  bf16x8 q[FwdCfg<D>::kSteps];
  float m_run;  // exponent reference, log2 units
  float l_run;  // this lane's share of the running sum
  float mx;     // row max of the pending score block, log2 units
};

// Global -> LDS load of K block blk by W waves. Lane offsets are relative to the block's first
// key row; in a partial last block, rows past the end of the segment read its last row.
template <int D, int W>
__device__ __forceinline__ void dma_k(const FwdCtx<D>& cx, uint32_t k_lds, int blk) {
  using C = FwdCfg<D, W>;
  const char* base = (const char*)cx.kbase + (int64_t)blk * cx.blk_bytes;
  if ((blk + 1) * C::kBk <= cx.n_kv) {
#pragma unroll
    for (int i = 0; i < C::kKDma; ++i)
      lds_dma16(k_lds + (i * W + cx.wave) * C::kGroupPitch, base + i * cx.k_dma_step, cx.koff_dma);
  } else {
    const int last = cx.n_kv - 1 - blk * C::kBk;
#pragma unroll
    for (int i = 0; i < C::kKDma; ++i) {
      const int row = min((i * W + cx.wave) * C::kGroupRows + cx.dma_krow, last);
      lds_dma16(k_lds + (i * W + cx.wave) * C::kGroupPitch, base, (uint32_t)row * cx.row_bytes + cx.dma_kcol);
    }
  }
}

// Each 1 KB of the V tile is 16 keys x 64 bytes of one column block; load i of wave w fills
// the (Wi + w)-th such piece: column block (Wi + w) / (kBk / 16), key group (Wi + w) % (kBk / 16).
template <int D, int W>
__device__ __forceinline__ void dma_v(const FwdCtx<D>& cx, uint32_t v_lds, int blk) {
  using C = FwdCfg<D, W>;
  const char* base = (const char*)cx.vbase + (int64_t)blk * cx.blk_bytes;
  if ((blk + 1) * C::kBk <= cx.n_kv) {
#pragma unroll
    for (int i = 0; i < C::kVDma; ++i)
      lds_dma16(v_lds + (i * W + cx.wave) * 1024, base + 64 * (W / (C::kBk / 16)) * i, cx.voff_dma);
  } else {
    const int row = min(cx.dma_vrow, cx.n_kv - 1 - blk * C::kBk);
#pragma unroll
    for (int i = 0; i < C::kVDma; ++i)
      lds_dma16(v_lds + (i * W + cx.wave) * 1024, base,
                (uint32_t)row * cx.row_bytes + cx.dma_vcol + 64 * (W / (C::kBk / 16)) * i);
  }
}

// Clears the queue counters, the split-item counters and the visit counters before a launch.
__global__ __launch_bounds__(256) void zero_counters_kernel(int32_t* counters, int32_t grid, int32_t* split_cnt,
                                                            int32_t n_split, int32_t* visits, int32_t n_visits) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < kQueues) counters[i * kCounterStride] = home_count(grid, i);  // past the static first items
  for (int j = i; j < n_split; j += gridDim.x * 256) split_cnt[j] = 0;
  if (visits)
    for (int j = i; j < n_visits; j += gridDim.x * 256) visits[j] = 0;
}

// S^T[key][q] of one block: kKb tiles of 32 keys, each a chain of k-steps over d.
template <int D>
__device__ __forceinline__ void score_block(const FwdCtx<D>& cx, uint32_t k_lds, const bf16x8 (&q)[FwdCfg<D>::kSteps],
                                            f32x16 (&s)[FwdCfg<D>::kKb]) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int kb = 0; kb < C::kKb; ++kb) {
    s[kb] = f32x16{};
#pragma unroll
    for (int st = 0; st < C::kSteps; ++st) {
      const uint32_t kp = k_lds + kb * C::kKbStride + (st & 1 ? cx.koff1 : cx.koff0) + 64 * (st >> 1);
      s[kb] = mfma32(*(ZL_LDS const bf16x8*)kp, q[st], s[kb]);
    }
  }
}

// O^T[c][q] += V^T[c][key] P^T[key][q], 16 keys per step. The k order of P^T in this lane is
// keys {16ks + 4hi + 0..3, 16ks + 8 + 4hi + 0..3}; the two transposed reads fetch V rows in
// that same order.
template <int D>
__device__ __forceinline__ void value_block(const FwdCtx<D>& cx, uint32_t v_lds, const bf16x8 (&pb)[FwdCfg<D>::kKs],
                                            f32x16 (&oacc)[FwdCfg<D>::kCb]) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int ks = 0; ks < C::kKs; ++ks)
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb) {
      const uint32_t vp = v_lds + cb * C::kVCbStride + ks * 1024 + cx.voff;
      const bf16x8 a = cat(lds_read_tr(vp), lds_read_tr(vp + 512));
      oacc[cb] = mfma32(a, pb[ks], oacc[cb]);
    }
}

// Keys at or past `valid` in a score block get -inf.
template <int KB>
__device__ __forceinline__ void mask_block(f32x16 (&s)[KB], int valid, int hi) {
  const int vr = valid - 4 * hi;  // compare lane-independent key offsets against one value
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (kb * 32 + 8 * (i / 4) + (i % 4) >= vr) s[kb][i] = -INFINITY;
}

template <int KB>
__device__ __forceinline__ float block_max(const f32x16 (&s)[KB]) {
  float mx = s[0][0];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
  return mx;
}

// In place: S -> exp2(S * scale_log2 - m).
template <int KB>
__device__ __forceinline__ void block_exp(f32x16 (&s)[KB], float scale_log2, float m) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(fmaf(s[kb][i], scale_log2, -m));
}

// Exponentials -> bf16 P in the B-operand layout (P^T k-steps of 16 keys). Returns this
// lane's sum of the rounded values (bf16 pair dot products with 1): the same weights that the
// P V product uses.
template <int KB>
__device__ __forceinline__ float block_round(const f32x16 (&e)[KB], bf16x8 (&pb)[2 * KB]) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      f32x8 v;
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = e[kb][8 * hs + u];
      const bf16x8 r = to_bf16x8(v);
      pb[2 * kb + hs] = r;
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(r, r, 0, 1), one, lsum, false);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(r, r, 2, 3), one, lsum, false);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(r, r, 4, 5), one, lsum, false);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(r, r, 6, 7), one, lsum, false);
    }
  return lsum;
}

// Operand reads at a per-lane base plus a constant (the constant folds into the instruction).
template <int D>
__device__ __forceinline__ bf16x8 v_operand(ZL_LDS const char* vb, int m) {
  using C = FwdCfg<D>;
  ZL_LDS const char* vp = vb + (m % C::kCb) * C::kVCbStride + (m / C::kCb) * 1024;
  return cat(lds_read_tr(vp), lds_read_tr(vp + 512));
}

template <int D>
__device__ __forceinline__ bf16x8 k_operand(ZL_LDS const char* kb0, ZL_LDS const char* kb1, int m) {
  using C = FwdCfg<D>;
  const int st = m % C::kSteps;
  return *(ZL_LDS const bf16x8*)((st & 1 ? kb1 : kb0) + (m / C::kSteps) * C::kKbStride + 64 * (st >> 1));
}

// Region 1 of a step, written in issue order: each P(t-1) V(t-1) MFMA (operands read two
// MFMAs ahead) is followed by its share of the in-place exponentials of S(t).
template <int D>
__device__ __forceinline__ void pv_exp_interleaved(const FwdCtx<D>& cx, uint32_t v_lds, const bf16x8 (&pb)[FwdCfg<D>::kKs],
                                                   f32x16 (&oacc)[FwdCfg<D>::kCb], f32x16 (&sc)[FwdCfg<D>::kKb],
                                                   float m_ref) {
  using C = FwdCfg<D>;
  constexpr int kM = C::kKs * C::kCb;
  constexpr int kAhead = C::kAhead;
  constexpr int kPer = 16 * C::kKb / kM;  // exponentials per MFMA
  static_assert(kPer * kM == 16 * C::kKb, "exponentials must divide evenly over the MFMAs");
  ZL_LDS const char* vb = (ZL_LDS const char*)(v_lds + cx.voff);
  bf16x8 a[kM];
#pragma unroll
  for (int m = 0; m < kAhead; ++m) a[m] = v_operand<D>(vb, m);
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    if (m + kAhead < kM) a[m + kAhead] = v_operand<D>(vb, m + kAhead);
    oacc[m % C::kCb] = mfma32(a[m], pb[m / C::kCb], oacc[m % C::kCb]);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = m * kPer + u;
      sc[e / 16][e % 16] = fast_exp2(fmaf(sc[e / 16][e % 16], cx.scale_log2, -m_ref));
    }
  }
}

// Region 2 of a step, written in issue order: the exponentials become bf16 P(t) (tile 0 before
// its score chain starts, tile 1 during it); the S(t+1) MFMAs (operands read two MFMAs ahead)
// accumulate into the freed registers; the row sum of P(t) and the row max of the finished
// tile 0 fill the slots of the later MFMAs; the max of tile 1 follows the last MFMA.
template <int D>
__device__ __forceinline__ void round_score_interleaved(const FwdCtx<D>& cx, uint32_t k_lds,
                                                        const bf16x8 (&q)[FwdCfg<D>::kSteps],
                                                        f32x16 (&sc)[2], bf16x8 (&pb)[4], float& lsum,
                                                        float& mx) {
  using C = FwdCfg<D>;
  static_assert(C::kKb == 2, "two score tiles per block");
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  auto half = [](const f32x16& t, int hs) {
    f32x8 v;
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = t[8 * hs + u];
    return to_bf16x8(v);
  };
  pb[0] = half(sc[0], 0);
  pb[1] = half(sc[0], 1);
  constexpr int kM = 2 * C::kSteps;
  constexpr int kAhead = C::kAhead;
  float ls0 = 0.f, ls1 = 0.f, mx0 = -INFINITY, mx1 = -INFINITY;
  ZL_LDS const char* kb0 = (ZL_LDS const char*)(k_lds + cx.koff0);
  ZL_LDS const char* kb1 = (ZL_LDS const char*)(k_lds + cx.koff1);
  bf16x8 ko[kM];
#pragma unroll
  for (int m = 0; m < kAhead; ++m) ko[m] = k_operand<D>(kb0, kb1, m);
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    if (m + kAhead < kM) ko[m + kAhead] = k_operand<D>(kb0, kb1, m + kAhead);
    const int kb = m / C::kSteps;
    const int st = m % C::kSteps;
    sc[kb] = mfma32(ko[m], q[st], st == 0 ? f32x16{} : sc[kb]);
    if (m == 0) pb[2] = half(sc[1], 0);
    if (m == 1) pb[3] = half(sc[1], 1);
    // 16 row-sum dot products spread over the slots after the rounding.
    if (m >= 2) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (2 + (j * (kM - 2)) / 16 == m) {
          const bf16x8 r = pb[j / 4];
          const bf16x2 pr = __builtin_shufflevector(r, r, 0, 1);
          const bf16x2 pr1 = __builtin_shufflevector(r, r, 2, 3);
          const bf16x2 pr2 = __builtin_shufflevector(r, r, 4, 5);
          const bf16x2 pr3 = __builtin_shufflevector(r, r, 6, 7);
          const bf16x2 sel = (j % 4) == 0 ? pr : (j % 4) == 1 ? pr1 : (j % 4) == 2 ? pr2 : pr3;
          if (j & 1)
            ls1 = __builtin_amdgcn_fdot2_f32_bf16(sel, one, ls1, false);
          else
            ls0 = __builtin_amdgcn_fdot2_f32_bf16(sel, one, ls0, false);
        }
    }
    // Row max of tile 0 over the slots of tile 1's chain (two values per slot).
    if (kb == 1) {
#pragma unroll
      for (int u = 0; u < 16 / C::kSteps; ++u) {
        const int i = st * (16 / C::kSteps) + u;
        mx0 = fmaxf(mx0, sc[0][i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) mx1 = fmaxf(mx1, sc[1][i]);
  lsum = ls0 + ls1;
  mx = fmaxf(mx0, mx1);
}

// One pipeline step t of an item (see the file comment). kPrev: block t-1 exists (P(t-1) is in
// `pb`, V(t-1) in LDS); kNext: block t+1 exists (K(t+1) in LDS). On entry `sc` holds S(t) and
// st.mx its row max; on return `pb` holds P(t), `sc` S(t+1) and st.mx its row max. The two
// register sets are reused in place, so steps need no copies:
//   region 1: the P(t-1) V(t-1) MFMAs, with the exponentials of S(t) computed in place;
//   region 2: rounding of those exponentials into `pb` (free once region 1 has issued its
//             MFMAs), with the S(t+1) MFMAs accumulating into `sc`, then its row max.
template <int D, int W, bool kPrev, bool kNext>
__device__ __forceinline__ void fwd_step(const FwdCtx<D>& cx, FwdState<D>& st, int t, uint32_t k_dma, uint32_t v_dma,
                                         uint32_t k_rd, uint32_t v_rd, f32x16 (&sc)[FwdCfg<D>::kKb],
                                         bf16x8 (&pb)[FwdCfg<D>::kKs], int hi) {
  using C = FwdCfg<D>;
  if (kNext && t + 2 < cx.n_blk) dma_k<D, W>(cx, k_dma, t + 2);
  dma_v<D, W>(cx, v_dma, t);

  // Lazy rescaling: the exponent reference only moves when the block max exceeds it by more
  // than kSlack, so exponentials stay below 2^kSlack. P(t) uses the new reference; the
  // accumulators move to it after the pending P(t-1) V(t-1) product (which belongs to the old
  // one) has been added, and only when some lane of the wave needs it. The result is the same
  // quantity; only the reference changes.
  const bool need = st.mx > st.m_run + C::kSlack;
  const bool rescale = __any(need);
  float alpha = 1.f;
  if (rescale) {
    const float m_new = need ? st.mx : st.m_run;
    alpha = fast_exp2(st.m_run - m_new);
    st.m_run = m_new;
  }

  __builtin_amdgcn_sched_barrier(0);
  if (kPrev)
    pv_exp_interleaved<D>(cx, v_rd, pb, st.oacc, sc, st.m_run);
  else
    block_exp(sc, cx.scale_log2, st.m_run);
#pragma unroll
  for (int kb = 0; kb < C::kKb; ++kb) asm volatile("" : "+v"(sc[kb]));  // keep the exponentials here
  __builtin_amdgcn_sched_barrier(0);
  if (rescale) {
    st.l_run *= alpha;
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb) st.oacc[cb] *= alpha;
  }
  __builtin_amdgcn_sched_barrier(0);
  float lsum, mxn = 0.f;
  if (kNext)
    round_score_interleaved<D>(cx, k_rd, st.q, sc, pb, lsum, mxn);
  else
    lsum = block_round(sc, pb);
  asm volatile("" : "+v"(lsum), "+v"(mxn));
  __builtin_amdgcn_sched_barrier(0);
  st.l_run += lsum;
  if (kNext) {
    const int valid = cx.n_kv - (t + 1) * C::kBk;
    if (valid < C::kBk) {
      mask_block(sc, valid, hi);
      mxn = block_max(sc);
    }
    st.mx = half_max(mxn) * cx.scale_log2;
  }
  dma_wait();
  __syncthreads();
}

template <int D, bool kPacked, int W>
__global__ __launch_bounds__(64 * W, 8 / W) void fwd_kernel(const FwdParams p) {
  using C = FwdCfg<D, W>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::kVBytes + 2 * C::kKBytes];
  // LDS byte addresses of the double-buffered V and K blocks.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(ZL_LDS char*)smem;
  const uint32_t v_lds0 = lds0, v_lds1 = lds0 + C::kVBytes;
  const uint32_t k_lds0 = lds0 + 2 * C::kVBytes, k_lds1 = k_lds0 + C::kKBytes;
  __shared__ int32_t s_item;
  __shared__ int32_t s_queue_mem[kQueues + 2];  // queue state of thread 0: bounds, then take_item's state
  ZL_LDS int32_t* const s_bounds = (ZL_LDS int32_t*)s_queue_mem;
  ZL_LDS int32_t* const s_taker = s_bounds + kQueues + 1;
  __shared__ int32_t s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bf16* __restrict__ gq = (const bf16*)p.q;

  FwdCtx<D> cx;
  cx.wave = __builtin_amdgcn_readfirstlane(wave);
  cx.scale_log2 = p.scale_log2;
  {
    const int g = (l32 / (C::kGroupRows / 4)) & 3;
    const int row = (l32 / C::kGroupRows) * C::kGroupPitch + (l32 % C::kGroupRows) * C::kRowBytes;
    cx.koff0 = row + 16 * (hi ^ g);
    cx.koff1 = row + 16 * ((2 + hi) ^ g);
    const int r_in = (lane & 15) >> 2;
    const int c_in = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    cx.voff = (4 * hi + r_in) * 64 + 2 * c_in;
    constexpr int kGroups = C::kBk / 16;
    cx.dma_krow = lane / C::kRowChunks;
    cx.dma_kcol = 16 * ((lane % C::kRowChunks) ^ ((lane >> 4) & 3));
    cx.dma_vrow = (wave % kGroups) * 16 + lane / 4;
    cx.dma_vcol = 64 * (wave / kGroups) + 16 * (lane & 3);
  }

  const int home = blockIdx.x % kQueues;
  if (tid == 0) {
    stage_bounds(p.queue, s_bounds);
    *s_taker = home << 8;
  }
  for (;;) {
    if (tid == 0) s_item = take_item(p.queue, s_bounds, s_taker, p.visits);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);  // the same for every lane
    if (item < 0) break;
    const Tile tile = p.queue.items[item];
    const SegDev sg = p.segs[tile.seg];
    const int nh = sg.nh;
    const int h = tile.head;
    const QkvRows qr = qkv_rows<kPacked>(sg);  // planar, or the QKV-packed layout
    cx.rs = (int64_t)qr.t_stride * D;          // K / V elements between consecutive tokens
    cx.row_bytes = (uint32_t)(cx.rs * 2);
    cx.blk_bytes = (int64_t)C::kBk * cx.rs * 2;
    cx.koff_dma = (uint32_t)(wave * C::kGroupRows + cx.dma_krow) * cx.row_bytes + cx.dma_kcol;
    cx.voff_dma = (uint32_t)cx.dma_vrow * cx.row_bytes + cx.dma_vcol;
    cx.k_dma_step = (int64_t)W * C::kGroupRows * cx.rs * 2;
    cx.n_kv = tile.kv_end - tile.kv_begin;  // the segment's keys, or one piece of them
    cx.n_blk = (cx.n_kv + C::kBk - 1) / C::kBk;
    cx.kbase = (const bf16*)p.k + (qr.k0 + (int64_t)tile.kv_begin * qr.t_stride + h) * D;
    cx.vbase = (const bf16*)p.v + (qr.k0 + qr.v_off + (int64_t)tile.kv_begin * qr.t_stride + h) * D;
    const int n = cx.n_blk;

    // Prologue: K(0), K(1) into LDS; this lane's query row into registers (clamped to the
    // last valid row; results of clamped rows are dropped); S(0) and its row max.
    dma_k<D, W>(cx, k_lds0, 0);
    if (n > 1) dma_k<D, W>(cx, k_lds1, 1);
    const int qi = wave * 32 + l32;
    const bool q_valid = qi < tile.nrows;
    const int qtok = tile.row0 + (q_valid ? qi : tile.nrows - 1);
    FwdState<D> st;
    {
      const bf16* qp = gq + (qr.q0 + (int64_t)qtok * qr.t_stride + h) * D + 8 * hi;
#pragma unroll
      for (int s = 0; s < C::kSteps; ++s) st.q[s] = *(const bf16x8*)(qp + 16 * s);
    }
#pragma unroll
    for (int cb = 0; cb < C::kCb; ++cb) st.oacc[cb] = f32x16{};
    st.m_run = -INFINITY;
    st.l_run = 0.f;
    f32x16 sc[C::kKb];
    bf16x8 pb[C::kKs];
    dma_wait();
    __syncthreads();
    score_block<D>(cx, k_lds0, st.q, sc);
    if (cx.n_kv < C::kBk) mask_block(sc, cx.n_kv, hi);
    st.mx = half_max(block_max(sc)) * cx.scale_log2;
    __syncthreads();  // every wave has read K(0) before step 0 refills its buffer

    // Step t reads K(t+1) from k_lds[(t+1)&1] and V(t-1) from v_lds[(t-1)&1], and refills
    // k_lds[t&1] with K(t+2) and v_lds[t&1] with V(t).
    if (n == 1) {
      fwd_step<D, W, false, false>(cx, st, 0, k_lds0, v_lds0, k_lds1, v_lds1, sc, pb, hi);
    } else {
      fwd_step<D, W, false, true>(cx, st, 0, k_lds0, v_lds0, k_lds1, v_lds1, sc, pb, hi);
      for (int t = 1; t < n - 1; ++t) {
        const bool odd = t & 1;
        fwd_step<D, W, true, true>(cx, st, t, odd ? k_lds1 : k_lds0, odd ? v_lds1 : v_lds0, odd ? k_lds0 : k_lds1,
                                odd ? v_lds0 : v_lds1, sc, pb, hi);
      }
      const bool odd = (n - 1) & 1;
      fwd_step<D, W, true, false>(cx, st, n - 1, odd ? k_lds1 : k_lds0, odd ? v_lds1 : v_lds0, odd ? k_lds0 : k_lds1,
                               odd ? v_lds0 : v_lds1, sc, pb, hi);
    }
    value_block<D>(cx, ((n - 1) & 1) ? v_lds1 : v_lds0, pb, st.oacc);  // P(n-1) V(n-1)

    // Epilogue: O = O_acc / l, LSE = ln(2) * (m + log2 l), natural log. A ring part writes
    // its normalised partial to the slab, or in accumulate mode folds it into the running
    // O and LSE of its rows (exact merge of two normalised results, §II-B):
    //   LSE' = M + ln(e^{LSE - M} + e^{LSE_b - M}),  O' = e^{LSE - LSE'} O + e^{LSE_b - LSE'} O_b.
    // Rows whose running LSE is -inf take the part as it is (their O is not read).
    const float l_tot = half_sum(st.l_run);
    float o_scale = 1.0f / l_tot;
    float lse_b = 0.69314718055994531f * (st.m_run + __log2f(l_tot));
    bool store = true;
    if (tile.split >= 0) {
      // One key piece of a split item: publish the normalised partial (device-coherent
      // stores), then count the pieces done; the last piece merges all of them (the same
      // exact merge) and stores the item's result. No fence: the partials bypass the
      // per-XCD caches, and each count is issued after this workgroup's stores completed.
      const int n_pieces = tile.piece >> 16;
      const int64_t slot = tile.split + (tile.piece & 0xffff);
      if (q_valid) {
        float* so = p.split_o + (slot * C::kRows + qi) * D;
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 val = {st.oacc[cb][4 * g] * o_scale, st.oacc[cb][4 * g + 1] * o_scale,
                               st.oacc[cb][4 * g + 2] * o_scale, st.oacc[cb][4 * g + 3] * o_scale};
            store_dev16(so + cb * 32 + 8 * g + 4 * hi, val);
          }
        if (hi == 0)
          __hip_atomic_store(p.split_lse + slot * C::kRows + qi, lse_b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      store_dev_wait();
      __syncthreads();
      if (tid == 0)
        s_last = __hip_atomic_fetch_add(p.split_cnt + tile.split, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 n_pieces - 1;
      __syncthreads();
      store = s_last;
      if (store && q_valid) {
        const float* sl = p.split_lse + (int64_t)tile.split * C::kRows + qi;
        float m = -INFINITY;
        for (int c = 0; c < n_pieces; ++c)
          m = fmaxf(m, __hip_atomic_load(sl + c * C::kRows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        float tot = 0.f;
        for (int c = 0; c < n_pieces; ++c)
          tot += expf(__hip_atomic_load(sl + c * C::kRows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - m);
        lse_b = m + logf(tot);
#pragma unroll
        for (int cb = 0; cb < C::kCb; ++cb) st.oacc[cb] = f32x16{};
        for (int c = 0; c < n_pieces; ++c) {
          const float w =
              expf(__hip_atomic_load(sl + c * C::kRows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - lse_b);
          const float* so = p.split_o + (((int64_t)tile.split + c) * C::kRows + qi) * D + 4 * hi;
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
            for (int e = 0; e < 4; ++e) st.oacc[k / 4][4 * (k % 4) + e] += w * x[k][e];
        }
        o_scale = 1.0f;
      }
    }
    if (store && q_valid) {
      const bool fold = sg.part >= 0 && p.accumulate;
      float* orow;
      int64_t lrow;
      float* lse_out;
      if (sg.part < 0 || fold) {
        lrow = sg.q_row0 + (int64_t)qtok * nh + h;
        orow = p.o + lrow * D;
        lse_out = p.lse;
      } else {
        lrow = sg.part_row0 + (int64_t)(qtok - sg.q_begin) * (sg.head_end - sg.head_begin) + (h - sg.head_begin);
        orow = p.o_part + lrow * D;
        lse_out = p.lse_part;
      }
      float w_old = 0.f, w_new = o_scale, lse_new = lse_b;
      if (fold) {
        const float lse_a = lse_out[lrow];
        if (lse_a != -INFINITY) {
          const float mx = fmaxf(lse_a, lse_b);
          lse_new = mx + logf(expf(lse_a - mx) + expf(lse_b - mx));
          w_old = expf(lse_a - lse_new);
          w_new = expf(lse_b - lse_new) * o_scale;
        }
      }
#pragma unroll
      for (int cb = 0; cb < C::kCb; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = cb * 32 + 8 * g + 4 * hi;
          f32x4 val = {st.oacc[cb][4 * g] * w_new, st.oacc[cb][4 * g + 1] * w_new, st.oacc[cb][4 * g + 2] * w_new,
                       st.oacc[cb][4 * g + 3] * w_new};
          if (w_old != 0.f) val += *(const f32x4*)(orow + c) * w_old;
          *(f32x4*)(orow + c) = val;
        }
      if (hi == 0) lse_out[lrow] = lse_new;
    }
    __syncthreads();
  }
}

// Resident forward workgroups per compute unit for W-wave items, queried once per instance (a
// function-local static, so concurrent first calls are safe); 0 if the query fails.
template <int D, int W>
int blocks_per_cu_impl() {
  static const int cached = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_kernel<D, false, W>, 64 * W, 0) != hipSuccess) n = 0;
    return n;
  }();
  return cached;
}

template <int D, int W>
void launch_fwd_impl(const FwdParams& p, int grid, hipStream_t s) {
  if (p.packed)
    hipLaunchKernelGGL((fwd_kernel<D, true, W>), dim3(grid), dim3(64 * W), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_kernel<D, false, W>), dim3(grid), dim3(64 * W), 0, s, p);
}

}  // namespace

int fwd_blocks_per_cu(int d, int rows) {
  if (rows == kFwdRowsWide) return d == 64 ? blocks_per_cu_impl<64, 8>() : blocks_per_cu_impl<128, 8>();
  return d == 64 ? blocks_per_cu_impl<64, 4>() : blocks_per_cu_impl<128, 4>();
}

int launch_fwd(int d, int rows, const FwdParams& p, int grid, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t nz = std::max<int64_t>(p.n_split, p.visits ? p.n_visits : 0);
  const int zgrid = nz > 0 ? (int)std::min<int64_t>(64, (nz + 255) / 256) : 1;
  hipLaunchKernelGGL(zero_counters_kernel, dim3(zgrid), dim3(256), 0, s, p.queue.counters, grid, p.split_cnt,
                     p.n_split, p.visits, p.n_visits);
  const bool wide = rows == kFwdRowsWide;
  if (d == 64 && wide)
    launch_fwd_impl<64, 8>(p, grid, s);
  else if (d == 64)
    launch_fwd_impl<64, 4>(p, grid, s);
  else if (wide)
    launch_fwd_impl<128, 8>(p, grid, s);
  else
    launch_fwd_impl<128, 4>(p, grid, s);
  return hipPeekAtLastError() == hipSuccess ? 0 : 1;
}

}  // namespace zl
