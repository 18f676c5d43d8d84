// flce_kernels.h -- the kernels of the fused linear cross-entropy engine.
//
// Notation: X [N, H] hidden states, W [V, H] output weight, y the per-row
// targets, n the number of rows with a target ("valid" rows), c the gradient
// scale (grad_scale / n for the mean, grad_scale for the sum).  All GEMM-shaped
// kernels compute one or more 256 x 256 tiles with flce_tile.h.
//
// Forward  (loss, lse):
//   k_prep_*    targets, validity, compaction of the valid rows (idx, tgt)
//   k_gather    Xc[k] = X[idx[k]] for k < n, zero rows up to a tile multiple
//   k_target    zt[k] = <Xc[k], W[tgt[k]]>
//   k_fwd_lse   logits tiles W.Xc^T on MFMA, online max / sum-exp2 per row
//               over a range of vocabulary tiles -> (m, s) partials
//   k_merge     lse = merge of the partials, loss_i = lse_i - zt_i, block sums
//   k_loss      fixed-order sum of the block sums -> loss
// Backward (dX, dW), over vocabulary blocks [v0, v0 + vb), as tiles of k_bwd:
//   G tiles     logits recomputed on MFMA, G = c * exp(z - lse) stored (bf16 or
//               fp32) into a bounded [rows x block] slab (two, alternating)
//   dW tiles    dW[v0 + m, :] = sum_k G[k, m] Xc[k, :] - OH[v0 + m]
//               (complete, stored once; OH: the one-hot part, k_oh_*)
//   dX tiles    dX32[k, :] += sum_m G[k, m] W[v0 + m, :] (FP32)
// one launch runs the dX and dW tiles of block b with the G tiles of block
// b + 1; k_dx_final takes off the one-hot part c_k W[y_k], rounds dX32 once
// and scatters it to the original rows.
#pragma once

#include "flce_tile.h"

namespace flce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Counters {
  int n;         // valid rows
  int status;    // 0 or FLCE_ERR_LABEL_RANGE
  float c;       // gradient scale (backward)
  int fwd_p;     // forward: vocabulary ranges per token tile
  int dx_parts;  // chunked mode, per chunk: vocabulary parts of the dX tiles
};

// The dX tiles of a backward launch number (vocabulary parts) x (hidden
// tiles) x (token tiles).  With few token tiles (narrow H, few rows, the
// short last row chunk) one part per tile would leave most compute units
// idle for a whole block's K loop, so the block's vocabulary range is cut
// into parts, each summed in its own FP32 buffer, until about `target` dX
// tiles are in flight: at most kMaxDxParts, and, where the extra parts share
// a buffer of `part_tiles` token tiles, only as many as it holds
// (part_tiles < 0: no such bound).
constexpr int kMaxDxParts = 8;
__host__ __device__ inline int dx_parts_for(int hidden_tiles, int token_tiles, int target,
                                            int part_tiles) {
  if (token_tiles <= 0) return 1;
  const int per = hidden_tiles * token_tiles;
  int s = (target + per - 1) / per;
  if (s > kMaxDxParts) s = kMaxDxParts;
  if (part_tiles >= 0 && s > 1 + part_tiles / token_tiles) s = 1 + part_tiles / token_tiles;
  return s < 1 ? 1 : s;
}


constexpr int kStatusLabelRange = 8;

// ---------------------------------------------------------------------------
// Targets, validity and compaction in three kernels over blocks of 1024 rows:
//   k_prep_count  valid rows and bad labels per block
//   k_prep_scan   one workgroup: block offsets (exclusive scan, block order),
//                 n, status, c and the forward split -> Counters
//   k_prep_write  each block's valid rows to idx / tgt in row order, rowpos
// so the compacted order is the row order (deterministic).  Labels are
// checked against V (the whole vocabulary); targets are stored relative to
// v_begin, the first vocabulary row of this call's W (V_local rows; a
// vocabulary shard), so a target outside the shard has an index outside
// [0, V_local).
// ---------------------------------------------------------------------------
constexpr int kPrepBlock = 1024;

// the target of row i (ignore when it has none) and whether it is valid
// (bad: neither ignore nor in [0, V))
__device__ __forceinline__ bool row_target(const int64_t* __restrict__ labels, int i, int N,
                                           int T, int64_t ignore, int64_t V, int shift,
                                           int64_t& y, bool& bad) {
  y = ignore;
  bad = false;
  if (i >= N) return false;
  if (shift) {
    const int t = i % T;
    y = (t + 1 < T) ? labels[i + 1] : ignore;
  } else {
    y = labels[i];
  }
  if (y == ignore) return false;
  if (y < 0 || y >= V) {
    bad = true;
    return false;
  }
  return true;
}

// per block: [0] valid rows, [1] 1 if a bad label
__global__ __launch_bounds__(kPrepBlock) void k_prep_count(
    const int64_t* __restrict__ labels, int N, int T, int64_t ignore, int64_t V, int shift,
    int* __restrict__ blk) {
  __shared__ int wsum[kPrepBlock / 64];
  __shared__ int bad_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) bad_s = 0;
  __syncthreads();
  int64_t y;
  bool bad;
  const bool valid = row_target(labels, blockIdx.x * kPrepBlock + tid, N, T, ignore, V, shift,
                                y, bad);
  if (bad) bad_s = 1;
  const uint64_t m = __ballot(valid);
  if (lane == 0) wsum[w] = __popcll(m);
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int q = 0; q < kPrepBlock / 64; ++q) tot += wsum[q];
    blk[2 * blockIdx.x] = tot;
    blk[2 * blockIdx.x + 1] = bad_s;
  }
}

// One workgroup: blk[2 b] becomes the block's first compacted index; n,
// status, c; the forward split: P vocabulary ranges per token tile, P * TTn
// items of about VT / P tiles each, at most max_items of them (P = 1 always
// fits).  With the items running in waves of `ncu` workgroups the time is
// about waves(P) * ceil(VT / P) tiles; thread t prices P = t + 1 and the
// cheapest (then the smallest) P wins.
__global__ __launch_bounds__(1024) void k_prep_scan(
    int* __restrict__ blk, int nblk, int reduction, const float* __restrict__ grad_scale,
    int ncu, int max_items, int64_t V_local, Counters* __restrict__ ctr,
    int32_t* __restrict__ status_out) {
  __shared__ int part[1024];
  __shared__ int bad_s;
  __shared__ unsigned long long best_s;
  const int tid = threadIdx.x;
  // thread t scans blocks t * per .. (t + 1) * per - 1 in order
  const int per = (nblk + 1023) / 1024;
  const int b0 = tid * per, b1 = min(b0 + per, nblk);
  int sum = 0, bad = 0;
  for (int b = b0; b < b1; ++b) {
    sum += blk[2 * b];
    bad |= blk[2 * b + 1];
  }
  if (tid == 0) bad_s = 0;
  part[tid] = sum;
  __syncthreads();
  if (bad) bad_s = 1;
  // inclusive scan of the 1024 partial sums (Hillis-Steele)
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid > 0 ? part[tid - 1] : 0;
  for (int b = b0; b < b1; ++b) {
    const int c = blk[2 * b];
    blk[2 * b] = run;
    run += c;
  }
  const int n = part[1023];
  const int64_t VT = (V_local + kTile - 1) / kTile;
  const int64_t TTn = n > 0 ? (n + kTile - 1) / kTile : 1;
  if (tid == 0) best_s = ~0ull;
  __syncthreads();
  {
    const int64_t P = tid + 1;
    if (P == 1 || (P <= VT && P * TTn <= max_items)) {
      const int64_t waves = (P * TTn + ncu - 1) / ncu;
      const int64_t pr = (VT + P - 1) / P;
      atomicMin(&best_s, (unsigned long long)(waves * pr) * 2048ull + (unsigned long long)P);
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int st = bad_s ? kStatusLabelRange : 0;
    const float gs = grad_scale ? *grad_scale : 1.0f;
    float c = reduction == 0 ? (n > 0 ? gs / (float)n : 0.0f) : gs;
    if (st) c = __builtin_nanf("");
    ctr->n = n;
    ctr->status = st;
    ctr->c = c;
    ctr->fwd_p = (int)(best_s & 2047ull);
    if (status_out) *status_out = st;
  }
}

__global__ __launch_bounds__(kPrepBlock) void k_prep_write(
    const int64_t* __restrict__ labels, int N, int T, int64_t ignore, int64_t V, int shift,
    const int* __restrict__ blk, int64_t v_begin, int* __restrict__ idx, int* __restrict__ tgt,
    int* __restrict__ rowpos) {
  __shared__ int wsum[kPrepBlock / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = blockIdx.x * kPrepBlock + tid;
  int64_t y;
  bool bad;
  const bool valid = row_target(labels, i, N, T, ignore, V, shift, y, bad);
  const uint64_t m = __ballot(valid);
  const int pre = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[w] = __popcll(m);
  __syncthreads();
  int pos = blk[2 * blockIdx.x] + pre;
  for (int q = 0; q < w; ++q) pos += wsum[q];
  if (i < N) {
    rowpos[i] = valid ? pos : -1;
    if (valid) {
      idx[pos] = i;
      tgt[pos] = (int)(y - v_begin);   // index into this call's W rows
    }
  }
}

// ---------------------------------------------------------------------------
// k_gather: one wave per compacted row k in [0, rows_pad).  Row k < n copies
// X[idx[k]]; the rest is zero.  In the backward it also stages
// lse2[k] = lse[idx[k]] * log2(e), clears row k of each of the dx_split
// FP32 dX accumulators (dx_stride floats apart) and sets the one-hot map
// (V_local entries) to -1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gather(
    const char* __restrict__ X, int row_bytes, const int* __restrict__ idx,
    const Counters* __restrict__ ctr, char* __restrict__ Xc, int rows_pad,
    const float* __restrict__ lse, float* __restrict__ lse2,
    float* __restrict__ dx32, int dx32_row_bytes, int dx_split, int64_t dx_stride,
    const float* __restrict__ rs_in, float* __restrict__ rs_c, int* __restrict__ map,
    int V_local) {
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (map != nullptr)
    for (int v = blockIdx.x * 256 + threadIdx.x; v < V_local; v += gridDim.x * 256) map[v] = -1;
  if (k >= rows_pad) return;
  const int n = ctr->n;
  const int chunks = row_bytes >> 4;
  i32x4* dst = (i32x4*)(Xc + (int64_t)k * row_bytes);
  if (k < n) {
    const i32x4* src = (const i32x4*)(X + (int64_t)idx[k] * row_bytes);
    for (int c = lane; c < chunks; c += 64) dst[c] = src[c];
  } else {
    for (int c = lane; c < chunks; c += 64) dst[c] = i32x4{0, 0, 0, 0};
  }
  if (lse2 != nullptr && lane == 0) lse2[k] = k < n ? lse[idx[k]] * kLog2e : 0.f;
  if (rs_c != nullptr && lane == 0) rs_c[k] = k < n ? rs_in[idx[k]] : 0.f;
  if (dx32 != nullptr) {
    for (int sp = 0; sp < dx_split; ++sp) {
      i32x4* d = (i32x4*)((char*)(dx32 + sp * dx_stride) + (int64_t)k * dx32_row_bytes);
      for (int c = lane; c < (dx32_row_bytes >> 4); c += 64) d[c] = i32x4{0, 0, 0, 0};
    }
  }
}

// ---------------------------------------------------------------------------
// k_target: zt[k] = <Xc[k], W[tgt[k]]> in fp32, one wave per valid row.
// ---------------------------------------------------------------------------
template <class E>
__global__ __launch_bounds__(256) void k_target(
    const char* __restrict__ Xc, const char* __restrict__ W, int H,
    const int* __restrict__ tgt, const Counters* __restrict__ ctr,
    float* __restrict__ zt, int V_local) {
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (k >= ctr->n) return;
  if (tgt[k] < 0 || tgt[k] >= V_local) {   // target in another vocabulary shard
    if (lane == 0) zt[k] = 0.f;
    return;
  }
  const int row_bytes = H * E::kBytes;
  const i32x4* x = (const i32x4*)(Xc + (int64_t)k * row_bytes);
  const i32x4* w = (const i32x4*)(W + (int64_t)tgt[k] * row_bytes);
  float acc = 0.f;
  for (int c = lane; c < (row_bytes >> 4); c += 64) {
    const i32x4 a = x[c], b = w[c];
    if constexpr (E::kBytes == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t ua = (uint32_t)a[q], ub = (uint32_t)b[q];
        acc = fmaf(bf2f(ua & 0xFFFFu), bf2f(ub & 0xFFFFu), acc);
        acc = fmaf(bf2f(ua >> 16), bf2f(ub >> 16), acc);
      }
    } else {
      // bit-cast whole vectors: casting single vector elements miscompiles
      const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = fmaf(af[q], bf[q], acc);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) zt[k] = acc;
}

// ---------------------------------------------------------------------------
// Online (max, sum of 2^(z - max)) pairs, kept in log2 units.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;            // both empty
  s = s * __builtin_amdgcn_exp2f(m - M) + s2 * __builtin_amdgcn_exp2f(m2 - M);
  m = M;
}

// Online update of the per-lane (max, sum) of 4 token columns with one tile
// of logits.  kMasked: tile rows r with (32i + 8(r/4) + r%4) >= lim are past
// the vocabulary end and are skipped (lim already holds the lane's offset).
template <bool kMasked>
__device__ __forceinline__ void lse_update(const f32x16 (&acc)[4][4], float (&m)[4],
                                           float (&s)[4], int lim) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!kMasked || 32 * i + 8 * (r >> 2) + (r & 3) < lim)
          tmax = fmaxf(tmax, acc[i][j][r]);
    // branch-free: with nothing seen yet (M = -inf) the sums stay 0
    const float M = fmaxf(m[j], tmax * kLog2e);
    const float Ms = M == -INFINITY ? 0.f : M;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(acc[i][j][r], kLog2e, -Ms));
        sum += (!kMasked || 32 * i + 8 * (r >> 2) + (r & 3) < lim) ? e : 0.f;
      }
    s[j] = s[j] * __builtin_amdgcn_exp2f(m[j] - Ms) + sum;
    m[j] = M;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------------------
// k_fwd_lse: work item (p, tau) = vocabulary range p x token tile tau.  The
// workgroup walks the range's 256-wide vocabulary tiles; A = W rows (vocab),
// B = Xc rows (tokens), so each lane's accumulators hold 64 vocabulary entries
// of 4 tokens and the per-token reduction is mostly in registers.
// ---------------------------------------------------------------------------
struct FwdArgs {
  const char* W;
  const char* Xc;
  int H, V, rows_pad;
  int VT;
  const Counters* ctr;
  float2* part;      // [item = p * TTn + tau][256 rows] (m in log2 units, s)
};

template <class E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fwd_lse(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem_[];
  lds_t* smem = (lds_t*)smem_;
  // the split k_prep_scan chose: P ranges x TTn token tiles, handed out XCD by XCD
  const int n = a.ctr->n, P = a.ctr->fwd_p;
  const int TTn = (n + kTile - 1) / kTile;
  const int nact = P * TTn, nact8 = (nact + 7) & ~7;
  if ((int)blockIdx.x >= nact8) return;
  const int item = xcd_item(blockIdx.x, nact8);
  if (item >= nact) return;
  int p, tau;
  grouped(item, P, TTn, p, tau);
  const int vt0 = (int)((int64_t)p * a.VT / P), vt1 = (int)((int64_t)(p + 1) * a.VT / P);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ldb = a.H * E::kBytes;
  const int steps = (ldb + kRowBytes - 1) / kRowBytes;

  Opnd B;
  B.base = a.Xc + (int64_t)tau * kTile * ldb;
  B.bytes = (int64_t)(a.rows_pad - tau * kTile) * ldb;
  B.ldb = ldb;
  B.kbytes = ldb;

  // The running (max, sum) of the lane's 4 token columns live in LDS between
  // tiles (each thread owns its slots): held in registers they would be live
  // across the K loop, which needs every register, and be spilled.
  __shared__ float2 ms_s[4][kThreads];
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) ms_s[j][t] = make_float2(-INFINITY, 0.f);
  f32x16 acc[4][4];
  auto w_tile = [&](int v) {
    Opnd A;
    A.base = a.W + (int64_t)v * kTile * ldb;
    A.bytes = (int64_t)(a.V - v * kTile) * ldb;
    A.ldb = ldb;
    A.kbytes = ldb;
    return A;
  };
  for (int vt = vt0; vt < vt1; ++vt) {
    const Opnd A = w_tile(vt);
    zero_acc(acc);
    if (vt == vt0) gemm_tile<E, LoadDirect, LoadDirect>(A, B, steps, smem, wm, wn, acc, opaque_tid());
    else gemm_tile_prefetched<E>(A, B, steps, smem, wm, wn, acc, opaque_tid());
    // rows at or past V (last tile only) take no part in the reduction
    const int vlim = a.V - vt * kTile;
    float m[4], s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float2 v = ms_s[j][t];
      m[j] = v.x;
      s[j] = v.y;
    }
    // the next tile's first two steps go straight into the (now idle) LDS
    // slabs while this tile's softmax update runs in registers
    if (vt + 1 < vt1) {
      const int tid = opaque_tid();
      prefetch_direct(w_tile(vt + 1), smem, steps, tid);
      prefetch_direct(B, smem + 2 * kSlab, steps, tid);
    }
    if (vlim >= kTile) lse_update<false>(acc, m, s, 0);
    else lse_update<true>(acc, m, s, vlim - wm * 128 - 4 * (lane >> 5));
#pragma unroll
    for (int j = 0; j < 4; ++j) ms_s[j][t] = make_float2(m[j], s[j]);
  }
  // combine the two lane halves and the two waves that share tokens
  typedef __attribute__((address_space(3))) float lf;
  lf* st = (lf*)smem;  // [wm][h][256 tokens][m, s]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = ((wm * 2 + (lane >> 5)) * kTile + acc_col(wn, j, lane)) * 2;
    const float2 v = ms_s[j][t];
    st[e] = v.x;
    st[e + 1] = v.y;
  }
  __syncthreads();
  float M = -INFINITY, S = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) lse_merge(M, S, st[(q * kTile + t) * 2], st[(q * kTile + t) * 2 + 1]);
  a.part[((int64_t)p * TTn + tau) * kTile + t] = make_float2(M, S);
}

// ---------------------------------------------------------------------------
// k_merge: one thread per original row.  Valid rows merge the P partials into
// lse and form loss_i = lse_i - zt_i; ignored rows get lse = 0.  Each block
// writes the fixed-order sum of its 256 row losses.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_merge(
    const float2* __restrict__ part, const Counters* __restrict__ ctr,
    const int* __restrict__ rowpos, const float* __restrict__ zt, int N,
    float* __restrict__ lse_out, float* __restrict__ blocksum, float* __restrict__ rloss_out,
    float* __restrict__ zt_out) {
  __shared__ float red[256];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int P = ctr->fwd_p, TTn = (ctr->n + kTile - 1) / kTile;
  float li = 0.f;
  if (i < N) {
    const int k = rowpos[i];
    float lse = 0.f;
    if (k >= 0) {
      const float2* pk = part + (int64_t)(k / kTile) * kTile + k % kTile;
      float M = -INFINITY, S = 0.f;
      for (int p = 0; p < P; ++p) {
        const float2 v = pk[(int64_t)p * TTn * kTile];
        const float Mn = fmaxf(M, v.x);
        if (Mn == -INFINITY) continue;
        S = S * exp2f(M - Mn) + v.y * exp2f(v.x - Mn);
        M = Mn;
      }
      lse = (M + log2f(S)) * kLn2;
      li = lse - zt[k];
    }
    lse_out[i] = lse;
    // per-row losses (reduction "none"): 0 on ignored rows, NaN after a bad label
    if (rloss_out) rloss_out[i] = ctr->status ? __builtin_nanf("") : li;
    // a vocabulary shard's target logits (0 where the target is elsewhere)
    if (zt_out) zt_out[i] = k >= 0 ? zt[k] : 0.f;
  }
  red[threadIdx.x] = li;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) blocksum[blockIdx.x] = red[0];
}

// k_loss: fixed-order sum of the block sums -> loss (mean or sum).
__global__ __launch_bounds__(256) void k_loss(
    const float* __restrict__ blocksum, int nb, const Counters* __restrict__ ctr,
    int reduction, float* __restrict__ loss, int64_t* __restrict__ n_valid) {
  __shared__ float red[256];
  float acc = 0.f;
  for (int b = threadIdx.x; b < nb; b += 256) acc += blocksum[b];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int n = ctr->n;
    float L = red[0];
    if (reduction == 0) L = n > 0 ? L / (float)n : 0.f;
    if (ctr->status != 0) L = __builtin_nanf("");
    if (loss) *loss = L;
    if (n_valid) *n_valid = n;
  }
}

// ---------------------------------------------------------------------------
// Backward GEMM tiles.  One launch of k_bwd runs three kinds of 256 x 256
// MFMA tiles, one per workgroup, longest first, so that the last wave of one
// kind is filled by the next instead of leaving compute units idle:
//   dX tiles of vocabulary block b     dX32[k, :] += G_b[k, :] W_b     (K = block)
//   dW tiles of block b                dW_b = G_b^T Xc                 (K = rows)
//   G tiles of block b + 1             G_{b+1} = c exp(Z - lse)        (K = H)
// Blocks b and b + 1 use the two halves of the softmax-gradient slab.
// ---------------------------------------------------------------------------
struct BwdArgs {
  const char* W;       // [V, H]
  const char* Xc;      // [rows_pad, H] compacted valid rows
  char* G;             // [rows_pad, Vb] this block's softmax-gradient slab
  const float* lse2;   // [rows_pad] lse * log2(e)
  const float* rs;     // [rows_pad] per-row gradient factors (reduction "none") or NULL
  const int* tgt;      // [n]
  float* dx32;         // [rows_pad, H]: the FP32 dX sum (vocabulary part 0)
  float* dx32p;        // parts 1 .. dx_split - 1, [rows_pad, H] each, dx_stride
  int64_t dx_stride;   //   floats apart
  int dx_split;        // dX tiles per (token tile, hidden tile): the block's
                       // vocabulary range cut into this many parts; 0: the
                       // count is ctr->dx_parts and the parts lie TTn * 256
                       // rows apart (chunked mode, set per chunk on the device)
  char* dW;            // [V, H] output (grad dtype)
  const Counters* ctr;
  int H, V, rows_pad, Vb;
  int v0, vb;          // block start and width
  int TT, HT, VTb;     // token tiles (bound), hidden tiles, block vocab tiles
  int dw_f32;          // dW written as fp32 (else bf16)
  int dw_acc;          // dW tiles add to dW (else overwrite it)
  const float* oh;     // [rows, H] one-hot sums (see k_oh_*) or NULL: dW tiles
  const int* oh_map;   //   then take off, for each column v, the part of the
  const char* ohx;     //   rows with target v (oh_map[v]: -1 none, k >= 0 the
                       //   one row k of ohx, the compacted rows with factors
                       //   rs; -2 - p row p of oh)
};

// G = c * 2^(z*log2e - lse2) for one tile, stored as G[token][vocab].
// kMasked: tile rows with (32i + 8g + q) >= vlim_lane lie past the vocabulary
// end and token columns >= nlim are padding; both become 0.
// l2[j], cs[j]: lse2 and gradient factor c (times the row's factor under
// reduction "none") of the lane's token column j, loaded before the K loop.
// bf16: through LDS (store_quarter_bf16); fp32: direct 16-byte stores.
template <class E, bool kMasked>
__device__ __forceinline__ void g_store(const BwdArgs& a, const f32x16 (&acc)[4][4],
                                        const float (&l2)[4], const float (&cs)[4], int vt,
                                        int tau, int wm, int wn, int lane, int vlim_lane,
                                        int nlim, lds_t* smem) {
  const rsrc_t gr = make_rsrc(a.G, (int64_t)a.rows_pad * a.Vb * E::kBytes);
  auto val = [&](int i, int j, int r) {
    const float v = cs[j] * __builtin_amdgcn_exp2f(fmaf(acc[i][j][r], kLog2e, -l2[j]));
    const bool ok = !kMasked || (acc_col(wn, j, lane) < nlim &&
                                 32 * i + 8 * (r >> 2) + (r & 3) < vlim_lane);
    return ok ? v : 0.f;
  };
  if constexpr (E::kBytes == 2) {
    const int wave = threadIdx.x >> 6;
    const int tok0 = tau * kTile + wn * 128, voc0 = vt * kTile + wm * 128;
    store_quarter_bf16(smem + wave * 32768, lane, val, [&](int o, int x0, i32x4 v) {
      __builtin_amdgcn_raw_buffer_store_b128(v, gr, ((tok0 + o) * a.Vb + voc0 + x0) * 2, 0, 0);
    });
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = tau * kTile + acc_col(wn, j, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row0 = acc_row(wm, i, 4 * g, lane);   // 4 consecutive rows
          const f32x4 fv = {val(i, j, 4 * g), val(i, j, 4 * g + 1), val(i, j, 4 * g + 2),
                            val(i, j, 4 * g + 3)};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, fv), gr,
                                                 (tok * a.Vb + vt * kTile + row0) * 4, 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// G tile (vocabulary tile vt of the block x token tile tau): the logits are
// recomputed (A = W rows, B = Xc rows, K = H) and turned into G on the way
// out; zero outside the vocabulary and on padding rows.
template <class E>
__device__ __forceinline__ void g_tile(const BwdArgs& a, int b, lds_t* smem) {
  const int n = a.ctr->n;
  const int TTn = (n + kTile - 1) / kTile;
  const int item = live_item(b, a.VTb * TTn);
  if (item < 0) return;
  int vt, tau;
  grouped(item, a.VTb, TTn, vt, tau);
  const float c = a.ctr->c;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ldb = a.H * E::kBytes;
  const int steps = (ldb + kRowBytes - 1) / kRowBytes;
  const int vbase = a.v0 + vt * kTile;

  Opnd A, B;
  A.base = a.W + (int64_t)vbase * ldb;
  A.bytes = (int64_t)(a.V - vbase) * ldb;
  A.ldb = ldb;
  A.kbytes = ldb;
  B.base = a.Xc + (int64_t)tau * kTile * ldb;
  B.bytes = (int64_t)(a.rows_pad - tau * kTile) * ldb;
  B.ldb = ldb;
  B.kbytes = ldb;
  // the rows' lse and gradient factors, fetched now so the epilogue does not
  // wait on them
  float l2[4], cs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = tau * kTile + acc_col(wn, j, lane);
    l2[j] = a.lse2[tok];
    cs[j] = a.rs ? c * a.rs[tok] : c;
  }
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_tile<E, LoadDirect, LoadDirect>(A, B, steps, smem, wm, wn, acc);

  const int vlim = a.V - vbase;
  if (vlim >= kTile && (tau + 1) * kTile <= n)
    g_store<E, false>(a, acc, l2, cs, vt, tau, wm, wn, lane, 0, 0, smem);
  else
    g_store<E, true>(a, acc, l2, cs, vt, tau, wm, wn, lane,
                     vlim - wm * 128 - 4 * (lane >> 5), n - tau * kTile, smem);
}

// dW tile in the output dtype: accumulator rows are hidden indices (4
// consecutive per lane and register group), columns vocabulary entries of the
// block.  kMasked: columns >= mlim lie past the block, rows >= hlim past H
// (H % 8 == 0, so a group of 4 is either inside or outside).  Branch-free:
// a masked lane stores to an offset past the descriptor's range, which the
// hardware drops (the descriptor covers the tile's 256 rows, < 2^31 bytes).
template <bool kMasked, class Fix>
__device__ __forceinline__ void dw_store(const BwdArgs& a, const f32x16 (&acc)[4][4],
                                         int vt, int ht, int wm, int wn, int lane,
                                         int mlim, int hlim, lds_t* smem, const Fix& fix) {
  const int es = a.dw_f32 ? 4 : 2;
  const int64_t row0 = (int64_t)(a.v0 + vt * kTile) * a.H + (int64_t)ht * kTile;
  const int64_t left = ((int64_t)a.V * a.H - row0) * es;
  const int64_t span = (int64_t)kTile * a.H * es;
  const rsrc_t wr = make_rsrc((char*)a.dW + row0 * es, left < span ? left : span);
  const int wave = threadIdx.x >> 6;
  lds_t* region = smem + wave * 32768;
  auto off = [&](int o, int x0) {
    const int m = wn * 128 + o, h = wm * 128 + x0;
    const bool ok = !kMasked || (m < mlim && h < hlim);
    return ok ? (m * a.H + h) * es : (int)0x80000000u;
  };
  auto store_f32 = [&](int o, int x0, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), wr, off(o, x0), 0, 0);
  };
  auto store_bf16 = [&](int o, int x0, f32x4 v) {
    i32x2 pk;
    pk[0] = pack_bf16(v[0], v[1]);
    pk[1] = pack_bf16(v[2], v[3]);
    __builtin_amdgcn_raw_buffer_store_b64(pk, wr, off(o, x0), 0, 0);
  };
  if (a.dw_acc) {
    // dW += tile (chunked mode): rows of 4-value groups through LDS, the sum
    // formed in fp32 and rounded once per call
    if (a.dw_f32) {
      rmw_quarter_f32(
          region, lane, acc,
          [&](int o, int x0) { return __builtin_bit_cast(f32x4, bload128(wr, off(o, x0))); },
          store_f32, fix);
    } else {
      rmw_quarter_f32(
          region, lane, acc,
          [&](int o, int x0) {
            const i32x2 u = __builtin_amdgcn_raw_buffer_load_b64(wr, off(o, x0), 0, 0);
            return f32x4{bf2f((uint32_t)u[0] & 0xFFFFu), bf2f((uint32_t)u[0] >> 16),
                         bf2f((uint32_t)u[1] & 0xFFFFu), bf2f((uint32_t)u[1] >> 16)};
          },
          store_bf16, fix);
    }
    return;
  }
  if (fix.any) {
    // one-hot sums to take off: the FP32 rows through LDS, where they are fixed
    if (a.dw_f32) rmw_quarter_f32(region, lane, acc, NoLoad{}, store_f32, fix);
    else rmw_quarter_f32(region, lane, acc, NoLoad{}, store_bf16, fix);
    return;
  }
  if (!a.dw_f32) {
    // bf16 rows through LDS: row o of the quarter is vocabulary entry
    // wn * 128 + o of the tile, inner x its hidden index wm * 128 + x
    store_quarter_bf16(
        region, lane, [&](int i, int j, int r) { return acc[i][j][r]; },
        [&](int o, int x0, i32x4 v) {
          const int m = wn * 128 + o, h = wm * 128 + x0;
          const bool ok = !kMasked || (m < mlim && h < hlim);
          __builtin_amdgcn_raw_buffer_store_b128(v, wr, ok ? (m * a.H + h) * 2 : (int)0x80000000u,
                                                 0, 0);
        });
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int mc = acc_col(wn, j, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int hc = acc_row(wm, i, 4 * g, lane);
        const bool ok = !kMasked || (mc < mlim && hc < hlim);
        const int off = ok ? (mc * a.H + hc) * 4 : (int)0x80000000u;
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                         acc[i][j][4 * g + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), wr, off, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The one-hot part of a dW tile, taken off in FP32 before the tile's one
// rounding: column m (vocabulary entry v = v0 + vt * 256 + m of this call's W)
// loses c_k Xc[k] summed over the rows k with target v: c_k Xc[k] itself for
// a target of one row, the row of the one-hot sums for several.
//
// Only the few columns with a target are touched.  After the K loop each wave
// fetches, for its columns that have one (in column order), the 128 values
// under its hidden rows into a 512-byte slot of its own 8 KiB past the tile's
// stages: all of the wave's loads go out together, one wait per tile.  The
// tile then leaves through the FP32 staging of rmw_quarter_f32, and this
// functor's fix step subtracts each slot from its column's staged row, two
// columns per wave instruction.  Columns past the kOhDataSlots data slots
// (dense targets) fetch their values in the fix step.  The last 512 bytes of
// the region list the map entry of every slot.
constexpr int kOhSlotBytes = 512;
constexpr int kOhDataSlots = 15;
constexpr int kOhWaveBytes = (kOhDataSlots + 1) * kOhSlotBytes;   // 8 KiB
constexpr int kBwdLdsBytes = kLdsBytes + 4 * kOhWaveBytes;         // 160 KiB
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) int lds_int;

// the map lookups, issued before the tile's K loop so that they arrive under
// it: idx[j] = map entry of this lane's column in block j (-1: none)
template <class A>
__device__ __forceinline__ void onehot_lookup(const A& a, int vt, int wn, int lane, int mlim,
                                              int (&idx)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = acc_col(wn, j, lane);
    idx[j] = a.oh != nullptr && m < mlim ? a.oh_map[a.v0 + vt * kTile + m] : -1;
  }
}

template <class E>
struct OneHotDW {
  const float* oh;
  const char* ohx;
  const float* rs;
  float c;
  lds_t* slots;        // this wave's slot region
  unsigned m[4];       // bit c of m[j]: column 32 j + c has a target
  int n0;              // targets among columns 0 .. 63
  int hcol, H;         // hidden index of this lane's 4 values in a slot
  bool any;
  // This lane's 4 values for map entry `e` (!= -1); hidden columns past H
  // are zeros.  A one-row target is scaled as the sums scale it.
  __device__ __forceinline__ f32x4 values(int e) const {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (hcol >= H) return v;
    if (e >= 0) {
      const float sc = rs ? c * rs[e] : c;
      f32x4 x;
      if constexpr (E::kBytes == 2) {
        const i32x2 u = *(const i32x2*)(ohx + ((int64_t)e * H + hcol) * 2);
        x = f32x4{bf2f((uint32_t)u[0] & 0xFFFFu), bf2f((uint32_t)u[0] >> 16),
                  bf2f((uint32_t)u[1] & 0xFFFFu), bf2f((uint32_t)u[1] >> 16)};
      } else {
        x = *(const f32x4*)(ohx + ((int64_t)e * H + hcol) * 4);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = fmaf(sc, x[q], 0.f);
    } else {
      v = *(const f32x4*)(oh + (int64_t)(-2 - e) * H + hcol);   // 64-bit: past 2^31 bytes
    }
    return v;
  }
  // After the K loop's last barrier (`slots_` is the wave's region).
  template <class A>
  __device__ __forceinline__ OneHotDW(const A& a, const int (&idx)[4], int ht, int wm, int lane,
                                      lds_t* slots_)
      : oh(a.oh), ohx(a.ohx), rs(a.rs), slots(slots_),
        hcol(ht * kTile + wm * 128 + 4 * (lane & 31)), H(a.H) {
    const int cl = lane & 31, hi = lane >> 5;
    int slot[4], total = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // lanes 32..63 hold the columns of lanes 0..31
      m[j] = (unsigned)__ballot(idx[j] != -1);
      slot[j] = total + __builtin_popcount(m[j] & ((1u << cl) - 1u));
      total += __builtin_popcount(m[j]);
      if (j == 1) n0 = total;
    }
    any = total > 0;
    if (!any) return;
    c = a.ctr->c;
    // slot -> map entry (LDS operations of one wave complete in order, so the
    // reads below see these writes)
    lds_int* tab = (lds_int*)(slots_ + kOhDataSlots * kOhSlotBytes);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (hi == 0 && idx[j] != -1) tab[slot[j]] = idx[j];
    // lanes 0..31 fill slot 2 q, lanes 32..63 slot 2 q + 1, 16 bytes each
    const int nload = total < kOhDataSlots ? total : kOhDataSlots;
    f32x4 v[(kOhDataSlots + 1) / 2];
#pragma unroll
    for (int q = 0; q < (kOhDataSlots + 1) / 2; ++q) {
      v[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int s = 2 * q + hi;
      if (2 * q < nload && s < nload) v[q] = values(tab[s]);
    }
#pragma unroll
    for (int q = 0; q < (kOhDataSlots + 1) / 2; ++q) {
      const int s = 2 * q + hi;
      if (2 * q < nload && s < nload) *(lds_f32x4*)(slots_ + s * kOhSlotBytes + 16 * cl) = v[q];
    }
  }
  // rmw_quarter_f32's fix step: staged row o of half hf (column 64 hf + o)
  // loses its slot; 16-byte unit u of a staged row sits at (u ^ (o % 32)).
  __device__ __forceinline__ void operator()(int hf, lds_t* region) const {
    if (!any) return;
    const int cl = threadIdx.x & 31, hi = (threadIdx.x >> 5) & 1;
    const lds_int* tab = (const lds_int*)(slots + kOhDataSlots * kOhSlotBytes);
    uint64_t hm = (uint64_t)m[2 * hf] | ((uint64_t)m[2 * hf + 1] << 32);
    int s = hf ? n0 : 0;
    while (hm != 0) {
      const int o0 = __builtin_ctzll(hm);
      hm &= hm - 1;
      const int o1 = hm != 0 ? __builtin_ctzll(hm) : -1;
      if (hm != 0) hm &= hm - 1;
      const int o = hi ? o1 : o0, sl = s + hi;
      s += 2;
      if (o >= 0) {
        const f32x4 p = sl < kOhDataSlots ? *(const lds_f32x4*)(slots + sl * kOhSlotBytes + 16 * cl)
                                          : values(tab[sl]);
        lds_f32x4* r = (lds_f32x4*)(region + o * 512 + ((cl ^ (o & 31)) << 4));
        const f32x4 x = *r;
        *r = f32x4{x[0] - p[0], x[1] - p[1], x[2] - p[2], x[3] - p[3]};
      }
    }
  }
};

// dW[v0 + m, h] = sum_k Xc[k, h] G[k, m] for one (hidden tile, vocabulary
// tile) of the block: A = Xc, B = G, both stored with K (rows) outer; K runs
// over the valid rows rounded up to one step (G and Xc are zero past n).
template <class E>
__device__ __forceinline__ void dw_tile(const BwdArgs& a, int b, lds_t* smem) {
  const int item = live_item(b, a.HT * a.VTb);
  if (item < 0) return;
  int ht, vt;
  grouped(item, a.HT, a.VTb, ht, vt);
  const int n = a.ctr->n;
  if (a.dw_acc && n == 0) return;   // nothing to add
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int es = E::kBytes;
  const int steps = (n + E::kKStep - 1) / E::kKStep;

  Opnd A, B;
  A.base = a.Xc + (int64_t)ht * kTile * es;
  A.bytes = (int64_t)a.rows_pad * a.H * es - (int64_t)ht * kTile * es;
  A.ldb = a.H * es;
  A.kbytes = 0;
  B.base = a.G + (int64_t)vt * kTile * es;
  B.bytes = (int64_t)a.rows_pad * a.Vb * es - (int64_t)vt * kTile * es;
  B.ldb = a.Vb * es;
  B.kbytes = 0;
  const int mlim = a.vb - vt * kTile, hlim = a.H - ht * kTile;
  int ohidx[4];
  onehot_lookup(a, vt, wn, lane, mlim, ohidx);
  f32x16 acc[4][4];
  zero_acc(acc);
  // K runs over the rows: past 2^31 bytes of an operand (very many rows) the
  // loaders rebase their descriptor per step
  const int64_t reach = (int64_t)steps * E::kKStep * (A.ldb > B.ldb ? A.ldb : B.ldb);
  if (reach <= 0x7FFFFFFF)
    gemm_tile<E, LoadMN<E>, LoadMN<E>>(A, B, steps, smem, wm, wn, acc);
  else
    gemm_tile<E, LoadMN<E, true>, LoadMN<E, true>>(A, B, steps, smem, wm, wn, acc);

  const OneHotDW<E> fix(a, ohidx, ht, wm, lane, smem + kLdsBytes + wave * kOhWaveBytes);
  if (mlim >= kTile && hlim >= kTile)
    dw_store<false>(a, acc, vt, ht, wm, wn, lane, 0, 0, smem, fix);
  else dw_store<true>(a, acc, vt, ht, wm, wn, lane, mlim, hlim, smem, fix);
}

// dX32 += tile, read-modify-write: each (token tile, hidden tile) belongs to
// one workgroup of a launch, and launches are ordered on the stream.
// Accumulator rows are hidden indices, columns tokens; the quarter goes
// through LDS (rmw_quarter_f32) so that each token row is read and written in
// 512-byte runs.  Token columns >= nlim (padding) and hidden rows >= hlim are
// skipped: their offset lies past the tile's rows (256 * H * 4 < 2^31), so
// the load returns zeros and the store is dropped.
template <bool kMasked>
__device__ __forceinline__ void dx_add(const BwdArgs& a, const f32x16 (&acc)[4][4],
                                       float* sum, int tau, int ht, int wm, int wn, int lane,
                                       int nlim, int hlim, lds_t* smem) {
  // sum: the part's [rows, H] FP32 array.  The descriptor starts at the token
  // tile's first row (64-bit base), so the offsets stay below 256 * H * 4
  // bytes whatever the row count
  float* base = sum + (int64_t)tau * kTile * a.H;
  const rsrc_t xr = make_rsrc(base, (int64_t)kTile * a.H * 4);
  const int wave = threadIdx.x >> 6;
  auto offset = [&](int o, int x0) {
    const int tcol = wn * 128 + o, hc = wm * 128 + x0;
    const bool ok = !kMasked || (tcol < nlim && hc < hlim);
    return ok ? (tcol * a.H + ht * kTile + hc) * 4 : (int)0x80000000u;
  };
  rmw_quarter_f32(
      smem + wave * 32768, lane, acc,
      [&](int o, int x0) { return __builtin_bit_cast(f32x4, bload128(xr, offset(o, x0))); },
      [&](int o, int x0, f32x4 v) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), xr, offset(o, x0),
                                               0, 0);
      });
}

// dX32_part[k, h] += sum_m W[v0 + m, h] G[k, m] for one (part, hidden tile,
// token tile), m over part `part` of the block's vocabulary range (parts of
// a multiple of 64 columns; the last may be shorter): A = W (K = vocabulary
// rows outer), B = G rows (K contiguous).  G reads past the part's last
// column are zero (kbytes), so the W rows a last partial step reaches add
// nothing.  Each part has its own FP32 accumulator, so the parts of one tile
// run in the same launch without sharing memory, and the final sum over the
// parts is in fixed order (k_dx_final).
template <class E>
__device__ __forceinline__ void dx_tile(const BwdArgs& a, int b, lds_t* smem) {
  const int n = a.ctr->n;
  const int TTn = (n + kTile - 1) / kTile;
  const int S = a.dx_split > 0 ? a.dx_split : a.ctr->dx_parts;
  const int64_t pstride = a.dx_split > 0 ? a.dx_stride : (int64_t)TTn * kTile * a.H;
  const int per_part = a.HT * TTn;
  const int item = live_item(b, S * per_part);
  if (item < 0) return;
  const int part = item / per_part;
  int ht, tau;
  grouped(item - part * per_part, a.HT, TTn, ht, tau);
  const int pw = (((a.vb + S - 1) / S) + 63) & ~63;
  const int m0 = part * pw;
  if (m0 >= a.vb) return;
  const int len = a.vb - m0 < pw ? a.vb - m0 : pw;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int es = E::kBytes;
  const int steps = (len + E::kKStep - 1) / E::kKStep;

  Opnd A, B;
  const int64_t aoff = ((int64_t)(a.v0 + m0) * a.H + (int64_t)ht * kTile) * es;
  A.base = a.W + aoff;
  A.bytes = (int64_t)a.V * a.H * es - aoff;
  A.ldb = a.H * es;
  A.kbytes = 0;
  const int64_t boff = ((int64_t)tau * kTile * a.Vb + m0) * es;
  B.base = a.G + boff;
  B.bytes = (int64_t)a.rows_pad * a.Vb * es - boff;
  B.ldb = a.Vb * es;
  B.kbytes = len * es;
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_tile<E, LoadMN<E>, LoadDirect>(A, B, steps, smem, wm, wn, acc);

  float* const sum = part == 0 ? a.dx32 : a.dx32p + (part - 1) * pstride;
  const int nlim = n - tau * kTile, hlim = a.H - ht * kTile;
  if (nlim >= kTile && hlim >= kTile)
    dx_add<false>(a, acc, sum, tau, ht, wm, wn, lane, 0, 0, smem);
  else dx_add<true>(a, acc, sum, tau, ht, wm, wn, lane, nlim, hlim, smem);
}

// One backward launch: nb_dx dX tiles and nb_dw dW tiles of block `cur`,
// then nb_g G tiles of block `nxt` (each count a multiple of 8, so every
// kind is spread over the XCDs on its own).  Workgroups start roughly in
// index order, so the kind with the longer K loop goes first (dw_first: the
// dW tiles, whose K runs over the rows, before the dX tiles, whose K runs
// over the block), and the shorter tiles fill the launch's last wave.
template <class E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_bwd(BwdArgs cur, BwdArgs nxt, int nb_dx, int nb_dw, int nb_g, int dw_first) {
  extern __shared__ __attribute__((aligned(16))) char smem_[];
  lds_t* smem = (lds_t*)smem_;
  int b = blockIdx.x;
  const int n1 = dw_first ? nb_dw : nb_dx, n2 = dw_first ? nb_dx : nb_dw;
  if (b < n1 + n2) {
    const bool dw = dw_first ? b < n1 : b >= n1;
    const int i = b < n1 ? b : b - n1;
    if (dw) dw_tile<E>(cur, i, smem);
    else dx_tile<E>(cur, i, smem);
    return;
  }
  b -= n1 + n2;
  if (b < nb_g) g_tile<E>(nxt, b, smem);
}

// ---------------------------------------------------------------------------
// Chunked mode: loss, lse, dX and dW in one call, over chunks of C compacted
// rows, with the chunk's softmax over the whole vocabulary held in a [C, Vp]
// slab (the pages' row-chunk recipe: three contractions instead of four,
// memory proportional to the chunk).  The slab keeps e = 2^(z log2e - R_k)
// against a per-row reference R_k, so the gradient G = f_k e needs no pass
// over the slab: f_k = c_k 2^(R_k - lse2_k) goes into the FP32 dX sums at the
// end and into a scaled copy of the chunk's rows for the dW tiles.  R_k is
// the row's target logit (known before the logits; the target's own entry is
// then 1 up to the two FP32 sums' rounding, so G at the target keeps its FP32
// precision), unless the row's largest z log2e lies more than kRefSpan above
// it (a target more than 44 nats below the row's best): such a row is stored
// again against its max by a second pass, so every stored row's largest
// entry lies in [1, 2^64] (no overflow, and what underflows is negligible
// next to it).  Per chunk:
//   k_chunk_z (pass 0)  logits tiles of the chunk's rows; each (row, 128-wide
//                       half of a vocabulary tile) keeps its max M (log2
//                       units) and s = sum 2^(z log2e - M); the slab gets e
//   k_chunk_lse         the rows' lse from the partials, row losses, f_k, the
//                       rows' flags for the second pass, the chunk's rows
//                       scaled by f_k (Xs), the chunk's counters
//   k_chunk_z (pass 1)  the flagged rows' slab rows against their max (token
//                       tiles without a flagged row exit at once)
//   k_bwd               dX and dW tiles per vocabulary block of the slab (dW
//                       added to the previous chunks' sum)
// ---------------------------------------------------------------------------
constexpr float kRefSpan = 64.f;
constexpr int kChunkZLdsBytes = kLdsBytes + 2 * kTile * 4;   // + the tokens' references, flags
struct ChunkArgs {
  const char* W;        // [V, H]
  const char* Xc;       // the chunk's first compacted row
  char* E;              // [C, Vp] slab
  float2* part;         // [C][2 VT] (M, s)
  const Counters* ctr;  // whole-call counters (n, status, c)
  Counters* cctr;       // this chunk's counters (n = rows in the chunk)
  const float* zt;      // [rows_pad] target logits (compacted rows)
  const int* tgt;       // [rows_pad] targets (compacted rows)
  const float* rs;      // [rows_pad] per-row gradient factors (reduction "none") or NULL
  float* lse_c;         // [rows_pad] lse per compacted row
  float* lse2;          // [rows_pad] lse * log2(e)
  float* rloss;         // [rows_pad] row losses lse - z_target
  float* fk;            // [rows_pad] G = fk * e per row
  float* mrow;          // [rows_pad] the row's max of z log2e
  int* redo;            // [rows_pad] 1: the row is stored against its max
  int* redo_t;          // [C / 256] some row of the chunk's token tile is
  char* Xs;             // [C, H] the chunk's rows times fk (the dW operand)
  float* dx32p;         // the dX tiles' extra vocabulary parts, part_tiles * 256 rows
  int H, V, Vp, C, row0, VT, TTc;
  int HT, dx_target, part_tiles;   // the chunk's dX part count (dx_parts_for)
};

__device__ __forceinline__ int chunk_rows(const ChunkArgs& a) {
  const int r = a.ctr->n - a.row0;
  return r < 0 ? 0 : (r < a.C ? r : a.C);
}

// Epilogue of a logits tile of the chunked mode: per (token, 128-row half of
// the tile) the max M of z log2e and s = sum 2^(z log2e - M) (pass 0), and
// e = 2^(z log2e - M) 2^(M - R) into the slab, R the token's reference
// (token rows past the chunk's rows store zeros; pass 1 stores the flagged
// tokens only).  kMasked: vocabulary rows 32i + 8g + q >= vlim (the lane's
// offset already in vlim) lie past V and count as absent; full tiles skip
// the test.
template <class E, int kPass, bool kMasked>
__device__ __forceinline__ void z_store(const ChunkArgs& a, const f32x16 (&acc)[4][4], int vt,
                                        int tau, int wm, int wn, int lane, int vlim,
                                        lds_t* smem) {
  const int nc = chunk_rows(a);
  // the tokens' references and (second pass) flags, staged in LDS by z_tile
  typedef const __attribute__((address_space(3))) float lds_cfloat;
  lds_cfloat* zref = (lds_cfloat*)(smem + kLdsBytes);
  lds_cint* zflag = (lds_cint*)(smem + kLdsBytes + kTile * 4);
  float ref[4];
  unsigned keep[4];   // bit c: token 32 j + c of the wave is stored
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ref[j] = zref[acc_col(wn, j, lane)];
    keep[j] = kPass == 0 ? ~0u : (unsigned)__ballot(zflag[acc_col(wn, j, lane)] != 0);
  }
  // lanes l and l ^ 32 hold the two halves of the 64 rows a wave keeps per
  // token column; each block j's max is taken right before its values
  float m2[4], sum[4], sc[4];
  auto begin = [&](int j) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!kMasked || 32 * i + 8 * (r >> 2) + (r & 3) < vlim) mx = fmaxf(mx, acc[i][j][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    m2[j] = mx == -INFINITY ? 0.f : mx * kLog2e;
    sum[j] = 0.f;
    const bool live = tau * kTile + acc_col(wn, j, lane) < nc;
    sc[j] = live ? __builtin_amdgcn_exp2f(m2[j] - ref[j]) : 0.f;
  };
  auto val = [&](int i, int j, int r) {
    const float e = __builtin_amdgcn_exp2f(fmaf(acc[i][j][r], kLog2e, -m2[j]));
    const float v = (!kMasked || 32 * i + 8 * (r >> 2) + (r & 3) < vlim) ? e : 0.f;
    sum[j] += v;
    return v * sc[j];
  };
  // the descriptor starts at the token tile's first slab row (64-bit base), so
  // the offsets stay below 256 * Vp * 4 bytes whatever the chunk's row count
  const rsrc_t er = make_rsrc(a.E + (int64_t)tau * kTile * a.Vp * E::kBytes,
                              (int64_t)kTile * a.Vp * E::kBytes);
  const int wave = threadIdx.x >> 6;
  if constexpr (E::kBytes == 2) {
    const int tok0 = wn * 128, voc0 = vt * kTile + wm * 128;   // tok0: within the tile
    store_quarter_bf16(
        smem + wave * 32768, lane, val,
        [&](int o, int x0, i32x4 v) {
          // row o of the quarter is token tok0 + o (= column 32 j + c of the wave)
          const bool st = (keep[o >> 5] >> (o & 31)) & 1;
          __builtin_amdgcn_raw_buffer_store_b128(
              v, er, st ? ((tok0 + o) * a.Vp + voc0 + x0) * 2 : (int)0x80000000u, 0, 0);
        },
        begin);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      begin(j);
      const int tok = acc_col(wn, j, lane);   // within the tile
      const bool st = (keep[j] >> (lane & 31)) & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row0 = acc_row(wm, i, 4 * g, lane);
          const f32x4 fv = {val(i, j, 4 * g), val(i, j, 4 * g + 1), val(i, j, 4 * g + 2),
                            val(i, j, 4 * g + 3)};
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(i32x4, fv), er,
              st ? (tok * a.Vp + vt * kTile + row0) * 4 : (int)0x80000000u, 0, 0);
        }
    }
  }
  if constexpr (kPass == 1) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float s2 = sum[j] + __shfl_xor(sum[j], 32);
    if (lane < 32)
      a.part[(int64_t)(tau * kTile + acc_col(wn, j, lane)) * (2 * a.VT) + 2 * vt + wm] =
          make_float2(m2[j], s2);
  }
}

// Logits tile (vocabulary tile vt x token tile tau of the chunk).
template <class E, int kPass>
__device__ __forceinline__ void z_tile(const ChunkArgs& a, int b, lds_t* smem) {
  // pass 0 clears the second pass's token-tile flags (k_chunk_lse sets them)
  if (kPass == 0 && b == 0)
    for (int t = threadIdx.x; t < a.TTc; t += kThreads) a.redo_t[t] = 0;
  const int TTn = (chunk_rows(a) + kTile - 1) / kTile;
  const int item = live_item(b, a.VT * TTn);
  if (item < 0) return;
  int vt, tau;
  grouped(item, a.VT, TTn, vt, tau);
  if (kPass == 1 && !a.redo_t[tau]) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ldb = a.H * E::kBytes;
  const int steps = (ldb + kRowBytes - 1) / kRowBytes;
  Opnd A, B;
  A.base = a.W + (int64_t)vt * kTile * ldb;
  A.bytes = (int64_t)(a.V - vt * kTile) * ldb;
  A.ldb = ldb;
  A.kbytes = ldb;
  B.base = a.Xc + (int64_t)tau * kTile * ldb;
  B.bytes = (int64_t)(a.C - tau * kTile) * ldb;
  B.ldb = ldb;
  B.kbytes = ldb;
  // thread t fetches token t's reference now and stages it after the K loop:
  // the target logit (pass 0) or the row's max (pass 1), log2 units
  const int nc = chunk_rows(a);
  const int tk = tau * kTile + (int)threadIdx.x;
  const float zr = tk >= nc ? 0.f : (kPass ? a.mrow[a.row0 + tk] : a.zt[a.row0 + tk] * kLog2e);
  const int zf = kPass && tk < nc ? a.redo[a.row0 + tk] : 0;
  f32x16 acc[4][4];
  zero_acc(acc);
  gemm_tile<E, LoadDirect, LoadDirect>(A, B, steps, smem, wm, wn, acc);
  ((__attribute__((address_space(3))) float*)(smem + kLdsBytes))[threadIdx.x] = zr;
  if (kPass) ((__attribute__((address_space(3))) int*)(smem + kLdsBytes + kTile * 4))[threadIdx.x] = zf;
  __syncthreads();

  const int vlim = a.V - vt * kTile;
  if (vlim >= kTile) z_store<E, kPass, false>(a, acc, vt, tau, wm, wn, lane, 0, smem);
  else
    z_store<E, kPass, true>(a, acc, vt, tau, wm, wn, lane, vlim - wm * 128 - 4 * (lane >> 5),
                            smem);
}

template <class E, int kPass>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_chunk_z(ChunkArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem_[];
  z_tile<E, kPass>(a, blockIdx.x, (lds_t*)smem_);
}

// One wave per row of the chunk: lse from the row's 2 VT partials (each lane
// merges every 64th in order, then a fixed butterfly across lanes), the row
// loss lse - z_target; thread 0 of block 0 also writes the chunk's counters.
__device__ __forceinline__ void lse_pair_merge(float& M, float& S, float m2, float s2) {
  const float Mn = fmaxf(M, m2);
  if (Mn == -INFINITY) return;
  S = S * exp2f(M - Mn) + s2 * exp2f(m2 - Mn);
  M = Mn;
}

template <class E>
__global__ __launch_bounds__(256) void k_chunk_lse(ChunkArgs a) {
  const int lane = threadIdx.x & 63;
  const int kl = blockIdx.x * 4 + (threadIdx.x >> 6), k = a.row0 + kl;
  const int nc = chunk_rows(a);
  const int ttc = (nc + kTile - 1) / kTile;
  const int parts = dx_parts_for(a.HT, ttc, a.dx_target, a.part_tiles);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    Counters c = *a.ctr;
    c.n = nc;
    c.fwd_p = 0;
    c.dx_parts = parts;
    *a.cctr = c;
  }
  if (kl >= a.C) return;
  // the row's FP32 sums of the extra dX parts start at zero (parts lie
  // ttc * 256 rows apart; the dX tiles and k_dx_fold touch rows < nc only)
  if (kl < nc)
    for (int q = 1; q < parts; ++q) {
      i32x4* d = (i32x4*)(a.dx32p + ((int64_t)(q - 1) * ttc * kTile + kl) * a.H);
      for (int c = lane; c < a.H / 4; c += 64) d[c] = i32x4{0, 0, 0, 0};
    }
  const int pieces = a.H * E::kBytes / 16;
  i32x4* xs = (i32x4*)(a.Xs + (int64_t)kl * a.H * E::kBytes);
  if (kl >= nc) {
    // the dW tiles' K steps read up to the last token tile's end: zeros there
    if (kl < (nc + kTile - 1) / kTile * kTile)
      for (int c = lane; c < pieces; c += 64) xs[c] = i32x4{0, 0, 0, 0};
    return;
  }
  const float2* pr = a.part + (int64_t)kl * (2 * a.VT);
  float M = -INFINITY, S = 0.f;
  for (int h = lane; h < 2 * a.VT; h += 64) {
    const float2 v = pr[h];
    if (v.y != 0.f) lse_pair_merge(M, S, v.x, v.y);   // empty half-tiles carry s = 0
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float m2 = __shfl_xor(M, d), s2 = __shfl_xor(S, d);
    lse_pair_merge(M, S, m2, s2);
  }
  // the reference of the stored e: the target logit, or the row's max when
  // that lies more than kRefSpan above it (the row goes to the second pass)
  const float l2 = M + log2f(S);
  const float zt2 = a.zt[k] * kLog2e;
  const bool far = !(M - zt2 <= kRefSpan);
  const float ck = a.rs ? a.ctr->c * a.rs[k] : a.ctr->c;
  const float f = ck * exp2f((far ? M : zt2) - l2);
  if (lane == 0) {
    a.lse2[k] = l2;
    a.lse_c[k] = l2 * kLn2;
    a.rloss[k] = l2 * kLn2 - a.zt[k];
    a.fk[k] = f;
    a.mrow[k] = M;
    a.redo[k] = far ? 1 : 0;
    if (far) a.redo_t[kl / kTile] = 1;
  }
  // the row scaled by f for the dW tiles (one rounding to the input dtype)
  const i32x4* xc = (const i32x4*)(a.Xc + (int64_t)kl * a.H * E::kBytes);
  for (int c = lane; c < pieces; c += 64) {
    i32x4 u = xc[c];
    if constexpr (E::kBytes == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        u[q] = pack_bf16(bf2f((uint32_t)u[q] & 0xFFFFu) * f, bf2f((uint32_t)u[q] >> 16) * f);
    } else {
      f32x4 g = __builtin_bit_cast(f32x4, u);
#pragma unroll
      for (int q = 0; q < 4; ++q) g[q] *= f;
      u = __builtin_bit_cast(i32x4, g);
    }
    xs[c] = u;
  }
}

// Fixed-order sums of 256 row losses (compacted rows; rows >= n add 0).
__global__ __launch_bounds__(256) void k_block_sums(const float* __restrict__ rloss,
                                                    const Counters* __restrict__ ctr,
                                                    float* __restrict__ bsum) {
  __shared__ float red[256];
  const int k = blockIdx.x * 256 + threadIdx.x;
  red[threadIdx.x] = k < ctr->n ? rloss[k] : 0.f;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) bsum[blockIdx.x] = red[0];
}

// lse of every original row (0 for ignored rows) after the chunks.
__global__ __launch_bounds__(256) void k_lse_out(const float* __restrict__ lse_c,
                                                 const int* __restrict__ rowpos, int N,
                                                 float* __restrict__ lse_out,
                                                 const float* __restrict__ rloss,
                                                 const Counters* __restrict__ ctr,
                                                 float* __restrict__ rloss_out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const int k = rowpos[i];
  lse_out[i] = k >= 0 ? lse_c[k] : 0.f;
  // per-row losses (reduction "none"): 0 on ignored rows, NaN after a bad label
  if (rloss_out) rloss_out[i] = ctr->status ? __builtin_nanf("") : (k >= 0 ? rloss[k] : 0.f);
}

// out = s * in (s a device scalar; out may be in itself): gradients computed
// with grad_scale 1, rescaled by the upstream gradient.  Grid-stride, 16
// bytes per thread step.
__global__ __launch_bounds__(256) void k_scale_grads(const char* src, char* dst,
                                                     int64_t chunks, int f32,
                                                     const float* __restrict__ s) {
  const float k = *s;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < chunks; i += (int64_t)gridDim.x * 256) {
    i32x4 u = ((const i32x4*)src)[i];
    if (f32) {
      f32x4 g = __builtin_bit_cast(f32x4, u);
#pragma unroll
      for (int e = 0; e < 4; ++e) g[e] *= k;
      u = __builtin_bit_cast(i32x4, g);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        u[e] = pack_bf16(bf2f((uint32_t)u[e] & 0xFFFFu) * k, bf2f((uint32_t)u[e] >> 16) * k);
    }
    ((i32x4*)dst)[i] = u;
  }
}

// dst = round(s * src (+ dst)) from FP32 gradient sums, 4 values per thread
// step: one rounding to bf16 (or none for fp32), the caller's values added in
// FP32 first when `accumulate`.  s = *scale, or 1 with no scale.
__global__ __launch_bounds__(256) void k_convert_grads(const float* __restrict__ src,
                                                       char* __restrict__ dst, int64_t chunks,
                                                       int dst_f32, const float* __restrict__ scale,
                                                       int accumulate) {
  const float k = scale ? *scale : 1.0f;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < chunks; i += (int64_t)gridDim.x * 256) {
    f32x4 v = *(const f32x4*)(src + 4 * i);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= k;
    if (dst_f32) {
      f32x4* d = (f32x4*)dst + i;
      if (accumulate) {
        const f32x4 o = *d;
        v = f32x4{v[0] + o[0], v[1] + o[1], v[2] + o[2], v[3] + o[3]};
      }
      *d = v;
    } else {
      i32x2* d = (i32x2*)dst + i;
      if (accumulate) {
        const i32x2 o = *d;
        v = f32x4{v[0] + bf2f((uint32_t)o[0] & 0xFFFFu), v[1] + bf2f((uint32_t)o[0] >> 16),
                  v[2] + bf2f((uint32_t)o[1] & 0xFFFFu), v[3] + bf2f((uint32_t)o[1] >> 16)};
      }
      i32x2 pk;
      pk[0] = pack_bf16(v[0], v[1]);
      pk[1] = pack_bf16(v[2], v[3]);
      *d = pk;
    }
  }
}

// Vocabulary shards: row i's lse is the log-sum-exp of the shards' lse and its
// target logit the sum of the shards' (exactly one holds it); one thread per
// original row, fixed-order block sums of the row losses.
__global__ __launch_bounds__(256) void k_shard_merge(
    const float* __restrict__ lse_g, const float* __restrict__ zt_g, int shards, int N,
    const int* __restrict__ rowpos, const Counters* __restrict__ ctr,
    float* __restrict__ lse_out, float* __restrict__ blocksum, float* __restrict__ rloss_out) {
  __shared__ float red[256];
  const int i = blockIdx.x * 256 + threadIdx.x;
  float li = 0.f;
  if (i < N) {
    float lse = 0.f;
    if (rowpos[i] >= 0) {
      float M = -INFINITY, z = 0.f;
      for (int g = 0; g < shards; ++g) M = fmaxf(M, lse_g[(int64_t)g * N + i]);
      float S = 0.f;
      for (int g = 0; g < shards; ++g) {
        S += expf(lse_g[(int64_t)g * N + i] - M);
        z += zt_g[(int64_t)g * N + i];
      }
      lse = M + logf(S);
      li = lse - z;
    }
    lse_out[i] = lse;
    if (rloss_out) rloss_out[i] = ctr->status ? __builtin_nanf("") : li;
  }
  red[threadIdx.x] = li;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) blocksum[blockIdx.x] = red[0];
}

// dX = round(f_k dX32 - c_k W[y_k]) scattered to the original rows (0 for
// ignored rows): the softmax part summed in FP32 over the vocabulary (and
// over its vocabulary parts, in part order), times the row's factor f_k of
// the chunked mode (1 when fk is NULL), and the one-hot part, added in FP32
// before the one rounding.  Targets outside [0, V_local) (another vocabulary
// shard's) have no one-hot term here.  One wave per row.
template <class E>
__global__ __launch_bounds__(256) void k_dx_final(
    const float* __restrict__ dx32, int dx_split, int64_t dx_stride,
    const int* __restrict__ rowpos, int N, int H, char* __restrict__ dX, int out_f32,
    const char* __restrict__ W, const int* __restrict__ tgt, int V_local,
    const Counters* __restrict__ ctr, const float* __restrict__ rs,
    const float* __restrict__ fk) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= N) return;
  const int k = rowpos[i];
  const int y = k >= 0 ? tgt[k] : -1;
  const bool hot = y >= 0 && y < V_local;
  const float ck = k >= 0 ? (rs ? ctr->c * rs[k] : ctr->c) : 0.f;
  const int groups = H >> 2;  // 4 values per lane step
  for (int g = lane; g < groups; g += 64) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (k >= 0) {
      v = *(const f32x4*)(dx32 + (int64_t)k * H + 4 * g);
      for (int sp = 1; sp < dx_split; ++sp) {
        const f32x4 u = *(const f32x4*)(dx32 + sp * dx_stride + (int64_t)k * H + 4 * g);
        v = f32x4{v[0] + u[0], v[1] + u[1], v[2] + u[2], v[3] + u[3]};
      }
      if (fk) {
        const float f = fk[k];
        v = f32x4{v[0] * f, v[1] * f, v[2] * f, v[3] * f};
      }
      if (hot) {
        f32x4 wv;
        if constexpr (E::kBytes == 2) {
          const i32x2 u = *(const i32x2*)(W + ((int64_t)y * H + 4 * g) * 2);
          wv = f32x4{bf2f((uint32_t)u[0] & 0xFFFFu), bf2f((uint32_t)u[0] >> 16),
                     bf2f((uint32_t)u[1] & 0xFFFFu), bf2f((uint32_t)u[1] >> 16)};
        } else {
          wv = *(const f32x4*)(W + ((int64_t)y * H + 4 * g) * 4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(-ck, wv[e], v[e]);
      }
    }
    if (out_f32) {
      *(f32x4*)((float*)dX + (int64_t)i * H + 4 * g) = v;
    } else {
      i32x2 pk;
      pk[0] = pack_bf16(v[0], v[1]);
      pk[1] = pack_bf16(v[2], v[3]);
      *(i32x2*)((uint16_t*)dX + (int64_t)i * H + 4 * g) = pk;
    }
  }
}

// ---------------------------------------------------------------------------
// One-hot sums for dW: OH_v = sum over valid rows k with y_k = v of c_k Xc[k]
// (FP32), summed in row order.  The compacted rows are sorted by the unique
// 64-bit key (target << 32 | row), so the order of every sum is fixed.  A
// target held by one row needs no sum (the dW tiles scale that row of Xc
// themselves); the runs of several rows are summed position by position, per
// block of kOhBlock sorted positions and then across blocks in order.
// map[v] (v < V_local) afterwards: -1 no row has target v; k >= 0 the one
// row k; -2 - p the sum is row p of OH.
// ---------------------------------------------------------------------------

constexpr uint64_t kNoKey = ~0ull;

__device__ __forceinline__ uint32_t key_target(uint64_t k) { return (uint32_t)(k >> 32); }

// a value every lane holds, kept in scalar registers
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// key of sorted-array position i before sorting: compacted row i when it has
// a target in [0, V_local), else kNoKey (sorts last)
__device__ __forceinline__ uint64_t oh_key(const int* __restrict__ tgt, int n, int V_local,
                                           int i) {
  if (i < n) {
    const int y = tgt[i];
    if (y >= 0 && y < V_local) return ((uint64_t)(uint32_t)y << 32) | (uint32_t)i;
  }
  return kNoKey;
}

// Bitonic compare-exchange of positions i < j = i + stride: ascending where
// bit `s` of i is clear (the stage of sequences of length s).
__device__ __forceinline__ void bitonic_pair(uint64_t& a, uint64_t& b, int i, int s) {
  const bool up = (i & s) == 0;
  if ((a > b) == up) {
    const uint64_t t = a;
    a = b;
    b = t;
  }
}

// Builds the keys and sorts each block of kSortLocal of them (the whole array
// when P is no larger) in LDS: stages 2 .. min(P, kSortLocal).  The
// directions follow the global position (alternating blocks, as the bitonic
// stages past kSortLocal need) or, with `ascending`, the position in the block
// (every block ascending, as k_oh_merge_blocks needs).  256 threads, two
// pairs each per step.
constexpr int kSortLocal = 1024;
__global__ __launch_bounds__(256) void k_oh_sort_local(const int* __restrict__ tgt,
                                                       const Counters* __restrict__ ctr,
                                                       int V_local, int P, int ascending,
                                                       uint64_t* __restrict__ keys) {
  __shared__ uint64_t sk[kSortLocal];
  const int len = P < kSortLocal ? P : kSortLocal;
  const int base = blockIdx.x * kSortLocal;
  const int n = ctr->n;
  for (int t = threadIdx.x; t < len; t += 256) sk[t] = oh_key(tgt, n, V_local, base + t);
  __syncthreads();
  for (int s = 2; s <= len; s <<= 1)
    for (int stride = s >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < len / 2; t += 256) {
        const int i = (t / stride) * 2 * stride + t % stride;
        bitonic_pair(sk[i], sk[i + stride], ascending ? i : base + i, s);
      }
      __syncthreads();
    }
  for (int t = threadIdx.x; t < len; t += 256) keys[base + t] = sk[t];
}

// P <= kMergeMax: the P / kSortLocal ascending blocks merged in one pass.  Every
// workgroup holds all keys in LDS; a key's place is its index in its block
// plus, for every other block, the number of that block's keys below it
// (binary search; the keys are unique).  The kNoKey padding goes after the
// valid keys in block order.  Grid: P / 1024 workgroups of 1024 threads.
constexpr int kMergeMax = 8192;
__device__ __forceinline__ int lower_bound_lds(const uint64_t* b, int len, uint64_t key) {
  int lo = 0;
  for (int step = len >> 1; step > 0; step >>= 1)
    if (b[lo + step - 1] < key) lo += step;
  return lo + (lo < len && b[lo] < key ? 1 : 0);
}
__global__ __launch_bounds__(1024) void k_oh_merge_blocks(const uint64_t* __restrict__ keys,
                                                          int P, uint64_t* __restrict__ out) {
  __shared__ uint64_t sk[kMergeMax];
  const int nb = P / kSortLocal;
  for (int t = threadIdx.x; t < P; t += 1024) sk[t] = keys[t];
  __syncthreads();
  const int i = blockIdx.x * 1024 + threadIdx.x;
  if (i >= P) return;
  const int b = i / kSortLocal, li = i - b * kSortLocal;
  const uint64_t key = sk[i];
  int r = li;
  if (key != kNoKey) {
    for (int bb = 0; bb < nb; ++bb)
      if (bb != b) r += lower_bound_lds(sk + bb * kSortLocal, kSortLocal, key);
  } else {
    // after every valid key, then the padding of the blocks before b
    for (int bb = 0; bb < nb; ++bb) {
      const int valid = lower_bound_lds(sk + bb * kSortLocal, kSortLocal, kNoKey);
      r += bb == b ? 0 : (bb < b ? kSortLocal : valid);
    }
  }
  out[r] = key;
}

// P > kMergeMax: bitonic stages past kSortLocal.  One stride (>= kSortLocal)
// of stage s over the whole array: thread t handles one pair.
__global__ __launch_bounds__(256) void k_bsort_global(uint64_t* __restrict__ keys, int P, int s,
                                                      int stride) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= P / 2) return;
  const int i = (t / stride) * 2 * stride + t % stride;
  uint64_t a = keys[i], b = keys[i + stride];
  bitonic_pair(a, b, i, s);
  keys[i] = a;
  keys[i + stride] = b;
}

// Strides kSortLocal / 2 .. 1 of stage s (> kSortLocal) inside each block of
// kSortLocal keys.
__global__ __launch_bounds__(256) void k_bsort_merge(uint64_t* __restrict__ keys, int s) {
  __shared__ uint64_t sk[kSortLocal];
  const int base = blockIdx.x * kSortLocal;
  for (int t = threadIdx.x; t < kSortLocal; t += 256) sk[t] = keys[base + t];
  __syncthreads();
  for (int stride = kSortLocal / 2; stride > 0; stride >>= 1) {
    for (int t = threadIdx.x; t < kSortLocal / 2; t += 256) {
      const int i = (t / stride) * 2 * stride + t % stride;
      bitonic_pair(sk[i], sk[i + stride], base + i, s);
    }
    __syncthreads();
  }
  for (int t = threadIdx.x; t < kSortLocal; t += 256) keys[base + t] = sk[t];
}

// Per block of kOhBlock sorted positions and hidden chunk of 256 (one thread
// per hidden column): for every piece of a run of several rows inside the
// block, ohp[start] = the sum over the piece's positions of c_k Xc[k], in
// position order, where start is the piece's first position (the block's
// first, or the run's).  Positions of one-row runs are skipped; runs that
// cross blocks are completed by k_oh_final.
constexpr int kOhBlock = 64;   // one wave's lanes: the run masks come from ballots
template <class E>
__global__ __launch_bounds__(256) void k_oh_partial(const uint64_t* __restrict__ keys, int P,
                                                    const char* __restrict__ Xc, int H,
                                                    int rows_pad,
                                                    const Counters* __restrict__ ctr,
                                                    const float* __restrict__ rs,
                                                    float* __restrict__ ohp) {
  // sk[q + 1] = key of block position q; sk[0], sk[kOhBlock + 1] the neighbours
  __shared__ uint64_t sk[kOhBlock + 2];
  __shared__ float sc[kOhBlock];
  __shared__ uint64_t masks[2];   // positions in runs of several rows; piece ends
  const int base = blockIdx.x * kOhBlock;
  if (threadIdx.x < kOhBlock + 2) {
    const int p = base + (int)threadIdx.x - 1;
    sk[threadIdx.x] = p >= 0 && p < P ? keys[p] : kNoKey;
  }
  __syncthreads();
  if (threadIdx.x < kOhBlock) {
    const int q = threadIdx.x;
    const uint64_t key = sk[q + 1];
    const bool valid = key != kNoKey;
    const bool ps = valid && sk[q] != kNoKey && key_target(sk[q]) == key_target(key);
    const bool ns = valid && sk[q + 2] != kNoKey && key_target(sk[q + 2]) == key_target(key);
    const bool m = ps || ns;
    const float c = ctr->c;
    sc[q] = m ? (rs ? c * rs[(uint32_t)key] : c) : 0.f;
    const uint64_t bm = __ballot(m), be = __ballot(m && !ns);
    if (q == 0) {
      masks[0] = bm;
      masks[1] = be;
    }
  }
  __syncthreads();
  const uint64_t mm = uniform64(masks[0]), me = uniform64(masks[1]);
  const int h = blockIdx.y * 256 + threadIdx.x;
  if (mm == 0 || h >= H) return;
  float x[kOhBlock];
#pragma unroll
  for (int q = 0; q < kOhBlock; ++q) {
    x[q] = 0.f;
    const int64_t row = (uint32_t)sk[q + 1];
    if (((mm >> q) & 1) && row < rows_pad) {
      if constexpr (E::kBytes == 2)
        x[q] = bf2f(((const uint16_t*)Xc)[row * H + h]);
      else
        x[q] = ((const float*)Xc)[row * H + h];
    }
  }
  float acc = 0.f;
  int start = 0;
#pragma unroll
  for (int q = 0; q < kOhBlock; ++q) {
    if (!((mm >> q) & 1)) {
      start = q + 1;
      continue;
    }
    acc = fmaf(sc[q], x[q], acc);
    if (q == kOhBlock - 1 || ((me >> q) & 1)) {
      ohp[(int64_t)(base + start) * H + h] = acc;
      acc = 0.f;
      start = q + 1;
    }
  }
}

// map and cross-block runs.  Every run start (the first position, or a
// target different from the previous position's) sets map[target].  The run
// of several rows that holds a block's last position, when it starts inside
// the block, is completed by that block: the partials that the following
// blocks' first positions hold for the same target are added to its own, in
// block order.  Grid: blocks of kOhBlock positions x hidden chunks of 256.
__global__ __launch_bounds__(256) void k_oh_final(const uint64_t* __restrict__ keys, int P,
                                                  int H, int rows_pad, float* __restrict__ ohp,
                                                  int* __restrict__ map) {
  __shared__ int open_at;
  const int base = blockIdx.x * kOhBlock;
  const int t = threadIdx.x;
  const int p = base + t;
  const uint64_t key = t < kOhBlock ? keys[p] : kNoKey;
  const bool prev_same = t < kOhBlock && p > 0 && keys[p - 1] != kNoKey &&
                         key_target(keys[p - 1]) == key_target(key);
  const bool next_same = t < kOhBlock && key != kNoKey && p + 1 < P && keys[p + 1] != kNoKey &&
                         key_target(keys[p + 1]) == key_target(key);
  const bool start = key != kNoKey && !prev_same;
  if (blockIdx.y == 0 && start) map[key_target(key)] = next_same ? -2 - p : (int)(uint32_t)key;
  if (t == 0) open_at = -1;
  __syncthreads();
  const uint64_t klast = keys[base + kOhBlock - 1];
  // the start of the run of several rows that holds the block's last position
  if (start && next_same && key_target(klast) == key_target(key)) open_at = t;
  __syncthreads();
  const int i0 = open_at;
  const int h = blockIdx.y * 256 + t;
  if (i0 < 0 || h >= H) return;
  const uint32_t tg = key_target(klast);
  float sum = ohp[(int64_t)(base + i0) * H + h];
  for (int b = base + kOhBlock; b < rows_pad; b += kOhBlock) {
    const uint64_t k0 = keys[b];
    if (k0 == kNoKey || key_target(k0) != tg) break;
    sum += ohp[(int64_t)b * H + h];
    const uint64_t k1 = keys[b + kOhBlock - 1];
    if (k1 == kNoKey || key_target(k1) != tg) break;
  }
  ohp[(int64_t)(base + i0) * H + h] = sum;
}

// dst[k, :] += sum over p = 0 .. parts - 1 of src_p[k, :] (src_p = src + p *
// stride floats), in that order, for rows k < rows of H floats: folds a row
// chunk's extra vocabulary parts of dX into the main FP32 sum.  The chunk's
// counters give rows (n), parts + 1 (dx_parts) and the stride (the chunk's
// token tiles times 256 rows).  Grid-stride, 4 floats per thread step.
__global__ __launch_bounds__(256) void k_dx_fold(float* __restrict__ dst,
                                                 const float* __restrict__ src,
                                                 const Counters* __restrict__ cctr, int H) {
  const int rows = cctr->n, parts = cctr->dx_parts - 1;
  if (parts <= 0) return;
  const int64_t stride = (int64_t)((rows + kTile - 1) / kTile) * kTile * H;
  const int64_t count4 = (int64_t)rows * H / 4;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < count4;
       i += (int64_t)gridDim.x * 256) {
    f32x4 v = *(const f32x4*)(dst + 4 * i);
    for (int p = 0; p < parts; ++p) {
      const f32x4 u = *(const f32x4*)(src + p * stride + 4 * i);
      v = f32x4{v[0] + u[0], v[1] + u[1], v[2] + u[2], v[3] + u[3]};
    }
    *(f32x4*)(dst + 4 * i) = v;
  }
}

// Zero fill, 16 bytes per thread step (graph-capture safe, unlike a memset).
__global__ __launch_bounds__(256) void k_zero(char* __restrict__ p, int64_t chunks) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < chunks; i += (int64_t)gridDim.x * 256)
    ((i32x4*)p)[i] = i32x4{0, 0, 0, 0};
}

// n == 0 rows (N == 0): loss = 0, n_valid = 0.
__global__ void k_empty(float* loss, int64_t* n_valid, int32_t* status) {
  if (loss) *loss = 0.f;
  if (n_valid) *n_valid = 0;
  if (status) *status = 0;
}

}  // namespace flce
