// flce_api.hip -- host side of the C ABI declared in include/flce.h:
// argument checks, workspace layout and the launch sequence on the caller's
// stream.  Nothing here allocates device memory or synchronises the host.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "flce.h"
#include "flce_kernels.h"

namespace flce {
namespace {

constexpr int64_t kAlign = 256;
#ifndef FLCE_SLAB_MIB
#define FLCE_SLAB_MIB 512
#endif
// backward: both softmax-gradient slabs together hold at most this many bytes
// (unless a single 256-wide vocabulary tile per row already needs more), or
// up to twice as many to bring blocks narrower than kMinVocabBlock closer to
// it: a dX tile's K loop runs over the block, and below 128 steps its fixed
// cost (first loads, the FP32 read-modify-write epilogue) weighs more than
// the larger slabs cost
constexpr int64_t kSlabBudget = (int64_t)FLCE_SLAB_MIB << 20;
#ifndef FLCE_MIN_VB
#define FLCE_MIN_VB 8192
#endif
constexpr int64_t kMinVocabBlock = FLCE_MIN_VB;
constexpr int64_t kMaxI32 = 0x7FFFFFFFll;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }
int64_t pow2_at_least(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}
// per-block counts of the prep kernels: two ints per 1024 rows
int64_t prep_blk_bytes(int64_t N) { return 8 * cdiv(N > 0 ? N : 1, kPrepBlock); }

// Problem geometry shared by the size query and the two calls.
struct Plan {
  int64_t N, rows_pad, H, V, es;
  int64_t TT, VT;           // token tiles (upper bound), vocabulary tiles
  int64_t fwd_items;        // forward work items (range x token tile), at most
  int64_t Vb;               // backward vocabulary block (multiple of 256)
  int64_t dx_split;         // dX tiles per (token tile, hidden tile) and block
  // workspace offsets (bytes)
  int64_t o_ctr, o_idx, o_tgt, o_rowpos, o_xc, o_blk;
  int64_t o_part, o_zt, o_bsum;            // forward region
  int64_t o_lse2, o_rs, o_g, o_dx32;       // backward region
  int64_t P;                               // sort length: rows_pad rounded up to 2^k
  int64_t o_keys, o_oh, o_map;             // one-hot sums for dW (backward)
  int64_t fwd_total;        // bytes the forward alone uses
  int64_t total;
};

// dX tiles in flight per launch that the vocabulary parts aim at
// (dx_parts_for).  The recompute path's launches also carry the G tiles (three
// tile kinds of equal total work, the chunked mode's two), and its token-tile
// count is a bound that the valid rows may not reach, hence the larger target.
// The recompute path fixes the part count on the host from that bound; the
// chunked mode sets it per chunk on the device from the chunk's rows, so the
// short last chunk gets more parts than the full ones.
#ifndef FLCE_DX_TILES
#define FLCE_DX_TILES 256
#endif
// token tiles of extra dX parts kept for a short last chunk (at most)
constexpr int64_t kShortChunkTiles = 16;
#ifndef FLCE_DX_TILES_CHUNKED
#define FLCE_DX_TILES_CHUNKED 176
#endif

int make_plan(int64_t B, int64_t T, int64_t H, int64_t V, int dtype, Plan* p) {
  if (B < 0 || T < 0 || H <= 0 || V <= 0) return FLCE_ERR_SHAPE;
  if (dtype != FLCE_DTYPE_F32 && dtype != FLCE_DTYPE_BF16) return FLCE_ERR_DTYPE;
  if (H % 8 != 0) return FLCE_ERR_ALIGN;
  const int64_t N = B * T;
  if (B > kMaxI32 || T > kMaxI32 || N > (1ll << 24) || H > 65536 || V > kMaxI32 - 512)
    return FLCE_ERR_SHAPE;
  Plan q;
  q.N = N;
  q.H = H;
  q.V = V;
  q.es = dtype == FLCE_DTYPE_BF16 ? 2 : 4;
  q.rows_pad = round_up(N > 0 ? N : 1, kTile);
  q.TT = q.rows_pad / kTile;
  q.VT = cdiv(V, kTile);
  // forward: the split itself is chosen on the device (k_prep_scan), once the
  // number of valid rows is known; this bounds its item count and partials
  q.fwd_items = std::max<int64_t>(2048, q.TT);
  // backward: the vocabulary block is as wide as the slab budget allows for
  // this many rows, whatever V is (and narrow enough for 32-bit offsets)
  // (the dX tiles address a whole block of W rows, and the dW tiles the
  // whole slab, from one descriptor each: both below 2^31 bytes)
  const int64_t per_col = 2 * q.rows_pad * q.es;   // both slabs, one column
  int64_t vb = std::max<int64_t>(kSlabBudget / per_col,
                                 std::min<int64_t>(kMinVocabBlock, 2 * kSlabBudget / per_col));
  vb = std::min<int64_t>({vb, kMaxI32 / (q.rows_pad * q.es), kMaxI32 / (H * q.es)});
  vb = std::max<int64_t>(kTile, vb / kTile * kTile);
  vb = std::min<int64_t>(vb, round_up(V, kTile));
  q.Vb = vb;
  q.dx_split = dx_parts_for((int)cdiv(H, kTile), (int)q.TT, FLCE_DX_TILES, -1);
  // 32-bit offsets inside the kernels
  if (q.rows_pad * q.Vb * q.es > kMaxI32 || (int64_t)kTile * H * q.es * 2 > kMaxI32)
    return FLCE_ERR_SHAPE;

  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = round_up(off + bytes, kAlign);
    return o;
  };
  q.o_ctr = take(sizeof(Counters));
  q.o_idx = take(4 * q.rows_pad);
  q.o_tgt = take(4 * q.rows_pad);
  q.o_rowpos = take(4 * q.rows_pad);
  q.o_xc = take(q.rows_pad * H * q.es);
  q.o_blk = take(prep_blk_bytes(N));
  const int64_t common = off;
  q.o_part = take(8 * kTile * q.fwd_items);
  q.o_zt = take(4 * q.rows_pad);
  q.o_bsum = take(4 * cdiv(q.rows_pad, 256));
  const int64_t fwd_end = off;
  off = common;
  q.o_lse2 = take(4 * q.rows_pad);
  q.o_rs = take(4 * q.rows_pad);
  q.o_g = take(2 * q.rows_pad * q.Vb * q.es);   // two slabs, alternating blocks
  q.o_dx32 = take(4 * q.dx_split * q.rows_pad * H);
  q.P = pow2_at_least(q.rows_pad);
  q.o_keys = take(16 * q.P);
  q.o_oh = take(4 * q.rows_pad * H);
  q.o_map = take(4 * V);
  const int64_t bwd_end = off;
  q.fwd_total = fwd_end;
  q.total = std::max(fwd_end, bwd_end);
  *p = q;
  return FLCE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// The two gradient outputs lie apart from each other and from the bytes of
// the workspace the call uses (dX of nx bytes may be absent: nx = 0).
bool grads_overlap(const void* dX, int64_t nx, const void* dW, int64_t nw, const void* ws,
                   int64_t nws) {
  return (nx > 0 && (overlaps(dX, nx, dW, nw) || overlaps(dX, nx, ws, nws))) ||
         overlaps(dW, nw, ws, nws);
}

// The GEMM kernels take 128 KiB of dynamic LDS.  The limit is raised once per
// kernel, device and process (the attribute belongs to the kernel, not to a
// call), so that calls made under stream capture issue no attribute changes.
constexpr int kAttrDevices = 64;
template <auto Kernel, int kBytes = kLdsBytes>
hipError_t allow_big_lds() {
  static std::once_flag once[kAttrDevices];
  static hipError_t err[kAttrDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kAttrDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] {
    err[dev] = hipFuncSetAttribute((const void*)Kernel,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, kBytes);
  });
  return err[dev];
}

// Launch bookkeeping: the first failing launch is remembered.
struct Launch {
  hipStream_t s;
  hipError_t err = hipSuccess;
  void check() {
    if (err == hipSuccess) err = hipGetLastError();
  }
};

int64_t pad8(int64_t n) { return round_up(n, 8); }

// Compute units of the current device (the forward split prices launch waves
// of this many workgroups); 256 if the query fails.
int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 256;
  return n;
}

// The calls' W may be a vocabulary shard: rows [v_begin, v_begin + V) of a
// vocabulary of V_total entries (labels index the whole vocabulary).
struct Shard {
  int64_t v_begin, V_total;
};

// Targets, validity and compaction (k_prep_*), counters and the forward
// split; blk: prep_blk_bytes(N) of workspace.
void launch_prep(Launch& L, const int64_t* labels, int64_t B, int64_t T, int64_t ignore,
                 int64_t V_total, int shift, int reduction, const float* grad_scale,
                 int max_items, int64_t v_begin, int64_t V_local, int* blk, int* idx, int* tgt,
                 int* rowpos, Counters* ctr, int32_t* status) {
  const int N = (int)(B * T);
  const int nblk = (int)cdiv(N > 0 ? N : 1, kPrepBlock);
  hipLaunchKernelGGL(k_prep_count, dim3((unsigned)nblk), dim3(kPrepBlock), 0, L.s, labels, N,
                     (int)T, ignore, V_total, shift, blk);
  L.check();
  hipLaunchKernelGGL(k_prep_scan, dim3(1), dim3(1024), 0, L.s, blk, nblk, reduction, grad_scale,
                     cu_count(), max_items, V_local, ctr, status);
  L.check();
  hipLaunchKernelGGL(k_prep_write, dim3((unsigned)nblk), dim3(kPrepBlock), 0, L.s, labels, N,
                     (int)T, ignore, V_total, shift, (const int*)blk, v_begin, idx, tgt, rowpos);
  L.check();
}

template <class E>
int forward_impl(const Plan& pl, const Shard& sh, const void* X, const void* W,
                 const int64_t* labels, int64_t B, int64_t T, int64_t ignore_index,
                 int reduction, int shift, float* loss, float* lse, int64_t* n_valid,
                 int32_t* status, float* zt_out, char* ws, hipStream_t stream) {
  Launch L{stream};
  Counters* ctr = (Counters*)(ws + pl.o_ctr);
  int* idx = (int*)(ws + pl.o_idx);
  int* tgt = (int*)(ws + pl.o_tgt);
  int* rowpos = (int*)(ws + pl.o_rowpos);
  char* xc = ws + pl.o_xc;
  float2* part = (float2*)(ws + pl.o_part);
  float* zt = (float*)(ws + pl.o_zt);
  float* bsum = (float*)(ws + pl.o_bsum);
  const int rows_pad = (int)pl.rows_pad;
  const int row_bytes = (int)(pl.H * E::kBytes);
  const bool none = reduction == FLCE_REDUCTION_NONE;

  launch_prep(L, labels, B, T, ignore_index, sh.V_total, shift, reduction, nullptr,
              (int)pl.fwd_items, sh.v_begin, pl.V, (int*)(ws + pl.o_blk), idx, tgt, rowpos, ctr,
              status);
  hipLaunchKernelGGL(k_gather, dim3((unsigned)cdiv(rows_pad, 4)), dim3(256), 0, stream,
                     (const char*)X, row_bytes, (const int*)idx, (const Counters*)ctr,
                     xc, rows_pad, (const float*)nullptr, (float*)nullptr,
                     (float*)nullptr, 0, 0, (int64_t)0, (const float*)nullptr, (float*)nullptr,
                     (int*)nullptr, 0);
  L.check();
  hipLaunchKernelGGL(k_target<E>, dim3((unsigned)cdiv(rows_pad, 4)), dim3(256), 0, stream,
                     (const char*)xc, (const char*)W, (int)pl.H, (const int*)tgt,
                     (const Counters*)ctr, zt, (int)pl.V);
  L.check();
  FwdArgs fa;
  fa.W = (const char*)W;
  fa.Xc = xc;
  fa.H = (int)pl.H;
  fa.V = (int)pl.V;
  fa.rows_pad = rows_pad;
  fa.VT = (int)pl.VT;
  fa.ctr = ctr;
  fa.part = part;
  if (L.err == hipSuccess) L.err = allow_big_lds<k_fwd_lse<E>>();
  // k_fwd_lse hands its items out XCD by XCD over the first pad8(P * TTn)
  // workgroups (P * TTn <= fwd_items), so the grid covers pad8(fwd_items)
  hipLaunchKernelGGL(k_fwd_lse<E>, dim3((unsigned)pad8(pl.fwd_items)), dim3(kThreads),
                     kLdsBytes, stream, fa);
  L.check();
  const int nb = (int)cdiv(pl.N, 256);
  hipLaunchKernelGGL(k_merge, dim3(nb), dim3(256), 0, stream, (const float2*)part,
                     (const Counters*)ctr, (const int*)rowpos, (const float*)zt,
                     (int)pl.N, lse, bsum, none ? loss : (float*)nullptr, zt_out);
  L.check();
  hipLaunchKernelGGL(k_loss, dim3(1), dim3(256), 0, stream, (const float*)bsum, nb,
                     (const Counters*)ctr, reduction, none ? (float*)nullptr : loss, n_valid);
  L.check();
  return L.err == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

// One-hot sums for the dW tiles (k_oh_*): sort the compacted rows by
// (target, row), sum the rows of each target held by several rows, in that
// order, and fill the map.  `keys` holds 2 P entries; the map must already
// be -1 (k_gather).
template <class E>
void onehot_sums(int64_t P, int64_t rows_pad, int64_t H, int64_t V_local, const int* tgt,
                 const Counters* ctr, const char* xc, const float* rs, uint64_t* keys,
                 float* oh, int* map, Launch& L) {
  hipStream_t s = L.s;
  const bool merge = P > kSortLocal && P <= kMergeMax;
  hipLaunchKernelGGL(k_oh_sort_local, dim3((unsigned)std::max<int64_t>(1, P / kSortLocal)),
                     dim3(256), 0, s, tgt, ctr, (int)V_local, (int)P, merge ? 1 : 0, keys);
  L.check();
  const uint64_t* sorted = keys;
  if (merge) {
    hipLaunchKernelGGL(k_oh_merge_blocks, dim3((unsigned)(P / 1024)), dim3(1024), 0, s,
                       (const uint64_t*)keys, (int)P, keys + P);
    L.check();
    sorted = keys + P;
  } else {
    for (int64_t st = 2 * kSortLocal; st <= P; st <<= 1) {
      for (int64_t stride = st / 2; stride >= kSortLocal; stride >>= 1) {
        hipLaunchKernelGGL(k_bsort_global, dim3((unsigned)cdiv(P / 2, 256)), dim3(256), 0, s,
                           keys, (int)P, (int)st, (int)stride);
        L.check();
      }
      hipLaunchKernelGGL(k_bsort_merge, dim3((unsigned)(P / kSortLocal)), dim3(256), 0, s, keys,
                         (int)st);
      L.check();
    }
  }
  const dim3 grid((unsigned)(rows_pad / kOhBlock), (unsigned)cdiv(H, 256));
  hipLaunchKernelGGL(k_oh_partial<E>, grid, dim3(256), 0, s, sorted, (int)P, xc, (int)H,
                     (int)rows_pad, ctr, rs, oh);
  L.check();
  hipLaunchKernelGGL(k_oh_final, grid, dim3(256), 0, s, sorted, (int)P, (int)H, (int)rows_pad,
                     oh, map);
  L.check();
}

template <class E>
int backward_impl(const Plan& pl, const Shard& sh, const void* X, const void* W,
                  const int64_t* labels, int64_t B, int64_t T, int64_t ignore_index,
                  int reduction, int shift, const float* lse, const float* grad_scale,
                  void* dX, void* dW, int dx_f32, int grad_f32, int dw_acc, int32_t* status,
                  char* ws, hipStream_t stream) {
  Launch L{stream};
  Counters* ctr = (Counters*)(ws + pl.o_ctr);
  int* idx = (int*)(ws + pl.o_idx);
  int* tgt = (int*)(ws + pl.o_tgt);
  int* rowpos = (int*)(ws + pl.o_rowpos);
  char* xc = ws + pl.o_xc;
  float* lse2 = (float*)(ws + pl.o_lse2);
  char* g = ws + pl.o_g;
  float* dx32 = (float*)(ws + pl.o_dx32);
  const int rows_pad = (int)pl.rows_pad;
  const int row_bytes = (int)(pl.H * E::kBytes);

  // reduction "none": grad_scale is per row, gathered into compacted order
  const bool none = reduction == FLCE_REDUCTION_NONE;
  float* rs = none && grad_scale ? (float*)(ws + pl.o_rs) : nullptr;
  launch_prep(L, labels, B, T, ignore_index, sh.V_total, shift, reduction,
              none ? nullptr : grad_scale, (int)pl.fwd_items, sh.v_begin, pl.V,
              (int*)(ws + pl.o_blk), idx, tgt, rowpos, ctr, status);
  hipLaunchKernelGGL(k_gather, dim3((unsigned)cdiv(rows_pad, 4)), dim3(256), 0, stream,
                     (const char*)X, row_bytes, (const int*)idx, (const Counters*)ctr,
                     xc, rows_pad, lse, lse2, dx32, (int)(pl.H * 4), (int)pl.dx_split,
                     (int64_t)pl.rows_pad * pl.H, grad_scale, rs, (int*)(ws + pl.o_map),
                     (int)pl.V);
  L.check();

  float* oh = (float*)(ws + pl.o_oh);
  int* oh_map = (int*)(ws + pl.o_map);
  onehot_sums<E>(pl.P, pl.rows_pad, pl.H, pl.V, tgt, ctr, xc, rs, (uint64_t*)(ws + pl.o_keys),
                 oh, oh_map, L);

  BwdArgs a;
  a.W = (const char*)W;
  a.Xc = xc;
  a.G = g;
  a.lse2 = lse2;
  a.rs = rs;
  a.oh = oh;
  a.oh_map = oh_map;
  a.ohx = xc;
  a.tgt = tgt;
  a.dx32 = dx32;
  a.dx32p = dx32 + (int64_t)pl.rows_pad * pl.H;
  a.dx_stride = (int64_t)pl.rows_pad * pl.H;
  a.dx_split = (int)pl.dx_split;
  a.dW = (char*)dW;
  a.ctr = ctr;
  a.H = (int)pl.H;
  a.V = (int)pl.V;
  a.rows_pad = rows_pad;
  a.Vb = (int)pl.Vb;
  a.TT = (int)pl.TT;
  a.HT = (int)cdiv(pl.H, kTile);
  a.dw_f32 = grad_f32;
  a.dw_acc = dw_acc;
  a.v0 = a.vb = a.VTb = 0;
  const int64_t slab = pl.rows_pad * pl.Vb * pl.es;
  auto block = [&](int64_t b) {
    BwdArgs r = a;
    r.v0 = (int)(b * pl.Vb);
    r.vb = (int)std::min<int64_t>(pl.Vb, pl.V - r.v0);
    r.VTb = (int)cdiv(r.vb, kTile);
    r.G = g + (b & 1) * slab;
    return r;
  };
  if (L.err == hipSuccess) L.err = allow_big_lds<k_bwd<E>, kBwdLdsBytes>();
  // launch b + 1 runs the dX / dW tiles of block b and the G tiles of block
  // b + 1
  const int64_t nblk = cdiv(pl.V, pl.Vb);
  // the dW tiles' K loop runs over the rows (bounded by rows_pad), the dX
  // tiles' over a part of the block: the longer kind starts first
  const int dw_first = pl.rows_pad > cdiv(pl.Vb, pl.dx_split) ? 1 : 0;
  for (int64_t b = -1; b < nblk && L.err == hipSuccess; ++b) {
    const BwdArgs cur = b >= 0 ? block(b) : a;
    const BwdArgs nxt = b + 1 < nblk ? block(b + 1) : a;
    const int nb_dx = b >= 0 ? (int)pad8((int64_t)a.dx_split * a.HT * a.TT) : 0;
    const int nb_dw = b >= 0 ? (int)pad8((int64_t)a.HT * cur.VTb) : 0;
    const int nb_g = b + 1 < nblk ? (int)pad8((int64_t)nxt.VTb * a.TT) : 0;
    hipLaunchKernelGGL(k_bwd<E>, dim3((unsigned)(nb_dx + nb_dw + nb_g)), dim3(kThreads),
                       kBwdLdsBytes, stream, cur, nxt, nb_dx, nb_dw, nb_g, dw_first);
    L.check();
  }
  hipLaunchKernelGGL(k_dx_final<E>, dim3((unsigned)cdiv(pl.N, 4)), dim3(256), 0, stream,
                     (const float*)dx32, (int)pl.dx_split, (int64_t)pl.rows_pad * pl.H,
                     (const int*)rowpos, (int)pl.N, (int)pl.H, (char*)dX, dx_f32,
                     (const char*)W, (const int*)tgt, (int)pl.V, (const Counters*)ctr,
                     (const float*)rs, (const float*)nullptr);
  L.check();
  return L.err == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}


// bytes % 16 == 0 (every caller's sizes are multiples of 8 bf16 / 4 fp32)
void zero_fill(void* p, int64_t bytes, hipStream_t s) {
  const int64_t chunks = bytes / 16;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(cdiv(chunks, 256), 4096));
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s, (char*)p, chunks);
}

// ---------------------------------------------------------------------------
// Chunked mode (one call for loss, lse, dX and dW)
// ---------------------------------------------------------------------------
#ifndef FLCE_CHUNK_MIB
#define FLCE_CHUNK_MIB 2048
#endif
// the [C, Vp] softmax-gradient slab of one row chunk holds at most this many
// bytes (unless one 256-row tile of it already needs more): 6912 rows at
// V = 152064 bf16.  Larger chunks give the dW tiles, whose K loop runs over
// the chunk's rows, deeper loops, and fewer chunks fewer launches and short
// last chunks; past 2 GiB the steps gain little more (about 2 % for four
// times the memory), so a caller with memory to spare passes chunk_rows
constexpr int64_t kChunkBudget = (int64_t)FLCE_CHUNK_MIB << 20;
// vocabulary block of the dX / dW launches inside a chunk
#ifndef FLCE_CHUNK_VB
#define FLCE_CHUNK_VB 32768
#endif
constexpr int64_t kChunkVocabBlock = FLCE_CHUNK_VB;

struct ChunkPlan {
  int64_t N, rows_pad, H, V, Vp, es, TT, VT;
  int64_t C, nchunks;       // chunk rows (multiple of 256), chunks covering rows_pad
  int64_t VB;               // vocabulary block of the dX / dW launches
  int64_t dx_split;         // dX parts of a full chunk
  int64_t part_tiles;       // token tiles the extra dX parts' buffer holds
  int64_t dx_blocks;        // workgroups of a launch's dX tiles, at most
  int64_t o_ctr, o_idx, o_tgt, o_rowpos, o_xc, o_zt, o_lse_c, o_lse2, o_rloss, o_bsum, o_cctr;
  int64_t o_blk;
  int64_t o_rs;
  int64_t o_part, o_slab, o_dx32, o_dx32p;
  int64_t o_fk, o_mrow, o_redo, o_redo_t, o_xs;   // per-row factors, second pass, scaled rows
  int64_t P, o_keys, o_oh, o_map;   // one-hot sums for dW
  int64_t total;
};

// chunk_rows: rows per chunk wanted (rounded up to 256); 0 = as many as the
// slab budget allows.  Never more than the padded row count.
int make_chunk_plan(int64_t B, int64_t T, int64_t H, int64_t V, int dtype, int64_t chunk_rows,
                    ChunkPlan* p) {
  Plan base;
  const int rc = make_plan(B, T, H, V, dtype, &base);
  if (rc != FLCE_OK) return rc;
  ChunkPlan q;
  q.N = base.N;
  q.rows_pad = base.rows_pad;
  q.H = H;
  q.V = V;
  q.es = base.es;
  q.TT = base.TT;
  q.VT = base.VT;
  q.Vp = q.VT * kTile;
  if (chunk_rows < 0) return FLCE_ERR_SHAPE;
  // one token tile of the slab within 32-bit offsets (each tile's accesses
  // start from its own 64-bit base)
  if (kTile * q.Vp * q.es > kMaxI32) return FLCE_ERR_SHAPE;
  int64_t c = chunk_rows > 0 ? round_up(chunk_rows, kTile)
                             : kChunkBudget / (q.Vp * q.es) / kTile * kTile;
  if (c < kTile) c = kTile;
  q.C = std::min(c, q.rows_pad);
  q.nchunks = cdiv(q.rows_pad, q.C);
  // vocabulary block of the dX / dW launches: its W rows stay below 2^31
  // bytes (one descriptor per dX tile operand)
  q.VB = std::max<int64_t>(kTile, std::min<int64_t>(kChunkVocabBlock, kMaxI32 / (H * q.es)) /
                                      kTile * kTile);
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = round_up(off + bytes, kAlign);
    return o;
  };
  q.o_ctr = take(sizeof(Counters));
  q.o_idx = take(4 * q.rows_pad);
  q.o_tgt = take(4 * q.rows_pad);
  q.o_rowpos = take(4 * q.rows_pad);
  q.o_xc = take(q.rows_pad * H * q.es);
  q.o_zt = take(4 * q.rows_pad);
  q.o_lse_c = take(4 * q.rows_pad);
  q.o_lse2 = take(4 * q.rows_pad);
  q.o_rloss = take(4 * q.rows_pad);
  q.o_rs = take(4 * q.rows_pad);
  q.o_bsum = take(4 * q.TT);
  q.o_cctr = take(sizeof(Counters) * q.nchunks);
  q.o_blk = take(prep_blk_bytes(q.N));
  q.o_part = take(8 * 2 * q.VT * q.C);
  q.o_fk = take(4 * q.rows_pad);
  q.o_mrow = take(4 * q.rows_pad);
  q.o_redo = take(4 * q.rows_pad);
  q.o_redo_t = take(4 * (q.C / kTile));
  q.o_xs = take(q.C * H * q.es);
  q.o_slab = take(q.C * q.Vp * q.es);
  // dX parts: a full chunk's as its token tiles ask; the buffer of the extra
  // parts holds that many full chunks' rows, and at least half a chunk's (at
  // most 16 token tiles of it), so a short last chunk (few token tiles) can
  // take more parts.  The parts cover one chunk's rows and are folded into the
  // main FP32 sum after it.
  const int HT = (int)cdiv(H, kTile), TTc = (int)(q.C / kTile);
  q.dx_split = dx_parts_for(HT, TTc, FLCE_DX_TILES_CHUNKED, -1);
  q.part_tiles = std::max<int64_t>((q.dx_split - 1) * TTc,
                                   std::min<int64_t>(cdiv(TTc, 2), kShortChunkTiles));
  q.dx_blocks = 0;
  for (int tt = 1; tt <= TTc; ++tt)
    q.dx_blocks = std::max<int64_t>(
        q.dx_blocks,
        (int64_t)dx_parts_for(HT, tt, FLCE_DX_TILES_CHUNKED, (int)q.part_tiles) * HT * tt);
  q.dx_blocks = pad8(q.dx_blocks);
  // every launch within a dispatch's 32-bit work-item count (blocks x 256
  // threads): the logits tiles of a chunk, and a block's dX and dW tiles
  constexpr int64_t kMaxBlocks = ((int64_t)1 << 32) / kThreads - 8;
  if (pad8(q.VT * TTc) > kMaxBlocks || q.dx_blocks + pad8(HT * cdiv(q.VB, kTile)) > kMaxBlocks)
    return FLCE_ERR_SHAPE;
  q.o_dx32 = take(4 * q.rows_pad * H);
  q.o_dx32p = take(4 * q.part_tiles * kTile * H);
  q.P = pow2_at_least(q.rows_pad);
  q.o_keys = take(16 * q.P);
  q.o_oh = take(4 * q.rows_pad * H);
  q.o_map = take(4 * V);
  q.total = off;
  *p = q;
  return FLCE_OK;
}

template <class E>
int chunked_impl(const ChunkPlan& pl, const void* X, const void* W, const int64_t* labels,
                 int64_t B, int64_t T, int64_t ignore_index, int reduction, int shift,
                 const float* grad_scale, float* loss, float* lse, int64_t* n_valid,
                 void* dX, void* dW, int grad_f32, int dw_acc, int32_t* status, char* ws,
                 hipStream_t stream) {
  Launch L{stream};
  Counters* ctr = (Counters*)(ws + pl.o_ctr);
  int* idx = (int*)(ws + pl.o_idx);
  int* tgt = (int*)(ws + pl.o_tgt);
  int* rowpos = (int*)(ws + pl.o_rowpos);
  char* xc = ws + pl.o_xc;
  float* zt = (float*)(ws + pl.o_zt);
  float* lse_c = (float*)(ws + pl.o_lse_c);
  float* lse2 = (float*)(ws + pl.o_lse2);
  float* rloss = (float*)(ws + pl.o_rloss);
  float* bsum = (float*)(ws + pl.o_bsum);
  Counters* cctr = (Counters*)(ws + pl.o_cctr);
  float2* part = (float2*)(ws + pl.o_part);
  char* slab = ws + pl.o_slab;
  float* dx32 = (float*)(ws + pl.o_dx32);
  float* dx32p = (float*)(ws + pl.o_dx32p);
  float* fk = (float*)(ws + pl.o_fk);
  float* mrow = (float*)(ws + pl.o_mrow);
  int* redo = (int*)(ws + pl.o_redo);
  int* redo_t = (int*)(ws + pl.o_redo_t);
  char* xs = ws + pl.o_xs;
  const int rows_pad = (int)pl.rows_pad;
  const int row_bytes = (int)(pl.H * E::kBytes);
  const int C = (int)pl.C, TTc = C / kTile, HT = (int)cdiv(pl.H, kTile);
  const bool none = reduction == FLCE_REDUCTION_NONE;
  float* rs = none && grad_scale ? (float*)(ws + pl.o_rs) : nullptr;

  launch_prep(L, labels, B, T, ignore_index, pl.V, shift, reduction, none ? nullptr : grad_scale,
              1, 0, pl.V, (int*)(ws + pl.o_blk), idx, tgt, rowpos, ctr, status);
  hipLaunchKernelGGL(k_gather, dim3((unsigned)cdiv(rows_pad, 4)), dim3(256), 0, stream,
                     (const char*)X, row_bytes, (const int*)idx, (const Counters*)ctr, xc,
                     rows_pad, (const float*)nullptr, (float*)nullptr, dx32,
                     (int)(pl.H * 4), 1, (int64_t)0, grad_scale, rs, (int*)(ws + pl.o_map),
                     (int)pl.V);
  L.check();
  hipLaunchKernelGGL(k_target<E>, dim3((unsigned)cdiv(rows_pad, 4)), dim3(256), 0, stream,
                     (const char*)xc, (const char*)W, (int)pl.H, (const int*)tgt,
                     (const Counters*)ctr, zt, (int)pl.V);
  L.check();
  float* oh = (float*)(ws + pl.o_oh);
  int* oh_map = (int*)(ws + pl.o_map);
  onehot_sums<E>(pl.P, pl.rows_pad, pl.H, pl.V, tgt, ctr, xc, rs, (uint64_t*)(ws + pl.o_keys),
                 oh, oh_map, L);
  if (L.err == hipSuccess) L.err = allow_big_lds<k_chunk_z<E, 0>, kChunkZLdsBytes>();
  if (L.err == hipSuccess) L.err = allow_big_lds<k_chunk_z<E, 1>, kChunkZLdsBytes>();
  if (L.err == hipSuccess) L.err = allow_big_lds<k_bwd<E>, kBwdLdsBytes>();
  for (int64_t ch = 0; ch < pl.nchunks && L.err == hipSuccess; ++ch) {
    ChunkArgs ca;
    ca.W = (const char*)W;
    ca.row0 = (int)(ch * C);
    ca.Xc = xc + (int64_t)ca.row0 * row_bytes;
    ca.E = slab;
    ca.part = part;
    ca.ctr = ctr;
    ca.cctr = cctr + ch;
    ca.zt = zt;
    ca.tgt = tgt;
    ca.rs = rs;
    ca.lse_c = lse_c;
    ca.lse2 = lse2;
    ca.rloss = rloss;
    ca.H = (int)pl.H;
    ca.V = (int)pl.V;
    ca.Vp = (int)pl.Vp;
    ca.C = C;
    ca.VT = (int)pl.VT;
    ca.TTc = TTc;
    ca.fk = fk;
    ca.mrow = mrow;
    ca.redo = redo;
    ca.redo_t = redo_t;
    ca.Xs = xs;
    ca.dx32p = dx32p;
    ca.HT = HT;
    ca.dx_target = FLCE_DX_TILES_CHUNKED;
    ca.part_tiles = (int)pl.part_tiles;
    const int nbz = (int)pad8(pl.VT * TTc);
    hipLaunchKernelGGL((k_chunk_z<E, 0>), dim3((unsigned)nbz), dim3(kThreads), kChunkZLdsBytes,
                       stream,
                       ca);
    L.check();
    hipLaunchKernelGGL(k_chunk_lse<E>, dim3((unsigned)(C / 4)), dim3(256), 0, stream, ca);
    L.check();
    // the rows whose largest logit lies far above the target logit, against
    // their max (token tiles without such a row exit at once)
    hipLaunchKernelGGL((k_chunk_z<E, 1>), dim3((unsigned)nbz), dim3(kThreads), kChunkZLdsBytes,
                       stream, ca);
    L.check();
    // dX and dW tiles of the chunk, one vocabulary block per launch; the dW
    // tiles contract the slab with the rows scaled by their factor
    BwdArgs b;
    b.W = (const char*)W;
    b.Xc = xs;
    b.lse2 = lse2;
    b.rs = rs;
    b.tgt = tgt;
    b.dx32 = dx32 + (int64_t)ca.row0 * pl.H;
    b.dx32p = dx32p;
    b.dx_stride = 0;
    b.dx_split = 0;   // the chunk's part count, from its counters (k_chunk_lse)
    b.dW = (char*)dW;
    b.ctr = cctr + ch;
    b.H = (int)pl.H;
    b.V = (int)pl.V;
    b.rows_pad = C;
    b.Vb = (int)pl.Vp;   // the slab's row pitch
    b.TT = TTc;
    b.HT = HT;
    b.dw_f32 = grad_f32;
    b.dw_acc = ch > 0 || dw_acc;
    // the one-hot part of dW (all rows) goes in with the first chunk's tiles
    b.oh = ch == 0 ? oh : nullptr;
    b.oh_map = oh_map;
    b.ohx = xc;
    for (int64_t v0 = 0; v0 < pl.V && L.err == hipSuccess; v0 += pl.VB) {
      b.v0 = (int)v0;
      b.vb = (int)std::min<int64_t>(pl.VB, pl.V - v0);
      b.VTb = (int)cdiv(b.vb, kTile);
      b.G = slab + v0 * E::kBytes;
      const int nb_dx = (int)pl.dx_blocks;
      const int nb_dw = (int)pad8((int64_t)HT * b.VTb);
      hipLaunchKernelGGL(k_bwd<E>, dim3((unsigned)(nb_dx + nb_dw)), dim3(kThreads), kBwdLdsBytes,
                         stream, b, b, nb_dx, nb_dw, 0, C > cdiv(b.vb, pl.dx_split) ? 1 : 0);
      L.check();
    }
    if (L.err == hipSuccess) {
      // the chunk's extra vocabulary parts (if it has any) into the main sum,
      // in part order, over the chunk's rows
      const int64_t count4 = (int64_t)C * pl.H / 4;
      hipLaunchKernelGGL(k_dx_fold, dim3((unsigned)std::min<int64_t>(cdiv(count4, 256), 4096)),
                         dim3(256), 0, stream, b.dx32, (const float*)dx32p,
                         (const Counters*)(cctr + ch), (int)pl.H);
      L.check();
    }
  }
  hipLaunchKernelGGL(k_lse_out, dim3((unsigned)cdiv(pl.N, 256)), dim3(256), 0, stream,
                     (const float*)lse_c, (const int*)rowpos, (int)pl.N, lse,
                     (const float*)rloss, (const Counters*)ctr, none ? loss : (float*)nullptr);
  L.check();
  hipLaunchKernelGGL(k_block_sums, dim3((unsigned)pl.TT), dim3(256), 0, stream,
                     (const float*)rloss, (const Counters*)ctr, bsum);
  L.check();
  hipLaunchKernelGGL(k_loss, dim3(1), dim3(256), 0, stream, (const float*)bsum, (int)pl.TT,
                     (const Counters*)ctr, reduction, none ? (float*)nullptr : loss, n_valid);
  L.check();
  hipLaunchKernelGGL(k_dx_final<E>, dim3((unsigned)cdiv(pl.N, 4)), dim3(256), 0, stream,
                     (const float*)dx32, 1, (int64_t)0, (const int*)rowpos, (int)pl.N,
                     (int)pl.H, (char*)dX, grad_f32, (const char*)W, (const int*)tgt,
                     (int)pl.V, (const Counters*)ctr, (const float*)rs, (const float*)fk);
  L.check();
  return L.err == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Allocation-free forward: a file-scope device array stands in for the
// caller's workspace.  Each device holds its own copy; its address on the
// current device is looked up once per device (hipGetSymbolAddress) and kept.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = FLCE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

}  // namespace
}  // namespace flce

// the array itself: never passed to a kernel by name (on the host the name is
// only a stand-in), only through the per-device address looked up below
static __device__ __align__(256) char scratch[flce::kScratchBytes];

namespace flce {
namespace {

// Device address of `scratch` on the current device, or an error.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return *out != nullptr ? hipSuccess : hipErrorInvalidSymbol;
}

}  // namespace
}  // namespace flce

using namespace flce;

extern "C" {

int flce_workspace_size(int64_t B, int64_t T, int64_t H, int64_t V, int dtype,
                        size_t* bytes) {
  if (bytes == nullptr) return FLCE_ERR_NULL;
  Plan p;
  const int rc = make_plan(B, T, H, V, dtype, &p);
  if (rc != FLCE_OK) return rc;
  *bytes = (size_t)p.total;
  return FLCE_OK;
}

int flce_forward(const void* X, const void* W, const int64_t* labels, int64_t B,
                 int64_t T, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                 int reduction, int shift, float* loss, float* lse, int64_t* n_valid,
                 int32_t* status, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (loss == nullptr) return FLCE_ERR_NULL;
  Plan p;
  int rc = make_plan(B, T, H, V, dtype, &p);
  if (rc != FLCE_OK) return rc;
  if (reduction != FLCE_REDUCTION_MEAN && reduction != FLCE_REDUCTION_SUM &&
      reduction != FLCE_REDUCTION_NONE)
    return FLCE_ERR_REDUCTION;
  hipStream_t s = (hipStream_t)stream;
  if (p.N == 0) {
    // reduction "none": the per-row loss array is empty
    hipLaunchKernelGGL(k_empty, dim3(1), dim3(1), 0, s,
                       reduction == FLCE_REDUCTION_NONE ? (float*)nullptr : loss, n_valid,
                       status);
    return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  if (X == nullptr || W == nullptr || labels == nullptr || lse == nullptr)
    return FLCE_ERR_NULL;
  if (!aligned16(X) || !aligned16(W) || ((uintptr_t)labels & 7u) ||
      ((uintptr_t)lse & 3u) || ((uintptr_t)loss & 3u))
    return FLCE_ERR_ALIGN;
  if (workspace == nullptr) return FLCE_ERR_WORKSPACE;
  if ((int64_t)workspace_bytes < p.total || !aligned16(workspace))
    return FLCE_ERR_WORKSPACE;
  if (dtype == FLCE_DTYPE_BF16)
    return forward_impl<BF16>(p, Shard{0, V}, X, W, labels, B, T, ignore_index, reduction,
                              shift, loss, lse, n_valid, status, nullptr, (char*)workspace, s);
  return forward_impl<F32>(p, Shard{0, V}, X, W, labels, B, T, ignore_index, reduction, shift,
                           loss, lse, n_valid, status, nullptr, (char*)workspace, s);
}

int flce_forward_noalloc(const void* X, const void* W, const int64_t* labels, int64_t B,
                         int64_t T, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                         int reduction, int shift, float* loss, float* lse, int64_t* n_valid,
                         int32_t* status, void* stream) {
  if (loss == nullptr) return FLCE_ERR_NULL;
  Plan p;
  int rc = make_plan(B, T, H, V, dtype, &p);
  if (rc != FLCE_OK) return rc;
  if (reduction != FLCE_REDUCTION_MEAN && reduction != FLCE_REDUCTION_SUM &&
      reduction != FLCE_REDUCTION_NONE)
    return FLCE_ERR_REDUCTION;
  if (p.fwd_total > kScratchBytes) return FLCE_ERR_TOO_LARGE;
  hipStream_t s = (hipStream_t)stream;
  if (p.N == 0) {
    hipLaunchKernelGGL(k_empty, dim3(1), dim3(1), 0, s,
                       reduction == FLCE_REDUCTION_NONE ? (float*)nullptr : loss, n_valid,
                       status);
    return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  if (X == nullptr || W == nullptr || labels == nullptr || lse == nullptr)
    return FLCE_ERR_NULL;
  if (!aligned16(X) || !aligned16(W) || ((uintptr_t)labels & 7u) ||
      ((uintptr_t)lse & 3u) || ((uintptr_t)loss & 3u))
    return FLCE_ERR_ALIGN;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return FLCE_ERR_HIP;
  // every byte of the forward's region that a kernel reads is written earlier
  // in the same call, so the array's previous contents never matter
  if (dtype == FLCE_DTYPE_BF16)
    return forward_impl<BF16>(p, Shard{0, V}, X, W, labels, B, T, ignore_index, reduction,
                              shift, loss, lse, n_valid, status, nullptr, (char*)ws, s);
  return forward_impl<F32>(p, Shard{0, V}, X, W, labels, B, T, ignore_index, reduction, shift,
                           loss, lse, n_valid, status, nullptr, (char*)ws, s);
}

int flce_backward(const void* X, const void* W, const int64_t* labels, int64_t B,
                  int64_t T, int64_t H, int64_t V, int dtype, int64_t ignore_index,
                  int reduction, int shift, const float* lse, const float* grad_scale,
                  void* dX, void* dW, int grad_dtype, int dW_accumulate, int32_t* status,
                  void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int rc = make_plan(B, T, H, V, dtype, &p);
  if (rc != FLCE_OK) return rc;
  if (reduction != FLCE_REDUCTION_MEAN && reduction != FLCE_REDUCTION_SUM &&
      reduction != FLCE_REDUCTION_NONE)
    return FLCE_ERR_REDUCTION;
  if (grad_dtype != dtype && grad_dtype != FLCE_DTYPE_F32) return FLCE_ERR_DTYPE;
  if (W == nullptr || dW == nullptr) return FLCE_ERR_NULL;
  if (p.N > 0 && (X == nullptr || labels == nullptr || lse == nullptr || dX == nullptr))
    return FLCE_ERR_NULL;
  const int64_t ges = grad_dtype == FLCE_DTYPE_F32 ? 4 : 2;
  if (!aligned16(W) || !aligned16(dW) || (p.N > 0 && (!aligned16(X) || !aligned16(dX))) ||
      ((uintptr_t)labels & 7u) || ((uintptr_t)lse & 3u))
    return FLCE_ERR_ALIGN;
  if (overlaps(dW, p.V * p.H * ges, W, p.V * p.H * p.es)) return FLCE_ERR_ALIAS;
  if (p.N > 0 && overlaps(dX, p.N * p.H * ges, X, p.N * p.H * p.es)) return FLCE_ERR_ALIAS;
  if (workspace == nullptr) return FLCE_ERR_WORKSPACE;
  if ((int64_t)workspace_bytes < p.total || !aligned16(workspace))
    return FLCE_ERR_WORKSPACE;
  if (grads_overlap(dX, p.N * p.H * ges, dW, p.V * p.H * ges, workspace, p.total))
    return FLCE_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  const int gf32 = grad_dtype == FLCE_DTYPE_F32 ? 1 : 0;
  if (p.N == 0) {
    // no rows: dW = 0 (dX is empty); accumulating adds nothing
    if (!dW_accumulate) zero_fill(dW, p.V * p.H * ges, s);
    if (status != nullptr)
      hipLaunchKernelGGL(k_empty, dim3(1), dim3(1), 0, s, (float*)nullptr,
                         (int64_t*)nullptr, status);
    return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  if (dtype == FLCE_DTYPE_BF16)
    return backward_impl<BF16>(p, Shard{0, V}, X, W, labels, B, T, ignore_index, reduction,
                               shift, lse, grad_scale, dX, dW, gf32, gf32,
                               dW_accumulate ? 1 : 0, status, (char*)workspace, s);
  return backward_impl<F32>(p, Shard{0, V}, X, W, labels, B, T, ignore_index, reduction, shift,
                            lse, grad_scale, dX, dW, gf32, gf32, dW_accumulate ? 1 : 0, status,
                            (char*)workspace, s);
}

int flce_shard_forward(const void* X, const void* W, const int64_t* labels, int64_t B,
                       int64_t T, int64_t H, int64_t V, int64_t v_begin, int64_t V_total,
                       int dtype, int64_t ignore_index, int shift, float* lse, float* zt,
                       int32_t* status, void* workspace, size_t workspace_bytes,
                       void* stream) {
  Plan p;
  int rc = make_plan(B, T, H, V, dtype, &p);
  if (rc != FLCE_OK) return rc;
  if (v_begin < 0 || V_total < V || v_begin > V_total - V || V_total > kMaxI32 - 512)
    return FLCE_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (p.N == 0) {
    hipLaunchKernelGGL(k_empty, dim3(1), dim3(1), 0, s, (float*)nullptr, (int64_t*)nullptr,
                       status);
    return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  if (X == nullptr || W == nullptr || labels == nullptr || lse == nullptr || zt == nullptr)
    return FLCE_ERR_NULL;
  if (!aligned16(X) || !aligned16(W) || ((uintptr_t)labels & 7u) || ((uintptr_t)lse & 3u) ||
      ((uintptr_t)zt & 3u))
    return FLCE_ERR_ALIGN;
  if (workspace == nullptr) return FLCE_ERR_WORKSPACE;
  if ((int64_t)workspace_bytes < p.total || !aligned16(workspace)) return FLCE_ERR_WORKSPACE;
  const Shard sh{v_begin, V_total};
  if (dtype == FLCE_DTYPE_BF16)
    return forward_impl<BF16>(p, sh, X, W, labels, B, T, ignore_index, FLCE_REDUCTION_SUM,
                              shift, nullptr, lse, nullptr, status, zt, (char*)workspace, s);
  return forward_impl<F32>(p, sh, X, W, labels, B, T, ignore_index, FLCE_REDUCTION_SUM, shift,
                           nullptr, lse, nullptr, status, zt, (char*)workspace, s);
}

int flce_shard_merge_workspace_size(int64_t B, int64_t T, size_t* bytes) {
  if (bytes == nullptr) return FLCE_ERR_NULL;
  if (B < 0 || T < 0 || B > kMaxI32 || T > kMaxI32 || B * T > (1ll << 24)) return FLCE_ERR_SHAPE;
  const int64_t rows_pad = round_up(B * T > 0 ? B * T : 1, kTile);
  *bytes = (size_t)(round_up(sizeof(Counters), kAlign) + 3 * round_up(4 * rows_pad, kAlign) +
                    round_up(4 * cdiv(rows_pad, 256), kAlign) +
                    round_up(prep_blk_bytes(B * T), kAlign));
  return FLCE_OK;
}

int flce_shard_merge(const float* lse_shards, const float* zt_shards, int shards,
                     const int64_t* labels, int64_t B, int64_t T, int64_t V_total,
                     int64_t ignore_index, int shift, int reduction, float* loss, float* lse,
                     int64_t* n_valid, int32_t* status, void* workspace,
                     size_t workspace_bytes, void* stream) {
  size_t need = 0;
  int rc = flce_shard_merge_workspace_size(B, T, &need);
  if (rc != FLCE_OK) return rc;
  if (shards <= 0 || V_total <= 0 || V_total > kMaxI32 - 512) return FLCE_ERR_SHAPE;
  if (reduction != FLCE_REDUCTION_MEAN && reduction != FLCE_REDUCTION_SUM &&
      reduction != FLCE_REDUCTION_NONE)
    return FLCE_ERR_REDUCTION;
  if (loss == nullptr) return FLCE_ERR_NULL;
  const int64_t N = B * T;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0) {
    hipLaunchKernelGGL(k_empty, dim3(1), dim3(1), 0, s,
                       reduction == FLCE_REDUCTION_NONE ? (float*)nullptr : loss, n_valid,
                       status);
    return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  if (lse_shards == nullptr || zt_shards == nullptr || labels == nullptr || lse == nullptr)
    return FLCE_ERR_NULL;
  if (((uintptr_t)labels & 7u) || ((uintptr_t)lse & 3u) || ((uintptr_t)loss & 3u))
    return FLCE_ERR_ALIGN;
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
    return FLCE_ERR_WORKSPACE;
  const int64_t rows_pad = round_up(N, kTile);
  char* ws = (char*)workspace;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = round_up(off + bytes, kAlign);
    return o;
  };
  Counters* ctr = (Counters*)(ws + take(sizeof(Counters)));
  int* idx = (int*)(ws + take(4 * rows_pad));
  int* tgt = (int*)(ws + take(4 * rows_pad));
  int* rowpos = (int*)(ws + take(4 * rows_pad));
  float* bsum = (float*)(ws + take(4 * cdiv(rows_pad, 256)));
  int* blk = (int*)(ws + take(prep_blk_bytes(N)));
  const bool none = reduction == FLCE_REDUCTION_NONE;
  Launch L{s};
  launch_prep(L, labels, B, T, ignore_index, V_total, shift, reduction, nullptr, 1, 0, V_total,
              blk, idx, tgt, rowpos, ctr, status);
  const int nb = (int)cdiv(N, 256);
  hipLaunchKernelGGL(k_shard_merge, dim3((unsigned)nb), dim3(256), 0, s, lse_shards, zt_shards,
                     shards, (int)N, (const int*)rowpos, (const Counters*)ctr, lse, bsum,
                     none ? loss : (float*)nullptr);
  L.check();
  hipLaunchKernelGGL(k_loss, dim3(1), dim3(256), 0, s, (const float*)bsum, nb,
                     (const Counters*)ctr, reduction, none ? (float*)nullptr : loss, n_valid);
  L.check();
  return L.err == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int flce_shard_backward(const void* X, const void* W, const int64_t* labels, int64_t B,
                        int64_t T, int64_t H, int64_t V, int64_t v_begin, int64_t V_total,
                        int dtype, int64_t ignore_index, int reduction, int shift,
                        const float* lse, const float* grad_scale, float* dX_partial, void* dW,
                        int grad_dtype, int dW_accumulate, int32_t* status, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Plan p;
  int rc = make_plan(B, T, H, V, dtype, &p);
  if (rc != FLCE_OK) return rc;
  if (v_begin < 0 || V_total < V || v_begin > V_total - V || V_total > kMaxI32 - 512)
    return FLCE_ERR_SHAPE;
  if (reduction != FLCE_REDUCTION_MEAN && reduction != FLCE_REDUCTION_SUM &&
      reduction != FLCE_REDUCTION_NONE)
    return FLCE_ERR_REDUCTION;
  if (grad_dtype != dtype && grad_dtype != FLCE_DTYPE_F32) return FLCE_ERR_DTYPE;
  if (W == nullptr || dW == nullptr) return FLCE_ERR_NULL;
  if (p.N > 0 && (X == nullptr || labels == nullptr || lse == nullptr || dX_partial == nullptr))
    return FLCE_ERR_NULL;
  const int64_t ges = grad_dtype == FLCE_DTYPE_F32 ? 4 : 2;
  if (!aligned16(W) || !aligned16(dW) ||
      (p.N > 0 && (!aligned16(X) || !aligned16(dX_partial))) || ((uintptr_t)labels & 7u) ||
      ((uintptr_t)lse & 3u))
    return FLCE_ERR_ALIGN;
  if (overlaps(dW, p.V * p.H * ges, W, p.V * p.H * p.es)) return FLCE_ERR_ALIAS;
  if (p.N > 0 && overlaps(dX_partial, p.N * p.H * 4, X, p.N * p.H * p.es)) return FLCE_ERR_ALIAS;
  if (workspace == nullptr) return FLCE_ERR_WORKSPACE;
  if ((int64_t)workspace_bytes < p.total || !aligned16(workspace)) return FLCE_ERR_WORKSPACE;
  if (grads_overlap(dX_partial, p.N * p.H * 4, dW, p.V * p.H * ges, workspace, p.total))
    return FLCE_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  const int gf32 = grad_dtype == FLCE_DTYPE_F32 ? 1 : 0;
  if (p.N == 0) {
    if (!dW_accumulate) zero_fill(dW, p.V * p.H * ges, s);
    if (status != nullptr)
      hipLaunchKernelGGL(k_empty, dim3(1), dim3(1), 0, s, (float*)nullptr, (int64_t*)nullptr,
                         status);
    return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  const Shard sh{v_begin, V_total};
  if (dtype == FLCE_DTYPE_BF16)
    return backward_impl<BF16>(p, sh, X, W, labels, B, T, ignore_index, reduction, shift, lse,
                               grad_scale, dX_partial, dW, 1, gf32, dW_accumulate ? 1 : 0,
                               status, (char*)workspace, s);
  return backward_impl<F32>(p, sh, X, W, labels, B, T, ignore_index, reduction, shift, lse,
                            grad_scale, dX_partial, dW, 1, gf32, dW_accumulate ? 1 : 0, status,
                            (char*)workspace, s);
}

int flce_chunked_workspace_size(int64_t B, int64_t T, int64_t H, int64_t V, int dtype,
                                int64_t chunk_rows, size_t* bytes) {
  if (bytes == nullptr) return FLCE_ERR_NULL;
  ChunkPlan p;
  const int rc = make_chunk_plan(B, T, H, V, dtype, chunk_rows, &p);
  if (rc != FLCE_OK) return rc;
  *bytes = (size_t)p.total;
  return FLCE_OK;
}

int flce_chunked(const void* X, const void* W, const int64_t* labels, int64_t B, int64_t T,
                 int64_t H, int64_t V, int dtype, int64_t ignore_index, int reduction,
                 int shift, int64_t chunk_rows, const float* grad_scale, float* loss,
                 float* lse, int64_t* n_valid, void* dX, void* dW, int grad_dtype,
                 int dW_accumulate, int32_t* status, void* workspace, size_t workspace_bytes,
                 void* stream) {
  ChunkPlan p;
  const int rc = make_chunk_plan(B, T, H, V, dtype, chunk_rows, &p);
  if (rc != FLCE_OK) return rc;
  if (reduction != FLCE_REDUCTION_MEAN && reduction != FLCE_REDUCTION_SUM &&
      reduction != FLCE_REDUCTION_NONE)
    return FLCE_ERR_REDUCTION;
  if (grad_dtype != dtype && grad_dtype != FLCE_DTYPE_F32) return FLCE_ERR_DTYPE;
  if (loss == nullptr || W == nullptr || dW == nullptr) return FLCE_ERR_NULL;
  if (p.N > 0 && (X == nullptr || labels == nullptr || lse == nullptr || dX == nullptr))
    return FLCE_ERR_NULL;
  const int64_t ges = grad_dtype == FLCE_DTYPE_F32 ? 4 : 2;
  if (!aligned16(W) || !aligned16(dW) || (p.N > 0 && (!aligned16(X) || !aligned16(dX))) ||
      ((uintptr_t)labels & 7u) || ((uintptr_t)lse & 3u) || ((uintptr_t)loss & 3u))
    return FLCE_ERR_ALIGN;
  if (overlaps(dW, p.V * p.H * ges, W, p.V * p.H * p.es)) return FLCE_ERR_ALIAS;
  if (p.N > 0 && overlaps(dX, p.N * p.H * ges, X, p.N * p.H * p.es)) return FLCE_ERR_ALIAS;
  if (grads_overlap(dX, p.N * p.H * ges, dW, p.V * p.H * ges, nullptr, 0)) return FLCE_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  const int gf32 = grad_dtype == FLCE_DTYPE_F32 ? 1 : 0;
  if (p.N == 0) {
    if (!dW_accumulate) zero_fill(dW, p.V * p.H * ges, s);
    hipLaunchKernelGGL(k_empty, dim3(1), dim3(1), 0, s,
                       reduction == FLCE_REDUCTION_NONE ? (float*)nullptr : loss, n_valid,
                       status);
    return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
  }
  if (workspace == nullptr) return FLCE_ERR_WORKSPACE;
  if ((int64_t)workspace_bytes < p.total || !aligned16(workspace))
    return FLCE_ERR_WORKSPACE;
  if (grads_overlap(dX, p.N * p.H * ges, dW, p.V * p.H * ges, workspace, p.total))
    return FLCE_ERR_ALIAS;
  if (dtype == FLCE_DTYPE_BF16)
    return chunked_impl<BF16>(p, X, W, labels, B, T, ignore_index, reduction, shift,
                              grad_scale, loss, lse, n_valid, dX, dW, gf32,
                              dW_accumulate ? 1 : 0, status, (char*)workspace, s);
  return chunked_impl<F32>(p, X, W, labels, B, T, ignore_index, reduction, shift, grad_scale,
                           loss, lse, n_valid, dX, dW, gf32, dW_accumulate ? 1 : 0, status,
                           (char*)workspace, s);
}

int flce_scale_grads(const void* dX_in, void* dX, int64_t nx, const void* dW_in, void* dW,
                     int64_t nw, int grad_dtype, const float* scale, void* stream) {
  if (scale == nullptr) return FLCE_ERR_NULL;
  if (grad_dtype != FLCE_DTYPE_F32 && grad_dtype != FLCE_DTYPE_BF16) return FLCE_ERR_DTYPE;
  const int per = grad_dtype == FLCE_DTYPE_F32 ? 4 : 8;
  const int64_t es = grad_dtype == FLCE_DTYPE_F32 ? 4 : 2;
  if (nx < 0 || nw < 0 || nx % per || nw % per) return FLCE_ERR_SHAPE;
  if ((nx > 0 && (dX == nullptr || dX_in == nullptr)) ||
      (nw > 0 && (dW == nullptr || dW_in == nullptr)))
    return FLCE_ERR_NULL;
  if ((nx > 0 && (!aligned16(dX) || !aligned16(dX_in))) ||
      (nw > 0 && (!aligned16(dW) || !aligned16(dW_in))))
    return FLCE_ERR_ALIGN;
  // each output is its input (in place) or lies apart from it
  if ((nx > 0 && dX != dX_in && overlaps(dX, nx * es, dX_in, nx * es)) ||
      (nw > 0 && dW != dW_in && overlaps(dW, nw * es, dW_in, nw * es)))
    return FLCE_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  const int f32 = grad_dtype == FLCE_DTYPE_F32;
  for (int t = 0; t < 2; ++t) {
    const int64_t chunks = (t == 0 ? nx : nw) / per;
    if (chunks == 0) continue;
    const int64_t blocks = std::min<int64_t>(cdiv(chunks, 256), 8192);
    hipLaunchKernelGGL(k_scale_grads, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const char*)(t == 0 ? dX_in : dW_in), (char*)(t == 0 ? dX : dW),
                       chunks, f32, scale);
  }
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int flce_convert_grads(const float* src, void* dst, int64_t n, int dst_dtype,
                       const float* scale, int accumulate, void* stream) {
  if (dst_dtype != FLCE_DTYPE_F32 && dst_dtype != FLCE_DTYPE_BF16) return FLCE_ERR_DTYPE;
  if (n < 0 || n % 4) return FLCE_ERR_SHAPE;
  if (n == 0) return FLCE_OK;
  if (src == nullptr || dst == nullptr) return FLCE_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return FLCE_ERR_ALIGN;
  const int64_t des = dst_dtype == FLCE_DTYPE_F32 ? 4 : 2;
  if (overlaps(src, n * 4, dst, n * des)) return FLCE_ERR_ALIAS;
  const int64_t chunks = n / 4;
  const int64_t blocks = std::min<int64_t>(cdiv(chunks, 256), 8192);
  hipLaunchKernelGGL(k_convert_grads, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     src, (char*)dst, chunks, dst_dtype == FLCE_DTYPE_F32 ? 1 : 0, scale,
                     accumulate ? 1 : 0);
  return hipGetLastError() == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

const char* flce_status_string(int code) {
  switch (code) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_NULL: return "a required pointer is NULL";
    case FLCE_ERR_SHAPE: return "sizes out of the supported range";
    case FLCE_ERR_ALIGN: return "H must be a multiple of 8 and buffers 16-byte aligned";
    case FLCE_ERR_DTYPE: return "unknown or unsupported dtype";
    case FLCE_ERR_REDUCTION: return "unknown reduction";
    case FLCE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FLCE_ERR_HIP: return "a HIP launch failed";
    case FLCE_ERR_LABEL_RANGE: return "a label is neither ignore_index nor in [0, V)";
    case FLCE_ERR_ALIAS:
      return "an output buffer overlaps an input, the other output or the workspace";
    case FLCE_ERR_TOO_LARGE:
      return "the problem needs more scratch than the allocation-free entry point holds";
    default: return "unknown status code";
  }
}

}  // extern "C"
