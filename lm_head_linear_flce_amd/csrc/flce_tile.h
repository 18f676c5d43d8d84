// flce_tile.h -- the 256 x 256 MFMA tile shared by every contraction of the
// fused linear cross-entropy engine (gfx950 / CDNA4).
//
// A workgroup of 256 threads (4 wave64s, one per SIMD) owns one 256 x 256 fp32
// accumulator tile C[m][n] = sum_k A[m][k] * B[n][k].  Each wave owns a
// 128 x 128 quarter held as 4 x 4 blocks of 32 x 32 MFMA accumulators
// (256 accumulator registers per lane).  K advances 128 bytes per step
// (64 bf16 or 32 fp32 values), double-buffered through LDS:
//
//   LDS = A[2 stages][256 rows][128 B] + B[2 stages][256 rows][128 B] = 128 KiB
//
// A K-major LDS row is K-contiguous, so one ds_read_b128 hands a lane the 8
// bf16 (or 4 fp32) K values an MFMA lane expects.  The 16-byte chunk
// c of row r is stored at a row-dependent XOR-permuted chunk position so that
// the lanes one LDS cycle serves touch distinct bank groups for fragment
// reads and for stores; see swz() for the exact pattern.
//
// Global memory is read with raw buffer loads whose descriptor covers exactly
// [base, end of tensor): a read past the end returns 0 in hardware, so ragged
// vocabulary / row tails need no branch and can never fault.  Two loaders:
//   * LoadDirect  -- the operand is stored with K contiguous (row-major
//                    [rows][K]), e.g. W [V, H] or X [N, H] contracted over H;
//   * LoadMN      -- the operand is stored with K as the outer index
//                    ([K][rows]), e.g. X [N, H] or W [V, H] contracted over N
//                    or V.  It keeps that layout in LDS and the fragment read
//                    transposes (ds_read_b64_tr_b16 on gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) char lds_t;   // LDS byte pointer

constexpr int kTile = 256;                 // tile extent in M and in N
constexpr int kRowBytes = 128;             // K bytes per tile row per step
constexpr int kThreads = 256;              // 4 waves
constexpr int kSlab = kTile * kRowBytes;   // 32 KiB: one operand, one stage
constexpr int kLdsBytes = 4 * kSlab;       // A0 A1 B0 B1
constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit dword format

// element traits --------------------------------------------------------------
struct BF16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;      // values per 16-byte chunk
  static constexpr int kKStep = 64;        // K values per main-loop step
};
struct F32 {
  static constexpr int kBytes = 4;
  static constexpr int kPerChunk = 4;
  static constexpr int kKStep = 32;
};

// Buffer descriptor over [base, base + bytes) (clamped to 32 bits).  Every
// caller passes workgroup-uniform values; saying so with readfirstlane keeps
// the descriptor in scalar registers even where the compiler cannot prove
// uniformity (it would otherwise wrap each load in a per-lane loop).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  uint32_t n = bytes <= 0 ? 0u
             : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  n = __builtin_amdgcn_readfirstlane(n);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)n, kRsrcWord3);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// fp32 -> bf16 with round-to-nearest-even (NaN stays NaN): gfx950 converts a
// pair in one v_cvt_pk_bf16_f32; `a` lands in the low half.
__device__ __forceinline__ int pack_bf16(float a, float b) {
  return __builtin_bit_cast(int, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ uint32_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float bf2f(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

__device__ __forceinline__ i32x4 bload128(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// gfx950 serves a 128-bit LDS read 16 lanes per cycle (64 banks): the 16
// rows one cycle touches must land on distinct 16-byte bank groups, i.e. the
// pair (row parity, physical chunk) must differ between them.  XOR-ing the
// chunk with (row & 7) ^ ((row >> 3) & 1) achieves that for any 16 aligned
// consecutive rows, and keeps 8 consecutive rows distinct for writes.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}

// One operand of a tile: where its first element is and how rows are strided.
//   direct: base = &op[row0][0];       element (r, k) at base + r*ldb + k*es
//   trans : base = &op[0][mn0];        element (k, c) at base + k*ldb + c*es
// `bytes` is the distance from base to the end of the tensor (reads beyond it
// return 0); `kbytes` (direct only) is the number of valid K bytes per row.
struct Opnd {
  const char* base;
  int64_t bytes;
  int ldb;
  int kbytes;
};

// ---------------------------------------------------------------------------
// Loaders: issue() starts the global reads of step s into registers, commit()
// writes them to an LDS slab.  Each thread moves 8 x 16 B per step.
// ---------------------------------------------------------------------------
struct LoadDirect {
  static constexpr bool kTransposed = false;
  struct Frag;
  i32x4 v[8];
  // Quarter `part` (0..3) of the loads of step s: register rows 2*part and
  // 2*part+1.  A chunk at or past the rows' K extent (it would hold the next
  // row's values) and every chunk of a step that is not `live` read zeros:
  // the descriptor covers at most the tile's 256 rows (< 2^31 bytes, as H is
  // bounded), so the offset 2^31 is always out of range.
  template <class E>
  __device__ __forceinline__ void issue_part(const Opnd& o, int s, int part, bool live,
                                             int tid) {
    const int c = tid & 7, rr = tid >> 3;
    const int64_t span = (int64_t)kTile * o.ldb;
    const rsrc_t r = make_rsrc(o.base, live ? (o.bytes < span ? o.bytes : span) : 0);
    const int kb = s * kRowBytes + c * 16;
    const bool ok = kb < o.kbytes;
#pragma unroll
    for (int i = 2 * part; i < 2 * part + 2; ++i)
      v[i] = bload128(r, ok ? (rr + 32 * i) * o.ldb + kb : (int)0x80000000u);
  }
  template <class E>
  __device__ __forceinline__ void issue(const Opnd& o, int s, bool live, int tid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_part<E>(o, s, q, live, tid);
  }
  // quarter `part` (0..3) of the stores: register rows 2*part, 2*part+1
  __device__ __forceinline__ void commit_part(lds_t* slab, int part, int tid) const {
    const int c = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int i = 2 * part; i < 2 * part + 2; ++i)
      *(__attribute__((address_space(3))) i32x4*)(slab + swz(rr + 32 * i, c)) = v[i];
  }
  __device__ __forceinline__ void commit(lds_t* slab, int tid) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) commit_part(slab, q, tid);
  }
};

typedef const __attribute__((address_space(3))) i32x4 lds_ci32x4;
typedef const __attribute__((address_space(3))) int lds_cint;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Fragment reader of a K-major slab: one ds_read_b128 per 32-row block.
struct LoadDirect::Frag {
  int off[4];   // per chunk pair p
  __device__ __forceinline__ Frag(int row_base, int lane) {
    const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int p = 0; p < 4; ++p) off[p] = swz(row_base + r32, 2 * p + h);
  }
  __device__ __forceinline__ i32x4 read(const lds_t* slab, int p, int i) const {
    return *(lds_ci32x4*)(slab + off[p] + i * 4096);
  }
  static constexpr int kReads = 1;
};

// K-outer storage, kept K-outer in LDS ("MN-major"): LDS row = one K index
// with the tile's 256 columns contiguous.  The loads are plain 16-byte copies;
// the transpose happens in the fragment read.
//   bf16: 64 K rows of 512 B; chunk c of K row k at chunk c ^ 4(k&3), which
//         keeps the transposing reads below free of bank conflicts.  Thread t
//         copies chunk t % 32 of K rows t / 32 + 8 i.
//   fp32: 32 K rows of 1 KiB, no permutation; thread t copies chunk t % 64 of
//         K rows t / 64 + 4 i.
//   kFar: K * ldb may pass 2^31 bytes; each step then gets a descriptor that
//         starts at its first K row (64-bit base), at a few scalar
//         instructions per step that the common case does without.
template <class E, bool kFar = false> struct LoadMN;

template <bool kFar>
struct LoadMN<BF16, kFar> {
  static constexpr bool kTransposed = true;
  i32x4 v[8];
  template <class E>
  __device__ __forceinline__ void issue_part(const Opnd& o, int s, int part, bool live,
                                             int tid) {
    const int c = tid & 31, kr = tid >> 5;
    if constexpr (kFar) {
      // the descriptor starts at the step's first K row, so the offsets stay
      // below 64 rows; a step that is not `live` gets an empty descriptor
      const int64_t skip = (int64_t)s * BF16::kKStep * o.ldb;
      const int64_t left = o.bytes - skip;
      const rsrc_t r =
          make_rsrc(o.base + skip, live ? (left < 0x7FFFFFFF ? left : 0x7FFFFFFF) : 0);
      const int off = kr * o.ldb + c * 16;
#pragma unroll
      for (int i = 2 * part; i < 2 * part + 2; ++i) v[i] = bload128(r, off + 8 * i * o.ldb);
    } else {
      // one descriptor for the whole operand (K * ldb below 2^31, so live
      // offsets are too); a step that is not `live` reads at 2^31 and up
      // (below 2^32: the rows it adds are within the tile), past the
      // descriptor's end, so it loads zeros
      const rsrc_t r = make_rsrc(o.base, o.bytes < 0x7FFFFFFF ? o.bytes : 0x7FFFFFFF);
      const uint32_t off = live ? (uint32_t)(s * BF16::kKStep + kr) * (uint32_t)o.ldb + c * 16
                                : 0x80000000u;
#pragma unroll
      for (int i = 2 * part; i < 2 * part + 2; ++i)
        v[i] = bload128(r, (int)(off + (uint32_t)(8 * i) * (uint32_t)o.ldb));
    }
  }
  template <class E>
  __device__ __forceinline__ void issue(const Opnd& o, int s, bool live, int tid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_part<E>(o, s, q, live, tid);
  }
  __device__ __forceinline__ void commit_part(lds_t* slab, int part, int tid) const {
    const int c = tid & 31, kr = tid >> 5;
    const int base = kr * 512 + ((c ^ (4 * (kr & 3))) << 4);
#pragma unroll
    for (int i = 2 * part; i < 2 * part + 2; ++i)
      *(__attribute__((address_space(3))) i32x4*)(slab + base + i * 4096) = v[i];
  }
  __device__ __forceinline__ void commit(lds_t* slab, int tid) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) commit_part(slab, q, tid);
  }
  // Lane l = 16 G + j of a wave: the group of 16 reads K rows 8(G/2) + j/4
  // (+ 16 p + 4 r), columns cb + 16 (G&1) + 4 (j&3) .. +3; ds_read_b64_tr_b16
  // then gives lane j the 4 K values of column cb + 16 (G&1) + j, r = 0 the
  // first four of its eight, r = 1 the last four.
  struct Frag {
    int off[4];   // per 32-column block i
    __device__ __forceinline__ Frag(int col_base, int lane) {
      const int G = lane >> 4, j = lane & 15;
      const int k = 8 * (G >> 1) + (j >> 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = col_base + 32 * i + 16 * (G & 1) + 4 * (j & 3);
        off[i] = k * 512 + (((col >> 3) ^ (4 * (k & 3))) << 4) + (col & 7) * 2;
      }
    }
    __device__ __forceinline__ i32x4 read(const lds_t* slab, int p, int i) const {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(slab + off[i] + (16 * p) * 512));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(slab + off[i] + (16 * p + 4) * 512));
      const i32x2 l2 = __builtin_bit_cast(i32x2, lo), h2 = __builtin_bit_cast(i32x2, hi);
      return i32x4{l2[0], l2[1], h2[0], h2[1]};
    }
    static constexpr int kReads = 2;
  };
};

template <bool kFar>
struct LoadMN<F32, kFar> {
  static constexpr bool kTransposed = true;
  i32x4 v[8];
  template <class E>
  __device__ __forceinline__ void issue_part(const Opnd& o, int s, int part, bool live,
                                             int tid) {
    const int c = tid & 63, kr = tid >> 6;
    // descriptors as for bf16
    if constexpr (kFar) {
      const int64_t skip = (int64_t)s * F32::kKStep * o.ldb;
      const int64_t left = o.bytes - skip;
      const rsrc_t r =
          make_rsrc(o.base + skip, live ? (left < 0x7FFFFFFF ? left : 0x7FFFFFFF) : 0);
      const int off = kr * o.ldb + c * 16;
#pragma unroll
      for (int i = 2 * part; i < 2 * part + 2; ++i) v[i] = bload128(r, off + 4 * i * o.ldb);
    } else {
      const rsrc_t r = make_rsrc(o.base, o.bytes < 0x7FFFFFFF ? o.bytes : 0x7FFFFFFF);
      const uint32_t off = live ? (uint32_t)(s * F32::kKStep + kr) * (uint32_t)o.ldb + c * 16
                                : 0x80000000u;
#pragma unroll
      for (int i = 2 * part; i < 2 * part + 2; ++i)
        v[i] = bload128(r, (int)(off + (uint32_t)(4 * i) * (uint32_t)o.ldb));
    }
  }
  template <class E>
  __device__ __forceinline__ void issue(const Opnd& o, int s, bool live, int tid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_part<E>(o, s, q, live, tid);
  }
  __device__ __forceinline__ void commit_part(lds_t* slab, int part, int tid) const {
    const int c = tid & 63, kr = tid >> 6;
#pragma unroll
    for (int i = 2 * part; i < 2 * part + 2; ++i)
      *(__attribute__((address_space(3))) i32x4*)(slab + (kr + 4 * i) * 1024 + c * 16) = v[i];
  }
  __device__ __forceinline__ void commit(lds_t* slab, int tid) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) commit_part(slab, q, tid);
  }
  // lane (column l%32, half h) takes k = 8p + 4h + e, e = 0..3
  struct Frag {
    int off;
    __device__ __forceinline__ Frag(int col_base, int lane) {
      off = 4 * (lane >> 5) * 1024 + (col_base + (lane & 31)) * 4;
    }
    __device__ __forceinline__ i32x4 read(const lds_t* slab, int p, int i) const {
      i32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = *(lds_cint*)(slab + off + (8 * p + e) * 1024 + i * 128);
      return v;
    }
    static constexpr int kReads = 4;
  };
};

// ---------------------------------------------------------------------------
// MFMA on one LDS slab pair.  For chunk pair p (K bytes 32p..32p+31) lane
// half h = lane/32 reads chunk 2p+h of its row: bf16 -> one
// v_mfma_f32_32x32x16_bf16; fp32 -> four v_mfma_f32_32x32x2f32, the j-th using
// the j-th value of the chunk.  A and B use the same (half, value) -> k map,
// so every k of the step is summed exactly once.
// ---------------------------------------------------------------------------
template <class E>
__device__ __forceinline__ void mma(const i32x4& a, const i32x4& b, f32x16& c);

template <>
__device__ __forceinline__ void mma<BF16>(const i32x4& a, const i32x4& b, f32x16& c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                              __builtin_bit_cast(bf16x8, b), c,
                                              0, 0, 0);
}

template <>
__device__ __forceinline__ void mma<F32>(const i32x4& a, const i32x4& b, f32x16& c) {
  const f32x4 af = __builtin_bit_cast(f32x4, a);
  const f32x4 bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[j], bf[j], c, 0, 0, 0);
}

// Fragments of one chunk pair: 4 A blocks and 4 B blocks, 16 B each.
struct Frags {
  i32x4 a[4], b[4];
};

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100,
              kSchedDsWrite = 0x200;

// The fragment reads of chunk pair p+1 are issued before the 16 MFMAs of pair
// p.  `mid(p)` then adds a quarter of the next step's LDS stores and of the
// step after's global loads.  The scheduling groups interleave them with the
// MFMAs: fragment reads over the first eight MFMAs, so that even the
// transposing loaders' two reads per fragment have half a pair to land, and
// stores and loads alternating over the last eight.
template <class E, class FA, class FB, class Mid>
__device__ __forceinline__ void mma_slab(const lds_t* sa, const lds_t* sb, const FA& fa,
                                         const FB& fb, f32x16 (&acc)[4][4], Mid&& mid) {
  constexpr int kDsr = 4 * (FA::kReads + FB::kReads);
  Frags f[2];
  // pair 0: A block 0 and all B blocks first, the order the first MFMAs use
  f[0].a[0] = fa.read(sa, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) f[0].b[j] = fb.read(sb, 0, j);
#pragma unroll
  for (int i = 1; i < 4; ++i) f[0].a[i] = fa.read(sa, 0, i);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (p + 1 < 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) f[(p + 1) & 1].a[i] = fa.read(sa, p + 1, i);
#pragma unroll
      for (int j = 0; j < 4; ++j) f[(p + 1) & 1].b[j] = fb.read(sb, p + 1, j);
    }
    const Frags& c = f[p & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma<E>(c.a[i], c.b[j], acc[i][j]);
    mid(p);
    if constexpr (E::kBytes == 2) {
      // all of pair 0's fragment reads go out before its first MFMA
      if (p == 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kDsr, 0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        // the next pair's fragment reads in the first half (two per MFMA when
        // there are more than 8), the stores and loads in the second
        constexpr int kPer = (kDsr + 7) / 8;
        if (p + 1 < 4 && q < 8) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPer, 0);
        if (q >= 8 && (q & 1) == 0) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
        if (q >= 8 && (q & 1) == 1) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct NoMid {
  __device__ __forceinline__ void operator()(int) const {}
};

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// Full K loop of one tile: acc += A . B^T over `steps` steps.
//
// Software pipeline: global loads run two steps ahead of the MFMAs, into two
// alternating register sets, and land in one of two LDS stages:
//   step s:  MFMAs on LDS stage s%2; between them, quarter by quarter, the
//            stores of regs[(s+1)%2] (step s+1) -> LDS stage (s+1)%2 and the
//            loads of step s+2 -> regs[s%2] (whose step s is already in LDS)
//            barrier
// so a quarter of the loads has one step of MFMA time to arrive before its
// registers are stored.  The loop runs step pairs with one branch-free body.
// Ends with a barrier, so the caller may reuse LDS right after.
template <class E, class LA, class LB>
struct TilePipe {
  LA la[2];
  LB lb[2];
  const Opnd& A;
  const Opnd& B;
  int steps;
  int tid;
  lds_t* sa;
  lds_t* sb;
  typename LA::Frag fa;
  typename LB::Frag fb;

  // `t`: the thread index (see gemm_tile)
  __device__ __forceinline__ TilePipe(const Opnd& a, const Opnd& b, int n, lds_t* smem,
                                      int wm, int wn, int t)
      : A(a), B(b), steps(n), tid(t), sa(smem), sb(smem + 2 * kSlab),
        fa(wm * 128, t & 63), fb(wn * 128, t & 63) {}

  // one step s with s % 2 == k: MFMAs on slab k, the loads of step s + 1 go to
  // slab k ^ 1, the loads of step s + 2 are issued into registers k.  Steps
  // at or past `steps` load zeros, so the loop needs no peeled tail (an odd
  // count runs one all-zero step).
  // kCommit = false: slab k ^ 1 already holds step s + 1 (a prefetched tile's
  // first step)
  template <int k, bool kCommit = true>
  __device__ __forceinline__ void step(int s, f32x16 (&acc)[4][4]) {
    const bool live = s + 2 < steps;
    mma_slab<E>(sa + k * kSlab, sb + k * kSlab, fa, fb, acc, [&](int part) {
      if constexpr (kCommit) {
        la[k ^ 1].commit_part(sa + (k ^ 1) * kSlab, part, tid);
        lb[k ^ 1].commit_part(sb + (k ^ 1) * kSlab, part, tid);
      }
      la[k].template issue_part<E>(A, s + 2, part, live, tid);
      lb[k].template issue_part<E>(B, s + 2, part, live, tid);
    });
    __syncthreads();
  }
  // run() for a tile whose steps 0 and 1 were put into slabs 0 and 1 by
  // prefetch_direct (during the previous tile's epilogue): wait for those
  // loads, then the same loop without the first loads and stores
  __device__ __forceinline__ void run_prefetched(f32x16 (&acc)[4][4]) {
    if (steps <= 0) return;
    __builtin_amdgcn_s_waitcnt(0);   // every counter: the direct-to-LDS loads
    __syncthreads();
    step<0, false>(0, acc);
    step<1>(1, acc);
    for (int s = 2; s < steps; s += 2) {
      step<0>(s, acc);
      step<1>(s + 1, acc);
    }
  }
  __device__ __forceinline__ void run(f32x16 (&acc)[4][4]) {
    if (steps <= 0) return;
    la[0].template issue<E>(A, 0, true, tid);
    lb[0].template issue<E>(B, 0, true, tid);
    // step 1 in the loop's order (A then B, quarter by quarter): the wait
    // before each of the loop's stores is the same on the first pass as on
    // every later one, instead of the deeper wait a different order here
    // would impose on all passes
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      la[1].template issue_part<E>(A, 1, q, steps > 1, tid);
      lb[1].template issue_part<E>(B, 1, q, steps > 1, tid);
      __builtin_amdgcn_sched_barrier(0);
    }
    la[0].commit(sa, tid);
    lb[0].commit(sb, tid);
    __syncthreads();
    for (int s = 0; s < steps; s += 2) {
      step<0>(s, acc);
      step<1>(s + 1, acc);
    }
  }
};

// One tile.  A kernel that runs several tiles in a loop passes the thread
// index through opaque_tid(), so that the loaders' address arithmetic is
// redone per tile instead of being hoisted out of that loop (where it would
// stay live across the loop's epilogue and be spilled).
template <class E, class LA, class LB>
__device__ __forceinline__ void gemm_tile(const Opnd& A, const Opnd& B, int steps,
                                          lds_t* smem, int wm, int wn,
                                          f32x16 (&acc)[4][4], int tid = threadIdx.x) {
  TilePipe<E, LA, LB> pipe(A, B, steps, smem, wm, wn, tid);
  pipe.run(acc);
}

// The second and later tiles of a kernel's tile loop, after prefetch_direct
// put their first two steps into LDS.
template <class E>
__device__ __forceinline__ void gemm_tile_prefetched(const Opnd& A, const Opnd& B, int steps,
                                                     lds_t* smem, int wm, int wn,
                                                     f32x16 (&acc)[4][4], int tid) {
  TilePipe<E, LoadDirect, LoadDirect> pipe(A, B, steps, smem, wm, wn, tid);
  pipe.run_prefetched(acc);
}

// Steps 0 and 1 of a K-contiguous operand straight from memory into LDS
// slabs 0 and 1 of that operand (slab0, slab0 + kSlab), in LoadDirect's
// swizzled layout, with no registers in between (buffer_load_dwordx4 ... lds:
// lane l of a wave writes 16 bytes at the wave's LDS address + 16 l, and an
// offset past the descriptor reads zeros).  Wave w fills rows 64 w .. 64 w +
// 63, eight rows (1 KiB) per instruction: lane l takes row 8 j + l / 8 of its
// block and the chunk whose swizzled slot is l % 8.  Steps at or past
// `steps`, and chunks past the rows' K extent, read zeros, as LoadDirect's.
// Only for slabs nothing else reads or writes until run_prefetched's wait.
__device__ __forceinline__ void prefetch_direct(const Opnd& o, lds_t* slab0, int steps,
                                                int tid) {
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t span = (int64_t)kTile * o.ldb;
  const rsrc_t r = make_rsrc(o.base, o.bytes < span ? o.bytes : span);
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row0 = 64 * w + 8 * j, row = row0 + (lane >> 3);
      const int c = (lane & 7) ^ (row & 7) ^ ((row >> 3) & 1);
      const int kb = s * kRowBytes + c * 16;
      const int off = s < steps && kb < o.kbytes ? row * o.ldb + kb : (int)0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(slab0 + s * kSlab + row0 * kRowBytes), 16,
          off, 0, 0, 0);
    }
}

__device__ __forceinline__ int opaque_tid() {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  __builtin_assume(tid >= 0 && tid < kThreads);
  return tid;
}

// Accumulator element (i, j, r) of lane `lane` in wave (wm, wn) sits at tile
// row  wm*128 + 32i + 8(r/4) + 4(lane/32) + (r%4)  and tile column
// wn*128 + 32j + lane%32  (the 32 x 32 MFMA output layout).
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * 128 + 32 * j + (lane & 31);
}

// Epilogue store of one wave's 128 x 128 quarter of a tile as bf16 rows.
// The accumulator layout gives each lane 4 consecutive values of a row's
// contiguous dimension ("inner" x = 32 i + 8 g + 4 (lane / 32) + q, the tile
// row index) for one row ("outer" o = 32 j + lane % 32, the tile column
// index), so direct stores would scatter 8-byte pieces over 32 rows.  The
// quarter goes through the wave's own 32 KiB of LDS instead ([128 rows][256
// B], 8-byte unit u of row o kept at u ^ (o % 32), conflict-free both ways)
// and leaves as 16-byte chunks, 16 lanes per 256-byte row segment.
//   val(i, j, r) -> float   value of accumulator register (i, j, r)
//   emit(o, x0, v)          store chunk v (8 bf16, inner x0 .. x0 + 7) of row o
// The region must be free (after the K loop's last barrier) and only this
// wave touches it, so no barrier is needed between the two phases.
// begin(j), when given, runs before block j's values are taken (a value that
// depends on the whole block, such as its max); the blocks are then kept
// apart in the schedule, so one block's registers are live at a time.
struct NoBegin {
  __device__ __forceinline__ void operator()(int) const {}
};

template <class Val, class Emit, class Begin = NoBegin>
__device__ __forceinline__ void store_quarter_bf16(lds_t* region, int lane, Val&& val,
                                                   Emit&& emit, Begin&& begin = NoBegin{}) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
  constexpr bool kBegin = !__is_same(__remove_cvref(Begin), NoBegin);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int o = 32 * j + (lane & 31);
    if constexpr (kBegin) {
      __builtin_amdgcn_sched_barrier(0);
      begin(j);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int u = 8 * i + 2 * g + (lane >> 5);
        i32x2 pk;
        pk[0] = pack_bf16(val(i, j, 4 * g), val(i, j, 4 * g + 1));
        pk[1] = pack_bf16(val(i, j, 4 * g + 2), val(i, j, 4 * g + 3));
        *(lds_i32x2*)(region + o * 256 + ((u ^ (o & 31)) << 3)) = pk;
      }
  }
  const int c = lane & 15;
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    const int o = 4 * t + (lane >> 4), x = o & 31;
    i32x4 v = *(const lds_i32x4*)(region + o * 256 + ((c ^ (x >> 1)) << 4));
    if (x & 1) v = i32x4{v[2], v[3], v[0], v[1]};
    emit(o, 8 * c, v);
  }
}

// fp32 counterpart for read-modify-write epilogues: the same quarter, in two
// halves of 64 rows (j = 0, 1 then j = 2, 3) of 512 B each, 16-byte unit u of
// row o kept at u ^ (o % 32).  For every 16-byte chunk (4 fp32, inner x0 ..
// x0 + 3) of row o, `load(o, x0)` fetches the old value (all of a half's
// loads are issued before its LDS traffic) and `store(o, x0, v)` writes v.
// `fix(hf, region)` may change the staged half (rows 64 hf .. 64 hf + 63,
// FP32, laid out as above) between the two phases.  With NoLoad for `load`
// the tile is stored as it is (a plain store through the same layout).
struct NoFix {
  __device__ __forceinline__ void operator()(int, lds_t*) const {}
};
struct NoLoad {
  __device__ __forceinline__ f32x4 operator()(int, int) const {
    return f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

template <class Load, class Store, class Fix>
__device__ __forceinline__ void rmw_quarter_f32(lds_t* region, int lane,
                                                const f32x16 (&acc)[4][4], Load&& load,
                                                Store&& store, Fix&& fix) {
  typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
  const int c = lane & 31;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f32x4 old[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) old[t] = load(64 * hf + 2 * t + (lane >> 5), 4 * c);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * hf + jj, o = 32 * jj + (lane & 31);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int u = 8 * i + 2 * g + (lane >> 5);
          const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                           acc[i][j][4 * g + 3]};
          *(lds_i32x4*)(region + o * 512 + ((u ^ (o & 31)) << 4)) = __builtin_bit_cast(i32x4, v);
        }
    }
    fix(hf, region);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int o = 2 * t + (lane >> 5);
      const f32x4 v = __builtin_bit_cast(
          f32x4, *(const lds_i32x4*)(region + o * 512 + ((c ^ (o & 31)) << 4)));
      if constexpr (__is_same(__remove_cvref(Load), NoLoad))
        store(64 * hf + o, 4 * c, v);
      else
        store(64 * hf + o, 4 * c, f32x4{old[t][0] + v[0], old[t][1] + v[1], old[t][2] + v[2],
                                        old[t][3] + v[3]});
    }
  }
}

template <class Load, class Store>
__device__ __forceinline__ void rmw_quarter_f32(lds_t* region, int lane,
                                                const f32x16 (&acc)[4][4], Load&& load,
                                                Store&& store) {
  rmw_quarter_f32(region, lane, acc, load, store, NoFix{});
}

// Maps a launch index to a work item so that items i, i+1, ... run on the same
// XCD: workgroups are handed to the 8 XCDs round-robin, so block b lands on XCD
// b % 8; grouping by b % 8 keeps neighbouring items (which share an operand
// slice) inside one XCD's L2.  `nblocks` is a multiple of 8.
__device__ __forceinline__ int xcd_item(int b, int nblocks) {
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

// Work item of block b (counted from the first block of its kind, which
// starts on XCD 0) when only `real` of the launched blocks have work, a count
// the device learns at run time (the launch is sized for the bound): the
// items go to the first real rounded up to 8 blocks, XCD by XCD, so every XCD
// gets the same share.  -1: no work.
__device__ __forceinline__ int live_item(int b, int real) {
  const int real8 = (real + 7) & ~7;
  if (b >= real8) return -1;
  const int item = xcd_item(b, real8);
  return item < real ? item : -1;
}

// Grouped tile order over an R x C item grid: items run through groups of
// kGroup consecutive rows, column by column inside a group.  The 32 workgroups
// an XCD runs at once then cover a 4 x 8 block of tiles, so each of the 4 row
// panels and each of the 8 column panels is fetched once into that XCD's L2
// and reused by the other tiles of the block.
#ifndef FLCE_GROUP
#define FLCE_GROUP 4
#endif
constexpr int kGroup = FLCE_GROUP;
__device__ __forceinline__ void grouped(int item, int R, int C, int& r, int& c) {
  const int group = item / (kGroup * C);
  const int r0 = group * kGroup;
  const int gsz = min(R - r0, kGroup);
  const int local = item - group * kGroup * C;
  r = r0 + local % gsz;
  c = local / gsz;
}

}  // namespace flce
