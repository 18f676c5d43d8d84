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
// Inside LDS every operand row is K-contiguous, so one ds_read_b128 hands a
// lane the 8 bf16 (or 4 fp32) K-values an MFMA lane expects.  The 16-byte chunk
// c of row r is stored at a row-dependent XOR-permuted chunk position so that
// the lanes one LDS cycle serves touch distinct bank groups for fragment
// reads and for stores; see swz() for the exact pattern.
//
// Global memory is read with raw buffer loads whose descriptor covers exactly
// [base, end of tensor): a read past the end returns 0 in hardware, so ragged
// vocabulary / row tails need no branch and can never fault.  Two loaders:
//   * LoadDirect  -- the operand is stored with K contiguous (row-major
//                    [rows][K]), e.g. W [V, H] or X [N, H] contracted over H;
//   * LoadTrans*  -- the operand is stored with K as the outer index
//                    ([K][rows]), e.g. X [N, H] or W [V, H] contracted over N
//                    or V.  Each thread reads an E x E block (E = 16 / bytes
//                    per element) with E row loads of 16 B, transposes it in
//                    registers (v_perm_b32 for bf16, plain moves for fp32) and
//                    writes E K-contiguous chunks.
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

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  uint32_t n = bytes <= 0 ? 0u
             : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)n, kRsrcWord3);
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
  i32x4 v[8];
  // kTail: the step may run past the end of the rows' K extent; chunks beyond
  // it are replaced by zeros (they would hold the next row's values).
  // quarter `part` (0..3) of the loads: register rows 2*part, 2*part+1
  template <class E, bool kTail>
  __device__ __forceinline__ void issue_part(const Opnd& o, int s, int part) {
    const int c = threadIdx.x & 7, rr = threadIdx.x >> 3;
    const rsrc_t r = make_rsrc(o.base, o.bytes);
    const int kb = s * kRowBytes + c * 16;
#pragma unroll
    for (int i = 2 * part; i < 2 * part + 2; ++i) {
      v[i] = bload128(r, (rr + 32 * i) * o.ldb + kb);
      if constexpr (kTail) {
        const bool ok = kb < o.kbytes;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[i][q] = ok ? v[i][q] : 0;
      }
    }
  }
  template <class E, bool kTail>
  __device__ __forceinline__ void issue(const Opnd& o, int s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_part<E, kTail>(o, s, q);
  }
  // quarter `part` (0..3) of the stores: register rows 2*part, 2*part+1
  __device__ __forceinline__ void commit_part(lds_t* slab, int part) const {
    const int c = threadIdx.x & 7, rr = threadIdx.x >> 3;
#pragma unroll
    for (int i = 2 * part; i < 2 * part + 2; ++i)
      *(__attribute__((address_space(3))) i32x4*)(slab + swz(rr + 32 * i, c)) = v[i];
  }
  __device__ __forceinline__ void commit(lds_t* slab) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) commit_part(slab, q);
  }
};

// bf16, K-outer storage: thread (kb = t % 8, mb = t / 8) reads K rows
// 8kb..8kb+7 of columns 8mb..8mb+7 and writes rows 8mb+i, chunk kb.
struct LoadTransBF16 {
  static constexpr bool kTransposed = true;
  i32x4 v[8];
  template <class E, bool kTail>
  __device__ __forceinline__ void issue_part(const Opnd& o, int s, int part) {
    const int kb = threadIdx.x & 7, mb = threadIdx.x >> 3;
    const int64_t k0 = (int64_t)s * BF16::kKStep;
    const rsrc_t r = make_rsrc(o.base + k0 * o.ldb, o.bytes - k0 * o.ldb);
#pragma unroll
    for (int j = 2 * part; j < 2 * part + 2; ++j)
      v[j] = bload128(r, (kb * 8 + j) * o.ldb + mb * 16);
  }
  template <class E, bool kTail>
  __device__ __forceinline__ void issue(const Opnd& o, int s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_part<E, kTail>(o, s, q);
  }
  __device__ __forceinline__ void commit(lds_t* slab) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) commit_part(slab, q);
  }
  __device__ __forceinline__ void commit_part(lds_t* slab, int part) const {
    const int kb = threadIdx.x & 7, mb = threadIdx.x >> 3;
#pragma unroll
    for (int i = 2 * part; i < 2 * part + 2; ++i) {
      const unsigned sel = (i & 1) ? 0x07060302u : 0x05040100u;
      i32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = (int)__builtin_amdgcn_perm((unsigned)v[2 * q + 1][i >> 1],
                                          (unsigned)v[2 * q][i >> 1], sel);
      *(__attribute__((address_space(3))) i32x4*)(slab + swz(mb * 8 + i, kb)) = o;
    }
  }
};

// fp32, K-outer storage: two 4 x 4 blocks per thread.
struct LoadTransF32 {
  static constexpr bool kTransposed = true;
  i32x4 v[8];
  template <class E, bool kTail>
  __device__ __forceinline__ void issue_part(const Opnd& o, int s, int part) {
    const int64_t k0 = (int64_t)s * F32::kKStep;
    const rsrc_t r = make_rsrc(o.base + k0 * o.ldb, o.bytes - k0 * o.ldb);
    const int blk = part >> 1;
    const int b = threadIdx.x + kThreads * blk;
    const int kb = b & 7, mb = b >> 3;
#pragma unroll
    for (int j = 2 * (part & 1); j < 2 * (part & 1) + 2; ++j)
      v[blk * 4 + j] = bload128(r, (kb * 4 + j) * o.ldb + mb * 16);
  }
  template <class E, bool kTail>
  __device__ __forceinline__ void issue(const Opnd& o, int s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_part<E, kTail>(o, s, q);
  }
  __device__ __forceinline__ void commit(lds_t* slab) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) commit_part(slab, q);
  }
  __device__ __forceinline__ void commit_part(lds_t* slab, int part) const {
    const int blk = part >> 1;
    {
      const int b = threadIdx.x + kThreads * blk;
      const int kb = b & 7, mb = b >> 3;
#pragma unroll
      for (int i = 2 * (part & 1); i < 2 * (part & 1) + 2; ++i) {
        i32x4 o = {v[blk * 4 + 0][i], v[blk * 4 + 1][i], v[blk * 4 + 2][i],
                   v[blk * 4 + 3][i]};
        *(__attribute__((address_space(3))) i32x4*)(slab + swz(mb * 4 + i, kb)) = o;
      }
    }
  }
};

template <class E> struct TransLoader;
template <> struct TransLoader<BF16> { using type = LoadTransBF16; };
template <> struct TransLoader<F32> { using type = LoadTransF32; };

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

// Per-lane LDS byte offsets of the fragment rows for chunk pair p, relative to
// an operand slab.  Block mb (or nb) adds mb * 32 rows = mb * 4096 bytes.
struct FragOffsets {
  int a[4], b[4];
  __device__ __forceinline__ FragOffsets(int wm, int wn) {
    const int lane = threadIdx.x & 63, r32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      a[p] = swz(wm * 128 + r32, 2 * p + h);
      b[p] = swz(wn * 128 + r32, 2 * p + h);
    }
  }
};

// Fragments of one chunk pair: 4 A blocks and 4 B blocks, 16 B each.
struct Frags {
  i32x4 a[4], b[4];
  __device__ __forceinline__ void load(const lds_t* sa, const lds_t* sb,
                                       const FragOffsets& fo, int p) {
    typedef const __attribute__((address_space(3))) i32x4 lv;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(lv*)(sa + fo.a[p] + i * 4096);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *(lv*)(sb + fo.b[p] + j * 4096);
  }
};

// The reads of chunk pair p+1 are issued before the 16 MFMAs of pair p; a
// scheduling barrier after each pair keeps the compiler from hoisting every
// read of the slab up front (which would need 128 fragment registers).
// `mid(p)` runs after the MFMAs of pair p are issued: the main loop stores a
// quarter of the next step's operands to LDS there while those MFMAs execute.
// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100,
              kSchedDsWrite = 0x200;

template <class E, bool kInterleave, class Mid>
__device__ __forceinline__ void mma_slab(const lds_t* sa, const lds_t* sb,
                                         const FragOffsets& fo,
                                         f32x16 (&acc)[4][4], Mid&& mid) {
  Frags f[2];
  f[0].load(sa, sb, fo, 0);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (p + 1 < 4) f[(p + 1) & 1].load(sa, sb, fo, p + 1);
    const Frags& c = f[p & 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma<E>(c.a[i], c.b[j], acc[i][j]);
    mid(p);
    // one memory instruction between consecutive MFMAs: the 8 fragment reads
    // of the next pair, then the pair's share of LDS stores and global loads
    // (not when both operands are transposed: their stores wait on VALU
    // permutes and are better left in a cluster)
    if constexpr (E::kBytes == 2 && kInterleave) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
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

// Full K loop of one tile: acc += A . B^T over `steps` steps; `tail` says the
// last step may cross the end of the K extent (direct operands only).
//
// Software pipeline: global loads run two steps ahead of the MFMAs, into two
// alternating register sets, and land in one of two LDS stages:
//   step s:  issue loads of step s+2 -> regs[s%2]   (their old content, step s,
//                                                    is already in LDS)
//            MFMAs on LDS stage s%2, with the stores of regs[(s+1)%2]
//            (step s+1) -> LDS stage (s+1)%2 interleaved between them
//            barrier
// so every load has about two steps of MFMA time to arrive.  The steady-state
// loop runs step pairs with no branch inside; the last 1-3 steps are peeled.
// Ends with a barrier, so the caller may reuse LDS right after.
template <class E, class LA, class LB>
struct TilePipe {
  LA la[2];
  LB lb[2];
  const Opnd& A;
  const Opnd& B;
  int steps;
  bool tail;
  lds_t* sa;
  lds_t* sb;
  const FragOffsets& fo;

  __device__ __forceinline__ TilePipe(const Opnd& a, const Opnd& b, int n, bool t,
                                      lds_t* smem, const FragOffsets& f)
      : A(a), B(b), steps(n), tail(t), sa(smem), sb(smem + 2 * kSlab), fo(f) {}

  template <int k>
  __device__ __forceinline__ void issue(int s) {
    if (tail && s == steps - 1) {
      la[k].template issue<E, true>(A, s);
      lb[k].template issue<E, true>(B, s);
    } else {
      la[k].template issue<E, false>(A, s);
      lb[k].template issue<E, false>(B, s);
    }
  }
  template <int k>
  __device__ __forceinline__ void commit() {
    la[k].commit(sa + k * kSlab);
    lb[k].commit(sb + k * kSlab);
  }
  // one step s with s % 2 == k
  template <int k>
  __device__ __forceinline__ void issue_part(int s, int part) {
    if (tail && s == steps - 1) {
      la[k].template issue_part<E, true>(A, s, part);
      lb[k].template issue_part<E, true>(B, s, part);
    } else {
      la[k].template issue_part<E, false>(A, s, part);
      lb[k].template issue_part<E, false>(B, s, part);
    }
  }
  static constexpr bool kInterleave = !(LA::kTransposed && LB::kTransposed);
  template <int k, bool kIssue, bool kCommit>
  __device__ __forceinline__ void step(int s, f32x16 (&acc)[4][4]) {
    if constexpr (kIssue && !kInterleave) {
      issue<k>(s + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    mma_slab<E, kInterleave>(sa + k * kSlab, sb + k * kSlab, fo, acc, [&](int part) {
      if constexpr (kCommit) {
        la[k ^ 1].commit_part(sa + (k ^ 1) * kSlab, part);
        lb[k ^ 1].commit_part(sb + (k ^ 1) * kSlab, part);
      }
      if constexpr (kIssue && kInterleave) issue_part<k>(s + 2, part);
    });
    __syncthreads();
  }
  __device__ __forceinline__ void run(f32x16 (&acc)[4][4]) {
    if (steps <= 0) return;
    issue<0>(0);
    if (steps > 1) issue<1>(1);
    commit<0>();
    __syncthreads();
    int s = 0;
    for (; s + 3 < steps; s += 2) {
      step<0, true, true>(s, acc);
      step<1, true, true>(s + 1, acc);
    }
    const int rem = steps - s;   // 1, 2 or 3, s even
    if (rem == 3) {
      step<0, true, true>(s, acc);
      step<1, false, true>(s + 1, acc);
      step<0, false, false>(s + 2, acc);
    } else if (rem == 2) {
      step<0, false, true>(s, acc);
      step<1, false, false>(s + 1, acc);
    } else {
      step<0, false, false>(s, acc);
    }
  }
};

template <class E, class LA, class LB>
__device__ __forceinline__ void gemm_tile(const Opnd& A, const Opnd& B, int steps,
                                          bool tail, lds_t* smem, const FragOffsets& fo,
                                          f32x16 (&acc)[4][4]) {
  TilePipe<E, LA, LB> pipe(A, B, steps, tail, smem, fo);
  pipe.run(acc);
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

// Maps a launch index to a work item so that items i, i+1, ... run on the same
// XCD: workgroups are handed to the 8 XCDs round-robin, so block b lands on XCD
// b % 8; grouping by b % 8 keeps neighbouring items (which share an operand
// slice) inside one XCD's L2.  `nblocks` is a multiple of 8.
__device__ __forceinline__ int xcd_item(int b, int nblocks) {
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

// Grouped tile order over an R x C item grid: items run through groups of
// kGroup consecutive rows, column by column inside a group.  The 32 workgroups
// an XCD runs at once then cover a 4 x 8 block of tiles, so each of the 4 row
// panels and each of the 8 column panels is fetched once into that XCD's L2
// and reused by the other tiles of the block.
constexpr int kGroup = 4;
__device__ __forceinline__ void grouped(int item, int R, int C, int& r, int& c) {
  const int group = item / (kGroup * C);
  const int r0 = group * kGroup;
  const int gsz = min(R - r0, kGroup);
  const int local = item - group * kGroup * C;
  r = r0 + local % gsz;
  c = local / gsz;
}

// float -> bfloat16 bits, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf2f(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

}  // namespace flce
