// mfma_ceiling.hip -- how much bf16 MFMA throughput the chip sustains with no
// memory traffic at all, as a function of the operand data.  Context for the
// roofline of the contraction kernels: the published dense peak assumes the
// top clock, and the clock a matrix-core load holds depends on how much the
// operand bits toggle.
//
// Every compute unit runs one 256-thread workgroup (one wave per SIMD), each
// wave a 128 x 128 block of FP32 accumulators (all 256 AGPRs, as the
// contraction tiles): 16 accumulators of v_mfma_f32_32x32x16_bf16 fed from 4 A
// and 4 B fragments, or 64 of v_mfma_f32_16x16x32_bf16 fed from 8 + 8, held in
// registers, every MFMA pairing a different (A, B) combination.  Three operand
// sets: constant 1.0; random sign and mantissa at one exponent; random sign,
// mantissa and exponent over eight binades (values of magnitude 2^-7 .. 2^1,
// like the inputs of a normalised LM head).  Each run lasts a few seconds of
// back-to-back launches (the clock settles within the first); the rate is
// the MFMA work over the elapsed time.  Prints a markdown table.
#include <hip/hip_runtime.h>
#include <stdio.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr double kPeakTflops = 2500.0;   // MI355X dense bf16
constexpr double kTopClockGHz = 2.4;

__device__ unsigned mix32(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// two bf16 values per 32-bit word; mode 0: 1.0, 1: random sign and
// mantissa, exponent 2^-7; 2: random sign, mantissa and 3 exponent bits
__device__ unsigned operand_bits(int mode, unsigned seed) {
  if (mode == 0) return 0x3F803F80u;
  const unsigned h = mix32(seed);
  const unsigned keep = mode == 1 ? 0x807F807Fu : 0x83FF83FFu;
  return (h & keep) | 0x3C003C00u;
}

// 16x16x32 form: 64 accumulators of 4 floats, 8 A and 8 B fragments
__global__ __launch_bounds__(kThreads) void k_mfma16(float* out, int iters, int mode) {
  f32x4 acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const unsigned t = blockIdx.x * kThreads + threadIdx.x;
  i32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[i][q] = (int)operand_bits(mode, t * 128 + i * 8 + q);
      b[i][q] = (int)operand_bits(mode, t * 128 + 64 + i * 8 + q);
    }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[8 * i + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]), acc[8 * i + j],
            0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[t] = s;
}

__global__ __launch_bounds__(kThreads) void k_mfma(float* out, int iters, int mode) {
  f32x16 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  const unsigned t = blockIdx.x * kThreads + threadIdx.x;
  i32x4 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[i][q] = (int)operand_bits(mode, t * 64 + i * 8 + q);
      b[i][q] = (int)operand_bits(mode, t * 64 + 32 + i * 8 + q);
    }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[4 * i + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]), acc[4 * i + j],
            0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  out[t] = s;   // keeps the work live; one float per thread of the grid
}

static bool ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

// Runs `mode` with the 32x32x16 (shape 32) or 16x16x32 (shape 16) form for
// about `seconds`; returns the rate in TFLOP/s (< 0: error).  Per wave and
// iteration: 16 x 32x32x16 = a 128 x 128 x 16 block (2^19 flop), or
// 64 x 16x16x32 = a 128 x 128 x 32 block (2^20 flop).
static void launch(int shape, int blocks, float* out, int iters, int mode) {
  if (shape == 16)
    hipLaunchKernelGGL(k_mfma16, dim3(blocks), dim3(kThreads), 0, 0, out, iters, mode);
  else
    hipLaunchKernelGGL(k_mfma, dim3(blocks), dim3(kThreads), 0, 0, out, iters, mode);
}

static double run(int shape, int mode, int blocks, float* out, double seconds) {
  hipEvent_t e0, e1;
  if (!ok(hipEventCreate(&e0), "event") || !ok(hipEventCreate(&e1), "event")) return -1;
  // calibrate the iteration count to ~10 ms per launch
  int iters = 2000;
  float ms = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    if (!ok(hipEventRecord(e0, 0), "event record")) return -1;
    launch(shape, blocks, out, iters, mode);
    if (!ok(hipEventRecord(e1, 0), "event record") || !ok(hipEventSynchronize(e1), "launch") ||
        !ok(hipEventElapsedTime(&ms, e0, e1), "elapsed"))
      return -1;
  }
  double it = iters * 10.0 / (ms > 0.f ? ms : 1.f);
  iters = it > 2e6 ? 2000000 : (it < 1 ? 1 : (int)it);
  const int reps = (int)(seconds * 100.0);
  if (!ok(hipEventRecord(e0, 0), "event record")) return -1;
  for (int r = 0; r < reps; ++r) launch(shape, blocks, out, iters, mode);
  if (!ok(hipEventRecord(e1, 0), "event record") || !ok(hipEventSynchronize(e1), "timed launches") ||
      !ok(hipEventElapsedTime(&ms, e0, e1), "elapsed"))
    return -1;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  const double per_iter = shape == 16 ? 1048576.0 : 524288.0;
  const double flop = (double)reps * blocks * (kThreads / 64) * (double)iters * per_iter;
  return flop / (ms * 1e-3) / 1e12;
}

int main() {
  setvbuf(stdout, NULL, _IONBF, 0);
  int dev = 0, cus = 0;
  if (!ok(hipGetDevice(&dev), "device") ||
      !ok(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "CUs"))
    return 1;
  float* out = nullptr;
  if (!ok(hipMalloc(&out, sizeof(float) * cus * kThreads), "hipMalloc")) return 1;
  const char* names[3] = {"constant operands (1.0)",
                          "random sign and mantissa, one exponent (2^-7)",
                          "random sign, mantissa and exponent (2^-7 .. 2^1)"};
  printf("| instruction | operands | TFLOP/s | %% of %.0f TFLOP/s | clock at 100 %% busy (GHz) |\n",
         kPeakTflops);
  printf("|---|---|---|---|---|\n");
  int rc = 0;
  const int runs[7][2] = {{32, 0}, {32, 1}, {32, 2}, {16, 0}, {16, 1}, {16, 2}, {32, 2}};
  for (const auto& sm : runs) {
    const double r = run(sm[0], sm[1], cus, out, 3.0);
    if (r < 0) {
      rc = 1;
      break;
    }
    printf("| %s | %s | %.0f | %.1f | %.2f |\n",
           sm[0] == 32 ? "v_mfma_f32_32x32x16_bf16" : "v_mfma_f32_16x16x32_bf16", names[sm[1]],
           r, 100.0 * r / kPeakTflops, kTopClockGHz * r / kPeakTflops);
  }
  (void)hipFree(out);
  return rc;
}
