// svdq_probe.hip -- measurement hooks of the C ABI (include/svdq.h): the
// shader clock a compute unit runs at, and the sustained rate of the scaled
// FP4 matrix instruction the MXFP4 GEMM is built on.  Not part of any
// forward; they exist so a benchmark can state what clock and what matrix
// rate the chip sustained next to the GEMM's own numbers.
//
// Both count shader-clock cycles with s_memtime and wall time with
// s_memrealtime (a constant-rate counter whose frequency the runtime
// reports as hipDeviceAttributeWallClockRate) on wave 0 of every workgroup.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "svdq.h"

// Target of a store that keeps the MFMA probe's results live (external
// linkage, so the compiler cannot treat the store as dead).
__device__ float svdq_probe_sink[64];

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kProbeSlots = 4096;   // workgroups recorded (one per compute unit is launched)

// per workgroup: wall clock and shader clock at the start, then at the end
__device__ unsigned long long probe_ticks[kProbeSlots][4];

// A spin of dependent integer adds (no memory traffic), timed by both counters.
__global__ __launch_bounds__(64) void k_probe_clock(int iters, unsigned seed) {
  unsigned x = seed + threadIdx.x;
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime(), c0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < iters; ++i) x = x * 1664525u + 1013904223u;
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime(), c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0 && blockIdx.x < kProbeSlots) {
    probe_ticks[blockIdx.x][0] = r0;
    probe_ticks[blockIdx.x][1] = c0;
    probe_ticks[blockIdx.x][2] = r1 + (x == 0xFFFFFFFFu ? 1u : 0u);   // keeps the spin live
    probe_ticks[blockIdx.x][3] = c1;
  }
}

// Eight waves per compute unit (two per SIMD), each issuing independent
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 (E2M1 operands, e8m0 scale 1.0) into 9
// accumulators: operands from a generator (fill = 0: zero codes, the
// cheapest case for the matrix core's power; else pseudo-random codes).
__global__ __launch_bounds__(512) void k_probe_mfma(int iters, unsigned fill) {
  const int lane = threadIdx.x & 63;
  unsigned x = fill * (0x9E3779B9u + threadIdx.x * 2654435761u + blockIdx.x * 40503u);
  auto next = [&]() { x = x * 1664525u + 1013904223u; return fill ? int(x) : 0; };
  const i32x8 a = {next(), next(), next(), next(), 0, 0, 0, 0};
  const i32x8 b = {next(), next(), next(), next(), 0, 0, 0, 0};
  const int s1 = 0x7F7F7F7F;   // e8m0 127 = 2^0 in every byte
  f32x16 acc[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) acc[i] = f32x16{};
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime(), c0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 9; ++i) acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], 4, 4, 0, s1, 0, s1);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 9; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[i][e];
  // the sums are stored (every workgroup's wave 0 writes the same 64 floats;
  // their values do not matter), so the loop cannot be dropped, and the end
  // of the timed region follows the store
  if (threadIdx.x < 64) svdq_probe_sink[lane] = s;
  // the two waves on a SIMD share its matrix core (the older one runs ahead),
  // so the workgroup ends with its last wave
  __syncthreads();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime(), c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0 && blockIdx.x < kProbeSlots) {
    probe_ticks[blockIdx.x][0] = r0;
    probe_ticks[blockIdx.x][1] = c0;
    probe_ticks[blockIdx.x][2] = r1;
    probe_ticks[blockIdx.x][3] = c1;
  }
}

std::mutex g_probe_mu;   // the probes share one result array per device

// Sums over workgroups of their own wall ticks and shader cycles, and the
// span from the first start to the last end in wall ticks (the launch may
// not hold every workgroup at once, so rates are taken over the span).
svdq_status read_ticks(int nblocks, double* wall_ticks, double* cycles, double* span_ticks) {
  std::vector<unsigned long long> t(size_t(nblocks) * 4);
  if (hipMemcpyFromSymbol(t.data(), HIP_SYMBOL(probe_ticks), t.size() * sizeof(unsigned long long), 0,
                          hipMemcpyDeviceToHost) != hipSuccess)
    return SVDQ_ERR_HIP;
  double w = 0.0, c = 0.0;
  unsigned long long first = ~0ull, last = 0ull;
  for (int b = 0; b < nblocks; ++b) {
    w += double(t[4 * b + 2] - t[4 * b]);
    c += double(t[4 * b + 3] - t[4 * b + 1]);
    first = t[4 * b] < first ? t[4 * b] : first;
    last = t[4 * b + 2] > last ? t[4 * b + 2] : last;
  }
  *wall_ticks = w;
  *cycles = c;
  *span_ticks = last > first ? double(last - first) : 0.0;
  return SVDQ_OK;
}

svdq_status device_info(int* cus, double* wall_hz) {
  int dev = 0, v = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SVDQ_ERR_HIP;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return SVDQ_ERR_HIP;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) return SVDQ_ERR_HIP;
  *cus = v < kProbeSlots ? v : kProbeSlots;
  *wall_hz = double(khz) * 1e3;
  return SVDQ_OK;
}

}  // namespace

extern "C" svdq_status svdq_probe_clock(hipStream_t stream, double* mhz) {
  if (!mhz) return SVDQ_ERR_INVALID_ARG;
  int cus = 0;
  double wall_hz = 0.0;
  svdq_status st = device_info(&cus, &wall_hz);
  if (st != SVDQ_OK) return st;
  std::lock_guard<std::mutex> lock(g_probe_mu);
  hipLaunchKernelGGL(k_probe_clock, dim3(unsigned(cus)), dim3(64), 0, stream, 20000, 7u);
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(stream) != hipSuccess) return SVDQ_ERR_HIP;
  double w = 0.0, c = 0.0, span = 0.0;
  if ((st = read_ticks(cus, &w, &c, &span)) != SVDQ_OK) return st;
  if (w <= 0.0) return SVDQ_ERR_NUMERIC;
  *mhz = c / w * wall_hz * 1e-6;
  return SVDQ_OK;
}

extern "C" svdq_status svdq_probe_mfma_rate(int random_operands, int iters, hipStream_t stream, double* tflops,
                                            double* mhz) {
  if (!tflops || !mhz || iters <= 0 || iters > (1 << 24)) return SVDQ_ERR_INVALID_ARG;
  int cus = 0;
  double wall_hz = 0.0;
  svdq_status st = device_info(&cus, &wall_hz);
  if (st != SVDQ_OK) return st;
  std::lock_guard<std::mutex> lock(g_probe_mu);
  hipLaunchKernelGGL(k_probe_mfma, dim3(unsigned(cus)), dim3(512), 0, stream, iters, random_operands ? 1u : 0u);
  if (hipGetLastError() != hipSuccess || hipStreamSynchronize(stream) != hipSuccess) return SVDQ_ERR_HIP;
  double w = 0.0, c = 0.0, span = 0.0;
  if ((st = read_ticks(cus, &w, &c, &span)) != SVDQ_OK) return st;
  if (w <= 0.0 || span <= 0.0) return SVDQ_ERR_NUMERIC;
  const double secs = span / wall_hz;
  const double flops = double(cus) * 8.0 * double(iters) * 9.0 * 2.0 * 32.0 * 32.0 * 64.0;
  *tflops = flops / secs * 1e-12;
  *mhz = c / w * wall_hz * 1e-6;
  return SVDQ_OK;
}
