// Measurement probes (include/rlk_probes.h): the HBM streaming-read rate and the sustained
// bf16 MFMA rate that this chip reaches outside the logprob kernels, so that the benchmark
// can state each kernel's rate against what is achievable as well as against the peak.

#include <hip/hip_runtime.h>

#include <cstring>
#include <stdint.h>

#include "rlk_probes.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kReadBlocks = 2048;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const f32x4* __restrict__ p,
                                                                int64_t n, float* sink) {
  float s = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)kReadBlocks * kThreads) {
    const f32x4 v = __builtin_nontemporal_load(p + i);
    s += (v.x + v.y) + (v.z + v.w);
  }
  if (s == 1234.5f) sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// Finite pseudo-random bf16 bits in (-2, 2): a 32-bit mix of (seed, index) for the
// mantissa and sign, exponent drawn from [2^-4, 2^0].
__device__ __forceinline__ uint16_t random_bf16(uint32_t seed, uint32_t i) {
  uint32_t h = (i + 0x9e3779b9u * (seed + 1u)) * 2654435761u;
  h ^= h >> 15;
  h *= 0x2c1b3c6du;
  h ^= h >> 12;
  const uint32_t sign = (h >> 31) << 15;
  const uint32_t exp = 123u + ((h >> 7) % 5u);  // 2^-4 .. 2^0
  return (uint16_t)(sign | (exp << 7) | (h & 0x7fu));
}

__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int iters, uint32_t seed,
                                                               float* sink) {
  const uint32_t gid = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 A[4], B[2];
#pragma unroll
  for (int f = 0; f < 6; ++f) {
    uint16_t bits[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bits[j] = random_bf16(seed, (gid * 6u + f) * 8u + j);
    const bf16x8 v = __builtin_bit_cast(bf16x8, bits);
    if (f < 4) A[f] = v; else B[f - 4] = v;
  }
  floatx16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  for (int it = 0; it < iters; it += 4) {
    // Four steps with the A fragments rotated by r and the B fragments by r % 2: every MFMA
    // of a step sees other data than in the step before.
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[(a + r) & 3], B[(b + r) & 1],
                                                              acc[a][b], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) s += acc[a][b][i];
  sink[gid] = s;
}

}  // namespace

extern "C" {

int rlk_probe_stream_read(const void* buf, size_t bytes, float* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(buf) % 16) != 0)
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kReadBlocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const f32x4*>(buf),
                     (int64_t)(bytes / 16), sink);
  return (int)hipGetLastError();
}

int rlk_probe_mfma(int32_t blocks, int32_t iters, uint32_t seed, float* sink, void* stream) {
  if (!sink || blocks < 1 || blocks > (1 << 20) || iters < 4 || iters % 4 != 0) return -1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), iters, seed, sink);
  return (int)hipGetLastError();
}

int rlk_probe_device_info(int32_t* compute_units, int32_t* engine_clock_khz,
                          int32_t* memory_clock_khz, int32_t* memory_bus_bits, char* arch,
                          size_t arch_len) {
  if (!compute_units || !engine_clock_khz || !memory_clock_khz || !memory_bus_bits || !arch ||
      arch_len == 0)
    return -1;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return (int)e;
  *compute_units = prop.multiProcessorCount;
  *engine_clock_khz = prop.clockRate;
  *memory_clock_khz = prop.memoryClockRate;
  *memory_bus_bits = prop.memoryBusWidth;
  std::strncpy(arch, prop.gcnArchName, arch_len - 1);
  arch[arch_len - 1] = '\0';
  return 0;
}

}  // extern "C"
