// Train-vs-rollout selected-logprob comparison: counts, max and means over active tokens.
//
// The figures are those of the RL-Kernel h100-pcp.json evidence page (the
// train_rollout_logprob block and the runtime_scalar_logprob rows) and of the RL-Kernel
// issue #342 runbook (section 2, per-row selected-logprob comparison): with
// d = train - rollout in fp64 over the active tokens,
//   active_tokens, mismatch_count (train != rollout as values), bitwise_mismatch_count,
//   max |d|, mean |d|, mismatch_kl = mean(-d), mismatch_k3_kl = mean(expm1(d) - d).
//
// Fixed reduction order, independent of the device and of what else runs: a workgroup of
// 256 threads owns tokens [4096 b, 4096 b + 4096); thread t folds tokens 4096 b + t + 256 k
// for k = 0..15 in increasing k; the 64 lanes of a wave combine by an xor butterfly
// (strides 32..1, lower lane first), the four waves as ((0,1),(2,3)).  The block partials
// are folded the same way by one workgroup (thread t takes blocks t, t + 256, ... in
// order).  Counts are exact integers and the maximum is exact; the sums are fp64.  No
// atomics.  The stream is HBM-bound (9 bytes per token) and tiny next to the logprob pass.

#include "rlk_launch.hpp"

namespace rlk {

namespace {

constexpr int kCmpThreads = 256;
constexpr int kCmpPerThread = 16;
constexpr int kCmpTokensPerBlock = kCmpThreads * kCmpPerThread;

struct Partial {
  long long n, mism, bitw;
  int nan;   // a NaN d among the active tokens
  int pad;
  double maxabs, sabs, sk1, sk3;
};

__device__ __forceinline__ Partial zero_partial() {
  Partial p;
  p.n = p.mism = p.bitw = 0;
  p.nan = 0;
  p.pad = 0;
  p.maxabs = p.sabs = p.sk1 = p.sk3 = 0.0;
  return p;
}

// lo covers lower token indices than hi; sums are taken lo + hi.
__device__ __forceinline__ Partial combine(const Partial& lo, const Partial& hi) {
  Partial r;
  r.n = lo.n + hi.n;
  r.mism = lo.mism + hi.mism;
  r.bitw = lo.bitw + hi.bitw;
  r.nan = lo.nan | hi.nan;
  r.pad = 0;
  r.maxabs = fmax(lo.maxabs, hi.maxabs);
  r.sabs = lo.sabs + hi.sabs;
  r.sk1 = lo.sk1 + hi.sk1;
  r.sk3 = lo.sk3 + hi.sk3;
  return r;
}

__device__ __forceinline__ Partial shfl_xor_partial(const Partial& p, int m) {
  Partial r;
  r.n = __shfl_xor(p.n, m, 64);
  r.mism = __shfl_xor(p.mism, m, 64);
  r.bitw = __shfl_xor(p.bitw, m, 64);
  r.nan = __shfl_xor(p.nan, m, 64);
  r.pad = 0;
  r.maxabs = __shfl_xor(p.maxabs, m, 64);
  r.sabs = __shfl_xor(p.sabs, m, 64);
  r.sk1 = __shfl_xor(p.sk1, m, 64);
  r.sk3 = __shfl_xor(p.sk3, m, 64);
  return r;
}

// Butterfly within the wave, then ((w0, w1), (w2, w3)) through LDS; thread 0 returns the
// workgroup total (other threads' return values are unspecified).
__device__ __forceinline__ Partial block_combine(Partial p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const Partial o = shfl_xor_partial(p, off);
    p = (lane & off) ? combine(o, p) : combine(p, o);
  }
  __shared__ Partial waves[kCmpThreads / 64];
  if (lane == 0) waves[wave] = p;
  __syncthreads();
  return combine(combine(waves[0], waves[1]), combine(waves[2], waves[3]));
}

__device__ __forceinline__ void add_token(Partial& p, float a, float b) {
  p.n += 1;
  p.mism += (a != b) ? 1 : 0;
  p.bitw += (__float_as_uint(a) != __float_as_uint(b)) ? 1 : 0;
  const double d = (double)a - (double)b;   // exact
  if (d != d) {
    p.nan = 1;
  } else {
    p.maxabs = fmax(p.maxabs, fabs(d));
  }
  p.sabs += fabs(d);
  p.sk1 += -d;
  p.sk3 += expm1(d) - d;
}

__global__ __launch_bounds__(kCmpThreads) void compare_blocks_kernel(
    const float* __restrict__ train, const float* __restrict__ rollout,
    const uint8_t* __restrict__ mask, int64_t T, Partial* __restrict__ partials) {
  const int64_t blk = linear_block();
  if (blk * kCmpTokensPerBlock >= T) return;
  const int64_t base = blk * kCmpTokensPerBlock + threadIdx.x;
  Partial p = zero_partial();
#pragma unroll
  for (int k = 0; k < kCmpPerThread; ++k) {
    const int64_t i = base + (int64_t)k * kCmpThreads;
    if (i < T && (!mask || mask[i] != 0)) add_token(p, train[i], rollout[i]);
  }
  const Partial r = block_combine(p);
  if (threadIdx.x == 0) partials[blk] = r;
}

__global__ __launch_bounds__(kCmpThreads) void compare_final_kernel(
    const Partial* __restrict__ partials, int64_t n_blocks, CompareResult* __restrict__ out) {
  Partial p = zero_partial();
  for (int64_t j = threadIdx.x; j < n_blocks; j += kCmpThreads) p = combine(p, partials[j]);
  const Partial r = block_combine(p);
  if (threadIdx.x != 0) return;
  CompareResult o;
  o.active_tokens = r.n;
  o.mismatch_count = r.mism;
  o.bitwise_mismatch_count = r.bitw;
  o.reserved = 0;
  if (r.n == 0) {
    o.max_abs_diff = o.mean_abs_diff = o.mismatch_kl = o.mismatch_k3_kl = 0.0;
  } else {
    const double n = (double)r.n;
    o.max_abs_diff = r.nan ? __builtin_nan("") : r.maxabs;
    o.mean_abs_diff = r.sabs / n;
    o.mismatch_kl = r.sk1 / n;
    o.mismatch_k3_kl = r.sk3 / n;
  }
  *out = o;
}

}  // namespace

int64_t compare_blocks(int64_t T) { return (T + kCmpTokensPerBlock - 1) / kCmpTokensPerBlock; }

size_t compare_workspace_bytes(int64_t T) { return (size_t)compare_blocks(T) * sizeof(Partial); }

hipError_t launch_compare(const float* train, const float* rollout, const uint8_t* mask,
                          int64_t T, void* ws, CompareResult* out, hipStream_t stream) {
  const int64_t nb = compare_blocks(T);
  Partial* partials = static_cast<Partial*>(ws);
  if (nb > 0) {
    hipLaunchKernelGGL(compare_blocks_kernel, split_grid(nb), dim3(kCmpThreads), 0, stream,
                       train, rollout, mask, T, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(compare_final_kernel, dim3(1), dim3(kCmpThreads), 0, stream, partials, nb,
                     out);
  return hipGetLastError();
}

}  // namespace rlk
