// Logits path, backward: gradient of sum_r g_lp[r] logprob[r] + g_ent[r] entropy[r] with
// respect to the fp32 logits.
//
// With z = x / tau, L = logsumexp(z), p = softmax(z), H the entropy (natural log):
//   d logprob / d x_i = (delta_it - p_i) / tau,    d H / d x_i = -p_i (z_i - L + H) / tau.
// Training consumes both outputs (the RL-Kernel h100-pcp.json evidence page's train/loss,
// entropy_loss and grad_norm records; its weight and norm comparisons across parallel
// configurations ask for a deterministic gradient).
//
// Pass 1 is the forward row reducer (canonical order, any vocab split) writing each row's
// root state (m, s, u) -- skipped when the caller passes the states its forward call
// saved.  Pass 2, below, streams the row again: per element
//   a = c (x - m)          (fp32, as in the forward leaf),   q = a - log2 s,
//   p = 2^q,  ln p = q ln 2,
//   grad = beta (g_lp (delta_it - p) - g_ent p (ln p + H)),
// with p (ln p + H) taken as 0 where p = 0 (a -inf logit).  Every element is a function of
// its own logit and the row's root state only, so the gradient is bitwise independent of
// the batch, the row order and the vocab split.  HBM-bound: 4 bytes read + 4 bytes
// written per element.

#include "rlk_launch.hpp"
#include "rlk_state.hpp"

namespace rlk {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGradThreads = 256;
constexpr int kGradQuadsPerThread = 4;
constexpr int kGradColsPerBlock = kGradThreads * kGradQuadsPerThread * 4;  // 4096

struct GradRow {
  float m, lg2s, H, beta, gl, ge;
  int64_t t;
  int mode;  // 0 compute, 1 all-zero row (both upstream gradients 0), 2 NaN row
};

__device__ __forceinline__ float grad_elem(float x, float delta, const GradRow& r, float c) {
  const float a = (x - r.m) * c;
  const float q = a - r.lg2s;
  const float p = exp2_hw(q);
  const float lnp = q * 0.693147180559945309f;
  const float ent = mul_zero_wins(p, lnp + r.H);  // 0 where p = 0
  return r.beta * (r.gl * (delta - p) - r.ge * ent);
}

template <bool VEC>
__global__ __launch_bounds__(kGradThreads) void logits_grad_kernel(
    const float* X, int64_t ld, int64_t V, const int64_t* __restrict__ targets,
    float c, double beta, const float* __restrict__ g_lp, const float* __restrict__ g_ent,
    const WireState* __restrict__ root, float* G, int64_t ldg, int64_t T) {
  const int64_t row = linear_block();
  if (row >= T) return;
  __shared__ GradRow rc;
  if (threadIdx.x == 0) {
    GradRow r;
    r.gl = g_lp ? g_lp[row] : 0.0f;
    r.ge = g_ent ? g_ent[row] : 0.0f;
    r.t = targets ? targets[row] : -1;
    r.beta = (float)beta;
    r.m = 0.0f;
    r.lg2s = 0.0f;
    r.H = 0.0f;
    if (r.gl == 0.0f && r.ge == 0.0f) {
      r.mode = 1;
    } else {
      const State st = from_wire(root[row]);
      const bool ok = (st.m != kNegInf) && (st.s > 0.0) && (st.s < __builtin_inf()) &&
                      (st.u == st.u);
      const bool has = (r.t >= 0) && (r.t < V);
      r.mode = (!ok || (!has && r.gl != 0.0f)) ? 2 : 0;
      if (r.mode == 0) {
        r.m = st.m;
        r.lg2s = (float)log2(st.s);
        r.H = (float)(log(st.s) - kLn2 * (st.u / st.s));
      }
    }
    rc = r;
  }
  __syncthreads();
  const GradRow r = rc;
  const float* x = X + row * ld;  // G may be X (in place): each element is read, then written
  float* g = G + row * ldg;
  const float fill = r.mode == 1 ? 0.0f : __builtin_nanf("");
  // Column spans of kGradColsPerBlock; grid.y is capped, so a block may take several.
  for (int64_t col0 = (int64_t)blockIdx.y * kGradColsPerBlock; col0 < V;
       col0 += (int64_t)gridDim.y * kGradColsPerBlock) {
#pragma unroll
    for (int k = 0; k < kGradQuadsPerThread; ++k) {
      const int64_t col = col0 + 4 * ((int64_t)threadIdx.x + (int64_t)kGradThreads * k);
      if (col >= V) break;
      if (VEC && col + 4 <= V) {
        f32x4 o;
        if (r.mode != 0) {
          o = f32x4{fill, fill, fill, fill};
        } else {
          const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + col));
          o.x = grad_elem(v.x, col + 0 == r.t ? 1.0f : 0.0f, r, c);
          o.y = grad_elem(v.y, col + 1 == r.t ? 1.0f : 0.0f, r, c);
          o.z = grad_elem(v.z, col + 2 == r.t ? 1.0f : 0.0f, r, c);
          o.w = grad_elem(v.w, col + 3 == r.t ? 1.0f : 0.0f, r, c);
        }
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(g + col));
      } else {
        for (int j = 0; j < 4 && col + j < V; ++j) {
          const int64_t cj = col + j;
          g[cj] = r.mode != 0 ? fill : grad_elem(x[cj], cj == r.t ? 1.0f : 0.0f, r, c);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_logits_backward(const LogitsArgs& a, const float* g_lp, const float* g_ent,
                                  float* G, int64_t ldg, bool vec, bool have_states,
                                  hipStream_t stream) {
  if (!have_states) {
    hipError_t e = launch_logits_path(a, stream);  // a.root receives the row states
    if (e != hipSuccess) return e;
  }
  const int64_t spans = (a.V + kGradColsPerBlock - 1) / kGradColsPerBlock;
  const dim3 grid = split_grid(a.T, (unsigned)(spans < 4096 ? spans : 4096));
  if (vec)
    hipLaunchKernelGGL((logits_grad_kernel<true>), grid, dim3(kGradThreads), 0, stream, a.X, a.ld,
                       a.V, a.targets, a.c, a.beta, g_lp, g_ent, a.root, G, ldg, a.T);
  else
    hipLaunchKernelGGL((logits_grad_kernel<false>), grid, dim3(kGradThreads), 0, stream, a.X,
                       a.ld, a.V, a.targets, a.c, a.beta, g_lp, g_ent, a.root, G, ldg, a.T);
  return hipGetLastError();
}

}  // namespace rlk
