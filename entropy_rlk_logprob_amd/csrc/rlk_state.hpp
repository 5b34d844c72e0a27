// Device-side reduction state shared by every kernel of the library.
//
// A state summarises the tempered softmax over a contiguous vocabulary range R:
//     m = max_{i in R} x_i                       (raw logit, fp32)
//     s = sum_{i in R} 2^{a_i}                   (fp64 once above a leaf)
//     u = sum_{i in R} 2^{a_i} * a_i             (fp64 once above a leaf)
// with a_i = c * (x_i - m) and c = log2(e) / tau rounded once to fp32 on the host.
// Identity: (-inf, 0, 0).  The selected-token logprob and the entropy of a full row are
//     logprob = (x_t - m) / tau - ln s,     entropy = ln s - ln(2) * u / s,
// evaluated in fp64 (finalize) from the root state.
//
// Strictness: every merge of two states goes through rlk_merge() below, always with the
// lower vocabulary range as its first operand; the one many-way merge, wave_merge() (the
// 64 lane states of a logits-path chunk), is likewise one fixed function.  The library is
// compiled with -ffp-contract=off so that no compiler contraction changes a rounding.
// Trees are fixed functions of the vocabulary position only, never of the number of rows,
// the row's place in a tile, the launch shape or the vocab split count.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlk {

constexpr float kNegInf = -__builtin_inff();
constexpr float kMaxFloat = 3.40282346638528859811704183484516925e+38f;
constexpr double kLn2 = 0.693147180559945309417232121458176568;

// 2^x on the hardware transcendental unit (v_exp_f32): exact at x = 0, 0 at x = -inf.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

struct State {
  float m;
  double s;
  double u;
};

// Exchange / workspace format of a state plus the captured target logit (24 bytes).
struct alignas(8) WireState {
  float m;
  float xt;   // target logit if the target lies in this range, else unused
  double s;
  double u;
};

__device__ __forceinline__ State identity_state() { return State{kNegInf, 0.0, 0.0}; }

// Merge of two states over adjacent ranges, `a` covering the lower vocabulary indices.
// Only the operand with the smaller max is rescaled (2^0 = 1 exactly for the other),
// a range of all -inf contributes nothing, and NaN in s or u propagates.
__device__ __forceinline__ State rlk_merge(const State& a, const State& b, float c) {
  const bool a_ge = a.m >= b.m;
  const float M = a_ge ? a.m : b.m;
  const float lo = a_ge ? b.m : a.m;
  const float Mref = (M == kNegInf) ? 0.0f : M;
  const float dlo = (lo - Mref) * c;           // <= 0, or -inf, or NaN if M = +inf
  const float elo = exp2_hw(dlo);
  const float dlo_c = fmaxf(dlo, -kMaxFloat);  // keeps 0 * (-inf) out of u
  const double ea = a_ge ? 1.0 : (double)elo;
  const double eb = a_ge ? (double)elo : 1.0;
  const double da = a_ge ? 0.0 : (double)dlo_c;
  const double db = a_ge ? (double)dlo_c : 0.0;
  State r;
  r.m = M;
  r.s = fma(a.s, ea, b.s * eb);
  const double ua = fma(da, a.s, a.u);
  const double ub = fma(db, b.s, b.u);
  r.u = fma(ua, ea, ub * eb);
  return r;
}

// Final per-row evaluation in fp64 from the root state; one rounding to fp32.
// beta = 1/tau in fp64.  has_target: the target lies in [0, V) (xt is its logit).
__device__ __forceinline__ void rlk_finalize(const State& st, float xt, bool has_target,
                                             double beta, float* lp, float* ent) {
  const double qnan = __builtin_nan("");
  const bool ok = (st.m != kNegInf) && (st.s > 0.0) && (st.s < __builtin_inf()) &&
                  (st.u == st.u);
  double l = ok ? log(st.s) : qnan;
  double e = ok ? (l - kLn2 * (st.u / st.s)) : qnan;
  double p = (ok && has_target) ? (beta * ((double)xt - (double)st.m) - l) : qnan;
  if (lp) *lp = (float)p;
  if (ent) *ent = (float)e;
}

__device__ __forceinline__ State from_wire(const WireState& w) { return State{w.m, w.s, w.u}; }

__device__ __forceinline__ WireState to_wire(const State& s, float xt) {
  WireState w;
  w.m = s.m;
  w.xt = xt;
  w.s = s.s;
  w.u = s.u;
  return w;
}

// x * y with 0 * (anything) = 0 (v_mul_legacy_f32): a zero-probability term (2^a = 0 at
// a = -inf) then adds nothing to u instead of 0 * (-inf) = NaN.  Otherwise equal to x * y.
__device__ __attribute__((const, noconvergent)) float mul_zero_wins(float, float) __asm("llvm.amdgcn.fmul.legacy");

// Wave-wide shuffle of a state (64 lanes).
__device__ __forceinline__ State shfl_xor_state(const State& s, int mask) {
  State r;
  r.m = __shfl_xor(s.m, mask, 64);
  r.s = __shfl_xor(s.s, mask, 64);
  r.u = __shfl_xor(s.u, mask, 64);
  return r;
}

// The state of the union of a wave's 64 lane states, in one fixed order: the wave max M
// of the lane maxima (exact, so its grouping does not matter), each lane's sums rescaled
// to M once -- s 2^d and (u + d s) 2^d with d = c (m - M), one v_exp_f32, and 2^0 = 1
// exactly for a lane at M -- then the fp64 sums over the lanes by an xor butterfly
// (strides 32, 16, 8, 4, 2, 1).  Both partners of a butterfly step add the same two values,
// so every lane ends with the same bits.  A lane of only -inf (m = -inf, s = u = 0) adds
// 0; with M = -inf every lane is such a lane and the result is the identity; NaN in s or u
// propagates.  A lane whose m is +inf has NaN sums already (its +inf term is NaN), and its
// d = c (inf - inf) is NaN too, so M = +inf always yields NaN sums.  Against the
// pairwise butterfly of rlk_merge this rounds each lane's contribution through one scale
// factor instead of up to six, at a tenth of the instructions.
__device__ __forceinline__ State wave_merge(const State& st, float c) {
  float M = st.m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float Mref = (M == kNegInf) ? 0.0f : M;
  const float d = (st.m - Mref) * c;          // <= 0; -inf for a lane of only -inf
  const double e = (double)exp2_hw(d);
  const double dc = (double)fmaxf(d, -kMaxFloat);  // keeps 0 * (-inf) out of u
  double s = st.s * e;
  double u = fma(dc, st.s, st.u) * e;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    s += __shfl_xor(s, off, 64);
    u += __shfl_xor(u, off, 64);
  }
  return State{M, s, u};
}

// Balanced tree over n = 1, 2, 4 or 8 consecutive states (lower index first):
// ((0,1),(2,3)),((4,5),(6,7)).
__device__ __forceinline__ State tree8(const State* v, int n, float c) {
  if (n == 1) return v[0];
  if (n == 2) return rlk_merge(v[0], v[1], c);
  if (n == 4) return rlk_merge(rlk_merge(v[0], v[1], c), rlk_merge(v[2], v[3], c), c);
  State l = rlk_merge(rlk_merge(v[0], v[1], c), rlk_merge(v[2], v[3], c), c);
  State r = rlk_merge(rlk_merge(v[4], v[5], c), rlk_merge(v[6], v[7], c), c);
  return rlk_merge(l, r, c);
}

}  // namespace rlk
