// Fused path, backward: gradients of sum_r g_lp[r] logprob[r] + g_ent[r] entropy[r] with
// respect to the hidden states and the LM-head weight, for logits x = H W^T (bf16).
//
//   dX[r, v] = ( g_lp[r] (delta(v, t_r) - p_rv) - g_ent[r] p_rv (ln p_rv + H_r) ) / tau
//   dH = dX W   (contraction over the vocabulary),   dW = dX^T H   (over the tokens).
// The RL-Kernel h100-pcp.json evidence page's training records consume the logprob and
// entropy; its comparison block finds the trained weights and norms equal across parallel
// configurations, which asks for a deterministic gradient with fixed reduction orders.
//
// Steps (all on the caller's stream, no atomics):
//   1. the forward fused path in row-state mode: each token's root state (m, s, u) --
//      skipped when the caller passes the states its forward call saved;
//   2. per-token constants (m, log2 s, entropy, upstream gradients, target, row mode);
//   3. the logits tile is recomputed on MFMA (same tile loop and K order as the forward)
//      and its gradient dX is written in bf16, row-major [T, Vp] (for dH) and transposed
//      [V, Tp] (for dW), with zero K padding;
//   4. dH = dX . W on the shared tile loop, dX K-contiguous and W read in place as a
//      K-major operand (gfx950 LDS transpose loads, so no transposed copy of W is made);
//      K = Vp split into 4 fixed ranges (boundaries depend on V only), partials summed in
//      the fixed tree (0,1),(2,3);
//   5. dW = dX^T . H with dX^T and a transposed copy of H (small), K = Tp in one
//      increasing-order pass per output tile.
// A token's row of dH depends only on that token (its place among the GEMM's columns does
// not change the accumulation order), so dH is batch-invariant like the forward; dW sums
// over the batch in increasing token order.

#include <algorithm>

#include "rlk_launch.hpp"
#include "rlk_mma_tile.hpp"
#include "rlk_state.hpp"

namespace rlk {

namespace {

using mma::floatx16;
using mma::kBK;
using mma::kStageBytes;
using mma::kThreads;

constexpr int kTile = 256;
// Fixed K ranges of dH.  4 against 8: half the fp32 partials (134 against 268 MB at
// T = 2048, d = 4096) and half the per-job fixed costs, in 2 rounds of 512 jobs instead of 4 of
// 1024 on 256 CUs: the whole backward 0.8% faster at that shape (same-process A/B, 3 of 3).
constexpr int kDhSplits = 4;

// Per-token constants of the logit gradient: the root state's m and log2 s, the entropy H,
// the upstream gradients times 1/tau (bgl, bge), the row mode and the value a row that is
// not computed takes (0 for a row whose upstream gradients are both 0, NaN for a row whose
// forward outputs are NaN).
struct GradRowC {
  float m, lg2s, H, bgl, bge, fill;
  int32_t mode;  // 0 compute, 1 all-zero row, 2 NaN row
  int32_t pad;
  int64_t t;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (round to nearest even) and packed, the first in the low
// half: v_cvt_pk_bf16_f32.  On every one of the 2^32 fp32 bit patterns it gives the bits of
// the plain round-to-nearest-even formula (b + 0x7fff + ((b >> 16) & 1)) >> 16, and a NaN
// for a NaN (checked exhaustively on the device).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

__global__ __launch_bounds__(256) void row_consts_kernel(
    const WireState* __restrict__ root, int64_t T, int64_t V, const int64_t* __restrict__ targets,
    const float* __restrict__ g_lp, const float* __restrict__ g_ent, double beta,
    GradRowC* __restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= T) return;
  GradRowC r;
  const float gl = g_lp ? g_lp[row] : 0.0f;
  const float ge = g_ent ? g_ent[row] : 0.0f;
  r.t = targets ? targets[row] : -1;
  r.bgl = (float)beta * gl;
  r.bge = (float)beta * ge;
  r.m = 0.0f;
  r.lg2s = 0.0f;
  r.H = 0.0f;
  r.pad = 0;
  if (gl == 0.0f && ge == 0.0f) {
    r.mode = 1;
  } else {
    const State st = from_wire(root[row]);
    const bool ok =
        (st.m != kNegInf) && (st.s > 0.0) && (st.s < __builtin_inf()) && (st.u == st.u);
    const bool has = (r.t >= 0) && (r.t < V);
    r.mode = (!ok || (!has && gl != 0.0f)) ? 2 : 0;
    if (r.mode == 0) {
      r.m = st.m;
      r.lg2s = (float)log2(st.s);
      r.H = (float)(log(st.s) - kLn2 * (st.u / st.s));
    }
  }
  r.fill = r.mode == 1 ? 0.0f : __builtin_nanf("");
  out[row] = r;
}

// Gradient of one logit: with a = c (x - m), q = a - log2 s (log2 p), p = 2^q,
//   g = bgl (delta - p) - bge p (q ln 2 + H)      (bgl = g_lp / tau, bge = g_ent / tau),
// p (ln p + H) taken as 0 where p = 0.  Every logit of a token is formed by these same fp32
// steps whatever tile it falls in, so a row of dX, and so of dH, does not depend on the
// batch.
__device__ __forceinline__ float logit_grad(float x, bool is_target, const GradRowC& r, float c) {
  const float q = (x - r.m) * c - r.lg2s;
  const float p = exp2_hw(q);
  const float ent = mul_zero_wins(p, __builtin_fmaf(q, 0.693147180559945309f, r.H));
  float g = __builtin_fmaf(r.bgl, (is_target ? 1.0f : 0.0f) - p, -(r.bge * ent));
  // g is formed on every lane and then selected: left to itself the compiler branches around
  // the formula per logit (an exec-mask branch each time) for the rows that take r.fill.
  asm volatile("" : "+v"(g));
  return r.mode == 0 ? g : r.fill;
}

// Output tile id -> (row tile, column tile): column tiles in groups of 8, row-tile-major
// within a group (see grouped_tile_of).
__device__ __forceinline__ bool tile_of(int64_t n_rt, int64_t n_ct, int64_t& rt, int64_t& ct) {
  return mma::grouped_tile_of<8>(n_rt, n_ct, rt, ct);
}

// Step 3: logits tile (vocab rows x tokens), then its gradient in bf16.
__global__ __launch_bounds__(kThreads, 1) void dx_tile_kernel(
    const uint16_t* __restrict__ H, int64_t ldh, const uint16_t* __restrict__ W, int64_t ldw,
    int64_t d, int64_t T, int64_t V, float c, const GradRowC* __restrict__ rc,
    uint16_t* __restrict__ dX, int64_t ldx, uint16_t* __restrict__ dXT, int64_t ldxt) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  int64_t vt, tt;
  // Tile order as in the forward, which runs the same tile loop: with 5 to 8 token tiles, groups
  // of 4 token tiles (0.1-0.5% faster for the whole backward at T = 2048 in a same-process A/B,
  // 3 of 3, bits equal), else of 8.
  const int64_t n_vt = (V + kTile - 1) / kTile, n_tt = (T + kTile - 1) / kTile;
  if (!((n_tt > 4 && n_tt <= 8) ? mma::grouped_tile_of<4>(n_vt, n_tt, vt, tt)
                                : tile_of(n_vt, n_tt, vt, tt)))
    return;
  const int64_t v_lo = vt * kTile;
  const int64_t t_lo = tt * kTile;
  const int n_v = (int)min((int64_t)kTile, V - v_lo);
  const int n_t = (int)min((int64_t)kTile, T - t_lo);
  floatx16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  // Row strides of W and H are at most 2^22 (the ABI's limit): buffer loads to LDS.
  mma::mma_tile_buf(W + v_lo * ldw, ldw, n_v - 1, H + t_lo * ldh, ldh, n_t - 1, 0, (int)(d / kBK),
                smem, acc);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wv = wave >> 2, wt = wave & 3;
  const int frow = lane & 31, fhalf = lane >> 5;
  // Lane (wv, wt, lane) holds, for tokens t_lo + wt 64 + b 32 + frow (b = 0, 1), the logits
  // of rows v_lo + wv 128 + a 32 + 8 g4 + 4 fhalf + j (a, g4, j = 0..3) in acc[a][b][4 g4 + j].
  const int64_t row0 = v_lo + wv * 128 + 4 * fhalf;  // this lane's first row
  if (v_lo + kTile <= V && t_lo + kTile <= T) {
    // Full tile: the bf16 gradient tile (128 KiB) goes through the LDS, which the K loop no
    // longer needs, once per layout, so that dX and dX^T are both written with 16-byte stores
    // whose 32 lanes cover 512 contiguous bytes of a row (four whole 128-byte lines).  Written
    // straight from the MFMA layout, dX took 8-byte stores that touch 32 lines each and dX^T
    // 2-byte stores, and the tile's stores cost several times its MFMAs' last steps.
    uint32_t w[2][4][4][2];  // token b; rows row0 + a 32 + 8 g4 + {0,1} and {2,3}, packed
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t tok = t_lo + wt * 64 + b * 32 + frow;
      const GradRowC r = rc[tok];
      const int tgt = (r.t >= row0 && r.t < row0 + 128) ? (int)(r.t - row0) : -1;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int off = a * 32 + 8 * g4;  // row offset from row0 (compile-time)
          float g[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) g[j] = logit_grad(acc[a][b][4 * g4 + j], tgt == off + j, r, c);
          w[b][a][g4][0] = pack_bf16(g[0], g[1]);
          w[b][a][g4][1] = pack_bf16(g[2], g[3]);
        }
      }
    }
    // LDS tile: 256 rows of 512 bytes (32 16-byte columns).  dX: row = token, column c of a
    // row at c ^ (row % 32); dX^T: row = vocabulary row, column c at c ^ 4 ((row / 4) % 8).
    // Both keep the 32 lanes of a write or read instruction off each other's banks.
    char* const tile = smem;
    const int wvrow = wv * 128 + 4 * fhalf;  // this lane's first vocabulary row in the tile
    if (dX) {
      __syncthreads();  // every wave is done with the K loop's stages (or the last dX^T pass)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int tl = wt * 64 + b * 32 + frow;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int vl = wvrow + a * 32 + 8 * g4;  // 4 rows: bytes 2 vl .. 2 vl + 7
            *reinterpret_cast<uint2*>(tile + tl * 512 + (((vl >> 3) ^ (tl & 31)) << 4) +
                                      ((vl & 4) << 1)) =
                make_uint2(w[b][a][g4][0], w[b][a][g4][1]);
          }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tl = wave * 32 + 2 * i + (lane >> 5);
        const int col = lane & 31;
        const uint4 q = *reinterpret_cast<const uint4*>(tile + tl * 512 + ((col ^ (tl & 31)) << 4));
        *reinterpret_cast<uint4*>(dX + (t_lo + tl) * ldx + v_lo + 8 * col) = q;
      }
    }
    if (dXT) {
      __syncthreads();
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int tl = wt * 64 + b * 32 + frow;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int vl = wvrow + a * 32 + 8 * g4 + j;
              const uint32_t word = w[b][a][g4][j >> 1];
              *reinterpret_cast<uint16_t*>(tile + vl * 512 +
                                           (((tl >> 3) ^ (4 * ((vl >> 2) & 7))) << 4) +
                                           ((tl & 7) << 1)) =
                  (uint16_t)((j & 1) ? (word >> 16) : word);
            }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int vl = wave * 32 + 2 * i + (lane >> 5);
        const int col = lane & 31;
        const uint4 q = *reinterpret_cast<const uint4*>(
            tile + vl * 512 + ((col ^ (4 * ((vl >> 2) & 7))) << 4));
        *reinterpret_cast<uint4*>(dXT + (v_lo + vl) * ldxt + t_lo + 8 * col) = q;
      }
    }
    return;
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t tok = t_lo + wt * 64 + b * 32 + frow;
    if (tok >= T) continue;
    const GradRowC r = rc[tok];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int64_t v0 = row0 + a * 32 + 8 * g4;
        if (v0 >= V) continue;
        float g[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) g[j] = logit_grad(acc[a][b][4 * g4 + j], v0 + j == r.t, r, c);
        const uint32_t w0 = pack_bf16(g[0], g[1]), w1 = pack_bf16(g[2], g[3]);
        const uint16_t bits[4] = {(uint16_t)w0, (uint16_t)(w0 >> 16), (uint16_t)w1,
                                  (uint16_t)(w1 >> 16)};
        if (dX) {
          uint16_t* dst = dX + tok * ldx + v0;
          if (v0 + 4 <= V) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
          } else {
            for (int j = 0; j < 4 && v0 + j < V; ++j) dst[j] = bits[j];
          }
        }
        if (dXT) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (v0 + j < V) dXT[(v0 + j) * ldxt + tok] = bits[j];
        }
      }
    }
  }
}

// H^T for the dW contraction: out[c][r] = in[r][c] for r < R, c < C; out[c][r] = 0 for
// R <= r < Rp.
// 64 x 64 tiles through LDS; each lane moves 16 contiguous bytes (8 elements) per global
// access when the row strides and the tile allow it (the common case), else elements.
__global__ __launch_bounds__(256) void transpose_pad_kernel(
    const uint16_t* __restrict__ in, int64_t ldin, int64_t R, int64_t C,
    uint16_t* __restrict__ out, int64_t ldout, int64_t Rp) {
  __shared__ uint16_t tile[64][64 + 8];
  const int64_t r0 = linear_block() * 64;
  const int64_t c0 = (int64_t)blockIdx.y * 64;
  if (r0 >= Rp) return;
  const int tid = threadIdx.x;
  // load: thread -> rows tid / 8 and tid / 8 + 32, columns 8 (tid % 8) .. + 8
  const bool vec_in = (ldin % 8 == 0) && (c0 + 64 <= C);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = tid / 8 + 32 * h, cc = 8 * (tid % 8);
    const int64_t r = r0 + rr;
    uint16_t v[8];
    if (r < R && vec_in) {
      const uint4 q = *reinterpret_cast<const uint4*>(in + r * ldin + c0 + cc);
      v[0] = q.x & 0xffff; v[1] = q.x >> 16; v[2] = q.y & 0xffff; v[3] = q.y >> 16;
      v[4] = q.z & 0xffff; v[5] = q.z >> 16; v[6] = q.w & 0xffff; v[7] = q.w >> 16;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (r < R && c0 + cc + j < C) ? in[r * ldin + c0 + cc + j] : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[rr][cc + j] = v[j];
  }
  __syncthreads();
  // store: thread -> output rows (= input columns) tid / 8 and tid / 8 + 32, 8 consecutive r
  const bool vec_out = (ldout % 8 == 0) && (r0 + 64 <= Rp);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cl = tid / 8 + 32 * h, rl = 8 * (tid % 8);
    const int64_t cc = c0 + cl;
    if (cc >= C) continue;
    uint16_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = tile[rl + j][cl];
    if (vec_out) {
      const uint4 q = make_uint4((uint32_t)v[0] | ((uint32_t)v[1] << 16),
                                 (uint32_t)v[2] | ((uint32_t)v[3] << 16),
                                 (uint32_t)v[4] | ((uint32_t)v[5] << 16),
                                 (uint32_t)v[6] | ((uint32_t)v[7] << 16));
      *reinterpret_cast<uint4*>(out + cc * ldout + r0 + rl) = q;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (r0 + rl + j < Rp) out[cc * ldout + r0 + rl + j] = v[j];
    }
  }
}

// Zero columns [c_begin, c_end) of rows [0, rows) of a bf16 matrix (the padding of dX).
__global__ __launch_bounds__(256) void zero_cols_kernel(uint16_t* __restrict__ p, int64_t ld,
                                                        int64_t rows, int64_t c_begin,
                                                        int64_t c_end) {
  const int64_t width = c_end - c_begin;
  const int64_t n = rows * width;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[(i / width) * ld + c_begin + i % width] = 0;
}

// Zero an fp32 matrix [rows, cols] with row stride ld (the weight gradient of an empty
// batch).
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t ld,
                                                       int64_t rows, int64_t cols) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[(i / cols) * ld + i % cols] = 0.0f;
}

// Steps 4 and 5: C(m, n) = sum_k A[m, k] B[n, k] over the split's K range (ACCUM: C(m, n)
// plus that sum, the accumulators starting from the stored C), in 256 x 256 tiles on the
// shared MFMA loop.  An operand is K-contiguous ([rows, K], row r at
// X + r ld) or K-major ([K, rows], k row at X + k ld; its k rows beyond k_last are
// clamped, the other operand holding zeros there).  Stored row-major at C[m * ldc + n]
// (32 lanes write 128 contiguous bytes of a row).  Split s (blockIdx.y) covers K steps
// [s * steps, (s + 1) * steps) and writes C + s * split_stride; an empty range writes 0.
// Tile order: SHARE_B groups row tiles by 4 and runs column-tile-major within a group
// (consecutive logical tiles share a B slice), else the reverse with groups of 8 (they share
// an A slice): the larger operand is fetched from HBM once and shared in an XCD's L2.  For
// dH (SHARE_B) each XCD then takes 4 W column tiles x 4 token tiles of a K range instead of
// 2 x 8, so that each XCD no longer reads the whole token range of dX: 6.994-6.998 ms against
// 7.005-7.013 ms for the whole backward at T = 2048, d = 4096, V = 151936 (groups of 2:
// 7.028-7.030 ms).
// BUF: stages staged by buffer loads to LDS (every row stride at most 2^22; see mma_tile_op).
template <bool A_KMAJOR, bool B_KMAJOR, bool SHARE_B, bool ACCUM = false, bool BUF = true>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t M, int64_t a_klast,
    const uint16_t* __restrict__ B, int64_t ldb, int64_t N, int64_t b_klast, int64_t K,
    int64_t steps, float* __restrict__ C, int64_t ldc, int64_t split_stride) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  int64_t mt, nt;
  const int64_t n_mt = (M + kTile - 1) / kTile, n_nt = (N + kTile - 1) / kTile;
  if (!(SHARE_B ? mma::grouped_tile_of<4>(n_nt, n_mt, nt, mt) : tile_of(n_mt, n_nt, mt, nt)))
    return;
  const int64_t m_lo = mt * kTile, n_lo = nt * kTile;
  const int64_t k_begin = (int64_t)blockIdx.y * steps * kBK;
  const int64_t k_end = min(k_begin + steps * kBK, K);
  const int nk = k_end > k_begin ? (int)((k_end - k_begin) / kBK) : 0;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int wv = wave >> 2, wt = wave & 3;
  const int frow = lane & 31, fhalf = lane >> 5;
  float* __restrict__ Cs = C + (int64_t)blockIdx.y * split_stride;
  floatx16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  if constexpr (ACCUM) {
    // Continue the accumulation of the stored C: the same places the epilogue stores.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t n = n_lo + wt * 64 + b * 32 + frow;
      if (n >= N) continue;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int64_t m0 = m_lo + wv * 128 + a * 32 + 8 * g4 + 4 * fhalf;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (m0 + j < M) acc[a][b][4 * g4 + j] = Cs[(m0 + j) * ldc + n];
        }
    }
  }
  if (nk > 0) {
    const int a_last = (int)min((int64_t)kTile, M - m_lo) - 1;
    const int b_last = (int)min((int64_t)kTile, N - n_lo) - 1;
    const mma::Operand Aop{A_KMAJOR ? A + m_lo : A + m_lo * lda, lda, a_last, a_klast};
    const mma::Operand Bop{B_KMAJOR ? B + n_lo : B + n_lo * ldb, ldb, b_last, b_klast};
    mma::mma_tile_op<A_KMAJOR, B_KMAJOR, 2, false, BUF>(Aop, Bop, k_begin, nk, smem, acc);
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t n = n_lo + wt * 64 + b * 32 + frow;
    if (n >= N) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int64_t m0 = m_lo + wv * 128 + a * 32 + 8 * g4 + 4 * fhalf;
        if (m0 >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (m0 + j < M) Cs[(m0 + j) * ldc + n] = acc[a][b][4 * g4 + j];
      }
    }
  }
}

// out[t, k] = (P0 + P1) + (P2 + P3), P_s = part + s * stride, part rows of d floats; 4
// consecutive k per thread (d is a multiple of 64).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            int64_t stride, int64_t T, int64_t d,
                                                            float* __restrict__ out, int64_t ldo) {
  const int64_t q = linear_block() * 256 + threadIdx.x;  // quad index
  const int64_t nq = T * (d / 4);
  if (q >= nq) return;
  const int64_t t = q / (d / 4), k = 4 * (q % (d / 4));
  float4 v[kDhSplits];
#pragma unroll
  for (int s = 0; s < kDhSplits; ++s)
    v[s] = *reinterpret_cast<const float4*>(part + s * stride + t * d + k);
  auto add = [](float4 x, float4 y) { return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w); };
  static_assert(kDhSplits == 4, "the reduction tree below");
  const float4 r = add(add(v[0], v[1]), add(v[2], v[3]));
  float* dst = out + t * ldo + k;
  dst[0] = r.x;
  dst[1] = r.y;
  dst[2] = r.z;
  dst[3] = r.w;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

LinearBackwardWorkspace linear_backward_layout(int64_t T, int64_t V, int64_t d, int S) {
  LinearBackwardWorkspace L;
  L.chunk = std::min<int64_t>(T, kBackwardChunkTokens);
  L.Vp = (V + kBK - 1) / kBK * kBK;
  L.Tp = (L.chunk + kBK - 1) / kBK * kBK;
  size_t off = align256(linear_workspace_layout(L.chunk, V, S).total);
  L.root = off;
  off += align256((size_t)L.chunk * sizeof(WireState));
  L.rowc = off;
  off += align256((size_t)L.chunk * sizeof(GradRowC));
  L.ht = off;
  off += align256((size_t)d * (size_t)L.Tp * 2);
  L.dx = off;
  off += align256((size_t)L.chunk * (size_t)L.Vp * 2);
  L.dxt = off;
  off += align256((size_t)V * (size_t)L.Tp * 2);
  L.part = off;
  off += align256((size_t)kDhSplits * (size_t)L.chunk * (size_t)d * sizeof(float));
  L.total = off;
  return L;
}

hipError_t launch_zero_f32(float* p, int64_t ld, int64_t rows, int64_t cols,
                           hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t n = rows * cols;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, ld, rows,
                     cols);
  return hipGetLastError();
}

namespace {

// One chunk of at most L.chunk tokens (the caller offsets every per-token pointer); accum:
// dW continues the sum of the chunks before (their tokens precede this chunk's).
hipError_t backward_chunk(const LinearArgs& fwd, const LinearBackwardWorkspace& L,
                          const float* g_lp, const float* g_ent, float* dH, int64_t ld_dh,
                          float* dW, int64_t ld_dw, const WireState* states, bool accum,
                          hipStream_t stream) {
  const int64_t T = fwd.T, V = fwd.V, d = fwd.d;
  const int64_t Tp = (T + kBK - 1) / kBK * kBK;
  char* base = static_cast<char*>(fwd.ws);
  LinearArgs a = fwd;
  a.root = reinterpret_cast<WireState*>(base + L.root);
  a.lp = nullptr;
  a.ent = nullptr;
  hipError_t e = hipSuccess;
  if (!states) {
    e = launch_linear_path(a, stream);  // step 1
    if (e != hipSuccess) return e;
  }
  GradRowC* rc = reinterpret_cast<GradRowC*>(base + L.rowc);
  hipLaunchKernelGGL(row_consts_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, stream,
                     states ? states : a.root, T, V, a.targets, g_lp, g_ent, a.beta, rc);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // Step 3 writes dX [T, Vp] (for dH) and dX^T [V, Tp] (for dW); their K padding
  // (columns [V, Vp), resp. [T, Tp)) is zeroed here, so the contractions see zeros there.
  uint16_t* dx = dH ? reinterpret_cast<uint16_t*>(base + L.dx) : nullptr;
  uint16_t* dxt = dW ? reinterpret_cast<uint16_t*>(base + L.dxt) : nullptr;
  const unsigned fill_blocks = 2048;
  if (dx && L.Vp > V)
    hipLaunchKernelGGL(zero_cols_kernel, dim3(fill_blocks), dim3(256), 0, stream, dx, L.Vp, T, V,
                       L.Vp);
  if (dxt && Tp > T)
    hipLaunchKernelGGL(zero_cols_kernel, dim3(fill_blocks), dim3(256), 0, stream, dxt, Tp, V, T,
                       Tp);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const int64_t tiles_x = ((V + kTile - 1) / kTile) * ((T + kTile - 1) / kTile);
  hipLaunchKernelGGL(dx_tile_kernel, split_grid((tiles_x + 7) / 8 * 8), dim3(kThreads), 0,
                     stream, a.H, a.ldh, a.W, a.ldw, d, T, V, a.c, rc, dx, L.Vp, dxt, Tp);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  if (dH) {
    // dH[t, k] = sum_v dX[t, v] W[v, k]: A = dX K-contiguous (M = T), B = W read in place
    // as a K-major operand (N = d; k rows v clamped to V - 1, where dX is zero), K = Vp;
    // column-tile-major so that the tiles sharing a W slice run together.
    float* part = reinterpret_cast<float*>(base + L.part);
    const int64_t steps = (L.Vp / kBK + kDhSplits - 1) / kDhSplits;
    const int64_t tiles = ((T + kTile - 1) / kTile) * ((d + kTile - 1) / kTile);
    // Buffer loads to LDS need dX's row stride Vp at most 2^22 (W's is, by the ABI's limit);
    // larger vocabularies take the global-address loads.  Same bits either way.
    if (L.Vp <= (int64_t(1) << 22))
      hipLaunchKernelGGL((gemm_kernel<false, true, true, false, true>),
                         split_grid((tiles + 7) / 8 * 8, kDhSplits), dim3(kThreads), 0,
                         stream, dx, L.Vp, T, (int64_t)0, a.W, a.ldw, d, V - 1, L.Vp, steps, part,
                         d, T * d);
    else
      hipLaunchKernelGGL((gemm_kernel<false, true, true, false, false>),
                         split_grid((tiles + 7) / 8 * 8, kDhSplits), dim3(kThreads), 0,
                         stream, dx, L.Vp, T, (int64_t)0, a.W, a.ldw, d, V - 1, L.Vp, steps, part,
                         d, T * d);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nq = T * (d / 4);
    hipLaunchKernelGGL(splitk_reduce_kernel, split_grid((nq + 255) / 256), dim3(256), 0,
                       stream, part, T * d, T, d, dH, ld_dh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (dW) {
    // dW[v, k] = sum_t dX^T[v, t] H^T[k, t]: A = dX^T (M = V), B = H^T (N = d; a transposed
    // copy of the chunk's H, small), both K-contiguous, K = Tp; row-tile-major within groups
    // of 8 column tiles, so that the tiles sharing a dX^T slice run together; stored
    // row-major (32 lanes write 128 contiguous bytes of a dW row).  After the first chunk
    // the accumulators start from the stored dW, so the sum over all tokens runs in the
    // one increasing K order whatever the chunking.  (Reading dX in place as a K-major A
    // operand measured 0.6 ms slower at T = 2048, d = 4096, V = 151936 than writing dX^T
    // in step 3.)
    uint16_t* ht = reinterpret_cast<uint16_t*>(base + L.ht);
    hipLaunchKernelGGL(transpose_pad_kernel, split_grid(Tp / 64, (unsigned)(d / 64)), dim3(256),
                       0, stream, a.H, a.ldh, T, d, ht, Tp, Tp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t tiles = ((V + kTile - 1) / kTile) * ((d + kTile - 1) / kTile);
    if (accum)
      hipLaunchKernelGGL((gemm_kernel<false, false, false, true>),
                         split_grid((tiles + 7) / 8 * 8), dim3(kThreads), 0, stream, dxt, Tp, V,
                         (int64_t)0, ht, Tp, d, (int64_t)0, Tp, Tp / kBK, dW, ld_dw, (int64_t)0);
    else
      hipLaunchKernelGGL((gemm_kernel<false, false, false>),
                         split_grid((tiles + 7) / 8 * 8), dim3(kThreads), 0, stream, dxt, Tp, V,
                         (int64_t)0, ht, Tp, d, (int64_t)0, Tp, Tp / kBK, dW, ld_dw, (int64_t)0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_linear_backward(const LinearArgs& fwd, const float* g_lp, const float* g_ent,
                                  float* dH, int64_t ld_dh, float* dW, int64_t ld_dw,
                                  const WireState* states, hipStream_t stream) {
  const LinearBackwardWorkspace L = linear_backward_layout(fwd.T, fwd.V, fwd.d, fwd.S);
  for (int64_t t0 = 0; t0 < fwd.T; t0 += L.chunk) {
    LinearArgs a = fwd;
    a.T = std::min<int64_t>(L.chunk, fwd.T - t0);
    a.H = fwd.H + t0 * fwd.ldh;
    a.targets = fwd.targets ? fwd.targets + t0 : nullptr;
    const hipError_t e = backward_chunk(
        a, L, g_lp ? g_lp + t0 : nullptr, g_ent ? g_ent + t0 : nullptr,
        dH ? dH + t0 * ld_dh : nullptr, ld_dh, dW, ld_dw, states ? states + t0 : nullptr,
        t0 > 0, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace rlk
