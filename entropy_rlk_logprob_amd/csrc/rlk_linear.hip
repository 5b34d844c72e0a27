// Fused path ("linear-logp"): logits = H W^T on bf16 MFMA tiles, folded tile by tile
// into softmax states that never leave the chip as logits.
//
// Canonical order (independent of the number of rows, the row's place in a token tile,
// the launch shape and the vocab split):
//   * the 8 canonical chunks of Vc columns (as on the logits path); inside a chunk,
//     vocabulary tiles of kTileV = 256 rows start at the chunk start, the last one short;
//   * a logit is one fp32 accumulation over the hidden dimension in fixed order:
//     64-wide K steps in increasing order, each four v_mfma_f32_32x32x16_bf16 steps
//     (16 consecutive k each);
//   * tile state of (token, tile): the 256 vocab rows split into two 128-row halves, each
//     into four 32-row MFMA blocks; within block a a lane holds 16 rows
//     8*(i/4) + 4*(lane/32) + (i%4), i = 0..15; a lane's 64 rows of a half form one leaf
//     (leaf64: their max, then pairwise fp32 sums within quads, quad pairs and blocks
//     ((0,1),(2,3))), then lane halves merge (lane < 32 first), then the two 128-row halves;
//   * tiles of a chunk: balanced binary tree over tile index (padded with identities);
//     chunks: ((0,1),(2,3)),((4,5),(6,7)), the top log2(S) levels in the shard merge.
//
// Workgroup: 8 waves, a 256 (vocab) x 256 (token) output tile, waves arranged 2 (vocab)
// x 4 (token), each wave 128 x 64 = 4 x 2 MFMA blocks.  K step 64 with two LDS stages
// (64 KiB each: the W and H slices with an XOR swizzle on 16-byte columns so that
// ds_read_b128 of 16 consecutive rows hits distinct banks).  Workgroup ids are remapped
// so that each XCD runs a few vocabulary tiles times a group of 8 token tiles at once,
// sharing their W and H slices in that XCD's L2.

#include <hip/hip_runtime.h>

#include <type_traits>

#include <algorithm>
#include <atomic>

#include "rlk_launch.hpp"
#include "rlk_mma_tile.hpp"
#include "rlk_state.hpp"

namespace rlk {

namespace {

using mma::bf16x8;
using mma::floatx16;
using mma::kBK;
using mma::kStageBytes;
using mma::kThreads;
using mma::kTileT;
using mma::kTileV;

// Binary-counter stack of the tile tree: at most floor(log2(tiles per chunk)) + 1 entries.
// The vocabulary limit of the fused path (2^26) bounds tiles per chunk by 2^15.
constexpr int kMaxTreeDepth = 17;

struct TileGeom {
  int64_t n_vt;       // vocabulary tiles (8 * tiles_per_chunk)
  int64_t n_tt;       // token tiles
  int64_t tpc;        // tiles per chunk
  int64_t block_tiles;  // tiles per block of the tile tree: max(1, P / 8), P = next_pow2(tpc)
  int64_t Vc, V, T;
};

// State of the 64 vocabulary rows a lane holds for one token (four 16-row groups, one per
// MFMA block): m = their max, then fp32 terms 2^{c (x - m)} and 2^{c (x - m)} c (x - m)
// summed pairwise -- within each quad, quad pairs, then the groups as ((0,1),(2,3)).
// With every value in registers the max comes first and no state merge is needed.
// WITH_U = false (no entropy or row state requested) leaves u at 0 and skips its terms;
// m and s, and so every logprob bit, are the same either way.
template <bool WITH_U>
__device__ __forceinline__ State leaf64(const float (&v)[4][16], float c) {
  float mg = v[0][0];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = (a == 0 ? 1 : 0); i < 16; ++i) mg = fmaxf(mg, v[a][i]);
  const float mref = (mg == kNegInf) ? 0.0f : mg;
  float sg[4], ug[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    float e[16], t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float x = (v[a][i] - mref) * c;
      e[i] = exp2_hw(x);
      if constexpr (WITH_U) t[i] = mul_zero_wins(e[i], x);  // 0 where e = 0 (a masked row)
    }
    float sq[4], uq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sq[j] = (e[4 * j] + e[4 * j + 1]) + (e[4 * j + 2] + e[4 * j + 3]);
      if constexpr (WITH_U) uq[j] = (t[4 * j] + t[4 * j + 1]) + (t[4 * j + 2] + t[4 * j + 3]);
    }
    sg[a] = (sq[0] + sq[1]) + (sq[2] + sq[3]);
    if constexpr (WITH_U) ug[a] = (uq[0] + uq[1]) + (uq[2] + uq[3]);
  }
  State r;
  r.m = mg;
  r.s = (double)((sg[0] + sg[1]) + (sg[2] + sg[3]));
  r.u = WITH_U ? (double)((ug[0] + ug[1]) + (ug[2] + ug[3])) : 0.0;
  return r;
}

// G: token tiles per group of the tile order (see grouped_tile_at and launch_linear_path).
// Persistent: the grid is a multiple of 8 workgroups, at most one per compute unit, and
// workgroup b takes the tile-order ids b, b + gridDim.x, b + 2 gridDim.x, ... (the same XCD,
// b mod 8, for all of them).  Right after a tile's K loop the workgroup issues the next
// tile's first stage and targets, which land while this tile's epilogue runs; the epilogue
// waits for no global load.  Every tile's arithmetic, and so every bit, is that of a
// workgroup that takes the tile alone.
template <bool WITH_U, int G = 8>
__global__ __launch_bounds__(kThreads, 1) void linear_tile_kernel(
    const uint16_t* __restrict__ H, int64_t ldh, const uint16_t* __restrict__ W, int64_t ldw,
    int64_t d, TileGeom g, const int64_t* __restrict__ targets, float c,
    WireState* __restrict__ tile_states, float* __restrict__ target_logit) {
  // Two K-loop stages, then the targets of a tile's 256 tokens in two buffers (tile parity),
  // staged by LDS-DMA with the tile's first stage so that the epilogue reads them from LDS
  // and waits for no load.  One LDS array for every LDS-DMA destination: with a second one
  // the compiler cannot tell a stage load from a fragment read and waits for every load in
  // flight before the fragment reads that follow the stage loads.
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes + 2 * kTileT * 8];
  int64_t (*tgt_lds)[kTileT] = reinterpret_cast<int64_t (*)[kTileT]>(smem + 2 * kStageBytes);

  const int64_t nb = g.n_vt * g.n_tt;
  const int64_t n_ids = 8 * ((nb + 7) / 8);
  const int64_t stride = gridDim.x;
  const int nk = (int)(d / kBK);
  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int wv = wave >> 2;  // vocab half (0, 1)
  const int wt = wave & 3;   // token quarter (0..3)

  // 32-bit tile coordinates (V < 2^26, T < 2^31): the tile loop keeps them in scalar
  // registers across the K loop, which needs nearly all of them.
  struct TileRef {
    int vt, v_lo, v_hi, t_lo;
  };
  const int T32 = (int)g.T, V32 = (int)g.V, Vc32 = (int)g.Vc, tpc32 = (int)g.tpc;
  // The next tile with vocabulary rows at or after id `id` of the tile order; empty tiles
  // (short chunks) met on the way get identity states, so that the tile tree sees no data.
  auto next_tile = [&](int64_t& id, TileRef& r) -> bool {
    for (; id < n_ids; id += stride) {
      int64_t vt, tt;
      if (!mma::grouped_tile_at<G>(id, g.n_vt, g.n_tt, vt, tt)) continue;
      const int vt32 = (int)vt;
      const int chunk = vt32 / tpc32;
      const int kin = vt32 - chunk * tpc32;
      const int chunk_lo = min(chunk * Vc32, V32);
      const int chunk_hi = min(chunk_lo + Vc32, V32);
      const int v_lo = chunk_lo + kin * kTileV;
      const int v_hi = min(v_lo + kTileV, chunk_hi);
      const int t_lo = (int)tt * kTileT;
      if (v_lo >= v_hi) {
        for (int j = tid; j < kTileT; j += kThreads) {
          const int tok = t_lo + j;
          if (tok < T32) tile_states[(int64_t)vt32 * T32 + tok] = to_wire(identity_state(), 0.0f);
        }
        continue;
      }
      r = TileRef{vt32, v_lo, v_hi, t_lo};
      id += stride;
      return true;
    }
    return false;
  };
  auto operand_w = [&](const TileRef& r) {
    return mma::Operand{W + (int64_t)r.v_lo * ldw, ldw, min(V32 - 1 - r.v_lo, kTileV - 1), 0};
  };
  auto operand_h = [&](const TileRef& r) {
    return mma::Operand{H + (int64_t)r.t_lo * ldh, ldh, min(T32 - 1 - r.t_lo, kTileT - 1), 0};
  };

  // One dword per lane: wave w stages bytes 256 w .. 256 w + 255 of the tile's 2 KiB of
  // targets (tokens at or beyond T read token T - 1's and are never used).
  auto issue_targets = [&](int t_lo, int buf) {
    if (!targets) return;
    const int dw = wave * 64 + mma::lane_id_here();
    const int tok = min(t_lo + (dw >> 1), T32 - 1);
    const char* src = reinterpret_cast<const char*>(targets + tok) + 4 * (dw & 1);
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)src,
        (__attribute__((address_space(3))) void*)(reinterpret_cast<char*>(tgt_lds[buf]) +
                                                  wave * 256),
        4, 0, 0);
  };

  int64_t id = blockIdx.x;
  TileRef cur;
  if (!next_tile(id, cur)) return;
  int p = 0;   // buffer of the current tile's first stage
  int tb = 0;  // buffer of the current tile's targets
  bool issued = false;
  issue_targets(cur.t_lo, tb);
  while (true) {
    TileRef nxt;
    const bool has_next = next_tile(id, nxt);
    const mma::Operand A = operand_w(cur), B = operand_h(cur);
    floatx16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
    mma::mma_tile_op<false, false, 2, true>(A, B, 0, nk, smem, acc, p, issued);
    // The next tile's first stage and targets, landing while this tile's epilogue runs.
    if (has_next) {
      mma::issue_first_stage(operand_w(nxt), operand_h(nxt), smem, (p + nk) & 1);
      issue_targets(nxt.t_lo, tb ^ 1);
    }
    // Every wave is done reading this tile's stages; the next tile's first stage may still
    // be landing in the other buffer, so the barrier waits for LDS work only.
    mma::lds_barrier();

    // -------------------------------------------------------------- epilogue
    // Each lane owns tokens wt*64 + b*32 + (lane%32), b = 0, 1, and for each of them the
    // 64 vocab rows wv*128 + a*32 + 8*(i/4) + 4*(lane/32) + (i%4).
    const int elane = mma::lane_id_here();
    const int frow = elane & 31;
    const int fhalf = elane >> 5;
    const int t_lo = cur.t_lo, v_lo = cur.v_lo, v_hi = cur.v_hi;
    const int n_valid = v_hi - v_lo;
    State half_state[2];
    // Two instantiations: only the last tile of a chunk has rows at or beyond n_valid to
    // mask, and keeping that test out of the common one keeps its selects and copies out too.
    auto token_epilogue = [&](auto masked) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int tok = t_lo + wt * 64 + b * 32 + frow;
        // A target outside [0, V) is in no tile.
        const int64_t t64 = (tok < T32 && targets) ? tgt_lds[tb][wt * 64 + b * 32 + frow] : -1;
        const int tg = (t64 >= 0 && t64 < V32) ? (int)t64 : -1;
        // Target row relative to this tile (-1 when the target is not in the tile), and
        // relative to this wave's vocab half.  Row r of the half is held by the lanes with
        // fhalf = (r / 4) % 2, in register i = 4 ((r / 8) % 4) + r % 4 of block a = r / 32.
        const int tloc = (tg >= v_lo && tg < v_hi) ? tg - v_lo : -1;
        const int r = tloc - wv * 128;
        const bool mine = tloc >= 0 && (unsigned)r < 128u && ((r >> 2) & 1) == fhalf;
        // Only about one token in twenty per wave has its target in this wave's rows, so
        // the capture sits behind a branch that whole waves skip.
        if (mine) {
          const int idx = ((r >> 5) << 4) | (((r >> 3) & 3) << 2) | (r & 3);  // 16 a + i
          float xt = 0.0f;
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 16; ++i) xt = (idx == 16 * a + i) ? acc[a][b][i] : xt;
          target_logit[tok] = xt;
        }

        float v[4][16];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            v[a][i] = acc[a][b][i];
            if constexpr (decltype(masked)::value) {
              const int vr = wv * 128 + a * 32 + 8 * (i >> 2) + 4 * fhalf + (i & 3);
              v[a][i] = (vr < n_valid) ? v[a][i] : kNegInf;
            }
          }
        const State st = leaf64<WITH_U>(v, c);
        const State o = shfl_xor_state(st, 32);
        half_state[b] = fhalf ? rlk_merge(o, st, c) : rlk_merge(st, o, c);
      }
    };
    if (n_valid < kTileV)
      token_epilogue(std::true_type{});
    else
      token_epilogue(std::false_type{});

    // Cross-half merge through LDS, in the buffer of this tile's last stage (the next tile's
    // first stage goes to the other one): the upper vocab half (wv = 1) publishes its
    // states, the lower half merges (lower range first) and stores the tile state.
    State* xch = reinterpret_cast<State*>(smem + ((p + nk - 1) & 1) * kStageBytes);
    if (wv == 1 && fhalf == 0) {
#pragma unroll
      for (int b = 0; b < 2; ++b) xch[wt * 64 + b * 32 + frow] = half_state[b];
    }
    mma::lds_barrier();
    if (wv == 0 && fhalf == 0) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int tok_in_tile = wt * 64 + b * 32 + frow;
        const int tok = t_lo + tok_in_tile;
        if (tok < T32) {
          const State r = rlk_merge(half_state[b], xch[tok_in_tile], c);
          tile_states[(int64_t)cur.vt * T32 + tok] = to_wire(r, 0.0f);
        }
      }
    }
    if (!has_next) break;
    cur = nxt;
    p = (p + nk) & 1;
    tb ^= 1;
    issued = true;
  }
  mma::wait_dma();  // every stage load of this workgroup has landed before it ends
}

// Batches of at most 128 tokens: one workgroup takes a pair of consecutive vocabulary tiles
// of a chunk (tiles 2p and 2p + 1, the second absent when the chunk has an odd count) as a
// 512 x 128 output tile, so that half the workgroups do the same MFMA work as 256 x 256
// tiles whose tokens would be mostly padding.  Each wave still holds 128 vocabulary rows x 64
// tokens at the same places within its tile, and each tile's state is formed exactly as in
// linear_tile_kernel (same leaves, same merges), so the bits are the same.
template <bool WITH_U>
__global__ __launch_bounds__(kThreads, 1) void linear_pair_kernel(
    const uint16_t* __restrict__ H, int64_t ldh, const uint16_t* __restrict__ W, int64_t ldw,
    int64_t d, TileGeom g, const int64_t* __restrict__ targets, float c,
    WireState* __restrict__ tile_states, float* __restrict__ target_logit) {
  constexpr int kPairStage = (2 * kTileV + 128) * kBK * 2;  // 80 KiB
  __shared__ __attribute__((aligned(16))) char smem[2 * kPairStage];
  const int64_t pp = (g.tpc + 1) / 2;  // pairs per chunk
  int64_t pr, tt;
  if (!mma::grouped_tile_of<8>(8 * pp, 1, pr, tt)) return;
  const int64_t chunk = pr / pp;
  const int64_t k0 = 2 * (pr % pp);
  const bool has_second = k0 + 1 < g.tpc;
  const int64_t vt0 = chunk * g.tpc + k0;
  const int64_t chunk_lo = min(chunk * g.Vc, g.V);
  const int64_t chunk_hi = min(chunk_lo + g.Vc, g.V);
  const int64_t v_lo = chunk_lo + k0 * kTileV;
  const int n_pair = (int)max((int64_t)0, min(v_lo + 2 * (int64_t)kTileV, chunk_hi) - v_lo);
  if (n_pair == 0) {
    // Empty tiles (short chunk): identity states so that the tile tree sees no data.
    for (int j = threadIdx.x; j < 2 * 128; j += kThreads) {
      const int pt = j >> 7;
      const int64_t tok = j & 127;
      if (tok < g.T && (pt == 0 || has_second))
        tile_states[(vt0 + pt) * g.T + tok] = to_wire(identity_state(), 0.0f);
    }
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int wv = wave >> 1;  // 128-row slice of the pair (0..3)
  const int wt = wave & 1;   // token half (0, 1)
  const int pt = wv >> 1;    // tile of the pair
  const int hv = wv & 1;     // vocab half of that tile
  const int64_t v_lo_t = v_lo + (int64_t)pt * kTileV;
  const int n_valid = max(0, min(n_pair - pt * kTileV, kTileV));

  floatx16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  const int w_last = (int)min(g.V - 1 - v_lo, (int64_t)(2 * kTileV - 1));
  const int h_last = (int)min(g.T - 1, (int64_t)127);
  mma::mma_tile_op<false, false, 4>(mma::Operand{W + v_lo * ldw, ldw, w_last, 0},
                                    mma::Operand{H, ldh, h_last, 0}, 0, (int)(d / kBK), smem,
                                    acc);
  __syncthreads();
  const int frow = lane & 31;
  const int fhalf = lane >> 5;

  // Epilogue as in linear_tile_kernel, per tile of the pair: lane tokens wt*64 + b*32 +
  // (lane%32), vocab rows hv*128 + a*32 + 8*(i/4) + 4*(lane/32) + (i%4) of tile pt.
  State half_state[2];
  auto token_epilogue = [&](auto masked) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int tok_in_tile = wt * 64 + b * 32 + frow;
      const int64_t tok = tok_in_tile;
      const int64_t tgt = (tok < g.T && targets) ? targets[tok] : -1;
      const int tloc = (tgt >= v_lo_t && tgt < v_lo_t + n_valid) ? (int)(tgt - v_lo_t) : -1;
      const int r = tloc - hv * 128;
      const bool mine = tloc >= 0 && (unsigned)r < 128u && ((r >> 2) & 1) == fhalf;
      if (mine) {
        const int idx = ((r >> 5) << 4) | (((r >> 3) & 3) << 2) | (r & 3);  // 16 a + i
        float xt = 0.0f;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int i = 0; i < 16; ++i) xt = (idx == 16 * a + i) ? acc[a][b][i] : xt;
        target_logit[tok] = xt;
      }
      float v[4][16];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          v[a][i] = acc[a][b][i];
          if constexpr (decltype(masked)::value) {
            const int vr = hv * 128 + a * 32 + 8 * (i >> 2) + 4 * fhalf + (i & 3);
            v[a][i] = (vr < n_valid) ? v[a][i] : kNegInf;
          }
        }
      const State st = leaf64<WITH_U>(v, c);
      const State o = shfl_xor_state(st, 32);
      half_state[b] = fhalf ? rlk_merge(o, st, c) : rlk_merge(st, o, c);
    }
  };
  if (n_valid < kTileV)
    token_epilogue(std::true_type{});
  else
    token_epilogue(std::false_type{});

  State* xch = reinterpret_cast<State*>(smem);
  if (hv == 1 && fhalf == 0) {
#pragma unroll
    for (int b = 0; b < 2; ++b) xch[pt * 128 + wt * 64 + b * 32 + frow] = half_state[b];
  }
  __syncthreads();
  if (hv == 0 && fhalf == 0 && (pt == 0 || has_second)) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int tok_in_tile = wt * 64 + b * 32 + frow;
      const int64_t tok = tok_in_tile;
      if (tok < g.T) {
        const State r = n_valid > 0 ? rlk_merge(half_state[b], xch[pt * 128 + tok_in_tile], c)
                                    : identity_state();
        tile_states[(vt0 + pt) * g.T + tok] = to_wire(r, 0.0f);
      }
    }
  }
}

// Tiles of each chunk -> chunk state, chunks of a shard -> shard state (tree8), then
// either the fp64 finalize (S = 1) or the shard's wire state for the cross-shard merge.
//
// The tile tree is the perfect binary tree over tile index, padded with identity states up
// to P = max(8, next power of two >= tiles per chunk) leaves (merging a state with the
// identity on its right returns it unchanged, up to the sign of a zero u).  A wave serves
// 8 consecutive tokens x 8 aligned blocks of B = P / 8 tiles: lane = 8 blk + token, so each
// load instruction reads 8 runs of 8 consecutive tokens' states (192 bytes each).  A lane
// reduces its block -- the subtree of that block, identities elided -- and an xor-butterfly
// over the block bits (strides 8, 16, 32; lower block first) applies the top three levels.
// Block: CPS waves (the shard's chunks); grid (ceil(T / 8), S).
//
// LB = log2 B when B <= 16 (every vocabulary up to 8 * 128 * 256 = 262144): the lane issues
// all B loads at once and reduces them level by level in registers.  LB = kStackLB for
// larger blocks: one load at a time, folded into a binary-counter stack.  Both evaluate the
// same tree, so they give the same bits.
constexpr int kStackLB = 5;

// Subtree of leaves [k0, k1) of a block of 2^LB, k0 < k1 <= k0 + 2^LB; a right subtree with
// no leaves is elided (its parent is its left subtree).
template <int LB>
__device__ __forceinline__ State block_subtree(const WireState* __restrict__ base, int64_t k0,
                                               int64_t k1, int64_t stride, float c) {
  constexpr int B = 1 << LB;
  const int n = (int)(k1 - k0);
  State v[B];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    // Leaves past the end re-read the last one (in bounds); they are never merged.
    const int64_t k = k0 + min(i, n - 1);
    v[i] = from_wire(base[k * stride]);
  }
#pragma unroll
  for (int w = B / 2; w >= 1; w /= 2) {
    const int span = B / w / 2;  // leaves under each child at this level
#pragma unroll
    for (int i = 0; i < w; ++i)
      if ((2 * i + 1) * span < n) v[i] = rlk_merge(v[2 * i], v[2 * i + 1], c);
      else v[i] = v[2 * i];
  }
  return v[0];
}

template <>
__device__ __forceinline__ State block_subtree<kStackLB>(const WireState* __restrict__ base,
                                                         int64_t k0, int64_t k1, int64_t stride,
                                                         float c) {
  State stk[kMaxTreeDepth];
  int top = 0;
  for (int64_t k = k0; k < k1; ++k) {
    State cur = from_wire(base[k * stride]);
    for (int64_t b = k - k0; b & 1; b >>= 1) cur = rlk_merge(stk[--top], cur, c);
    stk[top++] = cur;
  }
  State r = stk[--top];
  while (top > 0) r = rlk_merge(stk[--top], r, c);
  return r;
}

template <int CPS, int LB>
__global__ __launch_bounds__(64 * CPS) void tile_tree_kernel(
    const WireState* __restrict__ tile_states, const float* __restrict__ target_logit,
    TileGeom g, const int64_t* __restrict__ targets, float c, double beta,
    float* __restrict__ lp_out, float* __restrict__ ent_out, WireState* __restrict__ shard_ws,
    WireState* __restrict__ root) {
  const int lane = threadIdx.x & 63;
  const int ci = threadIdx.x >> 6;
  const int tl8 = lane & 7;
  const int blk = lane >> 3;
  const int64_t tok = linear_block() * 8 + tl8;
  const int shard = blockIdx.y;
  const int64_t chunk = (int64_t)shard * CPS + ci;
  __shared__ State cs[CPS][8];

  const int64_t k0 = (int64_t)blk * g.block_tiles;
  const int64_t k1 = min(k0 + g.block_tiles, g.tpc);
  State r = identity_state();
  if (tok < g.T && k0 < k1)
    r = block_subtree<LB>(tile_states + chunk * g.tpc * g.T + tok, k0, k1, g.T, c);
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
    const State o = shfl_xor_state(r, off);
    r = (lane & off) ? rlk_merge(o, r, c) : rlk_merge(r, o, c);
  }
  if (blk == 0) cs[ci][tl8] = r;
  __syncthreads();
  if (ci != 0 || blk != 0 || tok >= g.T) return;
  State chunks[CPS];
#pragma unroll
  for (int j = 0; j < CPS; ++j) chunks[j] = cs[j][tl8];
  const State top_state = tree8(chunks, CPS, c);
  const int64_t t = targets ? targets[tok] : -1;
  if constexpr (CPS == 8) {
    const bool has = (t >= 0) && (t < g.V);
    const float xt = has ? target_logit[tok] : 0.0f;
    if (root) root[tok] = to_wire(top_state, xt);
    if (lp_out || ent_out)
      rlk_finalize(top_state, xt, has, beta, lp_out ? lp_out + tok : nullptr,
                   ent_out ? ent_out + tok : nullptr);
  } else {
    const int64_t s_lo = min((int64_t)shard * CPS * g.Vc, g.V);
    const int64_t s_hi = min(s_lo + (int64_t)CPS * g.Vc, g.V);
    const bool mine = (t >= s_lo) && (t < s_hi);
    shard_ws[(int64_t)shard * g.T + tok] = to_wire(top_state, mine ? target_logit[tok] : 0.0f);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// tile_tree_kernel for a shard of CPS chunks and blocks of 2^lb tiles (the stack form above 16).
template <int CPS>
void launch_tile_tree(int lb, dim3 grid, hipStream_t stream, const WireState* tiles,
                      const float* tl, const TileGeom& g, const int64_t* targets, float c,
                      double beta, float* lp, float* ent, WireState* sws, WireState* root) {
  const dim3 block(64 * CPS);
#define RLK_TREE(L)                                                                          \
  hipLaunchKernelGGL((tile_tree_kernel<CPS, L>), grid, block, 0, stream, tiles, tl, g, targets, \
                     c, beta, lp, ent, sws, root)
  switch (lb) {
    case 0: RLK_TREE(0); break;
    case 1: RLK_TREE(1); break;
    case 2: RLK_TREE(2); break;
    case 3: RLK_TREE(3); break;
    case 4: RLK_TREE(4); break;
    default: RLK_TREE(kStackLB); break;
  }
#undef RLK_TREE
}

}  // namespace

LinearWorkspace linear_workspace_layout(int64_t T, int64_t V, int S) {
  LinearWorkspace L;
  const int64_t Vc = chunk_cols(V);
  L.tiles_per_chunk = (Vc + kTileV - 1) / kTileV;
  L.n_tiles = 8 * L.tiles_per_chunk;
  size_t off = 0;
  L.tile_states = off;
  off += align256((size_t)L.n_tiles * (size_t)T * sizeof(WireState));
  L.target_logit = off;
  off += align256((size_t)T * sizeof(float));
  L.shard_states = off;
  off += (S > 1) ? align256((size_t)S * (size_t)T * sizeof(WireState)) : 0;
  L.total = off;
  return L;
}

// Compute units of the current device rounded down to a multiple of 8 (the XCD count), so
// that a persistent workgroup b stays on XCD b mod 8 for every tile it takes.  Cached per
// device.
static int64_t persistent_workgroups() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu < 8)
      cu = 256;
    n = cu / 8 * 8;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_linear_path(const LinearArgs& a, hipStream_t stream) {
  const LinearWorkspace L = linear_workspace_layout(a.T, a.V, a.S);
  TileGeom g;
  g.tpc = L.tiles_per_chunk;
  if (g.tpc > (int64_t(1) << (kMaxTreeDepth - 1))) return hipErrorInvalidValue;
  int64_t pow2 = 1;
  while (pow2 < g.tpc) pow2 <<= 1;
  g.block_tiles = pow2 > 8 ? pow2 / 8 : 1;
  g.n_vt = L.n_tiles;
  g.n_tt = (a.T + kTileT - 1) / kTileT;
  g.Vc = a.Vc;
  g.V = a.V;
  g.T = a.T;
  char* base = static_cast<char*>(a.ws);
  const int64_t nb = g.n_vt * g.n_tt;
  const int64_t nb_pad = ((nb + 7) / 8) * 8;
  // Entropy terms only when an entropy or a row state is asked for.
  const bool with_u = a.ent || a.root;
  if (a.T <= 128) {
    const int64_t n_pairs = 8 * ((g.tpc + 1) / 2);
    const dim3 pgrid = split_grid((n_pairs + 7) / 8 * 8);
    if (with_u)
      hipLaunchKernelGGL(linear_pair_kernel<true>, pgrid, dim3(kThreads), 0, stream, a.H, a.ldh,
                         a.W, a.ldw, a.d, g, a.targets, a.c,
                         reinterpret_cast<WireState*>(base + L.tile_states),
                         reinterpret_cast<float*>(base + L.target_logit));
    else
      hipLaunchKernelGGL(linear_pair_kernel<false>, pgrid, dim3(kThreads), 0, stream, a.H, a.ldh,
                         a.W, a.ldw, a.d, g, a.targets, a.c,
                         reinterpret_cast<WireState*>(base + L.tile_states),
                         reinterpret_cast<float*>(base + L.target_logit));
  } else {
    // Token tiles per group of the tile order: an XCD runs ~32 tiles at once, i.e. a few
    // vocabulary tiles times one group.  With 5 to 8 token tiles (1024 < T <= 2048), groups
    // of 4 (8 vocabulary tiles at once, H of 4 token tiles re-read from the infinity cache
    // every 8 vocabulary tiles, W read by two XCDs) measured +0.2 to +0.5 points at T = 2048
    // over one group of 8 (three same-process A/Bs on three boxes, bits equal); with up to 4 token tiles both give
    // one group, and with more than 8, groups of 8 (T = 16384: 51.9% against 51.0% with 4).
    // Persistent: at most one workgroup per compute unit, a multiple of 8 of them.
    const int64_t grid = std::min<int64_t>(nb_pad, persistent_workgroups());
    auto launch = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a.H, a.ldh, a.W,
                         a.ldw, a.d, g, a.targets, a.c,
                         reinterpret_cast<WireState*>(base + L.tile_states),
                         reinterpret_cast<float*>(base + L.target_logit));
    };
    const bool g4 = g.n_tt > 4 && g.n_tt <= 8;
    if (with_u)
      g4 ? launch(linear_tile_kernel<true, 4>) : launch(linear_tile_kernel<true, 8>);
    else
      g4 ? launch(linear_tile_kernel<false, 4>) : launch(linear_tile_kernel<false, 8>);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const WireState* tiles = reinterpret_cast<const WireState*>(base + L.tile_states);
  const float* tl = reinterpret_cast<const float*>(base + L.target_logit);
  WireState* sws = reinterpret_cast<WireState*>(base + L.shard_states);
  const dim3 tgrid = split_grid((a.T + 7) / 8, (unsigned)a.S);
  int lb = 0;
  while ((int64_t(1) << lb) < g.block_tiles) ++lb;
  switch (a.S) {
    case 1:
      launch_tile_tree<8>(lb, tgrid, stream, tiles, tl, g, a.targets, a.c, a.beta, a.lp, a.ent,
                          sws, a.root);
      return hipGetLastError();
    case 2:
      launch_tile_tree<4>(lb, tgrid, stream, tiles, tl, g, a.targets, a.c, a.beta, a.lp, a.ent,
                          sws, a.root);
      break;
    case 4:
      launch_tile_tree<2>(lb, tgrid, stream, tiles, tl, g, a.targets, a.c, a.beta, a.lp, a.ent,
                          sws, a.root);
      break;
    case 8:
      launch_tile_tree<1>(lb, tgrid, stream, tiles, tl, g, a.targets, a.c, a.beta, a.lp, a.ent,
                          sws, a.root);
      break;
    default:
      return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_shard_merge(sws, a.T, a.targets, a.V, (int64_t)(8 / a.S) * a.Vc, a.c, a.beta,
                            a.S, a.lp, a.ent, a.root, stream);
}

}  // namespace rlk
