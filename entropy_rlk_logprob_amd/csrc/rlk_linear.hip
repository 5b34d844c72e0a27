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
//     into four 32-row MFMA blocks; within a block a lane holds 16 rows
//     8*(i/4) + 4*(lane/32) + (i%4), i = 0..15, which form one 16-element leaf (the same
//     leaf as on the logits path: pairwise fp32 sums); the four leaves of a lane merge as
//     ((0,1),(2,3)), then lane halves (lane < 32 first), then the two 128-row halves;
//   * tiles of a chunk: balanced binary tree over tile index (padded with identities);
//     chunks: ((0,1),(2,3)),((4,5),(6,7)), the top log2(S) levels in the shard merge.
//
// Workgroup: 8 waves, a 256 (vocab) x 256 (token) output tile, waves arranged 2 (vocab)
// x 4 (token), each wave 128 x 64 = 4 x 2 MFMA blocks.  K step 64 with two LDS stages
// (64 KiB each: the W and H slices with an XOR swizzle on 16-byte columns so that
// ds_read_b128 of 16 consecutive rows hits distinct banks).  Workgroup ids are remapped
// so that the token tiles of one vocabulary tile run back to back on the same XCD and
// share its W slice in that XCD's L2.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "rlk_launch.hpp"
#include "rlk_state.hpp"

namespace rlk {

namespace {

constexpr int kTileV = 256;   // vocab rows per tile
constexpr int kTileT = 256;   // tokens per tile
constexpr int kBK = 64;       // hidden elements per K step
constexpr int kThreads = 512; // 8 waves
constexpr int kStageBytes = (kTileV + kTileT) * kBK * 2;  // 64 KiB

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

struct alignas(16) U4 {
  uint32_t x, y, z, w;
};

// All LDS-DMA loads of this wave have landed.
// Scheduling groups (llvm.amdgcn.sched.group.barrier): the instructions of the current
// scheduling region are placed in the order of the groups requested.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedVmemRead = 0x020;
#define sched_group(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier ordering LDS reads (this wave's ds_reads done, then s_barrier).  The
// LDS-DMA stage that the next step reads was waited for by every wave before it arrives.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS slab layout: rows of kBK bf16 = 128 bytes; 16-byte column c16 of row r sits at
// physical column c16 ^ ((r / 2) % 8).  The XOR key makes the 16 rows that one 16-lane
// ds_read_b128 pass touches land in 16 distinct 16-byte bank groups of the 64-bank LDS.
__device__ __forceinline__ int lds_offset(int row, int c16) {
  return row * 128 + ((c16 ^ ((row >> 1) & 7)) << 4);
}

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

__global__ __launch_bounds__(kThreads, 1) void linear_tile_kernel(
    const uint16_t* __restrict__ H, int64_t ldh, const uint16_t* __restrict__ W, int64_t ldw,
    int64_t d, TileGeom g, const int64_t* __restrict__ targets, float c,
    WireState* __restrict__ tile_states, float* __restrict__ target_logit) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];

  // Remap the hardware id (dispatched round-robin over the 8 XCDs) so that logically
  // consecutive tiles -- the token tiles of one vocabulary tile -- share an XCD.
  const int64_t nb = g.n_vt * g.n_tt;
  const int64_t per_xcd = (nb + 7) / 8;
  const int64_t hw = blockIdx.x;
  const int64_t logical = (hw % 8) * per_xcd + hw / 8;
  if (logical >= nb) return;
  const int64_t vt = logical / g.n_tt;
  const int64_t tt = logical % g.n_tt;
  const int64_t chunk = vt / g.tpc;
  const int64_t kin = vt % g.tpc;
  const int64_t chunk_lo = min(chunk * g.Vc, g.V);
  const int64_t chunk_hi = min(chunk_lo + g.Vc, g.V);
  const int64_t v_lo = chunk_lo + kin * kTileV;
  const int64_t v_hi = min(v_lo + (int64_t)kTileV, chunk_hi);
  const int64_t t_lo = tt * kTileT;
  if (v_lo >= v_hi) {
    // Empty tile (short chunk): identity states so that the tile tree sees no data.
    for (int j = threadIdx.x; j < kTileT; j += kThreads) {
      const int64_t tok = t_lo + j;
      if (tok < g.T) tile_states[vt * g.T + tok] = to_wire(identity_state(), 0.0f);
    }
    return;
  }

  const int n_valid = (int)(v_hi - v_lo);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = wave >> 2;  // vocab half (0, 1)
  const int wt = wave & 3;   // token quarter (0..3)

  // Global -> LDS: direct 16-byte-per-lane loads into LDS (global_load_lds_dwordx4).  One
  // wave instruction fills one 1 KiB block = 8 slab rows: lane l writes physical column
  // l % 8 of row r = 8 b + l / 8 of block b, so it fetches logical column
  // (l % 8) ^ ((r / 2) % 8), the layout of lds_offset().  Blocks 0..31 are the W slab,
  // 32..63 the H slab; wave w fills blocks w, w + 8, ..., w + 56.  Offsets are
  // tile-relative on workgroup-uniform bases; rows beyond the valid range are clamped to
  // the last valid row (their values are masked in the epilogue or never stored).
  constexpr int kBlocksPerWave = (kTileV + kTileT) / 8 / (kThreads / 64);  // 8
  constexpr int kWBlocks = kTileV / 8;
  const uint16_t* __restrict__ Wt = W + v_lo * ldw;
  const uint16_t* __restrict__ Ht = H + t_lo * ldh;
  const int w_last = (int)min(g.V - 1 - v_lo, (int64_t)(kTileV - 1));
  const int h_last = (int)min(g.T - 1 - t_lo, (int64_t)(kTileT - 1));
  int src_off[kBlocksPerWave];
#pragma unroll
  for (int i = 0; i < kBlocksPerWave; ++i) {
    const int blk = i * 8 + wave;
    const bool is_w = i < kWBlocks / 8;
    const int bb = is_w ? blk : blk - kWBlocks;
    const int row = bb * 8 + (lane >> 3);
    const int col = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
    src_off[i] = is_w ? (min(row, w_last) * (int)ldw + col) : (min(row, h_last) * (int)ldh + col);
  }
  auto issue_stage = [&](int64_t k0, int stage) {
#pragma unroll
    for (int i = 0; i < kBlocksPerWave; ++i) {
      const int blk = i * 8 + wave;
      const bool is_w = i < kWBlocks / 8;
      const uint16_t* src = (is_w ? Wt : Ht) + k0 + src_off[i];
      char* dst = smem + stage * kStageBytes + blk * 1024;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  };

  floatx16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  const int nk = (int)(d / kBK);
  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  issue_stage(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt has landed for every wave, and every wave is done reading stage kt - 1,
    // whose buffer the loads of stage kt + 1 now overwrite.
    wait_dma();
    lds_barrier();
    const char* wb = smem + (kt & 1) * kStageBytes;
    const char* hb = wb + kTileV * kBK * 2;
    // Fragments of step ks + 1 are read from LDS while the MFMAs of step ks run.
    bf16x8 af[2][4], bfr[2][2];
    auto read_frags = [&](int ks, int buf) {
      const int c16 = 2 * ks + fhalf;
#pragma unroll
      for (int a = 0; a < 4; ++a)
        af[buf][a] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const U4*>(wb + lds_offset(wv * 128 + a * 32 + frow, c16)));
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bfr[buf][b] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const U4*>(hb + lds_offset(wt * 64 + b * 32 + frow, c16)));
    };
    read_frags(0, 0);
    sched_group(kSchedDsRead, 6);
    // Loads of stage kt + 1 into the other buffer.  Issued on every stage (the last one
    // repeats stage nk - 1 into the idle buffer) so that they stay in this scheduling
    // region and can be spread between the MFMAs of step 0 instead of stalling the wave.
    issue_stage((int64_t)min(kt + 1, nk - 1) * kBK, (kt + 1) & 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) read_frags(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][a], bfr[ks & 1][b],
                                                              acc[a][b], 0, 0, 0);
      // Instruction order: step 0 interleaves its eight MFMAs with the eight loads of the
      // next stage, then reads the fragments of step 1; steps 1 and 2 interleave the six
      // LDS reads of the following step with their first six MFMAs.  Left to itself the
      // scheduler merges the two fragment buffers, waits on each read right away and
      // issues all stage loads in one burst ahead of the MFMAs.
      if (ks == 0) {
#pragma unroll
        for (int q = 0; q < kBlocksPerWave; ++q) {
          sched_group(kSchedMfma, 1);
          sched_group(kSchedVmemRead, 1);
        }
        sched_group(kSchedDsRead, 6);
      } else if (ks + 1 < 4) {
#pragma unroll
        for (int q = 0; q < 6; ++q) {
          sched_group(kSchedMfma, 1);
          sched_group(kSchedDsRead, 1);
        }
        sched_group(kSchedMfma, 2);
      } else {
        sched_group(kSchedMfma, 8);
      }
    }
  }
  wait_dma();  // the repeated last-stage loads land before the epilogue reuses the LDS
  __syncthreads();

  // ---------------------------------------------------------------- epilogue
  // Each lane owns tokens wt*64 + b*32 + (lane%32), b = 0, 1, and for each of them the
  // 64 vocab rows wv*128 + a*32 + 8*(i/4) + 4*(lane/32) + (i%4).
  State half_state[2];
  // Two instantiations: only the last tile of a chunk has rows at or beyond n_valid to mask,
  // and keeping that test out of the common one keeps its selects and copies out too.
  auto token_epilogue = [&](auto masked) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int tok_in_tile = wt * 64 + b * 32 + frow;
      const int64_t tok = t_lo + tok_in_tile;
      const int64_t tgt = (tok < g.T && targets) ? targets[tok] : -1;
      // Target row relative to this tile (-1 when the target is not in the tile), and
      // relative to this wave's vocab half.  Row r of the half is held by the lanes with
      // fhalf = (r / 4) % 2, in register i = 4 ((r / 8) % 4) + r % 4 of block a = r / 32.
      const int tloc = (tgt >= v_lo && tgt < v_hi) ? (int)(tgt - v_lo) : -1;
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

      State leaf[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          v[i] = acc[a][b][i];
          if constexpr (decltype(masked)::value) {
            const int vr = wv * 128 + a * 32 + 8 * (i >> 2) + 4 * fhalf + (i & 3);
            v[i] = (vr < n_valid) ? v[i] : kNegInf;
          }
        }
        leaf[a] = leaf16(v, c);
      }
      State st = rlk_merge(rlk_merge(leaf[0], leaf[1], c), rlk_merge(leaf[2], leaf[3], c), c);
      const State o = shfl_xor_state(st, 32);
      half_state[b] = fhalf ? rlk_merge(o, st, c) : rlk_merge(st, o, c);
    }
  };
  if (n_valid < kTileV)
    token_epilogue(std::true_type{});
  else
    token_epilogue(std::false_type{});

  // Cross-half merge through LDS: the upper vocab half (wv = 1) publishes its states,
  // the lower half merges (lower range first) and stores the tile state.
  State* xch = reinterpret_cast<State*>(smem);
  if (wv == 1 && fhalf == 0) {
#pragma unroll
    for (int b = 0; b < 2; ++b) xch[wt * 64 + b * 32 + frow] = half_state[b];
  }
  __syncthreads();
  if (wv == 0 && fhalf == 0) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int tok_in_tile = wt * 64 + b * 32 + frow;
      const int64_t tok = t_lo + tok_in_tile;
      if (tok < g.T) {
        const State r = rlk_merge(half_state[b], xch[tok_in_tile], c);
        tile_states[vt * g.T + tok] = to_wire(r, 0.0f);
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
// 8 consecutive tokens x 8 aligned blocks of P / 8 tiles: lane = 8 blk + token, so each
// load instruction reads 8 runs of 8 consecutive tokens' states (192 bytes each).  A lane
// folds its block with a binary-counter stack (identities elided) -- the subtree of that
// block -- and an xor-butterfly over the block bits (strides 8, 16, 32; lower block first)
// applies the top three levels.  Block: CPS waves (the shard's chunks); grid
// (ceil(T / 8), S).
template <int CPS>
__global__ __launch_bounds__(64 * CPS) void tile_tree_kernel(
    const WireState* __restrict__ tile_states, const float* __restrict__ target_logit,
    TileGeom g, const int64_t* __restrict__ targets, float c, double beta,
    float* __restrict__ lp_out, float* __restrict__ ent_out, WireState* __restrict__ shard_ws) {
  const int lane = threadIdx.x & 63;
  const int ci = threadIdx.x >> 6;
  const int tl8 = lane & 7;
  const int blk = lane >> 3;
  const int64_t tok = (int64_t)blockIdx.x * 8 + tl8;
  const int shard = blockIdx.y;
  const int64_t chunk = (int64_t)shard * CPS + ci;
  __shared__ State cs[CPS][8];

  const int64_t k0 = (int64_t)blk * g.block_tiles;
  const int64_t k1 = min(k0 + g.block_tiles, g.tpc);
  State r = identity_state();
  if (tok < g.T && k0 < k1) {
    const WireState* __restrict__ base = tile_states + chunk * g.tpc * g.T + tok;
    State stk[kMaxTreeDepth];
    int top = 0;
    for (int64_t k = k0; k < k1; ++k) {
      State cur = from_wire(base[k * g.T]);
      for (int64_t b = k - k0; b & 1; b >>= 1) cur = rlk_merge(stk[--top], cur, c);
      stk[top++] = cur;
    }
    r = stk[--top];
    while (top > 0) r = rlk_merge(stk[--top], r, c);
  }
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
  const State root = tree8(chunks, CPS, c);
  const int64_t t = targets ? targets[tok] : -1;
  if constexpr (CPS == 8) {
    const bool has = (t >= 0) && (t < g.V);
    const float xt = has ? target_logit[tok] : 0.0f;
    rlk_finalize(root, xt, has, beta, lp_out ? lp_out + tok : nullptr,
                 ent_out ? ent_out + tok : nullptr);
  } else {
    const int64_t s_lo = min((int64_t)shard * CPS * g.Vc, g.V);
    const int64_t s_hi = min(s_lo + (int64_t)CPS * g.Vc, g.V);
    const bool mine = (t >= s_lo) && (t < s_hi);
    shard_ws[(int64_t)shard * g.T + tok] = to_wire(root, mine ? target_logit[tok] : 0.0f);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

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
  hipLaunchKernelGGL(linear_tile_kernel, dim3((unsigned)nb_pad), dim3(kThreads), 0, stream, a.H,
                     a.ldh, a.W, a.ldw, a.d, g, a.targets, a.c,
                     reinterpret_cast<WireState*>(base + L.tile_states),
                     reinterpret_cast<float*>(base + L.target_logit));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const WireState* tiles = reinterpret_cast<const WireState*>(base + L.tile_states);
  const float* tl = reinterpret_cast<const float*>(base + L.target_logit);
  WireState* sws = reinterpret_cast<WireState*>(base + L.shard_states);
  const dim3 tgrid((unsigned)((a.T + 7) / 8), (unsigned)a.S);
  switch (a.S) {
    case 1:
      hipLaunchKernelGGL((tile_tree_kernel<8>), tgrid, dim3(512), 0, stream, tiles, tl, g,
                         a.targets, a.c, a.beta, a.lp, a.ent, sws);
      return hipGetLastError();
    case 2:
      hipLaunchKernelGGL((tile_tree_kernel<4>), tgrid, dim3(256), 0, stream, tiles, tl, g,
                         a.targets, a.c, a.beta, a.lp, a.ent, sws);
      break;
    case 4:
      hipLaunchKernelGGL((tile_tree_kernel<2>), tgrid, dim3(128), 0, stream, tiles, tl, g,
                         a.targets, a.c, a.beta, a.lp, a.ent, sws);
      break;
    case 8:
      hipLaunchKernelGGL((tile_tree_kernel<1>), tgrid, dim3(64), 0, stream, tiles, tl, g,
                         a.targets, a.c, a.beta, a.lp, a.ent, sws);
      break;
    default:
      return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_shard_merge(sws, a.T, a.targets, a.V, (int64_t)(8 / a.S) * a.Vc, a.c, a.beta,
                            a.S, a.lp, a.ent, nullptr, stream);
}

}  // namespace rlk
