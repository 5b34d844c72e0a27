// Internal launch interface between the C-ABI host layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rlk_logprob.h"

namespace rlk {

struct WireState;

// Launch grids.  A dispatch holds at most 2^32 - 1 work-items along each dimension, so a
// grid of n blocks is laid out as x = min(n, kGridX) blocks times z = ceil(n / x): the
// kernel's block index is blockIdx.z * gridDim.x + blockIdx.x (linear_block), and the
// blocks at or beyond n return at once.  kGridX = 2^22 keeps blocks of up to 512 threads
// at 2^31 work-items along x, and is a multiple of 8, so that a block's XCD (its index in
// dispatch order mod 8) stays blockIdx.x mod 8.
constexpr int64_t kGridX = int64_t(1) << 22;

inline dim3 split_grid(int64_t n, unsigned y = 1) {
  if (n < 1) n = 1;
  const int64_t x = n < kGridX ? n : kGridX;
  return dim3((unsigned)x, y, (unsigned)((n + x - 1) / x));
}

__device__ __forceinline__ int64_t linear_block() {
  return (int64_t)blockIdx.z * gridDim.x + blockIdx.x;
}

// The wave's index within its workgroup (threadIdx.x / 64, the same on every lane of a
// wave).  readfirstlane tells the compiler it is wave-uniform, so whatever derives from it
// (tile offsets, chunk bounds, loop counts, branches) stays in scalar registers and scalar
// branches instead of per-lane registers and exec masks.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Canonical vocabulary partition shared by both paths: 8 chunks of Vc columns,
// Vc = 4 * ceil(ceil(V / 8) / 4).
inline int64_t chunk_cols(int64_t V) {
  const int64_t v8 = (V + 7) / 8;
  return ((v8 + 3) / 4) * 4;
}

struct LogitsArgs {
  const float* X;          // fp32 logits, or null when Xh is given
  const uint16_t* Xh;      // bf16 logits (bit patterns), or null
  int64_t ld, T, V, Vc;
  const int64_t* targets;  // may be null (entropy only)
  float c;                 // log2(e) / tau, rounded once to fp32
  double beta;             // 1 / tau in fp64
  int S;                   // vocab splits: 1, 2, 4, 8
  bool vec;                // quad loads legal (base aligned to a quad, ld % 4 == 0)
  float* lp;               // may be null
  float* ent;              // may be null
  WireState* ws;           // S * T wire states when S > 1
  WireState* root;         // when non-null: each row's root state (as well as lp / ent)
};

hipError_t launch_logits_path(const LogitsArgs& a, hipStream_t stream);

// Backward of the logits path (rlk_backward.hip): the row states into a.root (which must be
// set), then the gradient G[T, ldg]; vec: 16-byte accesses legal for both X and G.
hipError_t launch_logits_backward(const LogitsArgs& a, const float* g_lp, const float* g_ent,
                                  float* G, int64_t ldg, bool vec, bool have_states,
                                  hipStream_t stream);

// Top log2(S) levels of the chunk tree over S shard states ([S][T] wire states), then
// the fp64 finalize of every row (when lp or ent is non-null) and / or each row's root
// state (when root is non-null).
// Shared by both paths.
hipError_t launch_shard_merge(const WireState* ws, int64_t T, const int64_t* targets, int64_t V,
                              int64_t shard_cols, float c, double beta, int S, float* lp,
                              float* ent, WireState* root, hipStream_t stream);

struct LinearArgs {
  const uint16_t* H;
  const uint16_t* W;
  int64_t ldh, ldw, T, d, V, Vc;
  const int64_t* targets;
  float c;
  double beta;
  int S;
  float* lp;
  float* ent;
  void* ws;  // tile states, target logits, shard states
  WireState* root;  // when non-null: each token's root state (as well as lp / ent)
};

// Workspace layout of the fused path (offsets in bytes from the workspace base).
struct LinearWorkspace {
  int64_t tiles_per_chunk;  // ceil(Vc / kTileV)
  int64_t n_tiles;          // 8 * tiles_per_chunk
  size_t tile_states;       // n_tiles * T_pad TileState
  size_t target_logit;      // T_pad floats
  size_t shard_states;      // S * T WireState
  size_t total;
};

LinearWorkspace linear_workspace_layout(int64_t T, int64_t V, int S);

hipError_t launch_linear_path(const LinearArgs& a, hipStream_t stream);

// Fused-path backward (rlk_linear_bwd.hip).  It runs over the tokens in chunks of at most
// kBackwardChunkTokens (each chunk: forward recompute if needed, logit gradient, its dH
// rows, and its share of dW, accumulated onto the earlier chunks' in token order), so the
// workspace is sized for one chunk: the forward layout, then the regions below (byte
// offsets from the workspace base).
constexpr int64_t kBackwardChunkTokens = 4096;

struct LinearBackwardWorkspace {
  int64_t chunk;   // tokens per chunk: min(T, kBackwardChunkTokens)
  int64_t Vp, Tp;  // V and the chunk rounded up to multiples of 64 (K padding of the GEMMs)
  size_t root;     // chunk root states
  size_t rowc;     // chunk per-token gradient constants
  size_t ht;       // H^T [d, Tp] bf16 of the chunk
  size_t dx;       // dX [chunk, Vp] bf16, zero in columns [V, Vp)
  size_t dxt;      // dX^T [V, Tp] bf16, zero in columns [chunk, Tp)
  size_t part;     // 8 split-K partials of dH [chunk, d] fp32
  size_t total;
};

LinearBackwardWorkspace linear_backward_layout(int64_t T, int64_t V, int64_t d, int S);

// dH [T, ld_dh] and / or dW [V, ld_dw] (either may be null); a.ws holds the workspace.
// When states is non-null it holds the forward's row states and the recompute is skipped.
hipError_t launch_linear_backward(const LinearArgs& a, const float* g_lp, const float* g_ent,
                                  float* dH, int64_t ld_dh, float* dW, int64_t ld_dw,
                                  const WireState* states, hipStream_t stream);

// p[r * ld + c] = 0 for r < rows, c < cols (fp32); the weight gradient of an empty batch.
hipError_t launch_zero_f32(float* p, int64_t ld, int64_t rows, int64_t cols, hipStream_t stream);

// Train-vs-rollout comparison (rlk_compare.hip).
using CompareResult = rlk_compare_result;
int64_t compare_blocks(int64_t T);
size_t compare_workspace_bytes(int64_t T);
hipError_t launch_compare(const float* train, const float* rollout, const uint8_t* mask,
                          int64_t T, void* ws, CompareResult* out, hipStream_t stream);

}  // namespace rlk
