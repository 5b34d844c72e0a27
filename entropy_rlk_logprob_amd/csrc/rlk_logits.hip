// Logits path: streaming fixed-order row reducer and the vocab-shard merge.
//
// Canonical order for a row of V fp32 logits (the contract that makes results independent
// of rows-per-call, row order, repeats and vocab split):
//   * 8 chunks of Vc = 4 * ceil(ceil(V / 8) / 4) columns (the last ones short or empty);
//   * within a chunk, quad q covers chunk columns [4q, 4q+4) and belongs to lane q % 64;
//     a lane's quads k = 0, 1, 2, ... (q = lane + 64 k) are grouped four at a time into
//     16-element leaves;
//   * groups are folded into the lane's state in increasing k (fold_group): the state
//     keeps a reference m (the lane's running max, up to 8 units of c (x - m)) and fp64
//     sums relative to it; a group whose max exceeds m by more than that first rebases
//     the sums to its max, then its fp32 terms 2^{c (x - m)} and 2^{c (x - m)} c (x - m)
//     are summed pairwise (within each quad, then quad pairs) and added in;
//   * lanes: wave_merge (the wave max of the lane maxima, each lane's sums rescaled to it
//     once, fp64 sums by an xor butterfly 32, 16, 8, 4, 2, 1);
//   * chunks: ((0,1),(2,3)),((4,5),(6,7)) by rlk_merge.
// A vocab shard (split count S) owns 8/S consecutive chunks, reduces them in one
// workgroup exactly as the unsplit case does, and hands its state to the merge kernel,
// which applies the top S-leaf part of the same chunk tree.
//
// Layout and launch: one workgroup per (row, shard), one wave per chunk (bf16: per two
// chunks of the shard); each lane streams 16-byte loads (bf16: 8-byte) whose 64 lanes
// cover 1 KiB (512 bytes) of contiguous HBM per instruction.
// The loads carry the non-temporal hint: every logit is read exactly once.

#include <type_traits>

#include "rlk_launch.hpp"
#include "rlk_state.hpp"

namespace rlk {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Quad4 {
  float v[16];
};

// Logit element types: fp32, or bf16 given as its 16-bit pattern (widened exactly).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// A lane's group g holds quads q = lane + 64 * (4 g + i), i = 0..3 (16 elements).  The raw
// form keeps what one load brings in (fp32: 4 x 16 bytes; bf16: 4 x 8 bytes, still packed)
// so that several groups can be in flight without spending 16 VGPRs on each.
template <typename E> struct RawGroup;
template <> struct RawGroup<float> { f32x4 q[4]; };
template <> struct RawGroup<uint16_t> { u32x2 q[4]; };

// Full group: four quad loads at 32-bit byte offsets from the chunk's first column, which
// is the same for the whole wave, so they take the scalar-base form (one address add per
// group, the four loads 64 quads apart by immediate offsets).  A chunk spans less than 2^30
// bytes (V < 2^31 columns, 8 chunks), so the offsets fit.
template <typename E>
__device__ __forceinline__ void load_raw(const E* __restrict__ p, int lane, int g,
                                         RawGroup<E>& r) {
  using Q = std::remove_reference_t<decltype(r.q[0])>;
  const char* b = reinterpret_cast<const char*>(p);
  const uint32_t off = (uint32_t)(lane + 256 * g) * (uint32_t)sizeof(Q);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.q[i] = __builtin_nontemporal_load(
        reinterpret_cast<const Q*>(b + off + (uint32_t)(i * 64 * (int)sizeof(Q))));
}

template <typename E>
__device__ __forceinline__ void widen(const RawGroup<E>& r, Quad4& out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(E) == 4) {
      out.v[4 * i + 0] = r.q[i].x;
      out.v[4 * i + 1] = r.q[i].y;
      out.v[4 * i + 2] = r.q[i].z;
      out.v[4 * i + 3] = r.q[i].w;
    } else {  // little endian: the lower half of each dword is the earlier element
      out.v[4 * i + 0] = __uint_as_float(r.q[i].x << 16);
      out.v[4 * i + 1] = __uint_as_float(r.q[i].x & 0xffff0000u);
      out.v[4 * i + 2] = __uint_as_float(r.q[i].y << 16);
      out.v[4 * i + 3] = __uint_as_float(r.q[i].y & 0xffff0000u);
    }
  }
}

// Element loads of a full group (rows whose stride or base rule out the wide loads).
template <typename E>
__device__ __forceinline__ void load_group_scalar(const E* __restrict__ p, int lane, int g,
                                                  Quad4& out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = lane + 64 * (4 * g + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) out.v[4 * i + j] = to_f32(__builtin_nontemporal_load(p + 4 * q + j));
  }
}

// Same, with columns at or beyond n replaced by -inf (the identity's contribution).
template <typename E>
__device__ __forceinline__ void load_group_masked(const E* __restrict__ p, int lane, int g,
                                                  int n, Quad4& out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = lane + 64 * (4 * g + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = 4 * q + j;
      out.v[4 * i + j] = (col < n) ? to_f32(__builtin_nontemporal_load(p + col)) : kNegInf;
    }
  }
}

// Wide-load form of a chunk's last (partial) group: a quad wholly inside the chunk takes
// the wide load, a quad wholly beyond it is four -inf (the identity's contribution; bf16
// -inf is 0xff80), and only a quad that straddles column n loads elements.  It yields the
// values load_group_masked yields, so the leaf sees the same bits either way.
template <typename E>
__device__ __forceinline__ void load_raw_masked(const E* __restrict__ p, int lane, int g, int n,
                                                RawGroup<E>& r) {
  using Q = std::remove_reference_t<decltype(r.q[0])>;
  Q neg;  // four -inf elements
  if constexpr (sizeof(E) == 4)
    neg = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
  else
    neg = u32x2{0xff80ff80u, 0xff80ff80u};
  if ((n & 3) == 0) {
    // Every quad lies wholly inside the chunk or wholly beyond it (the common case: the
    // chunk width is a multiple of 4 unless it is a row's short last chunk).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = lane + 64 * (4 * g + i);
      if (4 * q < n)
        r.q[i] = __builtin_nontemporal_load(reinterpret_cast<const Q*>(p) + q);
      else
        r.q[i] = neg;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = lane + 64 * (4 * g + i);
    if (4 * q + 4 <= n) {
      r.q[i] = __builtin_nontemporal_load(reinterpret_cast<const Q*>(p) + q);
    } else if (4 * q >= n) {
      r.q[i] = neg;
    } else if constexpr (sizeof(E) == 4) {
      f32x4 v;
      v.x = (4 * q + 0 < n) ? __builtin_nontemporal_load(p + 4 * q + 0) : kNegInf;
      v.y = (4 * q + 1 < n) ? __builtin_nontemporal_load(p + 4 * q + 1) : kNegInf;
      v.z = (4 * q + 2 < n) ? __builtin_nontemporal_load(p + 4 * q + 2) : kNegInf;
      v.w = (4 * q + 3 < n) ? __builtin_nontemporal_load(p + 4 * q + 3) : kNegInf;
      r.q[i] = v;
    } else {
      uint32_t e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        e[j] = (4 * q + j < n) ? (uint32_t)__builtin_nontemporal_load(p + 4 * q + j) : 0xff80u;
      r.q[i] = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
    }
  }
}

// A lane's running state over its groups: (m, s, u) of everything folded so far with
// s and u relative to the reference m, and ref = m, or 0 while m = -inf (every value
// seen so far is -inf and contributes 0).  A group whose max g exceeds the reference by
// more than kRebaseUnits units of a, c (g - m) > kRebaseUnits, first rebases the sums to g
// in fp64: s <- s 2^d, u <- (u + d s) 2^d with d = c (m - g); its 16 terms 2^a and 2^a a,
// a = c (x - ref) <= kRebaseUnits, are then summed pairwise in fp32 (within each quad, then
// quad pairs) and added to s and u.  So m stays within kRebaseUnits ln(2) tau of the lane's
// max, every rebase divides the weight of what came before by at least 2^kRebaseUnits (a
// long run of tiny rebases would otherwise compound the rounding of their factors), and
// the terms stay at most 2^kRebaseUnits.  The rebase is a per-lane branch, so a wave runs
// it whenever any of its lanes needs it: with a margin of 1 unit that was nearly every
// group on N(0, 3^2) logits, with 8 about a third of them.
constexpr float kRebaseUnits = 8.0f;

struct LaneFold {
  State st;
  float ref;
};

__device__ __forceinline__ LaneFold lane_fold_init() { return LaneFold{identity_state(), 0.0f}; }

__device__ __forceinline__ void fold_group(LaneFold& f, const float* v, float c) {
  float gm = v[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) gm = fmaxf(gm, v[i]);
  if ((gm - f.st.m) * c > kRebaseUnits) {  // false for NaN: a NaN group poisons s below
    const float d = (f.st.m - gm) * c;  // < -kRebaseUnits; -inf when m = -inf or gm = +inf
    const double scale = (double)exp2_hw(d);
    const double dc = (double)fmaxf(d, -kMaxFloat);  // keeps 0 * (-inf) out of u
    f.st.u = (f.st.u + dc * f.st.s) * scale;
    f.st.s = f.st.s * scale;
    f.st.m = gm;
    f.ref = gm;
  }
  float e[16], t[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = (v[i] - f.ref) * c;
    e[i] = exp2_hw(a);
    t[i] = mul_zero_wins(e[i], a);  // 0 where e = 0 (a = -inf)
  }
  float sq[4], uq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sq[j] = (e[4 * j] + e[4 * j + 1]) + (e[4 * j + 2] + e[4 * j + 3]);
    uq[j] = (t[4 * j] + t[4 * j + 1]) + (t[4 * j + 2] + t[4 * j + 3]);
  }
  f.st.s += (double)((sq[0] + sq[1]) + (sq[2] + sq[3]));
  f.st.u += (double)((uq[0] + uq[1]) + (uq[2] + uq[3]));
}

template <typename E>
__device__ __forceinline__ void issue_group(const E* __restrict__ p, int lane, int g, int n,
                                            int n_full, RawGroup<E>& r) {
  if (g < n_full)
    load_raw(p, lane, g, r);
  else
    load_raw_masked(p, lane, g, n, r);
}

template <typename E>
__device__ __forceinline__ void fold_raw(LaneFold& f, const RawGroup<E>& r, float c) {
  Quad4 v;
  widen(r, v);
  fold_group(f, v.v, c);
}

// Chunks per wave for a shard of CPS chunks.  fp32 logits: one (8192 waves for 1024 rows),
// of which 4096 are resident at a time (four per SIMD, capped by rows_resident_lds), each
// with two groups in flight.  bf16 logits, which are bound by VALU issue: two when the shard
// has two or more (4096 waves, one round at four or more per SIMD), which leaves the
// registers to unroll the double buffer so that no register copies are issued per group --
// 6% faster.
template <typename E>
constexpr int chunks_per_wave(int cps) { return (sizeof(E) == 2 && cps >= 2) ? 2 : 1; }
template <typename E>
constexpr int waves_for(int cps) { return cps / chunks_per_wave<E>(cps); }

// Chunk k (0 <= k < n of the chunk) of one wave's stream of groups over its chunks.
template <typename E>
struct ChunkRef {
  const E* p;  // first column of the chunk in this row
  int n;       // columns
  int n_groups, n_full;
};

template <typename E>
__device__ __forceinline__ ChunkRef<E> chunk_ref(const E* row_base, int64_t chunk, int64_t Vc,
                                                 int64_t V) {
  const int64_t lo = min(chunk * Vc, V);
  const int64_t hi = min(lo + Vc, V);
  ChunkRef<E> r;
  r.p = row_base + lo;
  r.n = (int)(hi - lo);
  r.n_groups = (((r.n + 3) >> 2) + 255) >> 8;  // ceil(ceil(n/4) / 256)
  r.n_full = (r.n >> 2) >> 8;                   // groups with every column inside
  return r;
}

// One workgroup = one (row, shard) of CPS = 8 / S chunks; wave w folds chunks w and
// w + WAVES of the shard (or just w when CPS = 1), each into its own lane state.  Which
// wave folds a chunk does not change its bits.
template <typename E, int CPS, bool VEC>
__global__ __launch_bounds__(64 * waves_for<E>(CPS))
__attribute__((amdgpu_waves_per_eu((chunks_per_wave<E>(CPS) == 2 || sizeof(E) == 4) ? 4 : 8)))
void row_reduce_kernel(
    const E* __restrict__ X, int64_t ld, int64_t T, int64_t V, int64_t Vc,
    const int64_t* __restrict__ targets, float c, double beta, float* __restrict__ lp_out,
    float* __restrict__ ent_out, WireState* __restrict__ ws, WireState* __restrict__ root) {
  constexpr int WAVES = waves_for<E>(CPS);
  constexpr int CPW = chunks_per_wave<E>(CPS);
  const int64_t row = linear_block();
  if (row >= T) return;
  const int shard = blockIdx.y;
  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const E* __restrict__ base = X + row * ld;
  const ChunkRef<E> A = chunk_ref(base, (int64_t)shard * CPS + wave, Vc, V);
  ChunkRef<E> B = A;
  B.n_groups = 0;
  if constexpr (CPW == 2) B = chunk_ref(base, (int64_t)shard * CPS + wave + WAVES, Vc, V);

  // A's lane state, then B's: one LaneFold, saved to sa and reset at the chunk boundary
  // (a uniform branch), so that the fold never selects its state by a runtime index.
  State sa = identity_state(), sb = identity_state();
  if constexpr (VEC) {
    // One stream of groups over the wave's chunks (A's, then B's), double buffered: the
    // loads of the next group are in flight while a group is folded, across the chunk
    // boundary and into each chunk's partial last group, so no load latency is exposed
    // before the end of the stream.  (Deeper prefetch measured no faster.)
    if constexpr (CPW == 2) {
      // The wave's two chunks side by side: group g of A, then group g of B, each folded
      // into its own lane state in its own increasing order (so a chunk's bits are those of
      // a wave that folds it alone).  Each chunk streams through two buffers, so the next
      // two groups of each chunk are in flight while a group is folded; a buffer is
      // reloaded right after it is folded (unrolled by two: no register copies).
      LaneFold fa = lane_fold_init(), fb = lane_fold_init();
      RawGroup<E> ra0, ra1, rb0, rb1;
      const int n = max(A.n_groups, B.n_groups);
      // Main loop: while both chunks' next groups are full, only wide loads are issued,
      // so every iteration issues the same loads in the same order and the compiler can
      // wait for exactly the group being folded (with the masked loads of a chunk's last
      // group in the same loop it waited for every load in flight at each group).  The
      // loop is entered only from the first branch below, which issues the same four wide
      // loads in the same order as an iteration does: a conditional or masked first load
      // in front of the loop made the compiler wait for every load at the loop's head.
      const int n_full = min(A.n_full, B.n_full);
      int g = 0;
      if (n_full >= 4) {
        load_raw(A.p, lane, 0, ra0);
        load_raw(B.p, lane, 0, rb0);
        load_raw(A.p, lane, 1, ra1);
        load_raw(B.p, lane, 1, rb1);
        for (; g + 3 < n_full; g += 2) {
          fold_raw(fa, ra0, c);
          load_raw(A.p, lane, g + 2, ra0);
          fold_raw(fb, rb0, c);
          load_raw(B.p, lane, g + 2, rb0);
          fold_raw(fa, ra1, c);
          load_raw(A.p, lane, g + 3, ra1);
          fold_raw(fb, rb1, c);
          load_raw(B.p, lane, g + 3, rb1);
        }
      } else {
        if (A.n_groups > 0) issue_group(A.p, lane, 0, A.n, A.n_full, ra0);
        if (B.n_groups > 0) issue_group(B.p, lane, 0, B.n, B.n_full, rb0);
        if (A.n_groups > 1) issue_group(A.p, lane, 1, A.n, A.n_full, ra1);
        if (B.n_groups > 1) issue_group(B.p, lane, 1, B.n, B.n_full, rb1);
      }
      auto step = [&](int j, LaneFold& f, RawGroup<E>& r, const ChunkRef<E>& C) {
        if (j < C.n_groups) {
          fold_raw(f, r, c);
          if (j + 2 < C.n_groups) issue_group(C.p, lane, j + 2, C.n, C.n_full, r);
        }
      };
      for (; g < n; g += 2) {
        step(g, fa, ra0, A);
        step(g, fb, rb0, B);
        step(g + 1, fa, ra1, A);
        step(g + 1, fb, rb1, B);
      }
      sa = fa.st;
      sb = fb.st;
    } else {
      // One chunk through two buffers (unrolled by two: no register copies), the next two
      // groups in flight while a group is folded.  fp32 runs here at four waves per SIMD (see
      // rows_resident): fewer concurrent streams over the logits, each with two groups in flight.
      const int n = A.n_groups;
      LaneFold f = lane_fold_init();
      RawGroup<E> r0, r1;
      int g = 0;
      if (A.n_full >= 4) {  // wide loads only, entered with its own loads in flight (see above)
        load_raw(A.p, lane, 0, r0);
        load_raw(A.p, lane, 1, r1);
        for (; g + 3 < A.n_full; g += 2) {
          fold_raw(f, r0, c);
          load_raw(A.p, lane, g + 2, r0);
          fold_raw(f, r1, c);
          load_raw(A.p, lane, g + 3, r1);
        }
      } else {
        if (n > 0) issue_group(A.p, lane, 0, A.n, A.n_full, r0);
        if (n > 1) issue_group(A.p, lane, 1, A.n, A.n_full, r1);
      }
      for (; g < n; g += 2) {
        fold_raw(f, r0, c);
        if (g + 2 < n) issue_group(A.p, lane, g + 2, A.n, A.n_full, r0);
        if (g + 1 >= n) break;
        fold_raw(f, r1, c);
        if (g + 3 < n) issue_group(A.p, lane, g + 3, A.n, A.n_full, r1);
      }
      sa = f.st;
    }
  } else {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const ChunkRef<E>& C = i == 0 ? A : B;
      LaneFold f = lane_fold_init();
      for (int g = 0; g < C.n_full; ++g) {
        Quad4 v;
        load_group_scalar(C.p, lane, g, v);
        fold_group(f, v.v, c);
      }
      for (int g = C.n_full; g < C.n_groups; ++g) {
        Quad4 q;
        load_group_masked(C.p, lane, g, C.n, q);
        fold_group(f, q.v, c);
      }
      if (i == 0)
        sa = f.st;
      else
        sb = f.st;
    }
  }

  __shared__ State chunk_state[CPS];
  sa = wave_merge(sa, c);
  if (lane == 0) chunk_state[wave] = sa;
  if constexpr (CPW == 2) {
    sb = wave_merge(sb, c);
    if (lane == 0) chunk_state[wave + WAVES] = sb;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;

  const State r = tree8(chunk_state, CPS, c);
  const int64_t t = targets ? targets[row] : -1;
  if constexpr (CPS == 8) {
    const bool has = (t >= 0) && (t < V);
    const float xt = has ? to_f32(X[row * ld + t]) : 0.0f;
    if (root) root[row] = to_wire(r, xt);
    if (lp_out || ent_out)
      rlk_finalize(r, xt, has, beta, lp_out ? lp_out + row : nullptr,
                   ent_out ? ent_out + row : nullptr);
  } else {
    const int64_t s_lo = min((int64_t)shard * CPS * Vc, V);
    const int64_t s_hi = min(s_lo + (int64_t)CPS * Vc, V);
    const bool mine = (t >= s_lo) && (t < s_hi);
    const float xt = mine ? to_f32(X[row * ld + t]) : 0.0f;
    ws[(int64_t)shard * T + row] = to_wire(r, xt);
  }
}

// Top of the chunk tree across S shard states, then the fp64 finalize (when lp or ent is
// given) and / or the row's root state (when root is given); one thread per row.
template <int S>
__global__ __launch_bounds__(256) void shard_merge_kernel(
    const WireState* __restrict__ ws, int64_t T, const int64_t* __restrict__ targets, int64_t V,
    int64_t shard_cols, float c, double beta, float* __restrict__ lp_out,
    float* __restrict__ ent_out, WireState* __restrict__ root) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= T) return;
  State v[S];
#pragma unroll
  for (int s = 0; s < S; ++s) v[s] = from_wire(ws[(int64_t)s * T + row]);
  const State r = tree8(v, S, c);
  const int64_t t = targets ? targets[row] : -1;
  const bool has = (t >= 0) && (t < V);
  const int64_t owner = has ? (t / shard_cols) : 0;
  const float xt = has ? ws[owner * T + row].xt : 0.0f;
  if (root) root[row] = to_wire(r, xt);
  if (lp_out || ent_out)
    rlk_finalize(r, xt, has, beta, lp_out ? lp_out + row : nullptr,
                 ent_out ? ent_out + row : nullptr);
}

// fp32 logits: dynamic LDS that the kernel does not use, sized so that a CU holds 16 of its
// waves (4 per SIMD) instead of 32: n workgroups of w waves fit where n * bytes <= 160 KiB <
// (n + 1) * bytes.  The HBM stream then has 4096 concurrent streams (one per resident wave) of
// two groups in flight each instead of 8192 of one: 92.5-93.4 against 94.2-94.4 us for the
// 622 MB at T = 1024, V = 151936 (same-process A/B, bits equal; a plain read probe of the two
// patterns: 90.2 against 92.0 us).
template <typename E, int CPS>
constexpr unsigned rows_resident_lds() {
  if constexpr (sizeof(E) != 4) {
    return 0;
  } else {
    constexpr unsigned wgs_per_cu = 16 / waves_for<E>(CPS);
    return 160u * 1024u / (wgs_per_cu + 1) + 1;
  }
}

template <typename E, int CPS>
hipError_t launch_rows_t(const E* X, const LogitsArgs& a, hipStream_t stream) {
  const dim3 grid = split_grid(a.T, (unsigned)(8 / CPS));
  const dim3 block(64 * waves_for<E>(CPS));
  const unsigned lds = rows_resident_lds<E, CPS>();
  if (a.vec)
    hipLaunchKernelGGL((row_reduce_kernel<E, CPS, true>), grid, block, lds, stream, X, a.ld, a.T,
                       a.V, a.Vc, a.targets, a.c, a.beta, a.lp, a.ent, a.ws, a.root);
  else
    hipLaunchKernelGGL((row_reduce_kernel<E, CPS, false>), grid, block, 0, stream, X, a.ld, a.T,
                       a.V, a.Vc, a.targets, a.c, a.beta, a.lp, a.ent, a.ws, a.root);
  return hipGetLastError();
}

template <int CPS>
hipError_t launch_rows(const LogitsArgs& a, hipStream_t stream) {
  return a.Xh ? launch_rows_t<uint16_t, CPS>(a.Xh, a, stream)
              : launch_rows_t<float, CPS>(a.X, a, stream);
}

}  // namespace

hipError_t launch_logits_path(const LogitsArgs& a, hipStream_t stream) {
  hipError_t e = hipSuccess;
  switch (a.S) {
    case 1: return launch_rows<8>(a, stream);
    case 2: e = launch_rows<4>(a, stream); break;
    case 4: e = launch_rows<2>(a, stream); break;
    case 8: e = launch_rows<1>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_shard_merge(a.ws, a.T, a.targets, a.V, (int64_t)(8 / a.S) * a.Vc, a.c, a.beta,
                            a.S, a.lp, a.ent, a.root, stream);
}

hipError_t launch_shard_merge(const WireState* ws, int64_t T, const int64_t* targets, int64_t V,
                              int64_t shard_cols, float c, double beta, int S, float* lp,
                              float* ent, WireState* root, hipStream_t stream) {
  const dim3 grid((unsigned)((T + 255) / 256));
  switch (S) {
    case 2:
      hipLaunchKernelGGL((shard_merge_kernel<2>), grid, dim3(256), 0, stream, ws, T, targets, V,
                         shard_cols, c, beta, lp, ent, root);
      break;
    case 4:
      hipLaunchKernelGGL((shard_merge_kernel<4>), grid, dim3(256), 0, stream, ws, T, targets, V,
                         shard_cols, c, beta, lp, ent, root);
      break;
    case 8:
      hipLaunchKernelGGL((shard_merge_kernel<8>), grid, dim3(256), 0, stream, ws, T, targets, V,
                         shard_cols, c, beta, lp, ent, root);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rlk
