// 256 x 256 bf16 MFMA output tile, shared by the fused forward, the logit-gradient
// recompute and the GEMMs of the fused backward:
//   acc(r, c) += sum_k A[r, k] B[c, k]   over k in [k0, k0 + 64 nk),
// A rows r = 0..255 of the tile ("A side", e.g. vocabulary rows of W), B rows c = 0..255
// ("B side", e.g. tokens of H).  Each operand is either K-contiguous (row-major [rows, K],
// the layout of W and H in the forward) or K-major (row-major [K, rows], e.g. W read as
// the operand of dH = dX W): the latter is staged as is and its MFMA fragments are read
// with the LDS transpose load, so no transposed copy is ever written.
//
// Workgroup: 8 waves arranged 2 (A side) x 4 (B side), each wave 128 x 64 = 4 x 2 MFMA
// blocks (v_mfma_f32_32x32x16_bf16).  Accumulation order of every output: 64-wide K steps
// in increasing order, each four MFMA steps of 16 consecutive k -- independent of the
// output's place in the tile and of the operands' layouts.  Output layout: lane l of wave
// (wa, wb) holds, in acc[a][b][i], row wa*128 + a*32 + 8*(i/4) + 4*(l/32) + (i%4) and
// column wb*64 + b*32 + (l%32).
//
// LDS: two 64 KiB stages, each an A slab and a B slab of 32 KiB (256 rows x 64 k).  A
// K-contiguous slab holds 128-byte rows (64 k) with an XOR swizzle on their 16-byte
// columns so that ds_read_b128 of 16 consecutive rows hits distinct banks; a K-major slab
// holds 512-byte rows (one k, 256 tile rows) swizzled so that the four k rows one
// transpose load touches fall in four different bank groups.  Global -> LDS by direct
// LDS-DMA loads (global_load_lds_dwordx4; buffer_load_dwordx4 ... lds in the chained form
// of persistent kernels), issued one stage ahead.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rlk_launch.hpp"

namespace rlk {
namespace mma {

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

// The lane id from an opaque instruction pair: per-lane values derived from it are formed
// where they are used.  In a persistent kernel's tile loop, values derived from threadIdx
// alone would be hoisted out of the loop and held across the K loop in registers it needs.
__device__ __forceinline__ int lane_id_here() {
  int lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  return lane;
}

// Workgroup barrier ordering LDS reads (this wave's ds_reads done, then s_barrier).  The
// LDS-DMA stage that the next step reads was waited for by every wave before it arrives.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes per lane from base + voffset + soffset (bytes) into LDS at dst + 16 lane, by a
// buffer load to LDS on a raw buffer resource over base (stride 0, 0xffffffff records, so
// no offset is range-checked away; 32-bit data format).  Its only vector operand is the
// 32-bit offset register.  The resource type exists in the device pass only.
__device__ __forceinline__ void buffer_load_lds16(const uint16_t* base, uint32_t voffset,
                                                  int soffset, char* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voffset, soffset, 0, 0);
#else
  (void)base, (void)voffset, (void)soffset, (void)dst;
#endif
}

// Same with a given record count (bytes from base that may be read; lanes beyond read 0).
__device__ __forceinline__ void buffer_load_lds16_n(const uint16_t* base, uint32_t records,
                                                    uint32_t voffset, char* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base), (short)0, (int)records, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voffset, 0, 0, 0);
#else
  (void)base, (void)records, (void)voffset, (void)dst;
#endif
}

// LDS slab layout: rows of kBK bf16 = 128 bytes; 16-byte column c16 of row r sits at
// physical column c16 ^ ((r / 2) % 8).  The XOR key makes the 16 rows that one 16-lane
// ds_read_b128 pass touches land in 16 distinct 16-byte bank groups of the 64-bank LDS.
__device__ __forceinline__ int lds_offset(int row, int c16) {
  return row * 128 + ((c16 ^ ((row >> 1) & 7)) << 4);
}

// K-major slab layout: row k of 256 bf16 = 512 bytes; 16-byte column c of row k sits at
// physical column c ^ (4 (k % 4)), i.e. rows k = 0..3 (mod 4) are rotated by 64 bytes
// against each other.
__device__ __forceinline__ int lds_offset_kmajor(int k, int col) {  // col: element, % 4 == 0
  return k * 512 + ((((col >> 3) ^ ((k & 3) << 2))) << 4) + ((col & 4) << 1);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// gfx950 LDS transpose load (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane j
// supplies the address of 4 consecutive 16-bit elements, and lane i receives element
// i % 4 of the chunks of lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4, in that order
// (a 16 x 4 -> 4 x 16 transpose; verified on the device).  So if lane 4e + q points at
// k row kb + e, columns cb + 4q .. cb + 4q + 3, lane i receives column cb + i at rows
// kb .. kb + 3.
__device__ __forceinline__ v4i16 ds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<char*>(p)));
}

// One MFMA operand fragment (rows base .. base + 31 of the slab, k 16 ks .. 16 ks + 15):
// lane l holds row base + l % 32, k = 16 ks + 8 (l / 32) + j, j = 0..7.
// lane_in: the caller's lane id (a persistent kernel's, see lane_id_here), or -1 for
// threadIdx.x % 64.
template <bool KMAJOR>
__device__ __forceinline__ bf16x8 read_fragment(const char* slab, int base, int ks,
                                                int lane_in = -1) {
  const int lane = lane_in < 0 ? (int)(threadIdx.x & 63) : lane_in;
  if constexpr (!KMAJOR) {
    const int c16 = 2 * ks + (lane >> 5);
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const U4*>(slab + lds_offset(base + (lane & 31),
                                                                             c16)));
  } else {
    // Group g = l / 16 covers rows base + 16 (g % 2) + 0..15 at k 16 ks + 8 (g / 2) + 0..7,
    // in two transpose loads of four k each.
    const int g = lane >> 4, i = lane & 15;
    const int k = 16 * ks + 8 * (g >> 1) + (i >> 2);
    const int col = base + 16 * (g & 1) + 4 * (i & 3);
    const v4i16 lo = ds_read_tr16(slab + lds_offset_kmajor(k, col));
    const v4i16 hi = ds_read_tr16(slab + lds_offset_kmajor(k + 4, col));
    const v4i16 both[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8, both);
  }
}

// Scheduling groups spreading kReads LDS reads over six MFMAs (as evenly as possible).
template <int kReads, int Q>
__device__ __forceinline__ void sched_reads_over_mfmas() {
  if constexpr (Q < 6) {
    constexpr int n = kReads * (Q + 1) / 6 - kReads * Q / 6;
    sched_group(kSchedMfma, 1);
    if constexpr (n > 0) sched_group(kSchedDsRead, n);
    sched_reads_over_mfmas<kReads, Q + 1>();
  }
}

// An operand of the tile: K-contiguous ([rows, K], row r at p + r ld) or K-major
// ([K, rows], k row at p + k ld).
//   p      element (row 0 of the tile, k = 0)
//   ld     stride (elements) between rows (K-contiguous) or between k rows (K-major)
//   last   last valid row of the tile (rows beyond are clamped to it; the caller must not
//          use their outputs); K-major: last + 1 must be a multiple of 8
//   k_last K-major only: last k row that may be read (k rows beyond are clamped to it; the
//          other operand must hold zeros there)
struct Operand {
  const uint16_t* p;
  int64_t ld;
  int last;
  int64_t k_last;
};

// Runs the K loop; the caller zeroes acc and, after the return (which waits for the
// last DMA), issues a workgroup barrier before reusing smem.
//   k0, nk  first K element (multiple of 8) and number of 64-wide K steps (>= 1)
// WA = 4: a 512 x 128 tile instead (waves 4 (A side) x 2 (B side), each still 128 x 64;
// K-contiguous operands only), with 80 KiB stages: for batches of at most 128 tokens.
// CHAIN (persistent kernels, WA = 2, K-contiguous operands, k0 = 0): stage 0 sits in buffer
// p0 -- already issued when `issued` (by issue_first_stage, for instance while the previous
// tile's epilogue ran), else issued here; the last K step issues no loads, and nothing is
// waited for at the end, so the caller may issue the next tile's first stage into buffer
// (p0 + nk) % 2 right away (every wave has passed the barrier after which that buffer is
// no longer read); the next tile's first K step waits for it.
// BUF (implied by CHAIN): K-contiguous operands are staged by buffer loads to LDS as in the
// chained form; the caller guarantees row strides of at most 2^22 elements, so that every
// per-lane byte offset (255 rows at most) stays below 2^31.
template <bool A_KMAJOR, bool B_KMAJOR, int WA = 2, bool CHAIN = false, bool BUF = CHAIN>
__device__ __forceinline__ void mma_tile_op(const Operand& A, const Operand& B, int64_t k0,
                                            int nk, char* smem, floatx16 (&acc)[4][2],
                                            int p0 = 0, bool issued = false) {
  static_assert(!CHAIN || (WA == 2 && !A_KMAJOR && !B_KMAJOR), "chained tiles: K-contiguous");
  static_assert(WA == 2 || (WA == 4 && !A_KMAJOR && !B_KMAJOR), "512-row tiles: K-contiguous");
  constexpr int kARows = 128 * WA;                   // 256 or 512
  constexpr int kBRows = 64 * (8 / WA);              // 256 or 128
  constexpr int kStage = (kARows + kBRows) * kBK * 2;  // 64 or 80 KiB
  const int tid = threadIdx.x;
  // CHAIN: the per-lane address math below is formed anew for each tile (lane_id_here).
  int lane = tid & 63;
  if constexpr (CHAIN) lane = lane_id_here();
  const int wave = wave_id();
  const int wv = wave / (8 / WA);  // A-side 128-row slice (0, 1; or 0..3)
  const int wt = wave % (8 / WA);  // B-side 64-row slice (0..3; or 0, 1)
  // Global -> LDS: direct 16-byte-per-lane loads into LDS (global_load_lds_dwordx4); one
  // wave instruction fills one 1 KiB block with lane l's 16 bytes at byte 16 l.  Blocks
  // 0..31 are the A slab, 32..63 the B slab; wave w fills blocks w, w + 8, ..., w + 56.
  //   K-contiguous: a block is 8 slab rows of 128 bytes; lane l writes physical column
  //     l % 8 of row 8 b + l / 8 and so fetches logical column (l % 8) ^ ((row / 2) % 8).
  //   K-major: a block is 2 k rows of 512 bytes; lane l writes physical column l % 32 of
  //     k row 2 b + l / 32 and so fetches logical column (l % 32) ^ (4 (k % 4)).
  // Offsets are tile-relative on workgroup-uniform bases; rows beyond the valid range
  // are clamped as Operand describes.
  constexpr int kBlocksPerWave = (kARows + kBRows) / 8 / (kThreads / 64);  // 8 (WA = 4: 10)
  constexpr int kWBlocks = kARows / 8;
  int64_t src_off[kBlocksPerWave];  // K-contiguous: offset at k = 0
  int kmaj_row[kBlocksPerWave];     // K-major: k row within the step
  // CHAIN: the same K-contiguous offsets in bytes, 32-bit (rows < 256, ld <= 2^22, so below
  // 2^31), for buffer loads to LDS on one buffer resource per operand: the per-lane offset
  // register is the load's only vector operand, so there is no 64-bit address temporary
  // that the register allocator could hand to a fragment read while the load is in flight
  // (which costs a wait for every load in flight).
  uint32_t src_off_b[kBlocksPerWave];
#pragma unroll
  for (int i = 0; i < kBlocksPerWave; ++i) {
    const int blk = i * 8 + wave;
    const bool is_a = i < kWBlocks / 8;
    const int bb = is_a ? blk : blk - kWBlocks;
    const bool kmaj = is_a ? A_KMAJOR : B_KMAJOR;
    const Operand& op = is_a ? A : B;
    if (!kmaj) {
      const int row = bb * 8 + (lane >> 3);
      const int col = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
      src_off[i] = (int64_t)min(row, op.last) * op.ld + col;
      src_off_b[i] = (uint32_t)(min(row, op.last) * (uint32_t)op.ld + col) * 2u;
      kmaj_row[i] = 0;
    } else {
      const int k = bb * 2 + (lane >> 5);
      const int col = min(((lane & 31) ^ ((k & 3) << 2)) * 8, op.last & ~7);
      src_off[i] = col;
      // BUF: the byte offset within the stage's k rows (k < 64, ld <= 2^22: below 2^29).
      src_off_b[i] = ((uint32_t)k * (uint32_t)op.ld + (uint32_t)col) * 2u;
      kmaj_row[i] = k;
    }
  }
  auto issue_stage = [&](int64_t k, int stage) {
#pragma unroll
    for (int i = 0; i < kBlocksPerWave; ++i) {
      const int blk = i * 8 + wave;
      const bool is_a = i < kWBlocks / 8;
      const bool kmaj = is_a ? A_KMAJOR : B_KMAJOR;
      const Operand& op = is_a ? A : B;
      char* dst = smem + stage * kStage + blk * 1024;
      if (BUF && !kmaj) {
        buffer_load_lds16(is_a ? A.p : B.p, src_off_b[i], (int)(k * 2), dst);
      } else if (BUF && kmaj) {
        // The stage's k rows from k on: a resource based at row k whose records end after
        // row k_last, so that rows beyond it read as zeros (the other operand holds zeros
        // there).
        const int64_t rows = op.k_last - k + 1;
        const int64_t bytes = rows > 0 ? rows * op.ld * 2 : 0;
        buffer_load_lds16_n(op.p + k * op.ld, bytes < 0xffffffffll ? (uint32_t)bytes : 0xffffffffu,
                            src_off_b[i], dst);
      } else {
        const void* src;
        if (!kmaj)
          src = op.p + k + src_off[i];
        else
          src = op.p + min(k + kmaj_row[i], op.k_last) * op.ld + src_off[i];
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      }
    }
  };
  // LDS reads per MFMA step: four A fragments and two B fragments, two transpose loads
  // each on a K-major side.
  constexpr int kReads = (A_KMAJOR ? 8 : 4) + (B_KMAJOR ? 4 : 2);

  // Fragments of MFMA step ks live in buffer ks % 2; the fragments of step ks + 1 are read
  // from LDS while the MFMAs of step ks run.
  bf16x8 af[2][4], bfr[2][2];
  auto mfma_ab = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[2]) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], acc[a][b], 0, 0, 0);
  };
  auto mfma_step = [&](int buf) { mfma_ab(af[buf], bfr[buf]); };
  // A K-major B operand (and a K-contiguous A): all of a K step's B fragments are read right
  // after the barrier, before the step's stage loads are issued.  The compiler waits for
  // every LDS-DMA load in flight before a transpose load that follows one (it does not for
  // ds_read_b128), which with the transpose loads spread over the MFMA steps put a wait for
  // the next stage's loads in the middle of every K step.
  constexpr bool kBEarly = B_KMAJOR && !A_KMAJOR && WA == 2;
  // One K step.  The last MFMA step of K step kt - 1 (DEFERRED) is held back until after
  // the barrier that opens K step kt: its fragments are already in registers, so its
  // eight MFMAs keep the matrix unit busy while the first fragments of K step kt come
  // from LDS, instead of both waves of the SIMD idling through that latency.  Every
  // accumulator still sees its MFMAs in K order.
  auto k_step = [&](int kt, auto deferred, auto last) {
    // Stage kt has landed for every wave, and every wave is done reading stage kt - 1,
    // whose buffer the loads of stage kt + 1 now overwrite.  A wave waits at normal issue
    // priority and runs its MFMA steps at raised priority, so that the SIMD's arbiter
    // favours the wave that is feeding the matrix unit.
    __builtin_amdgcn_s_setprio(0);
    wait_dma();
    lds_barrier();
    const char* wb = smem + ((kt + p0) & 1) * kStage;
    const char* hb = wb + kARows * kBK * 2;
    auto read_frags = [&](int ks, int buf) {
#pragma unroll
      for (int a = 0; a < 4; ++a) af[buf][a] = read_fragment<A_KMAJOR>(wb, wv * 128 + a * 32, ks, CHAIN ? lane : -1);
#pragma unroll
      for (int b = 0; b < 2; ++b) bfr[buf][b] = read_fragment<B_KMAJOR>(hb, wt * 64 + b * 32, ks, CHAIN ? lane : -1);
    };
    bf16x8 bk[4][2];  // kBEarly: this K step's B fragments
    if constexpr (kBEarly) {
#pragma unroll
      for (int a = 0; a < 4; ++a) af[0][a] = read_fragment<false>(wb, wv * 128 + a * 32, 0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int b = 0; b < 2; ++b) bk[ks][b] = read_fragment<true>(hb, wt * 64 + b * 32, ks);
      __builtin_amdgcn_s_setprio(1);
      sched_group(kSchedDsRead, 4 + 16);
    } else {
      read_frags(0, 0);
      __builtin_amdgcn_s_setprio(1);
      sched_group(kSchedDsRead, kReads);
    }
    // Loads of stage kt + 1 into the other buffer.  Issued on every stage (the last one
    // repeats stage nk - 1 into the idle buffer; chained: the last one issues none) so that
    // they stay in this scheduling region and can be spread between MFMAs instead of
    // stalling the wave.
    if constexpr (!decltype(last)::value)
      issue_stage(k0 + (int64_t)min(kt + 1, nk - 1) * kBK, (kt + 1 + p0) & 1);
    // Instruction order (left to itself the scheduler merges the two fragment buffers,
    // waits on each read right away and issues all stage loads in one burst ahead of the
    // MFMAs): the deferred MFMAs interleaved with the eight stage loads; then MFMA steps
    // 0..2, each spreading the LDS reads of the following step over its MFMAs.
    if constexpr (decltype(deferred)::value) {
      mfma_step(1);
#pragma unroll
      for (int q = 0; q < kBlocksPerWave; ++q) {
        if (q < 8) sched_group(kSchedMfma, 1);
        sched_group(kSchedVmemRead, 1);
      }
    } else {
      sched_group(kSchedVmemRead, kBlocksPerWave);
    }
    if constexpr (kBEarly) {
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
          af[(ks + 1) & 1][a] = read_fragment<false>(wb, wv * 128 + a * 32, ks + 1);
        mfma_ab(af[ks & 1], bk[ks]);
        sched_reads_over_mfmas<4, 0>();
        sched_group(kSchedMfma, 2);
      }
      // MFMA step 3 is held back (it runs as the next K step's deferred step).
#pragma unroll
      for (int b = 0; b < 2; ++b) bfr[1][b] = bk[3][b];
    } else {
#pragma unroll
      for (int ks = 0; ks < 3; ++ks) {
        read_frags(ks + 1, (ks + 1) & 1);
        mfma_step(ks & 1);
        sched_reads_over_mfmas<kReads, 0>();
        sched_group(kSchedMfma, 2);
      }
    }
  };

  if constexpr (CHAIN) {
    if (!issued) issue_stage(k0, p0);
    if (nk == 1) {
      k_step(0, std::false_type{}, std::true_type{});
    } else {
      k_step(0, std::false_type{}, std::false_type{});
      for (int kt = 1; kt < nk - 1; ++kt) k_step(kt, std::true_type{}, std::false_type{});
      k_step(nk - 1, std::true_type{}, std::true_type{});
    }
    mfma_step(1);  // the last K step's deferred MFMA step
    __builtin_amdgcn_s_setprio(0);
  } else {
    issue_stage(k0, 0);
    k_step(0, std::false_type{}, std::false_type{});
    for (int kt = 1; kt < nk; ++kt) k_step(kt, std::true_type{}, std::false_type{});
    mfma_step(1);  // the last K step's deferred MFMA step
    __builtin_amdgcn_s_setprio(0);
    wait_dma();  // the repeated last-stage loads land before the caller reuses the LDS
  }
}

// The first stage (K offset 0) of a 256 x 256 tile with K-contiguous operands into LDS
// buffer `stage`, in mma_tile_op's layout (each wave its eight 1 KiB blocks): for a
// persistent kernel to issue the next tile's first stage ahead of that tile's K loop.
__device__ __forceinline__ void issue_first_stage(const Operand& A, const Operand& B,
                                                  char* smem, int stage) {
  const int lane = lane_id_here();
  const int wave = wave_id();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int blk = i * 8 + wave;
    const bool is_a = i < 4;
    const Operand& op = is_a ? A : B;
    const int row = (is_a ? blk : blk - 32) * 8 + (lane >> 3);
    const int col = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
    const uint16_t* src = op.p + (int64_t)min(row, op.last) * op.ld + col;
    char* dst = smem + stage * kStageBytes + blk * 1024;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  }
}

// Workgroup id -> (row tile, column tile) of an n_rt x n_ct grid of output tiles, launched
// as split_grid(8 ceil(n_rt n_ct / 8)).  The hardware hands workgroup ids out round-robin
// over the 8 XCDs; the remap gives each XCD a contiguous range of logical tiles.  Logical
// tiles run one group of up to G column tiles at a time, row-tile-major within the group,
// so that the ~32 tiles an XCD runs at once are a few row tiles times one column group and
// share both operands' slices in that XCD's L2.  Returns false for the padding ids beyond
// the grid.  grouped_tile_at takes the id explicitly (persistent kernels walk the ids b,
// b + gridDim.x, ... with gridDim.x a multiple of 8, so that id mod 8 stays b's XCD).
template <int G>
__device__ __forceinline__ bool grouped_tile_at(int64_t hw, int64_t n_rt, int64_t n_ct,
                                                int64_t& rt, int64_t& ct) {
  const int64_t nb = n_rt * n_ct;
  const int64_t per_xcd = (nb + 7) / 8;
  if (hw >= 8 * per_xcd) return false;
  const int64_t logical = (hw % 8) * per_xcd + hw / 8;
  if (logical >= nb) return false;
  const int64_t grp = logical / (G * n_rt);
  const int64_t gsz = min((int64_t)G, n_ct - grp * G);
  const int64_t idx = logical - grp * G * n_rt;
  rt = idx / gsz;
  ct = grp * G + idx % gsz;
  return true;
}
template <int G>
__device__ __forceinline__ bool grouped_tile_of(int64_t n_rt, int64_t n_ct, int64_t& rt,
                                                int64_t& ct) {
  return grouped_tile_at<G>(linear_block(), n_rt, n_ct, rt, ct);
}

// Both operands K-contiguous.
//   At, Bt       first row of the tile's A / B rows (element 0 of K)
//   lda, ldb     row strides (elements)
//   a_last, b_last  last valid row index within the tile
__device__ __forceinline__ void mma_tile(const uint16_t* __restrict__ At, int64_t lda,
                                         int a_last, const uint16_t* __restrict__ Bt,
                                         int64_t ldb, int b_last, int64_t k0, int nk, char* smem,
                                         floatx16 (&acc)[4][2]) {
  mma_tile_op<false, false>(Operand{At, lda, a_last, 0}, Operand{Bt, ldb, b_last, 0}, k0, nk,
                            smem, acc);
}
// Same, staged by buffer loads to LDS (row strides of at most 2^22 elements).
__device__ __forceinline__ void mma_tile_buf(const uint16_t* __restrict__ At, int64_t lda,
                                             int a_last, const uint16_t* __restrict__ Bt,
                                             int64_t ldb, int b_last, int64_t k0, int nk,
                                             char* smem, floatx16 (&acc)[4][2]) {
  mma_tile_op<false, false, 2, false, true>(Operand{At, lda, a_last, 0},
                                            Operand{Bt, ldb, b_last, 0}, k0, nk, smem, acc);
}

}  // namespace mma
}  // namespace rlk
