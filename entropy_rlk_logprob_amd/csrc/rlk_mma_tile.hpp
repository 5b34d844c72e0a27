// 256 x 256 bf16 MFMA output tile with K-contiguous operands, shared by the fused
// forward, the logit-gradient recompute and the NT GEMMs of the fused backward:
//   acc(r, c) += sum_k A[r, k] B[c, k]   over k in [k0, k0 + 64 nk),
// A rows r = 0..255 of the tile ("A side", e.g. vocabulary rows of W), B rows c = 0..255
// ("B side", e.g. tokens of H), both row-major with K contiguous.
//
// Workgroup: 8 waves arranged 2 (A side) x 4 (B side), each wave 128 x 64 = 4 x 2 MFMA
// blocks (v_mfma_f32_32x32x16_bf16).  Accumulation order of every output: 64-wide K steps
// in increasing order, each four MFMA steps of 16 consecutive k -- independent of the
// output's place in the tile.  Output layout: lane l of wave (wa, wb) holds, in
// acc[a][b][i], row wa*128 + a*32 + 8*(i/4) + 4*(l/32) + (i%4) and column
// wb*64 + b*32 + (l%32).
//
// LDS: two 64 KiB stages of (256 + 256) rows x 64 bf16, each 128-byte row with an XOR
// swizzle on its 16-byte columns so that ds_read_b128 of 16 consecutive rows hits
// distinct banks.  Global -> LDS by direct LDS-DMA loads (global_load_lds_dwordx4), issued
// one stage ahead.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Runs the K loop; the caller zeroes acc and, after the return (which waits for the
// last DMA), issues a workgroup barrier before reusing smem.
//   At, Bt       first row of the tile's A / B rows (element 0 of K)
//   lda, ldb     row strides (elements)
//   a_last, b_last  last valid row index within the tile (rows beyond are clamped to it;
//                the caller must not use their outputs)
//   k0, nk       first K element (multiple of 8) and number of 64-wide K steps (>= 1)
__device__ __forceinline__ void mma_tile(const uint16_t* __restrict__ At, int64_t lda,
                                         int a_last, const uint16_t* __restrict__ Bt,
                                         int64_t ldb, int b_last, int64_t k0, int nk, char* smem,
                                         floatx16 (&acc)[4][2]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = wave >> 2;  // A-side half (0, 1)
  const int wt = wave & 3;   // B-side quarter (0..3)
  const uint16_t* __restrict__ Wt = At + k0;
  const uint16_t* __restrict__ Ht = Bt + k0;
  const int w_last = a_last;
  const int h_last = b_last;
  const int64_t ldw = lda;
  const int64_t ldh = ldb;
  // Global -> LDS: direct 16-byte-per-lane loads into LDS (global_load_lds_dwordx4).  One
  // wave instruction fills one 1 KiB block = 8 slab rows: lane l writes physical column
  // l % 8 of row r = 8 b + l / 8 of block b, so it fetches logical column
  // (l % 8) ^ ((r / 2) % 8), the layout of lds_offset().  Blocks 0..31 are the A slab,
  // 32..63 the B slab; wave w fills blocks w, w + 8, ..., w + 56.  Offsets are
  // tile-relative on workgroup-uniform bases; rows beyond the valid range are clamped to
  // the last valid row (their values are masked in the epilogue or never stored).
  constexpr int kBlocksPerWave = (kTileV + kTileT) / 8 / (kThreads / 64);  // 8
  constexpr int kWBlocks = kTileV / 8;
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

  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  issue_stage(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt has landed for every wave, and every wave is done reading stage kt - 1,
    // whose buffer the loads of stage kt + 1 now overwrite.  A wave waits at normal issue
    // priority and runs its MFMA steps at raised priority, so that the SIMD's arbiter
    // favours the wave that is feeding the matrix unit.
    __builtin_amdgcn_s_setprio(0);
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
    __builtin_amdgcn_s_setprio(1);
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
  __builtin_amdgcn_s_setprio(0);
  wait_dma();  // the repeated last-stage loads land before the caller reuses the LDS
}

}  // namespace mma
}  // namespace rlk
