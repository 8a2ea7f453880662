// Building blocks shared by the grouped GEMM kernels on gfx950: tile
// constants, explicit vmcnt waits, the global -> LDS DMA of activation rows
// with its XOR swizzle, the LDS-only workgroup barrier, and the task logic of
// the fused gate_up + down launch.
#pragma once

#include "dg_common.h"
#include "launch.h"

namespace dg {
namespace gemm {

#ifndef DG_GEMM_WAVES
#define DG_GEMM_WAVES 4
#endif
constexpr int kWaves = DG_GEMM_WAVES;    // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kKS = 128;                  // K per pipeline step (four MFMA K steps of 32)
constexpr int kNS = kKS / 32;
constexpr int kSegs = kKS / 8;            // 16-byte segments per staged row
constexpr int kRowBytes = kKS * 2;
constexpr int kDmaRows = 1024 / kRowBytes;  // rows one wave-wide 16-byte-per-lane transfer fills
constexpr int kStageBytes = kTileRows * kRowBytes;
constexpr int kBMT = kTileRows / 16;      // m-tiles per tile
constexpr int kDmaInstr = kTileRows / (kWaves * kDmaRows);  // transfers per wave for a full tile

// vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS byte address of a shared-memory pointer (the address-space cast to
// the local address space; its value is the offset inside the workgroup's LDS).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// One 16-byte-per-lane global -> LDS transfer (global_load_lds_dwordx4): lane l
// writes LDS bytes lds_base + 16 l .. + 15. Issued from inline assembly so the
// compiler does not treat every later LDS read as depending on it; completion
// is awaited explicitly (vmcnt) before the workgroup barrier that publishes it.
// No register is written, so nothing is left in flight in a register.
// M0 is saved and restored around the transfer, so nothing the compiler keeps
// in M0 is disturbed. NT: with the non-temporal hint, for data read once
// (an embedding table streamed past the caches).
template <bool NT = false>
__device__ __forceinline__ void lds_dma16(uint32_t lds_base, const void* gaddr) {
  uint32_t saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(gaddr)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_base), "v"(gaddr)
        : "memory");
}

// DMA transfers per wave that stage ROWS activation rows with WV waves.
constexpr int dma_per_wave(int rows, int wv) { return (rows + wv * kDmaRows - 1) / (wv * kDmaRows); }

// Activation rows of one K step straight into LDS: instruction i of wave w
// (of WV waves) fills the kDmaRows rows starting at kDmaRows (w + WV i); lane l
// lands in row slot l / kSegs, 16-byte position l % kSegs and carries logical
// segment position ^ (row % kSegs), an XOR swizzle that makes the MFMA reads
// bank-conflict free. Segments past a short last step re-read a valid one.
// With 8 waves an odd count of 16-row tiles rounds up to whole transfers (the
// stage holds the extra rows).
template <int NMT, int NSEG, int NI, int WV = kWaves>
__device__ __forceinline__ void dma_a(char* stage, const uint16_t* const (&rowp)[NI], int k0, int wave,
                                      int lane) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(stage) + wave * kDmaRows * kRowBytes);
#pragma unroll
  for (int i = 0; i < (16 * NMT + WV * kDmaRows - 1) / (WV * kDmaRows); ++i) {
    const int r = kDmaRows * (wave + WV * i) + lane / kSegs;
    int sg = (lane % kSegs) ^ (r % kSegs);
    if (NSEG < kSegs) sg = sg % NSEG;
    lds_dma16(base + i * WV * kDmaRows * kRowBytes, rowp[i] + k0 + sg * 8);
  }
}

// Workgroup barrier that does not wait for this wave's outstanding global
// loads: the LDS-DMA writes the other waves are about to read are covered by
// the explicit vmcnt wait before it. The empty asm statements stop the
// compiler from moving memory operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The task logic of a fused launch of both GEMMs (tasks dealt whole expert
// by whole expert, so a tile's gate_up and down tasks share a queue, hence an
// XCD). Queue x, the workgroups b with b % 8 == x, runs its gate_up tasks,
// then its down tasks. A gate_up task, once its gated activations have
// reached this XCD's L2, counts itself on its tile; a down task starts once
// its tile's count holds all gate_up blocks. The workgroups of one XCD are
// dispatched in index order, so every gate_up task that a down task waits for
// is running or done and never waits itself. The wait is bounded
// (f.wait_polls, about a tenth of a second; none with DG_FWD_GEMM_NO_WAIT,
// which tests this path): past it the task writes NaN for its outputs instead of
// its product, so a broken assumption shows in the result and the launch
// still ends; it also raises DG_DEV_WAIT_TIMEOUT. The dispatcher may start a
// launch's round robin on any XCD (workgroup b then runs on XCD (b + c) % 8
// for a c fixed within the launch), which keeps every queue on one XCD. Each
// gate_up task also counts itself under the XCD it ran on, and a down task
// whose tile's gate_up tasks did not all run on its own XCD raises
// DG_DEV_XCD_GEMM. gate_up(tile) and down(tile) run one task's product.

template <int WV = kWaves, typename GateUp, typename Down>
__device__ __forceinline__ void fused_tasks(const FusedGemmArgs& f, GateUp gate_up, Down down) {
  __shared__ int ready;
  const int qx = blockIdx.x & (kQueues - 1), j = blockIdx.x / kQueues;
  const int ngu = f.gu.qlen[qx];
  const int tid = threadIdx.x;
  if (j < ngu) {
    const Tile tl = f.gu.tiles[(size_t)qx * f.gu.qmax + j];
    gate_up(tl);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have reached L2
    __syncthreads();
    if (tid == 0)
      atomicAdd(reinterpret_cast<unsigned long long*>(&f.tile_done[tl.row0]), 1ull | (1ull << (8 + 7 * xcc_id())));
    return;
  }
  const int jd = j - ngu;
  if (jd >= f.dn.qlen[qx]) return;
  const Tile tl = f.dn.tiles[(size_t)qx * f.dn.qmax + jd];
  const unsigned long long need = (unsigned long long)f.nb_gate_up;  // <= 64
  unsigned long long* cnt = reinterpret_cast<unsigned long long*>(&f.tile_done[tl.row0]);
  if (tid == 0) {
    unsigned long long v = 0;
    int n = 0;
    while (((v = atomicAdd(cnt, 0ull)) & 0xffull) < need && n < f.wait_polls) {
      __builtin_amdgcn_s_sleep(8);
      ++n;
    }
    ready = n < f.wait_polls;
    if (ready && ((v >> (8 + 7 * xcc_id())) & 127ull) != need) raise_flag(f.dev_flags, DG_DEV_XCD_GEMM);
  }
  __syncthreads();
  if (ready) {
    down(tl);
    return;
  }
  if (tid == 0) raise_flag(f.dev_flags, DG_DEV_WAIT_TIMEOUT);
  const int cols = 32 * WV;
  for (int i = tid; i < tl.mc * cols; i += 64 * WV)
    if (tl.nb * cols + i % cols < f.dn.D)
      f.dn.y[(size_t)(tl.row0 + i / cols) * f.dn.D + tl.nb * cols + i % cols] = 0x7fc0;  // bf16 NaN
}

}  // namespace gemm
}  // namespace dg
