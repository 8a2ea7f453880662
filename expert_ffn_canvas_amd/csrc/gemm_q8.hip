// Grouped expert GEMMs with Q8_0 expert weights on gfx950 fp16 matrix cores,
// dequantisation fused into the weight load.
//
// Weight format: the Q8 builds the pages measure (HF card "DiffusionGemma-
// 26B-A4B-it - ROCmFP4 / ROCmFPX GGUF", Variants) use Q8_0, which the pages do
// not spell out; it is read as the public ggml block of 32 consecutive inputs
// of a row: an fp16 scale d, then 32 int8 codes q (two's complement), each
// standing for q * d.
//
// Packed at create (the blocks are 34 bytes, unfit for 16-byte loads): per
// (expert e, 128-input step s, 16-row panel p), in that order, 2 KB of codes
// in MFMA fragment order and 64 fp16 scales. Lane l = n + 16 g of a code block
// holds 32 bytes for row 16 p + n, in two halves at 16 l and 1024 + 16 l:
// bytes 8 j .. 8 j + 7 of the pair are the codes of inputs 128 s + 32 j +
// 8 g .. + 7 (block 4 s + j), stored in the order k0 k2 k1 k3 k4 k6 k5 k7 so
// that the widening below yields natural order; the scales are [n][j].
// Blocks past the row (the 64-input tail of a 704 row) are padded with zero
// codes and scales. So a wave reads its weight fragments as two 1 KB
// contiguous loads (whole cache lines each, so the streaming hint never
// drops a line that the other load still needs), and the panels of one expert
// at one step lie together.
//
// Exact widening: a code byte masked into the low byte of each fp16 half, its
// sign bit flipped and 0x64 put above it gives fp16 1024 + q + 128 exactly; one
// packed fp16 add of -1152 gives q. These integers go into the fp16 MFMA
// against fp16 activations (products exact in fp32); each 32-input block's
// partial sum is multiplied by its scale in fp32 and added. So every weight
// enters as exactly q * d, as in the oracle.
//
// Mapping, activation path and work distribution as in the bf16 kernels (64-row
// tiles, or 32-row tiles where experts hold few rows; 4 waves, two 16-row
// panels per wave, activation rows staged in LDS by DMA, both GEMMs in one
// launch from the per-XCD queues).
#include "dg_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace dg {

namespace {

using namespace gemm;

constexpr int kQCodeBytes = 2048;  // codes of one (e, s, p)
constexpr int kQScales = 64;       // fp16 scales of one (e, s, p)

// One K step of a wave's two panels: 4 blocks of 8 codes per panel and lane,
// and the lane's row's 4 scales per panel.
struct QPanels {
  u32x4 c0[2], c1[2];
  uint2 s0, s1;
};

// Step `step`'s codes and scales; consecutive steps are `cstep` bytes and
// `sstep` scales apart.
// NT: past the caches (an expert in one tile reads its weights once); else
// normal loads, so that the expert's other tiles find them in L2.
template <bool NT>
__device__ __forceinline__ void load_q(const uint8_t* c0, const uint8_t* c1, const uint16_t* s0, const uint16_t* s1,
                                       int step, size_t cstep, size_t sstep, QPanels& p) {
  const uint8_t* a = c0 + (size_t)step * cstep;
  const uint8_t* b = c1 + (size_t)step * cstep;
  auto ld16 = [](const uint8_t* q) {
    return NT ? ld_stream(reinterpret_cast<const u32x4*>(q)) : *reinterpret_cast<const u32x4*>(q);
  };
  auto ld8 = [](const uint16_t* q) {
    return NT ? ld_stream(reinterpret_cast<const uint64_t*>(q)) : *reinterpret_cast<const uint64_t*>(q);
  };
  p.c0[0] = ld16(a);
  p.c0[1] = ld16(a + 1024);
  p.c1[0] = ld16(b);
  p.c1[1] = ld16(b + 1024);
  const uint64_t v0 = ld8(s0 + (size_t)step * sstep);
  const uint64_t v1 = ld8(s1 + (size_t)step * sstep);
  p.s0 = make_uint2((uint32_t)v0, (uint32_t)(v0 >> 32));
  p.s1 = make_uint2((uint32_t)v1, (uint32_t)(v1 >> 32));
}

// Bytes 0 and 2 of v as fp16 1024 + 128 + q: (v & 0x00FF00FF) ^ 0x64806480
// (one three-input bitwise instruction on gfx950).
__device__ __forceinline__ uint32_t q8_pair(uint32_t v) {
  return (v & 0x00FF00FFu) ^ 0x64806480u;
}

// 8 codes in the packed order (two dwords) -> 8 fp16 values q in natural order.
__device__ __forceinline__ f16x8 q8_to_f16(uint32_t lo, uint32_t hi) {
  const f16x2 bias = f16x2{(_Float16)-1152.0f, (_Float16)-1152.0f};
  const f16x2 p0 = __builtin_bit_cast(f16x2, q8_pair(lo)) + bias;       // k0 k1
  const f16x2 p1 = __builtin_bit_cast(f16x2, q8_pair(lo >> 8)) + bias;  // k2 k3
  const f16x2 p2 = __builtin_bit_cast(f16x2, q8_pair(hi)) + bias;       // k4 k5
  const f16x2 p3 = __builtin_bit_cast(f16x2, q8_pair(hi >> 8)) + bias;  // k6 k7
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ float scale_of(const uint2& s, int j) {
  const uint32_t w = (j < 2) ? s.x : s.y;
  const uint16_t h = (j & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
  return (float)__builtin_bit_cast(_Float16, h);
}

// NS blocks of one step: each block's MFMA into a zeroed accumulator, then
// scaled by the block's d into acc.
template <int NMT, int NS, int MB>
__device__ __forceinline__ void mma_q8(const char* stage, int lane, const QPanels& p, f32x4 (&acc0)[MB],
                                       f32x4 (&acc1)[MB]) {
  const int g = lane >> 4, m = lane & 15;
  const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int o = (j & 1) * 2;
    const f16x8 b0 = q8_to_f16(p.c0[j >> 1][o], p.c0[j >> 1][o + 1]);
    const f16x8 b1 = q8_to_f16(p.c1[j >> 1][o], p.c1[j >> 1][o + 1]);
    const float d0 = scale_of(p.s0, j), d1 = scale_of(p.s1, j);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int r = mt * 16 + m;
      const int pos = (j * 4 + g) ^ (r % kSegs);
      const f16x8 av = as_f16x8(*reinterpret_cast<const u32x4*>(stage + r * kRowBytes + pos * 16));
      const f32x4 t0 = mfma_f16(av, b0, zero);
      const f32x4 t1 = mfma_f16(av, b1, zero);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[mt][i] = fmaf(d0, t0[i], acc0[mt][i]);
        acc1[mt][i] = fmaf(d1, t1[i], acc1[mt][i]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one block's operands and partial sums live at a time
  }
}

// Weight streams of a wave: code and scale pointers of both panels at step 0
// and the distance between steps.
struct QStream {
  const uint8_t* c0;
  const uint8_t* c1;
  const uint16_t* s0;
  const uint16_t* s1;
  size_t cstep, sstep;
};

// One step, as in the bf16 kernels: DMA of the next step's activation rows,
// then its codes and scales, then the MFMAs of step `it` (NSP blocks) from
// `cur`; the wait lets the six weight loads fly.
template <int ROWS, bool NT, int NMT, int NS, int NSP>
__device__ __forceinline__ void qstep(char* As, const uint16_t* const (&rowp)[dma_per_wave(ROWS, kWaves)],
                                      const QStream& w, int k1, int it, int wave, int lane, const QPanels& cur,
                                      QPanels& nxt, f32x4 (&acc0)[ROWS / 16], f32x4 (&acc1)[ROWS / 16]) {
  constexpr int kSB = ROWS * kRowBytes;
  dma_a<NMT, NS * 4>(As + ((it + 1) & 1) * kSB, rowp, k1, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_q<NT>(w.c0, w.c1, w.s0, w.s1, it + 1, w.cstep, w.sstep, nxt);
  __builtin_amdgcn_sched_barrier(0);
  mma_q8<NMT, NSP>(As + (it & 1) * kSB, lane, cur, acc0, acc1);
  wait_vmcnt<6>();
  lds_barrier();
}

template <int ROWS, bool NT, int NMT>
__device__ __forceinline__ void qfinish(char* As, const uint16_t* const (&rowp)[dma_per_wave(ROWS, kWaves)],
                                        const QStream& w, int nfull, int ntail, int wave, int lane, const QPanels& cur,
                                        QPanels& nxt, f32x4 (&acc0)[ROWS / 16], f32x4 (&acc1)[ROWS / 16]) {
  constexpr int kSB = ROWS * kRowBytes;
  const int last = nfull - 1;
  if (ntail == 0) {
    mma_q8<NMT, 4>(As + (last & 1) * kSB, lane, cur, acc0, acc1);
  } else {  // one 64-wide step remains (K % 128 == 64): its two blocks
    qstep<ROWS, NT, NMT, 2, 4>(As, rowp, w, nfull * kKS, last, wave, lane, cur, nxt, acc0, acc1);
    wait_vmcnt<0>();
    mma_q8<NMT, 2>(As + (nfull & 1) * kSB, lane, nxt, acc0, acc1);
  }
}

// The K loop of one tile (K a multiple of 64), the bf16 kernels' ping-pong.
template <int ROWS, bool NT, int NMT>
__device__ __forceinline__ void qloop(char* As, const uint16_t* const (&rowp)[dma_per_wave(ROWS, kWaves)],
                                      const QStream& w, int K, int tid, f32x4 (&acc0)[ROWS / 16],
                                      f32x4 (&acc1)[ROWS / 16]) {
  const int lane = tid & 63, wave = tid >> 6;
  const int nfull = K / kKS;
  const int ntail = (K - nfull * kKS) / 32;
  QPanels p0, p1;
  if (nfull == 0) {  // K = 64
    dma_a<NMT, 8>(As, rowp, 0, wave, lane);
    load_q<NT>(w.c0, w.c1, w.s0, w.s1, 0, w.cstep, w.sstep, p0);
    wait_vmcnt<0>();
    lds_barrier();
    mma_q8<NMT, 2>(As, lane, p0, acc0, acc1);
    return;
  }
  dma_a<NMT, kSegs>(As, rowp, 0, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_q<NT>(w.c0, w.c1, w.s0, w.s1, 0, w.cstep, w.sstep, p0);
  wait_vmcnt<6>();
  lds_barrier();
  int it = 0;
  for (; it + 2 < nfull; it += 2) {
    qstep<ROWS, NT, NMT, 4, 4>(As, rowp, w, (it + 1) * kKS, it, wave, lane, p0, p1, acc0, acc1);
    qstep<ROWS, NT, NMT, 4, 4>(As, rowp, w, (it + 2) * kKS, it + 1, wave, lane, p1, p0, acc0, acc1);
  }
  if (it + 2 == nfull) {
    qstep<ROWS, NT, NMT, 4, 4>(As, rowp, w, (it + 1) * kKS, it, wave, lane, p0, p1, acc0, acc1);
    qfinish<ROWS, NT, NMT>(As, rowp, w, nfull, ntail, wave, lane, p1, p0, acc0, acc1);
  } else {
    qfinish<ROWS, NT, NMT>(As, rowp, w, nfull, ntail, wave, lane, p0, p1, acc0, acc1);
  }
}

// The product of one task: gate_up writes the gated activation as fp16 (the
// down GEMM's fp16 operand), down its fp32 sums as bf16.
template <bool GATE_UP, int ROWS, bool NT>
__device__ __forceinline__ void q8_body(const GemmArgs& a, const Tile& tl, char* As) {
  constexpr int MB = ROWS / 16, NI = dma_per_wave(ROWS, kWaves);
  const int F = a.F, D = a.D;
  const int K = GATE_UP ? D : F;
  const int nks = (K + kKS - 1) / kKS;
  const int nb = tl.nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4;
  const int nmt = (tl.mc + 15) >> 4;

  // source row of each DMA instruction of this lane (rows past the tile re-read
  // its last row; their results are never stored)
  const uint16_t* rowp[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = min(kDmaRows * (wave + kWaves * i) + lane / kSegs, tl.mc - 1);
    rowp[i] = GATE_UP ? a.h + (size_t)(a.sorted_slot[tl.row0 + r] / a.K) * D : a.act + (size_t)(tl.row0 + r) * F;
  }
  int col, p0, p1, np;
  if (GATE_UP) {
    col = nb * 16 * kWaves + wave * 16 + (lane & 15);
    np = 2 * F / 16;
    p0 = nb * kWaves + wave;
    p1 = p0 + F / 16;
  } else {
    col = nb * 32 * kWaves + wave * 32 + (lane & 15);
    np = D / 16;
    p0 = 2 * (nb * kWaves + wave);
    p1 = p0 + 1;
  }
  const uint8_t* C = static_cast<const uint8_t*>(GATE_UP ? a.w_gate_up : a.w_down);
  const uint16_t* S = GATE_UP ? a.s_gate_up : a.s_down;
  const size_t blk0 = (size_t)tl.e * nks * np;  // block (e, 0, 0)
  QStream w;
  w.c0 = C + (blk0 + p0) * kQCodeBytes + lane * 16;
  w.c1 = C + (blk0 + p1) * kQCodeBytes + lane * 16;
  w.s0 = S + (blk0 + p0) * kQScales + (lane & 15) * 4;
  w.s1 = S + (blk0 + p1) * kQScales + (lane & 15) * 4;
  w.cstep = (size_t)np * kQCodeBytes;
  w.sstep = (size_t)np * kQScales;

  f32x4 acc0[MB], acc1[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    acc0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (MB == 2) {
    if (nmt == 1)
      qloop<ROWS, NT, 1>(As, rowp, w, K, tid, acc0, acc1);
    else
      qloop<ROWS, NT, 2>(As, rowp, w, K, tid, acc0, acc1);
  } else {
    switch (nmt) {
      case 1: qloop<ROWS, NT, 1>(As, rowp, w, K, tid, acc0, acc1); break;
      case 2: qloop<ROWS, NT, 2>(As, rowp, w, K, tid, acc0, acc1); break;
      case 3: qloop<ROWS, NT, 3>(As, rowp, w, K, tid, acc0, acc1); break;
      default: qloop<ROWS, NT, 4>(As, rowp, w, K, tid, acc0, acc1); break;
    }
  }

#pragma unroll
  for (int mt = 0; mt < MB; ++mt) {
    if (mt < nmt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + g * 4 + i;
        if (r < tl.mc) {
          if (GATE_UP) {
            const _Float16 v = (_Float16)(gelu_tanh(acc0[mt][i]) * acc1[mt][i]);
            a.act[(size_t)(tl.row0 + r) * F + col] = __builtin_bit_cast(uint16_t, v);
          } else {
            uint16_t* yr = a.y + (size_t)(tl.row0 + r) * D + col;
            yr[0] = f32_to_bf16_bits(acc0[mt][i]);
            yr[16] = f32_to_bf16_bits(acc1[mt][i]);
          }
        }
      }
    }
  }
}

// One task: weights past the caches when the expert has one tile only.
template <bool GATE_UP, int ROWS>
__device__ __forceinline__ void q8_task(const FusedGemmArgs& f, const GemmArgs& a, const Tile& tl, char* As) {
  if ((f.counts[tl.e] + ROWS - 1) / ROWS > 1)
    q8_body<GATE_UP, ROWS, false>(a, tl, As);
  else
    q8_body<GATE_UP, ROWS, true>(a, tl, As);
}

// Both GEMMs in one launch (the task logic of fused_tasks): 64-row tiles at
// two workgroups per CU, or 32-row tiles at three.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_q8_fused(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[2 * kTileRows * kRowBytes];
  fused_tasks(
      f, [&](const Tile& tl) { q8_task<true, kTileRows>(f, f.gu, tl, As); },
      [&](const Tile& tl) { q8_task<false, kTileRows>(f, f.dn, tl, As); });
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_gemm_q8_fused_short(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[2 * kShortRows * kRowBytes];
  fused_tasks(
      f, [&](const Tile& tl) { q8_task<true, kShortRows>(f, f.gu, tl, As); },
      [&](const Tile& tl) { q8_task<false, kShortRows>(f, f.dn, tl, As); });
}

// One wave per packed block (e, s, p); lane l = n + 16 g reads its row's
// blocks 4 s .. 4 s + 3, 8 codes each.
__global__ __launch_bounds__(256) void k_pack_q8(const uint8_t* __restrict__ src, uint8_t* __restrict__ pcodes,
                                                 uint16_t* __restrict__ pscales, int E, int R, int K) {
  const int nkb = K / 32, nks = (K + kKS - 1) / kKS, np = R / 16;
  const size_t nblk = (size_t)E * nks * np;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  for (size_t b = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6); b < nblk; b += (size_t)gridDim.x * 4) {
    const int p = (int)(b % np);
    const size_t es = b / np;
    const int s = (int)(es % nks);
    const size_t e = es / nks;
    const size_t row = e * R + (size_t)p * 16 + n;
    u32x4 o[2];
    uint32_t sc[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = 4 * s + j;
      uint32_t q[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      uint32_t d = 0;
      if (kb < nkb) {
        const uint8_t* blk = src + (row * nkb + kb) * 34;
        d = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = blk[2 + 8 * g + i];
      }
      o[j >> 1][(j & 1) * 2] = q[0] | (q[2] << 8) | (q[1] << 16) | (q[3] << 24);
      o[j >> 1][(j & 1) * 2 + 1] = q[4] | (q[6] << 8) | (q[5] << 16) | (q[7] << 24);
      sc[j >> 1] |= d << (16 * (j & 1));
    }
    uint8_t* dst = pcodes + b * kQCodeBytes + lane * 16;
    *reinterpret_cast<u32x4*>(dst) = o[0];
    *reinterpret_cast<u32x4*>(dst + 1024) = o[1];
    if (g == 0) *reinterpret_cast<uint2*>(pscales + b * kQScales + n * 4) = make_uint2(sc[0], sc[1]);
  }
}

}  // namespace

hipError_t launch_pack_q8(const uint8_t* blocks, uint8_t* pcodes, uint16_t* pscales, int E, int R, int K,
                          hipStream_t stream) {
  k_pack_q8<<<dim3(4096), dim3(256), 0, stream>>>(blocks, pcodes, pscales, E, R, K);
  return hipGetLastError();
}

hipError_t launch_gemm_fused_q8(const FusedGemmArgs& f, int tile_rows, hipStream_t stream, const KernelEvents* ev) {
  return launch_kernel(tile_rows == kShortRows ? k_gemm_q8_fused_short : k_gemm_q8_fused,
                       dim3(kQueues * (f.gu.qmax + f.dn.qmax)), dim3(kThreads), stream, ev, f);
}

}  // namespace dg
