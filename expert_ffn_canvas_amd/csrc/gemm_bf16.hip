// Grouped expert GEMMs on gfx950 bf16 matrix cores (fp32 accumulation).
//
//  gate_up: for each tile (expert e, rows row0 .. row0+mc-1, mc <= 64) and
//           each block of 64 d_ff features: g = h W_gate[e]^T and
//           u = h W_up[e]^T over the full d_model, then act = gelu_tanh(g) * u
//           (bf16). Where the expert input is not materialised, the rows are
//           the raw x, the packed weight holds W diag(1 + gamma_e), and g and
//           u are scaled by each token's r: the same h W^T, with the norm
//           applied on the other side of the product.
//  down:    for each tile and each block of 128 d_model outputs:
//           y = act W_down[e]^T (fp32 sums, stored as bf16), one row per routed
//           slot (the combine applies the routing weights).
//
// Shapes (auto-round PR "Add quantization support for DiffusionGemma",
// transformers backend test log, expert module dump): gate_proj and up_proj
// are Linear(2816 -> 704), down_proj is Linear(704 -> 2816), no bias; the
// activation is GELUTanh. The fused gate_up tensor is [E, 2F, D] with the
// gate rows first (Quant-Tuner PR, "Answers to the motivating questions",
// names the fused 3D gate_up projection; the row order is this library's).
//
// Mapping: one workgroup = 4 waves = one (tile, column block). Each wave owns
// two 16-row weight panels (gate+up, or two down panels) for every row of the
// tile, so every weight byte is read by exactly one wave and goes straight
// from global memory into MFMA operand registers; the next K step of the
// panels (128 inputs) is in flight while the current one is multiplied. The
// tile's activation rows are staged once per K step into LDS (double-buffered)
// and shared by the four waves. The main loop is specialised on the number of
// 16-row MFMA tiles the tile needs (1..4, or up to 8 for 128-row tiles) and is
// branch-free inside (rows past the tile re-read its last row), so the next
// step's loads stay in flight across the current step's MFMAs.
//
// Work distribution: both GEMMs run in one launch. Workgroup b takes task
// b / 8 of queue b % 8 (its XCD): the queue's gate_up tasks, then its down
// tasks, each down task once its tile's gate_up blocks are done. The
// permutation dealt whole experts to balance the queues.
#include "dg_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace dg {

namespace {

using namespace gemm;

// The weight fragments of one K step (NS sub-steps of 32) of a wave's two
// panels, and the stride of the stream they come from: elements between
// consecutive 32-column blocks of a lane (32 in a row-major row; in the packed
// layout, all of the expert's panels: their count times 512).
struct Panels {
  u32x4 b0[kNS], b1[kNS];
  int wstep;
};

// Weight panels of one K step: NS sub-steps of 32.
template <bool PK, int NS, bool NT = true>
__device__ __forceinline__ void load_w(const uint16_t* w0, const uint16_t* w1, int k0, Panels& p) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if constexpr (NT) {
      p.b0[s] = ld_stream(reinterpret_cast<const u32x4*>(w0 + (size_t)((k0 + 32 * s) >> 5) * p.wstep));
      p.b1[s] = ld_stream(reinterpret_cast<const u32x4*>(w1 + (size_t)((k0 + 32 * s) >> 5) * p.wstep));
    } else {
      p.b0[s] = *reinterpret_cast<const u32x4*>(w0 + (size_t)((k0 + 32 * s) >> 5) * p.wstep);
      p.b1[s] = *reinterpret_cast<const u32x4*>(w1 + (size_t)((k0 + 32 * s) >> 5) * p.wstep);
    }
  }
}

template <int NMT, int NS, int BMT>
__device__ __forceinline__ void mma_step(const char* stage, int lane, const Panels& p, f32x4 (&acc0)[BMT],
                                         f32x4 (&acc1)[BMT]) {
  // activation fragments live at a time: two sub-steps, one above 8 tiles
  constexpr int kLive = NMT > 8 ? 1 : 2;
  const int g = lane >> 4, m = lane & 15;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bf16x8 bb0 = as_bf16x8(p.b0[s]);
    const bf16x8 bb1 = as_bf16x8(p.b1[s]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int r = mt * 16 + m;
      const int pos = (s * 4 + g) ^ (r % kSegs);
      const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4*>(stage + r * kRowBytes + pos * 16));
      acc0[mt] = mfma_bf16(av, bb0, acc0[mt]);
      acc1[mt] = mfma_bf16(av, bb1, acc1[mt]);
    }
    if (s % kLive == kLive - 1) __builtin_amdgcn_sched_barrier(0);
  }
}

// One step with NS sub-steps, issued after the previous one: DMA of the
// activation rows into stage (it + 1) & 1, then the weight panels into `nxt`,
// then the MFMAs of step `it` (NSP sub-steps) from `cur`.
template <bool PK, int NMT, int NS, int NSP, int ROWS, int WV, bool NT>
__device__ __forceinline__ void step(char* As, const uint16_t* const (&rowp)[dma_per_wave(ROWS, WV)], const uint16_t* w0,
                                     const uint16_t* w1, int k1, int it, int wave, int lane, const Panels& cur,
                                     Panels& nxt, f32x4 (&acc0)[ROWS / 16], f32x4 (&acc1)[ROWS / 16]) {
  constexpr int kSB = ROWS * kRowBytes;
  dma_a<NMT, NS * 4, dma_per_wave(ROWS, WV), WV>(As + ((it + 1) & 1) * kSB, rowp, k1, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_w<PK, NS, NT>(w0, w1, k1, nxt);
  __builtin_amdgcn_sched_barrier(0);
  mma_step<NMT, NSP>(As + (it & 1) * kSB, lane, cur, acc0, acc1);
  wait_vmcnt<2 * NS>();  // this wave's DMA has landed; its weight loads may still fly
  lds_barrier();
}

// The last full step `last` (panels in `cur`) and the short tail, if any.
template <bool PK, int NMT, int ROWS, int WV, bool NT>
__device__ __forceinline__ void finish(char* As, const uint16_t* const (&rowp)[dma_per_wave(ROWS, WV)], const uint16_t* w0,
                                       const uint16_t* w1, int nfull, int ntail, int wave, int lane,
                                       const Panels& cur, Panels& nxt, f32x4 (&acc0)[ROWS / 16],
                                       f32x4 (&acc1)[ROWS / 16]) {
  constexpr int kSB = ROWS * kRowBytes;
  const int last = nfull - 1;
  const int k1 = nfull * kKS;
  char* tail_stage = As + (nfull & 1) * kSB;
  if (ntail == 0) {
    mma_step<NMT, kNS>(As + (last & 1) * kSB, lane, cur, acc0, acc1);
  } else {  // one 64-wide step remains (K % 128 == 64)
    step<PK, NMT, 2, kNS, ROWS, WV, NT>(As, rowp, w0, w1, k1, last, wave, lane, cur, nxt, acc0, acc1);
    wait_vmcnt<0>();
    mma_step<NMT, 2>(tail_stage, lane, nxt, acc0, acc1);
  }
}

// The K loop of one tile with NMT 16-row MFMA tiles. K is a multiple of 64.
// Two panel buffers alternate roles (the loop is unrolled by two) so that no
// register copies are needed between steps.
template <bool PK, int NMT, int ROWS, int WV, bool NT>
__device__ __forceinline__ void k_loop(char* As, const uint16_t* const (&rowp)[dma_per_wave(ROWS, WV)], const uint16_t* w0,
                                       const uint16_t* w1, int K, int tid, f32x4 (&acc0)[ROWS / 16],
                                       f32x4 (&acc1)[ROWS / 16], int wstep) {
  const int lane = tid & 63, wave = tid >> 6;
  const int nfull = K / kKS;
  const int ntail = (K - nfull * kKS) / 32;  // 0, or 2 for a last 64-wide step (K is a multiple of 64)
  Panels p0, p1;
  p0.wstep = wstep;
  p1.wstep = wstep;
  if (nfull == 0) {
    // K = 64: one short step only
    dma_a<NMT, 8, dma_per_wave(ROWS, WV), WV>(As, rowp, 0, wave, lane);
    load_w<PK, 2, NT>(w0, w1, 0, p0);
    wait_vmcnt<0>();
    lds_barrier();
    mma_step<NMT, 2>(As, lane, p0, acc0, acc1);
    return;
  }
  dma_a<NMT, kSegs, dma_per_wave(ROWS, WV), WV>(As, rowp, 0, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_w<PK, kNS, NT>(w0, w1, 0, p0);
  wait_vmcnt<2 * kNS>();
  lds_barrier();
  int it = 0;
  for (; it + 2 < nfull; it += 2) {
    step<PK, NMT, kNS, kNS, ROWS, WV, NT>(As, rowp, w0, w1, (it + 1) * kKS, it, wave, lane, p0, p1, acc0, acc1);
    step<PK, NMT, kNS, kNS, ROWS, WV, NT>(As, rowp, w0, w1, (it + 2) * kKS, it + 1, wave, lane, p1, p0, acc0, acc1);
  }
  if (it + 2 == nfull) {
    step<PK, NMT, kNS, kNS, ROWS, WV, NT>(As, rowp, w0, w1, (it + 1) * kKS, it, wave, lane, p0, p1, acc0, acc1);
    finish<PK, NMT, ROWS, WV, NT>(As, rowp, w0, w1, nfull, ntail, wave, lane, p1, p0, acc0, acc1);
  } else {
    finish<PK, NMT, ROWS, WV, NT>(As, rowp, w0, w1, nfull, ntail, wave, lane, p0, p1, acc0, acc1);
  }
}

// The product of one task (tile `tl` of up to ROWS rows, 64, 128 or 160 for
// experts that receive many rows) by WV waves (4, or 8 with 160 rows: 128
// gate_up features or 256 down outputs per task); `As` holds two K steps of
// ROWS activation rows. A wave whose panels lie past the last column block's
// end (F or D not a multiple of the block) streams the block's last panels
// again (cache hits) and stores nothing.
template <bool GATE_UP, bool PK, int ROWS, int WV = kWaves, bool NT = true>
__device__ __forceinline__ void gemm_body(const GemmArgs& a, const Tile& tl, char* As, float* rrow) {
  constexpr int kBM = ROWS / 16;  // 16-row MFMA tiles, and activation transfers per wave per step
  const int F = a.F, D = a.D;
  const int K = GATE_UP ? D : F;
  const int nb = tl.nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4;
  const int nmt = (tl.mc + 15) >> 4;
  // gate_up: r of each row's token into LDS. In the 64-row kernel the two
  // dependent loads go to a register here and to LDS only after the K loop,
  // so they overlap it instead of delaying its start (canvas256 -0.8 us per
  // step); the wider kernels, short of registers, keep them up front.
  constexpr bool kLateR = ROWS == kTileRows;
  float my_r = 1.0f;
  if (GATE_UP) {
    if (tid < ROWS && a.rnorm != nullptr && tid < tl.mc) my_r = a.rnorm[a.sorted_slot[tl.row0 + tid] / a.K];
    if (!kLateR) {
      if (tid < ROWS) rrow[tid] = my_r;
      __syncthreads();
    }
  }

  // source row of each DMA instruction of this lane (rows past the tile re-read
  // its last row; their results are never stored)
  constexpr int kNI = dma_per_wave(ROWS, WV);
  const uint16_t* rowp[kNI];
#pragma unroll
  for (int i = 0; i < kNI; ++i) {
    const int r = min(kDmaRows * (wave + WV * i) + lane / kSegs, tl.mc - 1);
    rowp[i] = GATE_UP ? a.h + (size_t)(a.sorted_slot[tl.row0 + r] / a.K) * D : a.act + (size_t)(tl.row0 + r) * F;
  }
  int col;  // gate_up: feature f; down: first output d
  const uint16_t* w0;
  const uint16_t* w1;
  // this wave's panel (pair) inside the matrix, clamped to the last one
  const int pw = nb * WV + wave;           // gate_up: gate panel; down: panel pair
  const int npw = GATE_UP ? F / 16 : D / 32;
  const bool live = pw < npw;
  const int pc = live ? pw : npw - 1;
  if (GATE_UP) {
    col = pc * 16 + (lane & 15);
    const uint16_t* W = static_cast<const uint16_t*>(a.w_gate_up);
    if (PK) {  // gate panel pc, up panel F / 16 later, in the same K-step row
      const int p = pc;
      w0 = W + ((size_t)tl.e * (D / 32) * (2 * F / 16) + p) * 512 + lane * 8;
      w1 = w0 + (size_t)(F / 16) * 512;
    } else {
      w0 = W + ((size_t)tl.e * 2 * F + col) * D + g * 8;
      w1 = w0 + (size_t)F * D;
    }
  } else {
    col = pc * 32 + (lane & 15);
    const uint16_t* W = static_cast<const uint16_t*>(a.w_down);
    if (PK) {  // panels 2 pc and the next
      const int p = 2 * pc;
      w0 = W + ((size_t)tl.e * (F / 32) * (D / 16) + p) * 512 + lane * 8;
      w1 = w0 + 512;
    } else {
      w0 = W + ((size_t)tl.e * D + col) * F + g * 8;
      w1 = w0 + (size_t)16 * F;
    }
  }

  const int wstep = PK ? (GATE_UP ? 2 * F / 16 : D / 16) * 512 : 32;
  f32x4 acc0[kBM], acc1[kBM];
#pragma unroll
  for (int i = 0; i < kBM; ++i) {
    acc0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (ROWS == 64) {
    switch (nmt) {
      case 1: k_loop<PK, 1, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 2: k_loop<PK, 2, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 3: k_loop<PK, 3, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      default: k_loop<PK, 4, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
    }
  } else if constexpr (ROWS == 128) {
    switch (nmt) {
      case 1: k_loop<PK, 1, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 2: k_loop<PK, 2, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 3: k_loop<PK, 3, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 4: k_loop<PK, 4, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 5: k_loop<PK, 5, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 6: k_loop<PK, 6, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 7: k_loop<PK, 7, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      default: k_loop<PK, 8, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
    }
  } else {
    switch (nmt) {  // wide tiles: up to 80 rows run as 5 MFMA tiles
      case 1: case 2: case 3: case 4: case 5:
        k_loop<PK, 5, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 6: k_loop<PK, 6, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 7: k_loop<PK, 7, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 8: k_loop<PK, 8, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      case 9: k_loop<PK, 9, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
      default: k_loop<PK, 10, ROWS, WV, NT>(As, rowp, w0, w1, K, tid, acc0, acc1, wstep); break;
    }
  }

  if (GATE_UP && kLateR) {
    if (tid < ROWS) rrow[tid] = my_r;
    __syncthreads();
  }
#pragma unroll
  for (int mt = 0; mt < kBM; ++mt) {
    if (mt < nmt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + g * 4 + i;
        if (r < tl.mc && live) {
          if (GATE_UP) {
            const float rr = rrow[r];
            a.act[(size_t)(tl.row0 + r) * F + col] =
                f32_to_bf16_bits(gelu_tanh(acc0[mt][i] * rr) * (acc1[mt][i] * rr));
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

// One task of a fused launch. Expert weights are read once per launch and
// stream past the caches (ld_stream), except those of an expert cut into
// several tiles: each of its tiles reads the same weight blocks, close together
// in time (the tiles of one column block are neighbours in the queue), so they
// are loaded normally and the later tiles find them in L2 (30 stacked layers
// at 512 tokens, where the Zipf-loaded experts hold up to 8 tiles: 8.26 ->
// 7.53 ms per stack; canvas256 170.1 -> 167.8 us and encode 347 -> 341 us for
// the fused launch).
template <bool GATE_UP, bool PK, int ROWS, int WV = kWaves>
__device__ __forceinline__ void task_body(const FusedGemmArgs& f, const GemmArgs& a, const Tile& tl, char* As,
                                          float* rrow) {
  if ((f.counts[tl.e] + ROWS - 1) / ROWS > 1)
    gemm_body<GATE_UP, PK, ROWS, WV, false>(a, tl, As, rrow);
  else
    gemm_body<GATE_UP, PK, ROWS, WV, true>(a, tl, As, rrow);
}

// Both GEMMs in one launch (the task logic of fused_tasks). Three workgroups
// per CU (waves_per_eu 3): the register budget that keeps two K steps of
// weight panels per wave in flight without spilling.
template <bool PK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_gemm_fused(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[2 * kTileRows * kRowBytes];
  __shared__ float rrow[kTileRows];  // gate_up: r of each row's token, or 1
  fused_tasks(
      f, [&](const Tile& tl) { task_body<true, PK, kTileRows>(f, f.gu, tl, As, rrow); },
      [&](const Tile& tl) { task_body<false, PK, kTileRows>(f, f.dn, tl, As, rrow); });
}

// 128-row tiles: twice the accumulators and 64 KB of activation stages, two
// workgroups per CU.
template <bool PK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_fused_tall(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[2 * kTallRows * kRowBytes];
  __shared__ float rrow[kTallRows];
  fused_tasks(
      f, [&](const Tile& tl) { task_body<true, PK, kTallRows>(f, f.gu, tl, As, rrow); },
      [&](const Tile& tl) { task_body<false, PK, kTallRows>(f, f.dn, tl, As, rrow); });
}

// Wide tiles of up to 160 rows (every row an expert receives at the 2304-token
// encode, so each weight block is streamed once): 8 waves share the tile's
// activation stages (80 KB, one workgroup per CU, two waves per SIMD) and
// cover 128 gate_up features or 256 down outputs per task.
template <bool PK>
__global__ __launch_bounds__(64 * kWideWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_fused_wide(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[2 * kWideRows * kRowBytes];
  __shared__ float rrow[kWideRows];
  fused_tasks<kWideWaves>(
      f, [&](const Tile& tl) { task_body<true, PK, kWideRows, kWideWaves>(f, f.gu, tl, As, rrow); },
      [&](const Tile& tl) { task_body<false, PK, kWideRows, kWideWaves>(f, f.dn, tl, As, rrow); });
}

// One wave per block of 64 lanes x 16 bytes: source block (e, p, s) of 16 rows
// x 32 columns goes to position (e, s, p). With `gamma`, value k is scaled by
// (1 + gamma[k]) and rounded to bf16.
__global__ __launch_bounds__(256) void k_pack_panels(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                     int E, int R, int K, const float* __restrict__ gamma) {
  const int nks = K / 32, np = R / 16;
  const size_t nblk = (size_t)E * np * nks;
  const int lane = threadIdx.x & 63;
  for (size_t b = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6); b < nblk; b += (size_t)gridDim.x * 4) {
    const int s = (int)(b % nks);
    const size_t ep = b / nks;  // e * np + p
    const size_t row = ep * 16 + (lane & 15);
    const int k = 32 * s + 8 * (lane >> 4);
    u32x4 v = *reinterpret_cast<const u32x4*>(src + row * K + k);
    if (gamma != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = pack_bf16x2(bf16_lo(v[i]) * (1.0f + gamma[k + 2 * i]), bf16_hi(v[i]) * (1.0f + gamma[k + 2 * i + 1]));
    }
    const size_t e = ep / np, pp = ep % np;
    *reinterpret_cast<u32x4*>(dst + ((e * nks + s) * np + pp) * 512 + lane * 8) = v;
  }
}

}  // namespace

hipError_t launch_pack_panels(const uint16_t* src, uint16_t* dst, int E, int R, int K, const float* gamma,
                              hipStream_t stream) {
  k_pack_panels<<<dim3(4096), dim3(256), 0, stream>>>(src, dst, E, R, K, gamma);
  return hipGetLastError();
}

hipError_t launch_gemm_fused(const FusedGemmArgs& f, int tile_rows, hipStream_t stream, const KernelEvents* ev) {
  const dim3 grid(kQueues * (f.gu.qmax + f.dn.qmax));
  const bool pk = f.gu.w_packed != 0;
  if (tile_rows == kWideRows)
    return launch_kernel(pk ? k_gemm_fused_wide<true> : k_gemm_fused_wide<false>, grid, dim3(64 * kWideWaves), stream,
                         ev, f);
  auto k = tile_rows == kTallRows ? (pk ? k_gemm_fused_tall<true> : k_gemm_fused_tall<false>)
                                  : (pk ? k_gemm_fused<true> : k_gemm_fused<false>);
  return launch_kernel(k, grid, dim3(kThreads), stream, ev, f);
}

}  // namespace dg
