// Grouped expert GEMMs with OCP Microscaling expert weights (MXFP4 and MXFP8)
// on gfx950 bf16 matrix cores, the codes and their block scales widened by the
// hardware conversion inside the weight load.
//
// Weight formats: the FP4 and FP8 builds that the HF card "DiffusionGemma-
// 26B-A4B-it - ROCmFP4 / ROCmFPX GGUF" compares (introduction; "The 4-bit is
// NOT the fastest here"; Credits) are not spelled out on the pages; they are
// read as OCP Microscaling formats: blocks of 32 consecutive inputs of a row
// share an E8M0 scale 2^(e - 127) (e = 255: NaN), and each input is
//  * MXFP4: an E2M1 code (sign, two exponent bits with bias 1, one mantissa
//    bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6). The caller stores a block as the scale
//    byte, then 16 code bytes holding input j in the low nibble of byte j
//    (j < 16) or in the high nibble of byte j - 16;
//  * MXFP8: an E4M3 code (sign, four exponent bits with bias 7, three mantissa
//    bits, subnormal below 2^-6, 448 the largest, S.1111.111 NaN). The caller
//    stores a block as the scale byte, then the 32 code bytes in input order.
//
// Packed at create (17- and 33-byte blocks do not fit 16-byte loads): per
// (expert e, 128-input step s, 16-row panel p), in that order, the codes
// (1 KB for MXFP4, 2 KB for MXFP8) and 64 scale bytes. Lane l = n + 16 g of a
// code block holds its row 16 p + n's inputs 128 s + 32 j + 8 g .. + 7 (block
// 4 s + j) for j = 0..3: one dword per block for MXFP4 (two codes per byte,
// the even input in the low nibble; 16 bytes at 16 l), two for MXFP8 (one
// code per byte, in input order; 32 bytes in two halves at 16 l and
// 1024 + 16 l, so each 16-byte load of a wave reads whole cache lines); the
// scale bytes are [n][j]. Blocks past the row (the 64-input
// tail of a 704 row) are padded with zero codes and scale bytes.
//
// Exact widening: v_cvt_scalef32_pk_bf16_fp4 (one code byte) and
// v_cvt_scalef32_pk_bf16_fp8 (two code bytes) give two codes' values times
// the block scale 2^(e - 127) (built as an fp32 bit pattern) as bf16. An E2M1
// value has at most two significant bits, an E4M3 value four, and bf16 has
// fp32's exponent range, so the product is exact as long as it stays within
// bf16's range: always for MXFP4 (subnormal down to 2^-133; a scale of 2^127
// overflows to infinity for the codes 6 and -6, as in fp32), and for MXFP8
// whenever e >= 3 (below that, the smallest codes fall under bf16's smallest
// subnormal 2^-133 and are rounded to it). These weights go into the bf16 MFMA
// against bf16 activations (products exact in fp32), exactly like the bf16
// kernels: every weight enters as exactly its code's value times its block
// scale, as in the oracle.
//
// Mapping, activation path and work distribution as in the bf16 and Q8_0
// kernels (64-row tiles, or 32-row tiles where experts hold few rows; 4 waves,
// two 16-row panels per wave, activation rows staged in LDS by DMA, both GEMMs
// in one launch from the per-XCD queues), with a quarter (MXFP4) or a half
// (MXFP8) of the bf16 kernels' weight bytes per step.
#include "dg_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace dg {

namespace {

using namespace gemm;

constexpr int kMScaleBytes = 64;  // scale bytes of one (e, s, p)

// Code bytes of one (e, s, p), and per lane, for BITS-bit codes.
template <int BITS>
constexpr int kMCodeBytes = 64 * 4 * BITS;  // 4 blocks of 8 codes per lane

// One K step of a wave's two panels: 4 blocks of 8 codes per panel and lane
// (BITS / 4 vectors of 16 bytes each), and the lane's row's 4 scale bytes per
// panel.
template <int BITS>
struct MPanels {
  u32x4 c0[BITS / 4], c1[BITS / 4];
  uint32_t s0, s1;
};

// Loads per step and wave (codes and scales of both panels).
template <int BITS>
constexpr int kMLoads = 2 * (BITS / 4) + 2;

// Step `step`'s codes and scales; consecutive steps are `cstep` and `sstep`
// bytes apart.
// NT: past the caches (an expert in one tile reads its weights once); else
// normal loads, so that the expert's other tiles find them in L2.
template <int BITS, bool NT>
__device__ __forceinline__ void load_m(const uint8_t* c0, const uint8_t* c1, const uint8_t* s0, const uint8_t* s1,
                                       int step, size_t cstep, size_t sstep, MPanels<BITS>& p) {
  auto ld16 = [](const uint8_t* q) {
    return NT ? ld_stream(reinterpret_cast<const u32x4*>(q)) : *reinterpret_cast<const u32x4*>(q);
  };
  auto ld4 = [](const uint8_t* q) {
    return NT ? ld_stream(reinterpret_cast<const uint32_t*>(q)) : *reinterpret_cast<const uint32_t*>(q);
  };
#pragma unroll
  for (int h = 0; h < BITS / 4; ++h) {
    p.c0[h] = ld16(c0 + (size_t)step * cstep + 1024 * h);
    p.c1[h] = ld16(c1 + (size_t)step * cstep + 1024 * h);
  }
  p.s0 = ld4(s0 + (size_t)step * sstep);
  p.s1 = ld4(s1 + (size_t)step * sstep);
}

// 8 E2M1 codes of one dword (natural order, even input in the low nibble)
// times the block scale -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 mx4_to_bf16(uint32_t v, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// 8 E4M3 codes of two dwords (input order, byte by byte) times the block
// scale -> 8 bf16, exact (see above for the tiniest scales).
__device__ __forceinline__ bf16x8 mx8_to_bf16(uint32_t lo, uint32_t hi, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Block j's 8 codes of a lane's panel (c: the panel's code vectors).
template <int BITS>
__device__ __forceinline__ bf16x8 widen(const u32x4 (&c)[BITS / 4], int j, float scale) {
  if constexpr (BITS == 4)
    return mx4_to_bf16(c[0][j], scale);
  else
    return mx8_to_bf16(c[j >> 1][(j & 1) * 2], c[j >> 1][(j & 1) * 2 + 1], scale);
}

// Scale byte j of s as fp32: 2^(e - 127), its bit pattern e << 23 for
// e = 1 .. 254; e = 0 is 2^-127, the subnormal 0x00400000; e = 255 is NaN.
__device__ __forceinline__ float mx_scale(uint32_t s, int j) {
  const uint32_t e = (s >> (8 * j)) & 0xffu;
  const uint32_t bits = e == 0 ? 0x00400000u : e == 255 ? 0x7fc00000u : e << 23;
  return __uint_as_float(bits);
}

// NS blocks of one step, each one MFMA K step of 32 inputs.
template <int BITS, int NMT, int NS, int MB>
__device__ __forceinline__ void mma_mx(const char* stage, int lane, const MPanels<BITS>& p, f32x4 (&acc0)[MB],
                                       f32x4 (&acc1)[MB]) {
  const int g = lane >> 4, m = lane & 15;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const bf16x8 b0 = widen<BITS>(p.c0, j, mx_scale(p.s0, j));
    const bf16x8 b1 = widen<BITS>(p.c1, j, mx_scale(p.s1, j));
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int r = mt * 16 + m;
      const int pos = (j * 4 + g) ^ (r % kSegs);
      const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4*>(stage + r * kRowBytes + pos * 16));
      acc0[mt] = mfma_bf16(av, b0, acc0[mt]);
      acc1[mt] = mfma_bf16(av, b1, acc1[mt]);
    }
    if (j & 1) __builtin_amdgcn_sched_barrier(0);  // at most two blocks' operands live at a time
  }
}

// Weight streams of a wave: code and scale pointers of both panels at step 0
// and the distance between steps.
struct MStream {
  const uint8_t* c0;
  const uint8_t* c1;
  const uint8_t* s0;
  const uint8_t* s1;
  size_t cstep, sstep;
};

// One step, as in the bf16 kernels: DMA of the next step's activation rows,
// then its codes and scales, then the MFMAs of step `it` (NSP blocks) from
// `cur`; the wait lets the weight loads fly.
template <int BITS, int ROWS, bool NT, int NMT, int NS, int NSP>
__device__ __forceinline__ void mstep(char* As, const uint16_t* const (&rowp)[dma_per_wave(ROWS, kWaves)],
                                      const MStream& w, int k1, int it, int wave, int lane, const MPanels<BITS>& cur,
                                      MPanels<BITS>& nxt, f32x4 (&acc0)[ROWS / 16], f32x4 (&acc1)[ROWS / 16]) {
  constexpr int kSB = ROWS * kRowBytes;
  dma_a<NMT, NS * 4>(As + ((it + 1) & 1) * kSB, rowp, k1, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_m<BITS, NT>(w.c0, w.c1, w.s0, w.s1, it + 1, w.cstep, w.sstep, nxt);
  __builtin_amdgcn_sched_barrier(0);
  mma_mx<BITS, NMT, NSP>(As + (it & 1) * kSB, lane, cur, acc0, acc1);
  wait_vmcnt<kMLoads<BITS>>();
  lds_barrier();
}

template <int BITS, int ROWS, bool NT, int NMT>
__device__ __forceinline__ void mfinish(char* As, const uint16_t* const (&rowp)[dma_per_wave(ROWS, kWaves)],
                                        const MStream& w, int nfull, int ntail, int wave, int lane,
                                        const MPanels<BITS>& cur, MPanels<BITS>& nxt, f32x4 (&acc0)[ROWS / 16],
                                        f32x4 (&acc1)[ROWS / 16]) {
  constexpr int kSB = ROWS * kRowBytes;
  const int last = nfull - 1;
  if (ntail == 0) {
    mma_mx<BITS, NMT, 4>(As + (last & 1) * kSB, lane, cur, acc0, acc1);
  } else {  // one 64-wide step remains (K % 128 == 64): its two blocks
    mstep<BITS, ROWS, NT, NMT, 2, 4>(As, rowp, w, nfull * kKS, last, wave, lane, cur, nxt, acc0, acc1);
    wait_vmcnt<0>();
    mma_mx<BITS, NMT, 2>(As + (nfull & 1) * kSB, lane, nxt, acc0, acc1);
  }
}

// The K loop of one tile (K a multiple of 64), the bf16 kernels' ping-pong.
template <int BITS, int ROWS, bool NT, int NMT>
__device__ __forceinline__ void mloop(char* As, const uint16_t* const (&rowp)[dma_per_wave(ROWS, kWaves)],
                                      const MStream& w, int K, int tid, f32x4 (&acc0)[ROWS / 16],
                                      f32x4 (&acc1)[ROWS / 16]) {
  const int lane = tid & 63, wave = tid >> 6;
  const int nfull = K / kKS;
  const int ntail = (K - nfull * kKS) / 32;
  MPanels<BITS> p0, p1;
  if (nfull == 0) {  // K = 64
    dma_a<NMT, 8>(As, rowp, 0, wave, lane);
    load_m<BITS, NT>(w.c0, w.c1, w.s0, w.s1, 0, w.cstep, w.sstep, p0);
    wait_vmcnt<0>();
    lds_barrier();
    mma_mx<BITS, NMT, 2>(As, lane, p0, acc0, acc1);
    return;
  }
  dma_a<NMT, kSegs>(As, rowp, 0, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_m<BITS, NT>(w.c0, w.c1, w.s0, w.s1, 0, w.cstep, w.sstep, p0);
  wait_vmcnt<kMLoads<BITS>>();
  lds_barrier();
  int it = 0;
  for (; it + 2 < nfull; it += 2) {
    mstep<BITS, ROWS, NT, NMT, 4, 4>(As, rowp, w, (it + 1) * kKS, it, wave, lane, p0, p1, acc0, acc1);
    mstep<BITS, ROWS, NT, NMT, 4, 4>(As, rowp, w, (it + 2) * kKS, it + 1, wave, lane, p1, p0, acc0, acc1);
  }
  if (it + 2 == nfull) {
    mstep<BITS, ROWS, NT, NMT, 4, 4>(As, rowp, w, (it + 1) * kKS, it, wave, lane, p0, p1, acc0, acc1);
    mfinish<BITS, ROWS, NT, NMT>(As, rowp, w, nfull, ntail, wave, lane, p1, p0, acc0, acc1);
  } else {
    mfinish<BITS, ROWS, NT, NMT>(As, rowp, w, nfull, ntail, wave, lane, p0, p1, acc0, acc1);
  }
}

// The product of one task: gate_up writes the gated activation as bf16 (the
// down GEMM's bf16 operand), down its fp32 sums as bf16.
template <int BITS, bool GATE_UP, int ROWS, bool NT>
__device__ __forceinline__ void mx_body(const GemmArgs& a, const Tile& tl, char* As) {
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
  constexpr int kCB = kMCodeBytes<BITS>;
  const uint8_t* C = static_cast<const uint8_t*>(GATE_UP ? a.w_gate_up : a.w_down);
  const uint8_t* S = reinterpret_cast<const uint8_t*>(GATE_UP ? a.s_gate_up : a.s_down);
  const size_t blk0 = (size_t)tl.e * nks * np;  // block (e, 0, 0)
  MStream w;
  w.c0 = C + (blk0 + p0) * kCB + lane * 16;
  w.c1 = C + (blk0 + p1) * kCB + lane * 16;
  w.s0 = S + (blk0 + p0) * kMScaleBytes + (lane & 15) * 4;
  w.s1 = S + (blk0 + p1) * kMScaleBytes + (lane & 15) * 4;
  w.cstep = (size_t)np * kCB;
  w.sstep = (size_t)np * kMScaleBytes;

  f32x4 acc0[MB], acc1[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    acc0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (MB == 2) {
    if (nmt == 1)
      mloop<BITS, ROWS, NT, 1>(As, rowp, w, K, tid, acc0, acc1);
    else
      mloop<BITS, ROWS, NT, 2>(As, rowp, w, K, tid, acc0, acc1);
  } else {
    switch (nmt) {
      case 1: mloop<BITS, ROWS, NT, 1>(As, rowp, w, K, tid, acc0, acc1); break;
      case 2: mloop<BITS, ROWS, NT, 2>(As, rowp, w, K, tid, acc0, acc1); break;
      case 3: mloop<BITS, ROWS, NT, 3>(As, rowp, w, K, tid, acc0, acc1); break;
      default: mloop<BITS, ROWS, NT, 4>(As, rowp, w, K, tid, acc0, acc1); break;
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
            a.act[(size_t)(tl.row0 + r) * F + col] = f32_to_bf16_bits(gelu_tanh(acc0[mt][i]) * acc1[mt][i]);
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
template <int BITS, bool GATE_UP, int ROWS>
__device__ __forceinline__ void mx_task(const FusedGemmArgs& f, const GemmArgs& a, const Tile& tl, char* As) {
  if ((f.counts[tl.e] + ROWS - 1) / ROWS > 1)
    mx_body<BITS, GATE_UP, ROWS, false>(a, tl, As);
  else
    mx_body<BITS, GATE_UP, ROWS, true>(a, tl, As);
}

// Both GEMMs in one launch (the task logic of fused_tasks): 64-row tiles at
// three workgroups per CU as the bf16 kernels (162 registers for MXFP8, no
// spills), or 32-row tiles at four.
template <int BITS, int ROWS>
__device__ __forceinline__ void mx_fused(const FusedGemmArgs& f, char* As) {
  fused_tasks(
      f, [&](const Tile& tl) { mx_task<BITS, true, ROWS>(f, f.gu, tl, As); },
      [&](const Tile& tl) { mx_task<BITS, false, ROWS>(f, f.dn, tl, As); });
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_gemm_mx4_fused(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[2 * kTileRows * kRowBytes];
  mx_fused<4, kTileRows>(f, As);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_gemm_mx8_fused(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[2 * kTileRows * kRowBytes];
  mx_fused<8, kTileRows>(f, As);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_gemm_mx4_fused_short(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[2 * kShortRows * kRowBytes];
  mx_fused<4, kShortRows>(f, As);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_gemm_mx8_fused_short(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[2 * kShortRows * kRowBytes];
  mx_fused<8, kShortRows>(f, As);
}

// One wave per packed block (e, s, p); lane l = n + 16 g gathers its row's
// inputs 8 g .. 8 g + 7 of blocks 4 s .. 4 s + 3. Caller blocks are
// 1 + 4 BITS bytes: the scale byte, then the codes.
template <int BITS>
__global__ __launch_bounds__(256) void k_pack_mx(const uint8_t* __restrict__ src, uint8_t* __restrict__ pcodes,
                                                 uint8_t* __restrict__ pscales, int E, int R, int K) {
  constexpr int kSrcBlock = 1 + 4 * BITS;
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
    uint32_t o[BITS];  // BITS / 4 dwords per block
    uint32_t sc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = 4 * s + j;
      uint32_t v[2] = {0u, 0u}, ex = 0;
      if (kb < nkb) {
        const uint8_t* blk = src + (row * nkb + kb) * kSrcBlock;
        ex = blk[0];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int t = 8 * g + i;  // input of the block
          if constexpr (BITS == 4) {
            const uint32_t byte = blk[1 + (t & 15)];
            v[0] |= (t < 16 ? (byte & 0xfu) : (byte >> 4)) << (4 * i);
          } else {
            v[i >> 2] |= (uint32_t)blk[1 + t] << (8 * (i & 3));
          }
        }
      }
#pragma unroll
      for (int h = 0; h < BITS / 4; ++h) o[j * (BITS / 4) + h] = v[h];
      sc |= ex << (8 * j);
    }
    uint8_t* dst = pcodes + b * (64 * 4 * BITS) + lane * 16;
#pragma unroll
    for (int h = 0; h < BITS / 4; ++h)
      *reinterpret_cast<u32x4*>(dst + 1024 * h) = u32x4{o[4 * h], o[4 * h + 1], o[4 * h + 2], o[4 * h + 3]};
    if (g == 0) *reinterpret_cast<uint32_t*>(pscales + b * kMScaleBytes + n * 4) = sc;
  }
}

}  // namespace

hipError_t launch_pack_mx4(const uint8_t* blocks, uint8_t* pcodes, uint8_t* pscales, int E, int R, int K,
                           hipStream_t stream) {
  k_pack_mx<4><<<dim3(4096), dim3(256), 0, stream>>>(blocks, pcodes, pscales, E, R, K);
  return hipGetLastError();
}

hipError_t launch_pack_mx8(const uint8_t* blocks, uint8_t* pcodes, uint8_t* pscales, int E, int R, int K,
                           hipStream_t stream) {
  k_pack_mx<8><<<dim3(4096), dim3(256), 0, stream>>>(blocks, pcodes, pscales, E, R, K);
  return hipGetLastError();
}

hipError_t launch_gemm_fused_mx4(const FusedGemmArgs& f, int tile_rows, hipStream_t stream, const KernelEvents* ev) {
  return launch_kernel(tile_rows == kShortRows ? k_gemm_mx4_fused_short : k_gemm_mx4_fused,
                       dim3(kQueues * (f.gu.qmax + f.dn.qmax)), dim3(kThreads), stream, ev, f);
}

hipError_t launch_gemm_fused_mx8(const FusedGemmArgs& f, int tile_rows, hipStream_t stream, const KernelEvents* ev) {
  return launch_kernel(tile_rows == kShortRows ? k_gemm_mx8_fused_short : k_gemm_mx8_fused,
                       dim3(kQueues * (f.gu.qmax + f.dn.qmax)), dim3(kThreads), stream, ev, f);
}

}  // namespace dg
