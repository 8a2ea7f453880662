// Grouped expert GEMMs with int4-g128 expert weights on gfx950 fp16 matrix
// cores, dequantisation fused into the weight load.
//
// Weight format (auto-round PR "Add quantization support for DiffusionGemma",
// test log, quantization_config: bits 4, group_size 128, sym, int): a code q
// in [0, 15] stands for (q - 8) * s, with one fp16 scale s per (output row,
// group of 128 consecutive inputs). Two codes per byte, even input index in
// the low nibble. The last group of a down row holds the remaining 64 inputs
// (d_ff = 704 = 5 * 128 + 64).
//
// Exact dequantisation: OR-ing a nibble into the mantissa of fp16 1024.0
// (0x6400) gives exactly 1024 + q, and one packed fp16 add of -1032 gives
// q - 8 exactly. These small integers go into the MFMA against fp16
// activations (products exact in fp32); each group's partial sum is then
// multiplied by its scale in fp32. So every weight enters as exactly (q - 8) s.
//
// Work distribution as in the bf16 kernels: workgroup b takes queue b % 8 (its
// XCD), task b / 8 of that queue (a tile and a column block).
//
// Lane layout: lane (n = l % 16, g = l / 16) loads 16 bytes = 32 codes of
// row n covering inputs 32 g .. 32 g + 31 of a 128-input group; dword s of that
// load feeds MFMA step s. Unpacking a dword with the mask 0x000F000F pairs
// codes (0,4), (1,5), (2,6), (3,7); the activations are stored into LDS in the
// same order so that both MFMA operands agree on which k each element is.
#include "dg_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace dg {

namespace {

using namespace gemm;  // kThreads (256), kBMT (4: the borrowed kernels' 64-row tiles), the DMA and wait helpers

constexpr int kSlab = 128;              // inputs per scale group = K per step
constexpr int kPitch = kSlab + 8;       // LDS row pitch in fp16 elements
constexpr int kAPass = kTileRows / 16;  // 256 threads stage 16 rows x 128 K per pass

// 8 activations (a0..a7) -> order a0 a4 a1 a5 a2 a6 a3 a7.
__device__ __forceinline__ u32x4 interleave_k(const u32x4& v) {
  u32x4 o;
  o[0] = (v[0] & 0xffffu) | (v[2] << 16);
  o[1] = (v[0] >> 16) | (v[2] & 0xffff0000u);
  o[2] = (v[1] & 0xffffu) | (v[3] << 16);
  o[3] = (v[1] >> 16) | (v[3] & 0xffff0000u);
  return o;
}

// 8 int4 codes of one dword -> 8 fp16 values (q - 8), order k0 k4 k1 k5 k2 k6 k3 k7.
__device__ __forceinline__ f16x8 dequant8(uint32_t v) {
  const f16x2 bias = f16x2{(_Float16)-1032.0f, (_Float16)-1032.0f};
  f16x2 p0 = __builtin_bit_cast(f16x2, (v & 0x000F000Fu) | 0x64006400u) + bias;
  f16x2 p1 = __builtin_bit_cast(f16x2, ((v >> 4) & 0x000F000Fu) | 0x64006400u) + bias;
  f16x2 p2 = __builtin_bit_cast(f16x2, ((v >> 8) & 0x000F000Fu) | 0x64006400u) + bias;
  f16x2 p3 = __builtin_bit_cast(f16x2, ((v >> 12) & 0x000F000Fu) | 0x64006400u) + bias;
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ float half_bits(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Stage one 128-input step of the tile rows; segments at or past `k_end` are zero.
__device__ __forceinline__ void load_a(const uint16_t* const (&src)[kAPass], int k0, int seg, int k_end,
                                       u32x4 (&ra)[kAPass]) {
#pragma unroll
  for (int p = 0; p < kAPass; ++p) {
    if (src[p]) {
      if (k0 + seg * 8 < k_end)
        ra[p] = *reinterpret_cast<const u32x4*>(src[p] + k0);
      else
        ra[p] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void store_a(uint16_t* lds, const uint16_t* const (&src)[kAPass], int tid,
                                        const u32x4 (&ra)[kAPass]) {
#pragma unroll
  for (int p = 0; p < kAPass; ++p)
    if (src[p]) *reinterpret_cast<u32x4*>(lds + ((tid >> 4) + 16 * p) * kPitch + (tid & 15) * 8) = interleave_k(ra[p]);
}

__global__ __launch_bounds__(kThreads) void k_gate_up_i4(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTileRows * kPitch];
  const int F = a.F, D = a.D;
  const int qx = blockIdx.x & (kQueues - 1);
  const int jq = blockIdx.x / kQueues;
  if (jq >= a.qlen[qx]) return;
  const Tile tl = a.tiles[(size_t)qx * a.qmax + jq];
  const int fb = tl.nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nmt = (tl.mc + 15) >> 4;
  const int seg = tid & 15;

  const uint16_t* src[kAPass];
#pragma unroll
  for (int p = 0; p < kAPass; ++p) {
    const int r = (tid >> 4) + 16 * p;
    src[p] = (r < tl.mc) ? a.h + (size_t)(a.sorted_slot[tl.row0 + r] / a.K) * D + seg * 8 : nullptr;
  }
  const int G = D / kSlab;
  const int f = fb * 64 + wave * 16 + (lane & 15);
  const size_t rg = (size_t)tl.e * 2 * F + f;  // gate row; up row is rg + F
  const uint8_t* wg = static_cast<const uint8_t*>(a.w_gate_up) + rg * (D / 2) + (lane >> 4) * 16;
  const uint8_t* wu = wg + (size_t)F * (D / 2);
  const uint16_t* sg = a.s_gate_up + rg * G;
  const uint16_t* su = sg + (size_t)F * G;

  f32x4 accg[kBMT], accu[kBMT];
#pragma unroll
  for (int i = 0; i < kBMT; ++i) {
    accg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  u32x4 ra[kAPass];
  load_a(src, 0, seg, D, ra);
  u32x4 qg = ld_stream(reinterpret_cast<const u32x4*>(wg));
  u32x4 qu = ld_stream(reinterpret_cast<const u32x4*>(wu));
  uint16_t scg = ld_stream(sg), scu = ld_stream(su);
  store_a(As[0], src, tid, ra);
  __syncthreads();

  for (int it = 0; it < G; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < G;
    u32x4 qgn, qun;
    uint16_t scgn = 0, scun = 0;
    if (more) {
      const int k1 = (it + 1) * kSlab;
      load_a(src, k1, seg, D, ra);
      qgn = ld_stream(reinterpret_cast<const u32x4*>(wg + (size_t)(it + 1) * (kSlab / 2)));
      qun = ld_stream(reinterpret_cast<const u32x4*>(wu + (size_t)(it + 1) * (kSlab / 2)));
      scgn = ld_stream(sg + it + 1);
      scun = ld_stream(su + it + 1);
    }
    f16x8 bg[4], bu[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bg[s] = dequant8(qg[s]);
      bu[s] = dequant8(qu[s]);
    }
    const float fsg = half_bits(scg), fsu = half_bits(scu);
    const uint16_t* Ab = As[cur];
#pragma unroll
    for (int mt = 0; mt < kBMT; ++mt) {
      if (mt < nmt) {
        f32x4 tg = f32x4{0.f, 0.f, 0.f, 0.f}, tu = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f16x8 av = as_f16x8(
              *reinterpret_cast<const u32x4*>(Ab + (mt * 16 + (lane & 15)) * kPitch + (lane >> 4) * 32 + s * 8));
          tg = mfma_f16(av, bg[s], tg);
          tu = mfma_f16(av, bu[s], tu);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accg[mt][i] += fsg * tg[i];
          accu[mt][i] += fsu * tu[i];
        }
      }
    }
    if (more) {
      store_a(As[cur ^ 1], src, tid, ra);
      qg = qgn; qu = qun; scg = scgn; scu = scun;
    }
    __syncthreads();
  }

  uint16_t* out = a.act + (size_t)tl.row0 * F + f;
#pragma unroll
  for (int mt = 0; mt < kBMT; ++mt) {
    if (mt < nmt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + (lane >> 4) * 4 + i;
        if (r < tl.mc) {
          const _Float16 v = (_Float16)(gelu_tanh(accg[mt][i]) * accu[mt][i]);
          out[(size_t)r * F] = __builtin_bit_cast(uint16_t, v);
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_down_i4(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTileRows * kPitch];
  const int F = a.F, D = a.D;
  const int qx = blockIdx.x & (kQueues - 1);
  const int jq = blockIdx.x / kQueues;
  if (jq >= a.qlen[qx]) return;
  const Tile tl = a.tiles[(size_t)qx * a.qmax + jq];
  const int nb = tl.nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nmt = (tl.mc + 15) >> 4;
  const int seg = tid & 15;
  const int g = lane >> 4;

  const uint16_t* src[kAPass];
#pragma unroll
  for (int p = 0; p < kAPass; ++p) {
    const int r = (tid >> 4) + 16 * p;
    src[p] = (r < tl.mc) ? a.act + (size_t)(tl.row0 + r) * F + seg * 8 : nullptr;
  }
  const int G = (F + kSlab - 1) / kSlab;
  const int d0 = nb * 128 + wave * 32 + (lane & 15);
  const size_t r0 = (size_t)tl.e * D + d0;  // second row is r0 + 16
  const uint8_t* w0 = static_cast<const uint8_t*>(a.w_down) + r0 * (F / 2) + g * 16;
  const uint8_t* w1 = w0 + (size_t)16 * (F / 2);
  const uint16_t* s0 = a.s_down + r0 * G;
  const uint16_t* s1 = s0 + (size_t)16 * G;

  f32x4 acc0[kBMT], acc1[kBMT];
#pragma unroll
  for (int i = 0; i < kBMT; ++i) {
    acc0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // code 8 stands for 0: lanes whose 32 inputs lie past d_ff (the short last
  // group) feed exact zeros
  const u32x4 zero4 = u32x4{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
  u32x4 ra[kAPass];
  load_a(src, 0, seg, F, ra);
  u32x4 q0 = (g * 32 < F) ? ld_stream(reinterpret_cast<const u32x4*>(w0)) : zero4;
  u32x4 q1 = (g * 32 < F) ? ld_stream(reinterpret_cast<const u32x4*>(w1)) : zero4;
  uint16_t sc0 = ld_stream(s0), sc1 = ld_stream(s1);
  store_a(As[0], src, tid, ra);
  __syncthreads();

  for (int it = 0; it < G; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < G;
    u32x4 q0n = zero4, q1n = zero4;
    uint16_t sc0n = 0, sc1n = 0;
    if (more) {
      const int k1 = (it + 1) * kSlab;
      load_a(src, k1, seg, F, ra);
      if (k1 + g * 32 < F) {
        q0n = ld_stream(reinterpret_cast<const u32x4*>(w0 + (size_t)(it + 1) * (kSlab / 2)));
        q1n = ld_stream(reinterpret_cast<const u32x4*>(w1 + (size_t)(it + 1) * (kSlab / 2)));
      }
      sc0n = ld_stream(s0 + it + 1);
      sc1n = ld_stream(s1 + it + 1);
    }
    f16x8 b0[4], b1[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      b0[s] = dequant8(q0[s]);
      b1[s] = dequant8(q1[s]);
    }
    const float f0 = half_bits(sc0), f1 = half_bits(sc1);
    const uint16_t* Ab = As[cur];
#pragma unroll
    for (int mt = 0; mt < kBMT; ++mt) {
      if (mt < nmt) {
        f32x4 t0 = f32x4{0.f, 0.f, 0.f, 0.f}, t1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const f16x8 av = as_f16x8(
              *reinterpret_cast<const u32x4*>(Ab + (mt * 16 + (lane & 15)) * kPitch + g * 32 + s * 8));
          t0 = mfma_f16(av, b0[s], t0);
          t1 = mfma_f16(av, b1[s], t1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc0[mt][i] += f0 * t0[i];
          acc1[mt][i] += f1 * t1[i];
        }
      }
    }
    if (more) {
      store_a(As[cur ^ 1], src, tid, ra);
      q0 = q0n; q1 = q1n; sc0 = sc0n; sc1 = sc1n;
    }
    __syncthreads();
  }

#pragma unroll
  for (int mt = 0; mt < kBMT; ++mt) {
    if (mt < nmt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + g * 4 + i;
        if (r < tl.mc) {
          uint16_t* yr = a.y + (size_t)(tl.row0 + r) * D + d0;
          yr[0] = f32_to_bf16_bits(acc0[mt][i]);
          yr[16] = f32_to_bf16_bits(acc1[mt][i]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Packed layout (create-time): codes in MFMA fragment order, 1 KB block per
// (expert e, 16-row panel p, group gi); lane l = n + 16 g of the block holds
// 16 bytes for row 16 p + n: dword s carries the 8 codes of inputs
// 128 gi + 32 s + 8 g .. + 7, nibble-ordered so that the exact widening below
// yields them in natural order (nibble i holds input 2 i for i < 4 and
// input 2 (i - 4) + 1 for i >= 4). Inputs past K (the short last group) get
// code 8, which stands for 0. Scales: those of the two panels one task reads
// (gate_up: panel q and q + F/16, gate and up; down: panels 2 q and 2 q + 1)
// side by side, 16 rows x 2 fp16 per (e, pair q, gi), so a lane loads both of
// its row's scales of a group as one dword.
// So a wave reads one weight fragment as 1 KB contiguous, and the activation
// fragments are exactly the bf16 kernels' (same LDS layout and DMA).

// (a & mask) | 0x64006400 in one three-input bitwise operation (truth table
// 0xEA: (A & B) | C).
__device__ __forceinline__ uint32_t nib_pair(uint32_t a) {
  return __builtin_amdgcn_bitop3_b32(a, 0x000F000Fu, 0x64006400u, 0xEA);
}

// 8 codes of the packed order -> 8 fp16 values (q - 8) in natural order.
__device__ __forceinline__ f16x8 dequant8n(uint32_t v) {
  const f16x2 bias = f16x2{(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2 p0 = __builtin_bit_cast(f16x2, nib_pair(v)) + bias;        // k0 k1
  const f16x2 p1 = __builtin_bit_cast(f16x2, nib_pair(v >> 4)) + bias;   // k2 k3
  const f16x2 p2 = __builtin_bit_cast(f16x2, nib_pair(v >> 8)) + bias;   // k4 k5
  const f16x2 p3 = __builtin_bit_cast(f16x2, nib_pair(v >> 12)) + bias;  // k6 k7
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// One thread per (block, lane).
// pair_stride: panels between the two panels of a pair (R / 32 for gate_up,
// whose pairs are gate panel q and up panel q; 1 for down, panels 2 q, 2 q + 1).
__global__ __launch_bounds__(256) void k_pack_i4(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                                 uint8_t* __restrict__ pcodes, uint16_t* __restrict__ pscales, int E,
                                                 int R, int K, int pair_stride) {
  const int G = (K + 127) / 128, NP = R / 16;
  const size_t nblk = (size_t)E * NP * G;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  for (size_t b = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6); b < nblk; b += (size_t)gridDim.x * 4) {
    const int gi = (int)(b % G);
    const size_t ep = b / G;  // e * NP + p
    const size_t row = (ep / NP) * R + (ep % NP) * 16 + n;
    const uint8_t* src = codes + row * (K / 2);
    u32x4 o;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = 128 * gi + 32 * s + 8 * g + j;
        c[j] = (k < K) ? ((src[k >> 1] >> ((k & 1) * 4)) & 0xFu) : 8u;
      }
      o[s] = c[0] | (c[2] << 4) | (c[4] << 8) | (c[6] << 12) | (c[1] << 16) | (c[3] << 20) | (c[5] << 24) |
             (c[7] << 28);
    }
    *reinterpret_cast<u32x4*>(pcodes + (b * 64 + lane) * 16) = o;
    if (g == 0) {
      const int p = (int)(ep % NP);
      const int pair = pair_stride == 1 ? p >> 1 : (p < pair_stride ? p : p - pair_stride);
      const int slot = pair_stride == 1 ? p & 1 : (p < pair_stride ? 0 : 1);
      pscales[((((ep / NP) * (NP / 2) + pair) * G + gi) * 16 + n) * 2 + slot] = scales[row * G + gi];
    }
  }
}

// Weights of one group for this lane: codes of both panels and their two
// scales (fp16, first panel's in the low half).
struct WGroup {
  u32x4 c0, c1;
  uint32_t s;
};

// NT: past the caches (an expert in one tile reads its weights once); else
// normal loads, so that the expert's other tiles find them in L2.
// Three loads per group: the scale pair as one dword (two 2-byte loads, one
// per panel, had cost the T = 256 launch 7 us: 87 against 80 us).
template <bool NT>
__device__ __forceinline__ void load_wg(const uint8_t* c0, const uint8_t* c1, const uint32_t* sp, int gi, WGroup& w) {
  if constexpr (NT) {
    w.c0 = ld_stream(reinterpret_cast<const u32x4*>(c0 + (size_t)gi * 1024));
    w.c1 = ld_stream(reinterpret_cast<const u32x4*>(c1 + (size_t)gi * 1024));
    w.s = ld_stream(sp + gi * 16);
  } else {
    w.c0 = *reinterpret_cast<const u32x4*>(c0 + (size_t)gi * 1024);
    w.c1 = *reinterpret_cast<const u32x4*>(c1 + (size_t)gi * 1024);
    w.s = sp[gi * 16];
  }
}

// One group's MFMAs: partial sums over the 128 inputs in t, then scaled into acc.
template <int NMT, int MB>
__device__ __forceinline__ void mma_i4(const char* stage, int lane, const WGroup& w, f32x4 (&acc0)[MB],
                                       f32x4 (&acc1)[MB]) {
  const int g = lane >> 4, m = lane & 15;
  f32x4 t0[MB], t1[MB];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    t0[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    t1[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < kNS; ++s) {
    const f16x8 b0 = dequant8n(w.c0[s]);
    const f16x8 b1 = dequant8n(w.c1[s]);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int r = mt * 16 + m;
      const int pos = (s * 4 + g) ^ (r % kSegs);
      const f16x8 av = as_f16x8(*reinterpret_cast<const u32x4*>(stage + r * kRowBytes + pos * 16));
      t0[mt] = mfma_f16(av, b0, t0[mt]);
      t1[mt] = mfma_f16(av, b1, t1[mt]);
    }
    __builtin_amdgcn_sched_barrier(0);  // widen one sub-step's codes at a time
  }
  const float f0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.s & 0xffffu));
  const float f1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w.s >> 16));
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc0[mt][i] = fmaf(f0, t0[mt][i], acc0[mt][i]);
      acc1[mt][i] = fmaf(f1, t1[mt][i], acc1[mt][i]);
    }
}

constexpr int kDepthI4 = 3;  // LDS stages and weight buffers; step i + 2 is issued during step i

// The packed kernels' tile heights: 64 rows, or 32 where experts hold few rows
// (half the registers for the sums, so three workgroups share a CU).
template <int ROWS>
struct I4Tile {
  static constexpr int kMB = ROWS / 16;                       // m-tiles
  static constexpr int kStage = ROWS * kRowBytes;             // bytes of one LDS stage
  static constexpr int kNI = dma_per_wave(ROWS, kWaves);      // activation transfers per wave
};

template <int ROWS, int NMT, bool NT>
__device__ __forceinline__ void issue_i4(char* As, const uint16_t* const (&rowp)[I4Tile<ROWS>::kNI], const uint8_t* c0,
                                         const uint8_t* c1, const uint32_t* sp, int j, int K,
                                         int wave, int lane, WGroup& w) {
  char* st = As + (j % kDepthI4) * I4Tile<ROWS>::kStage;
  const int k0 = j * kKS;
  if (k0 + kKS <= K)
    dma_a<NMT, kSegs>(st, rowp, k0, wave, lane);
  else
    dma_a<NMT, kSegs / 2>(st, rowp, k0, wave, lane);
  __builtin_amdgcn_sched_barrier(0);
  load_wg<NT>(c0, c1, sp, j, w);
  __builtin_amdgcn_sched_barrier(0);
}

// Step i: wait until step i's transfers have landed (those of step i + 1,
// NMT DMA transfers and 3 weight loads, may still fly; WAIT = 0 for the last
// step), publish, issue step i + 2, multiply step i.
template <int ROWS, int NMT, bool NT, bool ISSUE, int WAIT>
__device__ __forceinline__ void step_i4(char* As, const uint16_t* const (&rowp)[I4Tile<ROWS>::kNI], const uint8_t* c0,
                                        const uint8_t* c1, const uint32_t* sp, int i, int K,
                                        int wave, int lane, const WGroup& wb, WGroup& wn2,
                                        f32x4 (&acc0)[I4Tile<ROWS>::kMB], f32x4 (&acc1)[I4Tile<ROWS>::kMB]) {
  wait_vmcnt<WAIT>();
  lds_barrier();
  if (ISSUE) issue_i4<ROWS, NMT, NT>(As, rowp, c0, c1, sp, i + 2, K, wave, lane, wn2);
  mma_i4<NMT>(As + (i % kDepthI4) * I4Tile<ROWS>::kStage, lane, wb, acc0, acc1);
}

// The group loop: unrolled by three (one weight buffer per position), the last
// two to four groups written out so that every wait count is exact.
template <int ROWS, int NMT, bool NT>
__device__ __forceinline__ void loop_i4(char* As, const uint16_t* const (&rowp)[I4Tile<ROWS>::kNI], const uint8_t* c0,
                                        const uint8_t* c1, const uint32_t* sp, int K, int tid,
                                        f32x4 (&acc0)[I4Tile<ROWS>::kMB], f32x4 (&acc1)[I4Tile<ROWS>::kMB]) {
  constexpr int kW = NMT + 3;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = (K + kKS - 1) / kKS;
  WGroup w0, w1, w2;
  issue_i4<ROWS, NMT, NT>(As, rowp, c0, c1, sp, 0, K, wave, lane, w0);
  if (n == 1) {
    step_i4<ROWS, NMT, NT, false, 0>(As, rowp, c0, c1, sp, 0, K, wave, lane, w0, w2, acc0, acc1);
    return;
  }
  issue_i4<ROWS, NMT, NT>(As, rowp, c0, c1, sp, 1, K, wave, lane, w1);
  int i = 0;
  for (; i + 5 <= n; i += 3) {
    step_i4<ROWS, NMT, NT, true, kW>(As, rowp, c0, c1, sp, i, K, wave, lane, w0, w2, acc0, acc1);
    step_i4<ROWS, NMT, NT, true, kW>(As, rowp, c0, c1, sp, i + 1, K, wave, lane, w1, w0, acc0, acc1);
    step_i4<ROWS, NMT, NT, true, kW>(As, rowp, c0, c1, sp, i + 2, K, wave, lane, w2, w1, acc0, acc1);
  }
  switch (n - i) {
    case 2:
      step_i4<ROWS, NMT, NT, false, kW>(As, rowp, c0, c1, sp, i, K, wave, lane, w0, w2, acc0, acc1);
      step_i4<ROWS, NMT, NT, false, 0>(As, rowp, c0, c1, sp, i + 1, K, wave, lane, w1, w0, acc0, acc1);
      break;
    case 3:
      step_i4<ROWS, NMT, NT, true, kW>(As, rowp, c0, c1, sp, i, K, wave, lane, w0, w2, acc0, acc1);
      step_i4<ROWS, NMT, NT, false, kW>(As, rowp, c0, c1, sp, i + 1, K, wave, lane, w1, w0, acc0, acc1);
      step_i4<ROWS, NMT, NT, false, 0>(As, rowp, c0, c1, sp, i + 2, K, wave, lane, w2, w1, acc0, acc1);
      break;
    default:  // 4
      step_i4<ROWS, NMT, NT, true, kW>(As, rowp, c0, c1, sp, i, K, wave, lane, w0, w2, acc0, acc1);
      step_i4<ROWS, NMT, NT, true, kW>(As, rowp, c0, c1, sp, i + 1, K, wave, lane, w1, w0, acc0, acc1);
      step_i4<ROWS, NMT, NT, false, kW>(As, rowp, c0, c1, sp, i + 2, K, wave, lane, w2, w1, acc0, acc1);
      step_i4<ROWS, NMT, NT, false, 0>(As, rowp, c0, c1, sp, i + 3, K, wave, lane, w0, w2, acc0, acc1);
      break;
  }
}

// Packed-weight grouped GEMMs: the bf16 kernels' mapping and activation path,
// int4 weights widened exactly to fp16 in registers. gate_up writes the gated
// activation as fp16, down its fp32 sums as bf16.
template <bool GATE_UP, int ROWS, bool NT>
__device__ __forceinline__ void i4p_body(const GemmArgs& a, const Tile& tl, char* As) {
  constexpr int MB = I4Tile<ROWS>::kMB, NI = I4Tile<ROWS>::kNI;
  const int F = a.F, D = a.D;
  const int K = GATE_UP ? D : F;
  const int G = (K + kKS - 1) / kKS;
  const int nb = tl.nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4;
  const int nmt = (tl.mc + 15) >> 4;

  const uint16_t* rowp[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = min(kDmaRows * (wave + kWaves * i) + lane / kSegs, tl.mc - 1);
    rowp[i] = GATE_UP ? a.h + (size_t)(a.sorted_slot[tl.row0 + r] / a.K) * D : a.act + (size_t)(tl.row0 + r) * F;
  }
  int col, p0, p1, NP;
  if (GATE_UP) {
    col = nb * 16 * kWaves + wave * 16 + (lane & 15);
    NP = 2 * F / 16;
    p0 = nb * kWaves + wave;
    p1 = p0 + F / 16;
  } else {
    col = nb * 32 * kWaves + wave * 32 + (lane & 15);
    NP = D / 16;
    p0 = 2 * (nb * kWaves + wave);
    p1 = p0 + 1;
  }
  const uint8_t* C = static_cast<const uint8_t*>(GATE_UP ? a.w_gate_up : a.w_down);
  const uint32_t* S = reinterpret_cast<const uint32_t*>(GATE_UP ? a.s_gate_up : a.s_down);
  const size_t b0 = ((size_t)tl.e * NP + p0) * G, b1 = ((size_t)tl.e * NP + p1) * G;
  const uint8_t* c0 = C + b0 * 1024 + lane * 16;
  const uint8_t* c1 = C + b1 * 1024 + lane * 16;
  // the scale pair of panels p0, p1 (pair nb * kWaves + wave in both GEMMs)
  const uint32_t* sp = S + ((size_t)tl.e * (NP / 2) + nb * kWaves + wave) * G * 16 + (lane & 15);

  f32x4 acc0[MB], acc1[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    acc0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (MB == 2) {
    if (nmt == 1)
      loop_i4<ROWS, 1, NT>(As, rowp, c0, c1, sp, K, tid, acc0, acc1);
    else
      loop_i4<ROWS, 2, NT>(As, rowp, c0, c1, sp, K, tid, acc0, acc1);
  } else {
    switch (nmt) {
      case 1: loop_i4<ROWS, 1, NT>(As, rowp, c0, c1, sp, K, tid, acc0, acc1); break;
      case 2: loop_i4<ROWS, 2, NT>(As, rowp, c0, c1, sp, K, tid, acc0, acc1); break;
      case 3: loop_i4<ROWS, 3, NT>(As, rowp, c0, c1, sp, K, tid, acc0, acc1); break;
      default: loop_i4<ROWS, 4, NT>(As, rowp, c0, c1, sp, K, tid, acc0, acc1); break;
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
__device__ __forceinline__ void i4p_task(const FusedGemmArgs& f, const GemmArgs& a, const Tile& tl, char* As) {
  if ((f.counts[tl.e] + ROWS - 1) / ROWS > 1)
    i4p_body<GATE_UP, ROWS, false>(a, tl, As);
  else
    i4p_body<GATE_UP, ROWS, true>(a, tl, As);
}

// Both packed GEMMs in one launch (the task logic of fused_tasks): 64-row
// tiles at two workgroups per CU, or 32-row tiles at three.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_i4p_fused(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[kDepthI4 * I4Tile<kTileRows>::kStage];
  fused_tasks(
      f, [&](const Tile& tl) { i4p_task<true, kTileRows>(f, f.gu, tl, As); },
      [&](const Tile& tl) { i4p_task<false, kTileRows>(f, f.dn, tl, As); });
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_gemm_i4p_fused_short(
    FusedGemmArgs f) {
  __shared__ __attribute__((aligned(16))) char As[kDepthI4 * I4Tile<kShortRows>::kStage];
  fused_tasks(
      f, [&](const Tile& tl) { i4p_task<true, kShortRows>(f, f.gu, tl, As); },
      [&](const Tile& tl) { i4p_task<false, kShortRows>(f, f.dn, tl, As); });
}

}  // namespace

hipError_t launch_pack_i4(const uint8_t* codes, const uint16_t* scales, uint8_t* pcodes, uint16_t* pscales, int E,
                          int R, int K, int pair_stride, hipStream_t stream) {
  k_pack_i4<<<dim3(4096), dim3(256), 0, stream>>>(codes, scales, pcodes, pscales, E, R, K, pair_stride);
  return hipGetLastError();
}

hipError_t launch_gate_up_i4(const GemmArgs& a, hipStream_t stream, const KernelEvents* ev) {
  return launch_kernel(k_gate_up_i4, dim3(kQueues * a.qmax), dim3(kThreads), stream, ev, a);
}

hipError_t launch_down_i4(const GemmArgs& a, hipStream_t stream, const KernelEvents* ev) {
  return launch_kernel(k_down_i4, dim3(kQueues * a.qmax), dim3(kThreads), stream, ev, a);
}

hipError_t launch_gemm_fused_i4(const FusedGemmArgs& f, int tile_rows, hipStream_t stream, const KernelEvents* ev) {
  return launch_kernel(tile_rows == kShortRows ? k_gemm_i4p_fused_short : k_gemm_i4p_fused,
                       dim3(kQueues * (f.gu.qmax + f.dn.qmax)), dim3(kThreads), stream, ev, f);
}

}  // namespace dg
