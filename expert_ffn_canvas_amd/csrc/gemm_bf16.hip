// Grouped expert GEMMs on gfx950 bf16 matrix cores (fp32 accumulation).
//
//  gate_up: for each tile (expert e, rows row0 .. row0+mc-1) and each block of
//           64 d_ff features: g = h W_gate[e]^T, u = h W_up[e]^T over the full
//           d_model, then act = gelu_tanh(g) * u (bf16).
//  down:    for each tile and each block of 128 d_model outputs:
//           y = row_w * (act W_down[e]^T) in fp32, one row per routed slot.
//
// Shapes (auto-round PR "Add quantization support for DiffusionGemma",
// transformers backend test log, expert module dump): gate_proj and up_proj
// are Linear(2816 -> 704), down_proj is Linear(704 -> 2816), no bias; the
// activation is GELUTanh. The fused gate_up tensor is [E, 2F, D] with the
// gate rows first (Quant-Tuner PR, "Answers to the motivating questions",
// names the fused 3D gate_up projection; the row order is this library's).
//
// Mapping: one workgroup = 4 waves = one (tile, column block). Each wave owns
// 16 output columns of each operand it needs (gate+up, or two down tiles)
// for every row of the tile, so every weight byte is read from HBM by exactly
// one wave and goes straight from global memory into MFMA operand registers.
// The tile's activation rows are shared by the 4 waves through LDS
// (double-buffered along K). Weights for the next K step are loaded while the
// current step's MFMAs run.
#include "dg_common.h"
#include "launch.h"

namespace dg {

namespace {

constexpr int kThreads = 256;
constexpr int kKStep = 64;               // K per pipeline step
constexpr int kPitch = kKStep + 8;       // LDS row pitch in 16-bit elements (144 B)
constexpr int kBMT = kTileRows / 16;     // m-tiles per tile
constexpr int kAPass = kTileRows / 32;   // 256 threads stage 32 rows x 64 K per pass

// Stage rows [0, mc) of a tile's K step into LDS. Thread (row r = tid/8 + 32 p,
// 16-byte segment tid % 8). `src[p]` is null for rows past mc.
__device__ __forceinline__ void load_a(const uint16_t* const (&src)[kAPass], int k0, u32x4 (&ra)[kAPass]) {
#pragma unroll
  for (int p = 0; p < kAPass; ++p)
    if (src[p]) ra[p] = *reinterpret_cast<const u32x4*>(src[p] + k0);
}

__device__ __forceinline__ void store_a(uint16_t* lds, const uint16_t* const (&src)[kAPass], int tid,
                                        const u32x4 (&ra)[kAPass]) {
#pragma unroll
  for (int p = 0; p < kAPass; ++p)
    if (src[p]) *reinterpret_cast<u32x4*>(lds + ((tid >> 3) + 32 * p) * kPitch + (tid & 7) * 8) = ra[p];
}

__global__ __launch_bounds__(kThreads) void k_gate_up_bf16(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTileRows * kPitch];
  const int F = a.F, D = a.D;
  const int NB = F / 64;
  const int ti = blockIdx.x / NB;
  const int fb = blockIdx.x - ti * NB;
  if (ti >= *a.n_tiles) return;
  const Tile tl = a.tiles[ti];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nmt = (tl.mc + 15) >> 4;

  const uint16_t* src[kAPass];
#pragma unroll
  for (int p = 0; p < kAPass; ++p) {
    const int r = (tid >> 3) + 32 * p;
    src[p] = (r < tl.mc) ? a.h + (size_t)a.sorted_token[tl.row0 + r] * D + (tid & 7) * 8 : nullptr;
  }
  const int f = fb * 64 + wave * 16 + (lane & 15);
  const uint16_t* wg = static_cast<const uint16_t*>(a.w_gate_up) + ((size_t)tl.e * 2 * F + f) * D + (lane >> 4) * 8;
  const uint16_t* wu = wg + (size_t)F * D;

  f32x4 accg[kBMT], accu[kBMT];
#pragma unroll
  for (int i = 0; i < kBMT; ++i) {
    accg[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    accu[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  u32x4 ra[kAPass];
  u32x4 wgc[2], wuc[2], wgn[2], wun[2];
  load_a(src, 0, ra);
  wgc[0] = *reinterpret_cast<const u32x4*>(wg);
  wgc[1] = *reinterpret_cast<const u32x4*>(wg + 32);
  wuc[0] = *reinterpret_cast<const u32x4*>(wu);
  wuc[1] = *reinterpret_cast<const u32x4*>(wu + 32);
  store_a(As[0], src, tid, ra);
  __syncthreads();

  const int nk = D / kKStep;
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nk;
    if (more) {
      const int k1 = (it + 1) * kKStep;
      load_a(src, k1, ra);
      wgn[0] = *reinterpret_cast<const u32x4*>(wg + k1);
      wgn[1] = *reinterpret_cast<const u32x4*>(wg + k1 + 32);
      wun[0] = *reinterpret_cast<const u32x4*>(wu + k1);
      wun[1] = *reinterpret_cast<const u32x4*>(wu + k1 + 32);
    }
    const uint16_t* Ab = As[cur];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 bg = as_bf16x8(wgc[ks]);
      const bf16x8 bu = as_bf16x8(wuc[ks]);
#pragma unroll
      for (int mt = 0; mt < kBMT; ++mt) {
        if (mt < nmt) {
          const bf16x8 av = as_bf16x8(
              *reinterpret_cast<const u32x4*>(Ab + (mt * 16 + (lane & 15)) * kPitch + ks * 32 + (lane >> 4) * 8));
          accg[mt] = mfma_bf16(av, bg, accg[mt]);
          accu[mt] = mfma_bf16(av, bu, accu[mt]);
        }
      }
    }
    if (more) {
      store_a(As[cur ^ 1], src, tid, ra);
      wgc[0] = wgn[0]; wgc[1] = wgn[1];
      wuc[0] = wun[0]; wuc[1] = wun[1];
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
        if (r < tl.mc) out[(size_t)r * F] = f32_to_bf16_bits(gelu_tanh(accg[mt][i]) * accu[mt][i]);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_down_bf16(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kTileRows * kPitch];
  const int F = a.F, D = a.D;
  const int NB = D / 128;
  const int ti = blockIdx.x / NB;
  const int nb = blockIdx.x - ti * NB;
  if (ti >= *a.n_tiles) return;
  const Tile tl = a.tiles[ti];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nmt = (tl.mc + 15) >> 4;

  const uint16_t* src[kAPass];
#pragma unroll
  for (int p = 0; p < kAPass; ++p) {
    const int r = (tid >> 3) + 32 * p;
    src[p] = (r < tl.mc) ? a.act + (size_t)(tl.row0 + r) * F + (tid & 7) * 8 : nullptr;
  }
  const int d0 = nb * 128 + wave * 32 + (lane & 15);
  const uint16_t* w0 = static_cast<const uint16_t*>(a.w_down) + ((size_t)tl.e * D + d0) * F + (lane >> 4) * 8;
  const uint16_t* w1 = w0 + (size_t)16 * F;

  f32x4 acc0[kBMT], acc1[kBMT];
#pragma unroll
  for (int i = 0; i < kBMT; ++i) {
    acc0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  u32x4 ra[kAPass];
  u32x4 b0c[2], b1c[2], b0n[2], b1n[2];
  load_a(src, 0, ra);
  b0c[0] = *reinterpret_cast<const u32x4*>(w0);
  b0c[1] = *reinterpret_cast<const u32x4*>(w0 + 32);
  b1c[0] = *reinterpret_cast<const u32x4*>(w1);
  b1c[1] = *reinterpret_cast<const u32x4*>(w1 + 32);
  store_a(As[0], src, tid, ra);
  __syncthreads();

  const int nk = F / kKStep;
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nk;
    if (more) {
      const int k1 = (it + 1) * kKStep;
      load_a(src, k1, ra);
      b0n[0] = *reinterpret_cast<const u32x4*>(w0 + k1);
      b0n[1] = *reinterpret_cast<const u32x4*>(w0 + k1 + 32);
      b1n[0] = *reinterpret_cast<const u32x4*>(w1 + k1);
      b1n[1] = *reinterpret_cast<const u32x4*>(w1 + k1 + 32);
    }
    const uint16_t* Ab = As[cur];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 bb0 = as_bf16x8(b0c[ks]);
      const bf16x8 bb1 = as_bf16x8(b1c[ks]);
#pragma unroll
      for (int mt = 0; mt < kBMT; ++mt) {
        if (mt < nmt) {
          const bf16x8 av = as_bf16x8(
              *reinterpret_cast<const u32x4*>(Ab + (mt * 16 + (lane & 15)) * kPitch + ks * 32 + (lane >> 4) * 8));
          acc0[mt] = mfma_bf16(av, bb0, acc0[mt]);
          acc1[mt] = mfma_bf16(av, bb1, acc1[mt]);
        }
      }
    }
    if (more) {
      store_a(As[cur ^ 1], src, tid, ra);
      b0c[0] = b0n[0]; b0c[1] = b0n[1];
      b1c[0] = b1n[0]; b1c[1] = b1n[1];
    }
    __syncthreads();
  }

#pragma unroll
  for (int mt = 0; mt < kBMT; ++mt) {
    if (mt < nmt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + (lane >> 4) * 4 + i;
        if (r < tl.mc) {
          const float w = a.row_w[tl.row0 + r];
          float* yr = a.y + (size_t)(tl.row0 + r) * D + d0;
          yr[0] = w * acc0[mt][i];
          yr[16] = w * acc1[mt][i];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gate_up_bf16(const GemmArgs& a, hipStream_t stream) {
  k_gate_up_bf16<<<dim3(a.max_tiles * (a.F / 64)), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_bf16(const GemmArgs& a, hipStream_t stream) {
  k_down_bf16<<<dim3(a.max_tiles * (a.D / 128)), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace dg
