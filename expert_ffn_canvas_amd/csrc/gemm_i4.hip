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
#include "launch.h"

namespace dg {

namespace {

constexpr int kThreads = 256;
constexpr int kSlab = 128;              // inputs per scale group = K per step
constexpr int kPitch = kSlab + 8;       // LDS row pitch in fp16 elements
constexpr int kBMT = kTileRows / 16;
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
  const Tile tl = a.tiles[(size_t)jq * kQueues + qx];
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
  u32x4 qg = *reinterpret_cast<const u32x4*>(wg);
  u32x4 qu = *reinterpret_cast<const u32x4*>(wu);
  uint16_t scg = sg[0], scu = su[0];
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
      qgn = *reinterpret_cast<const u32x4*>(wg + (size_t)(it + 1) * (kSlab / 2));
      qun = *reinterpret_cast<const u32x4*>(wu + (size_t)(it + 1) * (kSlab / 2));
      scgn = sg[it + 1];
      scun = su[it + 1];
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
  const Tile tl = a.tiles[(size_t)jq * kQueues + qx];
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
  u32x4 q0 = (g * 32 < F) ? *reinterpret_cast<const u32x4*>(w0) : zero4;
  u32x4 q1 = (g * 32 < F) ? *reinterpret_cast<const u32x4*>(w1) : zero4;
  uint16_t sc0 = s0[0], sc1 = s1[0];
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
        q0n = *reinterpret_cast<const u32x4*>(w0 + (size_t)(it + 1) * (kSlab / 2));
        q1n = *reinterpret_cast<const u32x4*>(w1 + (size_t)(it + 1) * (kSlab / 2));
      }
      sc0n = s0[it + 1];
      sc1n = s1[it + 1];
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

}  // namespace

hipError_t launch_gate_up_i4(const GemmArgs& a, hipStream_t stream, const KernelEvents* ev) {
  return launch_kernel(k_gate_up_i4, dim3(kQueues * a.qmax), dim3(kThreads), stream, ev, a);
}

hipError_t launch_down_i4(const GemmArgs& a, hipStream_t stream, const KernelEvents* ev) {
  return launch_kernel(k_down_i4, dim3(kQueues * a.qmax), dim3(kThreads), stream, ev, a);
}

}  // namespace dg
