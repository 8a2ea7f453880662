// Router of the MoE layer on gfx950, in three short kernels:
//
//  norm:   per token, r = 1/sqrt(mean x^2 + eps); the expert input
//          h = x r (1 + gamma_e) (bf16, or fp16 for int4 experts); and the
//          router input z = x r (1 + gamma_r) in fp32, stored as three exact
//          bf16 planes z = z0 + z1 + z2 (each plane holds the next 8
//          significant bits of the fp32 value).
//  logits: [T, E] = z W_r^T on the bf16 matrix cores. Each bf16 x bf16
//          product is exact in fp32 and the MFMA accumulates in fp32, so with
//          z in three planes (and an fp32 router weight split the same way at
//          create time) the logits have fp32 dot-product accuracy.
//  top-k:  per token, the k largest logits + bias (ties: lower expert id),
//          their softmax renormalised over the k, slots ordered by logit.
//
// Sources: Quant-Tuner PR "Add DiffusionGemma (Gemma-4 MoE block-diffusion)
// support", "Answers to the motivating questions" (the router reads the raw
// residual through its own norm; pre_feedforward_layernorm_2 with the (1+gamma)
// convention feeds the fused gate_up); 128 experts / 8 active from its Summary.
#include "dg_common.h"
#include "launch.h"

namespace dg {

namespace {

constexpr int kTokTile = 16;       // tokens per logits workgroup (MFMA M)
constexpr int kKChunk = 128;       // d_model columns staged per LDS round

__device__ __forceinline__ void split3(float z, uint16_t& b0, uint16_t& b1, uint16_t& b2) {
  b0 = f32_to_bf16_bits(z);
  const float r1 = z - bf16_bits_to_f32(b0);
  b1 = f32_to_bf16_bits(r1);
  const float r2 = r1 - bf16_bits_to_f32(b1);
  b2 = f32_to_bf16_bits(r2);
}

template <bool XF32>
__device__ __forceinline__ void load8(const void* x, size_t off, float (&v)[8]) {
  if (XF32) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(a[i]);
      v[2 * i + 1] = bf16_hi(a[i]);
    }
  }
}

// One workgroup of 256 threads per token; thread i owns the 8-column segments
// i, i + 256, ... (up to 8 of them, d_model <= 16384). All x loads of a thread
// are issued together, then one block reduction gives the RMS statistic.
template <bool XF32>
__global__ __launch_bounds__(256) void k_norm(RouterArgs a) {
  __shared__ float wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int D = a.D;
  const int nseg = D / 8;
  const size_t row = (size_t)t * D;
  float v[8][8];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sg = tid + 256 * i;
    if (sg < nseg) load8<XF32>(a.x, row + sg * 8, v[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sg = tid + 256 * i;
    if (sg < nseg)
#pragma unroll
      for (int k = 0; k < 8; ++k) ss += v[i][k] * v[i][k];
  }
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  if (lane == 0) wsum[wave] = ss;
  __syncthreads();
  const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float r = 1.0f / sqrtf(tot / (float)D + a.eps);
  const size_t plane = (size_t)a.T * D;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sg = tid + 256 * i;
    if (sg >= nseg) continue;
    const int c = sg * 8;
    const float4 gr0 = *reinterpret_cast<const float4*>(a.gamma_r + c);
    const float4 gr1 = *reinterpret_cast<const float4*>(a.gamma_r + c + 4);
    const float4 ge0 = *reinterpret_cast<const float4*>(a.gamma_e + c);
    const float4 ge1 = *reinterpret_cast<const float4*>(a.gamma_e + c + 4);
    const float gr[8] = {gr0.x, gr0.y, gr0.z, gr0.w, gr1.x, gr1.y, gr1.z, gr1.w};
    const float ge[8] = {ge0.x, ge0.y, ge0.z, ge0.w, ge1.x, ge1.y, ge1.z, ge1.w};
    uint16_t zb[3][8];
    float hv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float xr = v[i][k] * r;
      split3(xr * (1.0f + gr[k]), zb[0][k], zb[1][k], zb[2][k]);
      hv[k] = xr * (1.0f + ge[k]);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = (uint32_t)zb[p][2 * k] | ((uint32_t)zb[p][2 * k + 1] << 16);
      *reinterpret_cast<u32x4*>(a.z + p * plane + row + c) = o;
    }
    u32x4 ho;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      ho[k] = a.h_f16 ? pack_f16x2(hv[2 * k], hv[2 * k + 1]) : pack_bf16x2(hv[2 * k], hv[2 * k + 1]);
    *reinterpret_cast<u32x4*>(a.h + row + c) = ho;
  }
}

// Workgroup = 16 tokens x 16 experts, eight waves: wave h takes the 128-column
// chunks h, h + 8, ... of d_model and the eight partial sums are added through
// LDS in a fixed order. Both MFMA operands come straight from global memory
// (the z planes and the router weight are L2-resident); a wave has its first
// two chunks in flight before it multiplies the first.
constexpr int kLogitWaves = 8;

template <int NWP>
struct ZChunk {
  u32x4 z[4][3];
  u32x4 w[4][NWP];
};

template <int NWP>
__device__ __forceinline__ void load_chunk(const uint16_t* zr, size_t plane, const uint16_t* wrow, size_t wplane,
                                           int c, ZChunk<NWP>& ch) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int col = c * kKChunk + kk * 32;
#pragma unroll
    for (int p = 0; p < 3; ++p) ch.z[kk][p] = *reinterpret_cast<const u32x4*>(zr + p * plane + col);
#pragma unroll
    for (int p = 0; p < NWP; ++p) ch.w[kk][p] = *reinterpret_cast<const u32x4*>(wrow + p * wplane + col);
  }
}

template <int NWP>
__device__ __forceinline__ void mma_chunk(const ZChunk<NWP>& ch, f32x4& acc) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int zp = 0; zp < 3; ++zp)
#pragma unroll
      for (int p = 0; p < NWP; ++p) acc = mfma_bf16(as_bf16x8(ch.z[kk][zp]), as_bf16x8(ch.w[kk][p]), acc);
}

template <int NWP>
__global__ __launch_bounds__(64 * kLogitWaves) void k_logits(RouterArgs a) {
  __shared__ float part[kLogitWaves][kTokTile][17];
  const int tid = threadIdx.x, lane = tid & 63, kh = tid >> 6;
  const int n_et = a.Epad / 16;
  const int tt = blockIdx.x / n_et;
  const int et = blockIdx.x - tt * n_et;
  const int t0 = tt * kTokTile;
  const int D = a.D;
  const int m = lane & 15, g = lane >> 4;
  const int t = min(t0 + m, a.T - 1);  // rows past T re-read the last token; never stored
  const size_t plane = (size_t)a.T * D;
  const size_t wplane = (size_t)a.Epad * D;
  const uint16_t* zr = a.z + (size_t)t * D + g * 8;
  const uint16_t* wrow = a.wr + (size_t)(et * 16 + m) * D + g * 8;
  const int nc = D / kKChunk;
  const int n_my = (nc - kh + kLogitWaves - 1) / kLogitWaves;  // chunks kh, kh + 8, ...

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  ZChunk<NWP> cur, nxt;
  if (n_my > 0) {
    load_chunk<NWP>(zr, plane, wrow, wplane, kh, cur);
    for (int i = 0; i + 1 < n_my; ++i) {
      load_chunk<NWP>(zr, plane, wrow, wplane, kh + kLogitWaves * (i + 1), nxt);
      __builtin_amdgcn_sched_barrier(0);
      mma_chunk<NWP>(cur, acc);
      cur = nxt;
    }
    mma_chunk<NWP>(cur, acc);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[kh][g * 4 + i][m] = acc[i];
  __syncthreads();
  // [16 tokens x 16 experts]; the eight partial sums in a fixed order
  if (tid < kTokTile * 16) {
    const int mm = tid >> 4, n = tid & 15;
    float sum = part[0][mm][n];
#pragma unroll
    for (int w = 1; w < kLogitWaves; ++w) sum += part[w][mm][n];
    if (t0 + mm < a.T) a.logits[(size_t)(t0 + mm) * a.Epad + et * 16 + n] = sum;
  }
}

// One wave per token: k rounds of a wave-wide argmax over (logit desc, id asc).
__global__ __launch_bounds__(256) void k_topk(RouterArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int E = a.E, K = a.K;
  float v[4];
  bool taken[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = lane + 64 * u;
    float l = -INFINITY;
    if (e < E) l = a.logits[(size_t)t * a.Epad + e] + (a.bias ? a.bias[e] : 0.0f);
    v[u] = (l == l) ? l : -INFINITY;  // a NaN logit ranks last, so k valid ids are always chosen
    taken[u] = (e >= E);
  }
  float my_v = -INFINITY, vmax = 0.0f;
  int my_i = 0;
  for (int j = 0; j < K; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = lane + 64 * u;
      if (!taken[u] && (v[u] > bv || (v[u] == bv && e < bi))) { bv = v[u]; bi = e; }
    }
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (j == 0) vmax = bv;
    if (lane == j) { my_v = bv; my_i = bi; }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (bi == lane + 64 * u) taken[u] = true;
  }
  // softmax over the k selected logits (equal to the full softmax renormalised over them)
  const float ex = (lane < K) ? __expf(my_v - vmax) : 0.0f;
  float den = ex;
  for (int m = 32; m >= 1; m >>= 1) den += __shfl_xor(den, m);
  if (lane < K) {
    a.topk_idx[(size_t)t * K + lane] = my_i;
    a.topk_w[(size_t)t * K + lane] = ex / den;
  }
}

// Create-time: router weight [E, D] (fp32 or bf16) -> bf16 planes [P][Epad][D],
// rows e >= E zero. fp32 weights are split exactly into three planes.
__global__ void k_prep_router_w(const void* __restrict__ w, int w_f32, int E, int Epad, int D,
                                uint16_t* __restrict__ planes) {
  const size_t n = (size_t)Epad * D;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int e = (int)(i / D);
    if (w_f32) {
      const float v = (e < E) ? static_cast<const float*>(w)[i] : 0.0f;
      uint16_t b0, b1, b2;
      split3(v, b0, b1, b2);
      planes[i] = b0;
      planes[n + i] = b1;
      planes[2 * n + i] = b2;
    } else {
      planes[i] = (e < E) ? static_cast<const uint16_t*>(w)[i] : (uint16_t)0;
    }
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t stream) {
  const dim3 blk(256);
  if (a.x_f32)
    k_norm<true><<<dim3(a.T), blk, 0, stream>>>(a);
  else
    k_norm<false><<<dim3(a.T), blk, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 lg(((a.T + kTokTile - 1) / kTokTile) * (a.Epad / 16));
  if (a.n_wplanes == 3)
    k_logits<3><<<lg, dim3(64 * kLogitWaves), 0, stream>>>(a);
  else
    k_logits<1><<<lg, dim3(64 * kLogitWaves), 0, stream>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_topk<<<dim3((a.T + 3) / 4), blk, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_prep_router_w(const void* w, int w_f32, int E, int Epad, int D, uint16_t* planes,
                                hipStream_t stream) {
  k_prep_router_w<<<dim3(512), dim3(256), 0, stream>>>(w, w_f32, E, Epad, D, planes);
  return hipGetLastError();
}

}  // namespace dg
