// Router of the MoE layer on gfx950: the RMS statistic of each token, the
// router's own (1+gamma) RMSNorm, E logits, top-k with lower-id tie break,
// renormalised softmax weights over the k, and the expert-input norm
// h = x r (1 + gamma_e) written for the grouped GEMMs.
//
// Sources: Quant-Tuner PR "Add DiffusionGemma (Gemma-4 MoE block-diffusion)
// support", "Answers to the motivating questions" (router reads the raw
// residual through its own norm; pre_feedforward_layernorm_2 with the (1+gamma)
// convention feeds the fused gate_up); 128 experts / 8 active from its Summary.
//
// Precision: the router stays fp32 end to end. The normalised input z (fp32)
// is split exactly into three bf16 planes z = z0 + z1 + z2 (each plane holds
// the next 8 significant bits), and the router weight is one bf16 plane (bf16
// weights) or three planes (fp32 weights, split the same way at create time).
// Each bf16 x bf16 product is exact in fp32, and the MFMA accumulates in fp32,
// so the logits carry fp32 dot-product accuracy while running on the bf16
// matrix cores.
#include "dg_common.h"
#include "launch.h"

namespace dg {

namespace {

constexpr int kTokTile = 16;   // tokens per workgroup (MFMA M)
constexpr int kKChunk = 128;   // d_model columns staged per LDS round
constexpr int kZPitch = kKChunk + 8;
constexpr int kRouterThreads = 512;
constexpr int kMaxPlanes = 3;

__device__ __forceinline__ void split3(float z, uint16_t& b0, uint16_t& b1, uint16_t& b2) {
  b0 = f32_to_bf16_bits(z);
  const float r1 = z - bf16_bits_to_f32(b0);
  b1 = f32_to_bf16_bits(r1);
  const float r2 = r1 - bf16_bits_to_f32(b1);
  b2 = f32_to_bf16_bits(r2);
}

template <bool XF32, int NWP>
__global__ __launch_bounds__(kRouterThreads) void k_router(
    const void* __restrict__ x, int T, int D, int E, int Epad, int K, const uint16_t* __restrict__ wr,
    const float* __restrict__ gamma_r, const float* __restrict__ bias, const float* __restrict__ gamma_e,
    float eps, int h_f16, uint16_t* __restrict__ h_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  __shared__ __attribute__((aligned(16))) uint16_t zs[3][kTokTile * kZPitch];
  __shared__ float logits[kTokTile][257];
  __shared__ float rs[kTokTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * kTokTile;

  // --- RMS statistic: wave w reduces tokens 2w and 2w+1.
  for (int q = 0; q < 2; ++q) {
    const int tt = wave * 2 + q;
    const int t = t0 + tt;
    float ss = 0.0f;
    if (t < T) {
      for (int c = lane * 4; c < D; c += 256) {
        float v0, v1, v2, v3;
        if (XF32) {
          const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)t * D + c);
          v0 = v.x; v1 = v.y; v2 = v.z; v3 = v.w;
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + (size_t)t * D + c);
          v0 = bf16_lo(v.x); v1 = bf16_hi(v.x); v2 = bf16_lo(v.y); v3 = bf16_hi(v.y);
        }
        ss += v0 * v0 + v1 * v1 + v2 * v2 + v3 * v3;
      }
    }
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if (lane == 0) rs[tt] = (t < T) ? 1.0f / sqrtf(ss / (float)D + eps) : 0.0f;
  }
  __syncthreads();

  // --- logits: wave w owns expert tiles w and w + 8 (16 experts each).
  const int n_et = Epad >> 4;
  f32x4 acc[2];
  acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int zt = tid >> 5;          // token row this thread stages
  const int zc = (tid & 31) * 4;    // 4 columns inside the chunk
  const int t_z = t0 + zt;
  const float r_z = rs[zt];

  for (int c0 = 0; c0 < D; c0 += kKChunk) {
    // issue the router-weight loads of this chunk first so they overlap the staging math
    u32x4 wb[2][4][NWP];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int et = wave + 8 * s;
      if (et < n_et) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
          for (int p = 0; p < NWP; ++p) {
            const uint16_t* src = wr + ((size_t)p * Epad + et * 16 + (lane & 15)) * D + c0 + kk * 32 + (lane >> 4) * 8;
            wb[s][kk][p] = *reinterpret_cast<const u32x4*>(src);
          }
        }
      }
    }

    // stage z = x r (1 + gamma_r) as three bf16 planes, and write h = x r (1 + gamma_e)
    {
      const int c = c0 + zc;
      float xv[4] = {0.f, 0.f, 0.f, 0.f};
      if (t_z < T) {
        if (XF32) {
          const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)t_z * D + c);
          xv[0] = v.x; xv[1] = v.y; xv[2] = v.z; xv[3] = v.w;
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + (size_t)t_z * D + c);
          xv[0] = bf16_lo(v.x); xv[1] = bf16_hi(v.x); xv[2] = bf16_lo(v.y); xv[3] = bf16_hi(v.y);
        }
      }
      const float4 gr = *reinterpret_cast<const float4*>(gamma_r + c);
      const float4 ge = *reinterpret_cast<const float4*>(gamma_e + c);
      const float grv[4] = {gr.x, gr.y, gr.z, gr.w};
      const float gev[4] = {ge.x, ge.y, ge.z, ge.w};
      uint16_t zb[3][4];
      float hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xr = xv[i] * r_z;
        split3(xr * (1.0f + grv[i]), zb[0][i], zb[1][i], zb[2][i]);
        hv[i] = xr * (1.0f + gev[i]);
      }
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        uint2 packed;
        packed.x = (uint32_t)zb[p][0] | ((uint32_t)zb[p][1] << 16);
        packed.y = (uint32_t)zb[p][2] | ((uint32_t)zb[p][3] << 16);
        *reinterpret_cast<uint2*>(&zs[p][zt * kZPitch + zc]) = packed;
      }
      if (t_z < T) {
        uint2 hp;
        if (h_f16) {
          hp.x = pack_f16x2(hv[0], hv[1]);
          hp.y = pack_f16x2(hv[2], hv[3]);
        } else {
          hp.x = pack_bf16x2(hv[0], hv[1]);
          hp.y = pack_bf16x2(hv[2], hv[3]);
        }
        *reinterpret_cast<uint2*>(h_out + (size_t)t_z * D + c) = hp;
      }
    }
    __syncthreads();

#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int et = wave + 8 * s;
      if (et < n_et) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int off = (lane & 15) * kZPitch + kk * 32 + (lane >> 4) * 8;
#pragma unroll
          for (int zp = 0; zp < 3; ++zp) {
            const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&zs[zp][off]));
#pragma unroll
            for (int p = 0; p < NWP; ++p) acc[s] = mfma_bf16(a, as_bf16x8(wb[s][kk][p]), acc[s]);
          }
        }
      }
    }
    __syncthreads();
  }

  // --- scatter the logits (plus bias) into LDS; padding experts get -inf
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int et = wave + 8 * s;
    if (et < n_et) {
      const int e = et * 16 + (lane & 15);
      const float b = (bias != nullptr && e < E) ? bias[e] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = (lane >> 4) * 4 + i;
        logits[tt][e] = (e < E) ? acc[s][i] + b : -INFINITY;
      }
    }
  }
  __syncthreads();

  // --- top-k per token: wave w selects for tokens 2w and 2w+1
  for (int q = 0; q < 2; ++q) {
    const int tt = wave * 2 + q;
    const int t = t0 + tt;
    if (t >= T) continue;  // uniform across the wave
    float v[4];
    bool taken[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = lane + 64 * u;
      const float l = (e < E) ? logits[tt][e] : -INFINITY;
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
      topk_idx[(size_t)t * K + lane] = my_i;
      topk_w[(size_t)t * K + lane] = ex / den;
    }
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
  const dim3 grid((a.T + kTokTile - 1) / kTokTile);
  const dim3 block(kRouterThreads);
  if (a.x_f32) {
    if (a.n_wplanes == 3)
      k_router<true, 3><<<grid, block, 0, stream>>>(a.x, a.T, a.D, a.E, a.Epad, a.K, a.wr, a.gamma_r, a.bias,
                                                    a.gamma_e, a.eps, a.h_f16, a.h, a.topk_idx, a.topk_w);
    else
      k_router<true, 1><<<grid, block, 0, stream>>>(a.x, a.T, a.D, a.E, a.Epad, a.K, a.wr, a.gamma_r, a.bias,
                                                    a.gamma_e, a.eps, a.h_f16, a.h, a.topk_idx, a.topk_w);
  } else {
    if (a.n_wplanes == 3)
      k_router<false, 3><<<grid, block, 0, stream>>>(a.x, a.T, a.D, a.E, a.Epad, a.K, a.wr, a.gamma_r, a.bias,
                                                     a.gamma_e, a.eps, a.h_f16, a.h, a.topk_idx, a.topk_w);
    else
      k_router<false, 1><<<grid, block, 0, stream>>>(a.x, a.T, a.D, a.E, a.Epad, a.K, a.wr, a.gamma_r, a.bias,
                                                     a.gamma_e, a.eps, a.h_f16, a.h, a.topk_idx, a.topk_w);
  }
  return hipGetLastError();
}

hipError_t launch_prep_router_w(const void* w, int w_f32, int E, int Epad, int D, uint16_t* planes,
                                hipStream_t stream) {
  k_prep_router_w<<<dim3(512), dim3(256), 0, stream>>>(w, w_f32, E, Epad, D, planes);
  return hipGetLastError();
}

}  // namespace dg
