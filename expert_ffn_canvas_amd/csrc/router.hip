// Router of the MoE layer on gfx950, two kernels:
//  norm:   per token r = 1/sqrt(mean x^2 + eps); the expert input
//          h = x r (1 + gamma_e) (bf16, or fp16 for int4 experts); and the
//          router input z = x r (1 + gamma_r) in fp32, stored as three exact
//          bf16 planes z = z0 + z1 + z2 (each holds the next 8 significant
//          bits of the fp32 value).
//  router: logits = z W_r^T + b on the bf16 matrix cores (each bf16 x bf16
//          product is exact in fp32 and the MFMA accumulates in fp32, so with
//          z in three planes, and an fp32 router weight split the same way at
//          create time, the logits have fp32 dot-product accuracy); then per
//          token the k largest logits (ties: lower expert id) and their
//          softmax renormalised over the k, slots ordered by logit.
//
// Sources: Quant-Tuner PR "Add DiffusionGemma (Gemma-4 MoE block-diffusion)
// support", "Answers to the motivating questions" (the router reads the raw
// residual through its own norm; pre_feedforward_layernorm_2 with the (1+gamma)
// convention feeds the fused gate_up); 128 experts / 8 active from its Summary.
#include "dg_common.h"
#include "launch.h"

namespace dg {

namespace {

constexpr int kTokTile = 16;    // tokens per workgroup (MFMA M)
constexpr int kKChunk = 128;    // d_model columns per chunk
constexpr int kWaves = 8;       // waves per workgroup; wave h owns chunks h, h + 8, ...

// z = hi + mid + lo exactly: hi keeps the top 8 significant bits of z
// (truncated), mid the next 8 of the remainder, and the last remainder has at
// most 8 significant bits, so all three are exact bf16 values.
__device__ __forceinline__ void split3(float z, float& hi, float& mid, float& lo) {
  hi = __uint_as_float(__float_as_uint(z) & 0xffff0000u);
  const float r1 = z - hi;
  mid = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
  lo = r1 - mid;
}

// Upper halves of two floats that are exact bf16 values -> packed bf16 pair.
__device__ __forceinline__ uint32_t pack_hi(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// x values (fp32 or bf16) of one 8-column piece.
template <bool XF32>
struct XPiece {
  u32x4 v[XF32 ? 2 : 1];
};

template <bool XF32>
__device__ __forceinline__ void load_piece(const void* x, size_t off, XPiece<XF32>& p) {
  if constexpr (XF32) {
    p.v[0] = *reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + off);
    p.v[1] = *reinterpret_cast<const u32x4*>(static_cast<const float*>(x) + off + 4);
  } else {
    p.v[0] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + off);
  }
}

template <bool XF32>
__device__ __forceinline__ void piece_floats(const XPiece<XF32>& p, float (&f)[8]) {
  if constexpr (XF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(p.v[0][i]);
      f[4 + i] = __uint_as_float(p.v[1][i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(p.v[0][i]);
      f[2 * i + 1] = bf16_hi(p.v[0][i]);
    }
  }
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Number of lanes of the wave for which `pred` holds.
__device__ __forceinline__ int wave_count(bool pred) { return __popcll(__ballot(pred)); }

// Top-k of one token from its logits row in LDS (one wave, E <= 256; lane l
// holds experts l + 64 u). A radix select on the keys finds the k-th largest
// key t (the largest t with at least k keys >= t); the experts above t are
// taken, and of those equal to t the lowest ids fill the remaining places.
// The k chosen experts are then ordered by (logit desc, id asc) and their
// softmax over the k is summed in that order.
__device__ __forceinline__ void topk_row(const float* lrow, int E, int K, int lane, float* sel_v, int* sel_i,
                                         int32_t* idx_out, float* w_out) {
  const int nu = (E + 63) >> 6;
  float v[4];
  uint32_t key[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bool present = (u < nu) && (lane + 64 * u < E);
    v[u] = present ? lrow[lane + 64 * u] : -INFINITY;
    key[u] = present ? float_key(v[u]) : 0u;  // absent experts rank below every real one
  }
  uint32_t t = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = t | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < nu) cnt += wave_count(key[u] >= cand);
    if (cnt >= K) t = cand;
  }
  int above = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (u < nu) above += wave_count(key[u] > t);
  // keys equal to t in id order: experts l + 64 u come before l + 64 (u + 1)
  int need = K - above;
  bool sel[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bool present = (u < nu) && (lane + 64 * u < E);
    const bool eq = present && key[u] == t;
    const uint64_t msk = __ballot(eq);
    const int before = __popcll(msk & ((1ull << lane) - 1ull));
    sel[u] = present && (key[u] > t || (eq && before < need));
    need -= min(__popcll(msk), max(need, 0));
  }
  // order the chosen experts: rank = chosen ones with a larger key, or an equal key and a lower id
  int rank[4] = {0, 0, 0, 0};
#pragma unroll
  for (int u2 = 0; u2 < 4; ++u2) {
    if (u2 >= nu) break;
    uint64_t msk = __ballot(sel[u2]);
    while (msk) {
      const int src = __ffsll((long long)msk) - 1;
      msk &= msk - 1ull;
      const uint32_t ks = __shfl(key[u2], src);
      const int es = src + 64 * u2;
#pragma unroll
      for (int u = 0; u < 4; ++u) rank[u] += (ks > key[u]) || (ks == key[u] && es < lane + 64 * u);
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (sel[u]) {
      sel_v[rank[u]] = v[u];
      sel_i[rank[u]] = lane + 64 * u;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  if (lane < K) {
    const float vmax = sel_v[0];
    float den = 0.0f;
    for (int j = 0; j < K; ++j) den += __expf(sel_v[j] - vmax);
    idx_out[lane] = sel_i[lane];
    w_out[lane] = __expf(sel_v[lane] - vmax) / den;
  }
}

// One workgroup of 256 threads per token; thread i owns the 8-column pieces
// i, i + 256, ... (up to 8 of them: d_model <= 16384). All loads of a thread
// (x and both gammas) are issued together, one block reduction gives r.
template <bool XF32>
__global__ __launch_bounds__(256) void k_norm(RouterArgs a) {
  __shared__ float wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int D = a.D;
  const int nseg = D / 8;
  const size_t row = (size_t)t * D;
  XPiece<XF32> xp[8];
  float4 gr[8][2], ge[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sg = tid + 256 * i;
    if (sg < nseg) {
      load_piece<XF32>(a.x, row + sg * 8, xp[i]);
      gr[i][0] = *reinterpret_cast<const float4*>(a.gamma_r + sg * 8);
      gr[i][1] = *reinterpret_cast<const float4*>(a.gamma_r + sg * 8 + 4);
      ge[i][0] = *reinterpret_cast<const float4*>(a.gamma_e + sg * 8);
      ge[i][1] = *reinterpret_cast<const float4*>(a.gamma_e + sg * 8 + 4);
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (tid + 256 * i < nseg) {
      float f[8];
      piece_floats<XF32>(xp[i], f);
#pragma unroll
      for (int k = 0; k < 8; ++k) ss += f[k] * f[k];
    }
  }
  for (int msk = 32; msk >= 1; msk >>= 1) ss += __shfl_xor(ss, msk);
  if (lane == 0) wsum[wave] = ss;
  __syncthreads();
  const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float r = 1.0f / sqrtf(tot / (float)D + a.eps);
  const size_t plane = (size_t)a.T * D;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int sg = tid + 256 * i;
    if (sg >= nseg) continue;
    float f[8];
    piece_floats<XF32>(xp[i], f);
    const float g1[8] = {gr[i][0].x, gr[i][0].y, gr[i][0].z, gr[i][0].w, gr[i][1].x, gr[i][1].y, gr[i][1].z, gr[i][1].w};
    const float g2[8] = {ge[i][0].x, ge[i][0].y, ge[i][0].z, ge[i][0].w, ge[i][1].x, ge[i][1].y, ge[i][1].z, ge[i][1].w};
    float zh[8], zm[8], zl[8], hv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float xr = f[k] * r;
      split3(xr * (1.0f + g1[k]), zh[k], zm[k], zl[k]);
      hv[k] = xr * (1.0f + g2[k]);
    }
    u32x4 o0, o1, o2, ho;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o0[k] = pack_hi(zh[2 * k], zh[2 * k + 1]);
      o1[k] = pack_hi(zm[2 * k], zm[2 * k + 1]);
      o2[k] = pack_hi(zl[2 * k], zl[2 * k + 1]);
      ho[k] = a.h_f16 ? pack_f16x2(hv[2 * k], hv[2 * k + 1]) : pack_bf16x2(hv[2 * k], hv[2 * k + 1]);
    }
    const size_t off = row + sg * 8;
    *reinterpret_cast<u32x4*>(a.z + off) = o0;
    *reinterpret_cast<u32x4*>(a.z + plane + off) = o1;
    *reinterpret_cast<u32x4*>(a.z + 2 * plane + off) = o2;
    *reinterpret_cast<u32x4*>(a.h + off) = ho;
  }
}

// Workgroup (token tile tt, expert tile et): 16 tokens x 16 experts, 8 waves;
// wave h owns the 128-column chunks h, h + 8, ... of d_model. Lane
// (m = l % 16, g = l / 16) loads, in each chunk, the 8-column pieces g, g + 4,
// g + 8, g + 12 of token m's three z planes and of expert m's router weight:
// the MFMA operand layouts. A wave issues the loads of up to kGroup chunks at
// once, then multiplies. The eight partial sums are added through LDS in a
// fixed order.
// All expert tiles of a token tile run on one XCD (workgroup b runs on XCD
// b % 8) and share its L2: each one publishes its logits with a counter and
// the last to arrive ranks the full rows for the top-k.
template <int NWP>
__global__ __launch_bounds__(64 * kWaves) void k_logits(RouterArgs a) {
  constexpr int kGroup = (NWP == 1) ? 3 : 1;
  __shared__ float part[kWaves][kTokTile][17];
  __shared__ float lrow[kTokTile][260];
  __shared__ float sel_v[kWaves][8];
  __shared__ int sel_i[kWaves][8];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63, kh = tid >> 6;
  const int n_et = a.Epad / 16;
  const int n_tt = (a.T + kTokTile - 1) / kTokTile;
  const int xq = blockIdx.x % kQueues, jq = blockIdx.x / kQueues;
  const int tt = xq + kQueues * (jq / n_et);
  const int et = jq % n_et;
  if (tt >= n_tt) return;
  const int t0 = tt * kTokTile;
  const int D = a.D;
  const int m = lane & 15, g = lane >> 4;
  const int t = min(t0 + m, a.T - 1);  // rows past T re-read the last token; never stored
  const size_t plane = (size_t)a.T * D;
  const size_t wplane = (size_t)a.Epad * D;
  const uint16_t* zr = a.z + (size_t)t * D + g * 8;
  const uint16_t* wrow = a.wr + (size_t)(et * 16 + m) * D + g * 8;
  const int nc = D / kKChunk;
  const int n_my = (nc - kh + kWaves - 1) / kWaves;  // chunks kh, kh + 8, ...

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < n_my; c0 += kGroup) {
    u32x4 zb[kGroup][4][3], wb[kGroup][4][NWP];
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      if (c0 + q < n_my) {
        const int col = (kh + kWaves * (c0 + q)) * kKChunk;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
          for (int p = 0; p < 3; ++p) zb[q][kk][p] = *reinterpret_cast<const u32x4*>(zr + p * plane + col + kk * 32);
#pragma unroll
          for (int p = 0; p < NWP; ++p) wb[q][kk][p] = *reinterpret_cast<const u32x4*>(wrow + p * wplane + col + kk * 32);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      if (c0 + q < n_my) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int zp = 0; zp < 3; ++zp)
#pragma unroll
            for (int p = 0; p < NWP; ++p) acc = mfma_bf16(as_bf16x8(zb[q][kk][zp]), as_bf16x8(wb[q][kk][p]), acc);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[kh][g * 4 + i][m] = acc[i];
  __syncthreads();
  // [16 tokens x 16 experts] (+ bias); the eight partial sums in a fixed order
  if (tid < kTokTile * 16) {
    const int mm = tid >> 4, n = tid & 15;
    float sum = part[0][mm][n];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += part[w][mm][n];
    const int e = et * 16 + n;
    if (a.bias != nullptr && e < a.E) sum += a.bias[e];
    if (t0 + mm < a.T) a.logits[(size_t)(t0 + mm) * a.Epad + e] = sum;
  }
  // publish: every thread's stores have reached L2 before the counter moves
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int old = atomicAdd(&a.tile_count[tt], 1);
    is_last = (old == n_et - 1);
    if (is_last) a.tile_count[tt] = 0;  // ready for the next forward
  }
  __syncthreads();
  if (!is_last) return;
  // Last expert tile of this token tile: gather the full logit rows. They come
  // from this XCD's L2 (every writer ran on this XCD and waited for its
  // stores); no workgroup on this CU read these rows earlier in the launch, so
  // its L1 holds no stale copy.
  for (int i = tid; i < kTokTile * (a.Epad / 4); i += 64 * kWaves) {
    const int mm = i / (a.Epad / 4), c4 = i - mm * (a.Epad / 4);
    float4 l = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    if (t0 + mm < a.T) l = *reinterpret_cast<const float4*>(&a.logits[(size_t)(t0 + mm) * a.Epad + 4 * c4]);
    const float lv[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)  // a NaN logit ranks last, so k valid ids are always chosen
      lrow[mm][4 * c4 + q] = (lv[q] == lv[q]) ? lv[q] : -INFINITY;
  }
  __syncthreads();
  for (int q = 0; q < kTokTile / kWaves; ++q) {
    const int mm = kh * (kTokTile / kWaves) + q;
    if (t0 + mm < a.T)
      topk_row(lrow[mm], a.E, a.K, lane, sel_v[kh], sel_i[kh], a.topk_idx + (size_t)(t0 + mm) * a.K,
               a.topk_w + (size_t)(t0 + mm) * a.K);
    __builtin_amdgcn_wave_barrier();
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
      float b0, b1, b2;
      split3(v, b0, b1, b2);
      planes[i] = (uint16_t)(__float_as_uint(b0) >> 16);
      planes[n + i] = (uint16_t)(__float_as_uint(b1) >> 16);
      planes[2 * n + i] = (uint16_t)(__float_as_uint(b2) >> 16);
    } else {
      planes[i] = (e < E) ? static_cast<const uint16_t*>(w)[i] : (uint16_t)0;
    }
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t stream) {
  if (a.x_f32)
    k_norm<true><<<dim3(a.T), dim3(256), 0, stream>>>(a);
  else
    k_norm<false><<<dim3(a.T), dim3(256), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_tt = (a.T + kTokTile - 1) / kTokTile;
  const dim3 grid(kQueues * ((n_tt + kQueues - 1) / kQueues) * (a.Epad / 16));
  if (a.n_wplanes == 3)
    k_logits<3><<<grid, dim3(64 * kWaves), 0, stream>>>(a);
  else
    k_logits<1><<<grid, dim3(64 * kWaves), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_prep_router_w(const void* w, int w_f32, int E, int Epad, int D, uint16_t* planes,
                                hipStream_t stream) {
  k_prep_router_w<<<dim3(512), dim3(256), 0, stream>>>(w, w_f32, E, Epad, D, planes);
  return hipGetLastError();
}

}  // namespace dg
