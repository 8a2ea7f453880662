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

// Bits 0..31 (lanes 0..31) or 32..63 (lanes 32..63) of a wave-wide mask: the
// half-wave of the calling lane.
__device__ __forceinline__ uint32_t half_mask(uint64_t m, bool hi_half) {
  return hi_half ? (uint32_t)(m >> 32) : (uint32_t)m;
}

// Top-k of two tokens per wave, one per half-wave; lane j of a half holds the
// logits of experts j + 32 u (u < NU, E <= 32 NU), read from `row`.
// A radix select on order-preserving keys finds the k-th largest key kt (the
// largest value with at least k keys >= it). The experts above kt are taken,
// and of those equal to kt the lowest ids fill the remaining places. The k
// chosen are compacted in id order into cv/ci (LDS, 8 entries per half);
// then lane p < k of the half ranks entry p by (logit desc, id asc) and
// writes it to that slot, with its softmax over the k (exponentials summed in
// id order).
template <int NU>
__device__ __forceinline__ void topk_half(const float* row, bool active, int E, int K, int lane, float* cv,
                                          int* ci, int32_t* idx_out, float* w_out) {
  const bool hi_half = lane >= 32;
  const int j = lane & 31;
  const uint32_t lt = (1u << j) - 1u;
  float v[NU];
  uint32_t key[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int e = j + 32 * u;
    float l = -INFINITY;
    if (active && e < E) l = row[e];
    v[u] = (l == l) ? l : -INFINITY;  // a NaN logit ranks last
    key[u] = (active && e < E) ? float_key(v[u]) : 0u;  // absent experts rank below every real one
  }
  uint32_t kt = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = kt | (1u << b);
    int c = 0;
#pragma unroll
    for (int u = 0; u < NU; ++u) c += __popc(half_mask(__ballot(key[u] >= cand), hi_half));
    kt = (c >= K) ? cand : kt;
  }
  int above = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) above += __popc(half_mask(__ballot(key[u] > kt), hi_half));
  int need = K - above;
  int base = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const bool eq = key[u] == kt;
    const uint32_t me = half_mask(__ballot(eq), hi_half);
    const bool sel = key[u] > kt || (eq && __popc(me & lt) < need);
    need -= min(__popc(me), max(need, 0));
    const uint32_t ms = half_mask(__ballot(sel), hi_half);
    if (sel) {
      const int p = base + __popc(ms & lt);
      cv[p] = v[u];
      ci[p] = j + 32 * u;
    }
    base += __popc(ms);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  if (active && j < K) {
    const float vp = cv[j];
    const int ip = ci[j];
    float vmax = -INFINITY;
    int rank = 0;
    for (int q = 0; q < K; ++q) {
      const float vq = cv[q];
      vmax = fmaxf(vmax, vq);
      rank += (vq > vp) || (vq == vp && ci[q] < ip);
    }
    float den = 0.0f;
    for (int q = 0; q < K; ++q) den += __expf(cv[q] - vmax);
    idx_out[rank] = ip;
    w_out[rank] = __expf(vp - vmax) / den;
  }
}

// One workgroup of 256 threads per token; thread i owns the 8-column pieces
// i, i + 256, ... (up to NP of them: d_model <= 2048 NP). All loads of a
// thread (x and both gammas) are issued together, one block reduction gives r.
template <bool XF32, int NP>
__global__ __launch_bounds__(256) void k_norm(RouterArgs a) {
  __shared__ float wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int D = a.D;
  const int nseg = D / 8;
  const size_t row = (size_t)t * D;
  XPiece<XF32> xp[NP];
  float4 gr[NP][2], ge[NP][2];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
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
  for (int i = 0; i < NP; ++i) {
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
  for (int i = 0; i < NP; ++i) {
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
// the MFMA operand layouts. A wave issues the loads of kGroup chunks at once
// (a chunk past its last is re-read and multiplied by a zero weight, so the
// loop has no branches), then multiplies. The eight partial sums are added
// through LDS in a fixed order.
// All expert tiles of a token tile run on one XCD (workgroup b runs on XCD
// b % 8) and share its L2: each one publishes its logits with a counter and
// the last to arrive selects the top-k of the 16 rows.
// GROUPS: chunks whose loads a wave keeps in flight at once. Three (two for
// fp32 router weights) take one round trip per wave at d_model <= 3072 but
// hold about 200 registers, so one workgroup fits a CU; one group lets two
// workgroups share a CU, which pays when there are many token tiles.
template <int NWP, int NU, bool WIDE>
__global__ __launch_bounds__(64 * kWaves) void k_logits(RouterArgs a) {
  constexpr int kGroup = !WIDE ? 1 : (NWP == 1) ? 3 : 2;
  __shared__ float part[kWaves][kTokTile][17];
  __shared__ float cv[kWaves][2][8];
  __shared__ int ci[kWaves][2][8];
  __shared__ int is_last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int kh = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_et = a.Epad / 16;
  const int n_tt = (a.T + kTokTile - 1) / kTokTile;
  const int xq = blockIdx.x % kQueues, jq = blockIdx.x / kQueues;
  const int tt = xq + kQueues * (jq / n_et);
  const int et = jq % n_et;
  if (tt >= n_tt) return;
  const int t0 = tt * kTokTile;
  const int D = a.D;
  // bias of this thread's output column, fetched before the long loads
  float bias_v = 0.0f;
  {
    const int e = et * 16 + (tid & 15);
    if (tid < kTokTile * 16 && a.bias != nullptr && e < a.E) bias_v = a.bias[e];
  }
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
      const int col = (kh + kWaves * min(c0 + q, n_my - 1)) * kKChunk;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int p = 0; p < 3; ++p) zb[q][kk][p] = *reinterpret_cast<const u32x4*>(zr + p * plane + col + kk * 32);
#pragma unroll
        for (int p = 0; p < NWP; ++p) wb[q][kk][p] = *reinterpret_cast<const u32x4*>(wrow + p * wplane + col + kk * 32);
      }
    }
    // keep every load of the group ahead of the first multiply: one memory
    // round trip per group instead of one per operand
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
      const uint32_t keep = (c0 + q < n_my) ? 0xffffffffu : 0u;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int p = 0; p < NWP; ++p) {
          u32x4 w = wb[q][kk][p];
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] &= keep;
#pragma unroll
          for (int zp = 0; zp < 3; ++zp) acc = mfma_bf16(as_bf16x8(zb[q][kk][zp]), as_bf16x8(w), acc);
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
    sum += bias_v;
    if (t0 + mm < a.T) a.logits[(size_t)(t0 + mm) * a.Epad + et * 16 + n] = sum;
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
  // Last expert tile of this token tile: the full logit rows come from this
  // XCD's L2 (every writer ran on this XCD and waited for its stores); no
  // workgroup on this CU read these rows earlier in the launch, so its L1
  // holds no stale copy. Wave h takes tokens t0 + 2h (lanes 0..31) and
  // t0 + 2h + 1 (lanes 32..63).
  const int half = lane >> 5;
  const int tk = t0 + 2 * kh + half;
  const bool active = tk < a.T;
  const size_t trow = (size_t)min(tk, a.T - 1);
  topk_half<NU>(a.logits + trow * a.Epad, active, a.E, a.K, lane, cv[kh][half], ci[kh][half],
                a.topk_idx + trow * a.K, a.topk_w + trow * a.K);
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

hipError_t launch_router(const RouterArgs& a, hipStream_t stream, const KernelEvents* ev) {
  void (*kn)(RouterArgs);
  if (a.D <= 2048 * 2)
    kn = a.x_f32 ? k_norm<true, 2> : k_norm<false, 2>;
  else
    kn = a.x_f32 ? k_norm<true, 8> : k_norm<false, 8>;
  hipError_t e = launch_kernel(kn, dim3(a.T), dim3(256), stream, ev ? &ev[0] : nullptr, a);
  if (e != hipSuccess) return e;
  const int n_tt = (a.T + kTokTile - 1) / kTokTile;
  const int n_et = a.Epad / 16;
  const dim3 grid(kQueues * ((n_tt + kQueues - 1) / kQueues) * n_et);
  // more workgroups than CUs: the narrow variant keeps two per CU
  const bool wide = (size_t)n_tt * n_et <= 256;
  const int nu = a.Epad / 32;  // 1 .. 8
  void (*k)(RouterArgs);
#define DG_LOGITS(NWP, W) \
  (nu <= 1 ? k_logits<NWP, 1, W> : nu <= 2 ? k_logits<NWP, 2, W> : nu <= 4 ? k_logits<NWP, 4, W> : k_logits<NWP, 8, W>)
  if (a.n_wplanes == 3)
    k = wide ? DG_LOGITS(3, true) : DG_LOGITS(3, false);
  else
    k = wide ? DG_LOGITS(1, true) : DG_LOGITS(1, false);
#undef DG_LOGITS
  return launch_kernel(k, grid, dim3(64 * kWaves), stream, ev ? &ev[1] : nullptr, a);
}

hipError_t launch_prep_router_w(const void* w, int w_f32, int E, int Epad, int D, uint16_t* planes,
                                hipStream_t stream) {
  k_prep_router_w<<<dim3(512), dim3(256), 0, stream>>>(w, w_f32, E, Epad, D, planes);
  return hipGetLastError();
}

}  // namespace dg
