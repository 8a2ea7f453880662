// Router of the MoE layer on gfx950.
//
//  logits + top-k (one kernel): per token r = 1/sqrt(mean_d x^2 + eps) and
//          logits = r (W' x) + b with W' = W_r diag(1 + gamma_r), the router
//          norm's scale folded into the router weight at create time. W' is
//          kept in fp32 and split in registers into three exact bf16 planes
//          (W' = W0 + W1 + W2, each plane the next 8 significant bits), so
//          the products on the bf16 matrix cores are exact and accumulate in
//          fp32: the logits have fp32 dot-product accuracy. Then per token the
//          k largest logits (ties: lower expert id), in that order, with their
//          softmax renormalised over the k.
//  norm:   only where the expert input has to be materialised (fp32
//          activations, int4 experts, borrowed weights): r again and
//          h = x r (1 + gamma_e), bf16 (fp16 for int4 experts). Otherwise the
//          gate_up GEMM reads x itself, with (1 + gamma_e) folded into its
//          packed weight and r applied to its sums.
//
// Sources: Quant-Tuner PR "Add DiffusionGemma (Gemma-4 MoE block-diffusion)
// support", "Answers to the motivating questions" (the router reads the raw
// residual through its own norm; pre_feedforward_layernorm_2 with the (1+gamma)
// convention feeds the fused gate_up); 128 experts / 8 active from its Summary.
#include "dg_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace dg {

namespace {

constexpr int kKChunk = 128;  // d_model columns per chunk
constexpr int kWaves = 8;     // waves per workgroup; wave h owns chunks h, h + 8, ...
constexpr int kChunkRowBytes = kKChunk * 2;

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

// Order-preserving map of a float to uint32 (larger float -> larger key) and back.
__device__ __forceinline__ uint32_t float_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Keep the larger (key, -id) of this lane's and the partner lane's.
template <int CTRL>
__device__ __forceinline__ void argmax_step(uint32_t& key, uint32_t& id) {
  const uint32_t ok = dpp<CTRL>(key), oi = dpp<CTRL>(id);
  const bool take = ok > key || (ok == key && oi < id);
  key = take ? ok : key;
  id = take ? oi : id;
}

template <int CTRL>
__device__ __forceinline__ float add_step(float v) {
  return v + __uint_as_float(dpp<CTRL>(__float_as_uint(v)));
}

// Top-k of one token per 16-lane row: lane j holds the logits of experts
// j + 16 u (u < NU, E <= 16 NU), read from `row`. Round q takes the largest
// remaining (logit, lowest id) of the row and removes it, so the k rounds
// produce the selection in slot order (logit descending, ties by id). Lane
// q < k keeps round q's pick and writes slot q with its softmax over the k
// (the shift by the largest logit cancels in the renormalisation). A NaN
// logit ranks below every number; experts >= E are never picked.
template <int NU>
__device__ __forceinline__ void topk_row(const float* row, bool active, int E, int K, int j, int32_t* idx_out,
                                         float* w_out) {
  // all NU loads issued at once (a clamped index instead of a guarded load,
  // which would wait for each load in turn), masked afterwards
  float lv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) lv[u] = row[min(j + 16 * u, E - 1)];
  uint32_t key[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const float l = (lv[u] == lv[u]) ? lv[u] : -INFINITY;
    key[u] = (j + 16 * u < E) ? float_key(l) : 0u;  // every real expert's key is > 0
  }
  uint32_t my_key = 0, my_id = 0, top = 0;
  for (int q = 0; q < K; ++q) {
    uint32_t bk = key[0], bi = (uint32_t)j;
#pragma unroll
    for (int u = 1; u < NU; ++u) {
      const bool gt = key[u] > bk;  // strict: on equal keys the lower id stays
      bk = gt ? key[u] : bk;
      bi = gt ? (uint32_t)(j + 16 * u) : bi;
    }
    argmax_step<kDppXor1>(bk, bi);
    argmax_step<kDppXor2>(bk, bi);
    argmax_step<kDppHalfMirror>(bk, bi);
    argmax_step<kDppMirror>(bk, bi);
    top = (q == 0) ? bk : top;
    if (j == q) {
      my_key = bk;
      my_id = bi;
    }
    const bool own = (int)(bi & 15u) == j;
#pragma unroll
    for (int u = 0; u < NU; ++u) key[u] = (own && (int)(bi >> 4) == u) ? 0u : key[u];
  }
  const float ex = (j < K) ? __expf(key_float(my_key) - key_float(top)) : 0.0f;
  float den = add_step<kDppXor1>(ex);
  den = add_step<kDppXor2>(den);
  den = add_step<kDppHalfMirror>(den);
  den = add_step<kDppMirror>(den);
  if (active && j < K) {
    idx_out[j] = (int32_t)my_id;
    w_out[j] = ex / den;
  }
}

// bf16 x values of one MFMA operand (8 consecutive columns) -> sum of squares.
__device__ __forceinline__ float sumsq8(const u32x4& v) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s = fmaf(bf16_lo(v[i]), bf16_lo(v[i]), s);
    s = fmaf(bf16_hi(v[i]), bf16_hi(v[i]), s);
  }
  return s;
}

// Workgroup (token tile tt, expert tile et): 16 MT tokens x 16 experts, 8
// waves; wave h owns the 128-column chunks h, h + 8, ... of d_model and keeps
// G of them in flight. Per chunk, bf16 x rows are copied into the wave's own
// LDS slot by full-line transfers (row r's 16-byte segment s at position
// s ^ (r % 16)), and lane (m = l % 16, g = l / 16) reads token m's 8-column
// pieces from there in the MFMA operand layout; fp32 x is loaded in that
// layout directly and split into three exact bf16 planes in registers. W'
// is stored in fragment order, so every weight read is 1 KB contiguous per
// wave. A chunk past the wave's last re-reads its last one with a zero
// weight and no share of the sum of squares, so the loop has no branches.
// The partial sums (three accumulators per m-tile, one per W' plane, and
// the sums of squares) are added through LDS in a fixed order; every expert
// tile of a token tile computes the same r bit for bit.
// All expert tiles of a token tile run on one XCD (workgroup b runs on XCD
// b % 8) and share its L2: each publishes its logits with a counter and the
// last to arrive selects the top-k of all the tile's tokens, one per 16-lane
// row. With SPLIT = 2 (few token tiles) each expert tile is shared by two
// workgroups, one per half of its 16 experts: each loads only its half of
// every W' fragment (the other lanes' operands are zero), so the W' bytes a
// CU takes in are halved and twice as many CUs share them.
template <bool XF32, int MT, int G, int NU, int SPLIT>
__global__ __launch_bounds__(64 * kWaves) void k_logits(RouterArgs a) {
  constexpr int kRows = 16 * MT;
  constexpr int kXsBytes = XF32 ? 0 : kWaves * G * MT * 16 * kChunkRowBytes;
  constexpr int kPartBytes = kWaves * kRows * 17 * 4;
  constexpr int kBuf = kXsBytes > kPartBytes ? kXsBytes : kPartBytes;
  __shared__ __attribute__((aligned(16))) char smem[kBuf];
  __shared__ float ssq[kWaves][kRows];
  __shared__ int is_last;
  float(*part)[kRows][17] = reinterpret_cast<float(*)[kRows][17]>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int kh = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_eh = a.Epad / 16 * SPLIT;  // workgroups per token tile
  const int n_tt = (a.T + kRows - 1) / kRows;
  const int xq = blockIdx.x % kQueues, jq = blockIdx.x / kQueues;
  const int tt = xq + kQueues * (jq / n_eh);
  const int et = (jq % n_eh) / SPLIT, half = (jq % n_eh) % SPLIT;
  if (tt >= n_tt) return;
  const int t0 = tt * kRows;
  const int D = a.D;
  const int nks = D / 32;
  float bias_v = 0.0f;  // bias of this thread's output column, fetched before the long loads
  {
    const int e = et * 16 + (tid & 15);
    if (a.bias != nullptr && e < a.E) bias_v = a.bias[e];
  }
  const int m = lane & 15, g = lane >> 4;
  const bool wmine = SPLIT == 1 || (m >> 3) == half;  // this lane's expert is in the workgroup's half
  const float* wfrag = a.wr + (size_t)et * nks * 512 + lane * 4;
  const int nc = D / kKChunk;
  const int n_my = (nc - kh + kWaves - 1) / kWaves;  // chunks kh, kh + 8, ...

  f32x4 acc[3][MT];
  float ss[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    ss[mt] = 0.0f;
#pragma unroll
    for (int p = 0; p < 3; ++p) acc[p][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int c0 = 0; c0 < n_my; c0 += G) {
    u32x4 wb[G][4][2];
    u32x4 xf[XF32 ? G : 1][XF32 ? MT : 1][4][2];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const int chunk = kh + kWaves * min(c0 + q, n_my - 1);
      const int col = chunk * kKChunk;
      if constexpr (XF32) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float* xr = static_cast<const float*>(a.x) + (size_t)min(t0 + mt * 16 + m, a.T - 1) * D + col + g * 8;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            xf[q][mt][kk][0] = *reinterpret_cast<const u32x4*>(xr + kk * 32);
            xf[q][mt][kk][1] = *reinterpret_cast<const u32x4*>(xr + kk * 32 + 4);
          }
        }
      } else {
        const uint32_t base =
            __builtin_amdgcn_readfirstlane(gemm::lds_addr(smem) + (kh * G + q) * MT * 16 * kChunkRowBytes);
        const uint16_t* xb = static_cast<const uint16_t*>(a.x);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = mt * 16 + 4 * i + (lane >> 4);
            const int s = (lane & 15) ^ (r & 15);
            gemm::lds_dma16(base + (mt * 16 + 4 * i) * kChunkRowBytes,
                            xb + (size_t)min(t0 + r, a.T - 1) * D + col + s * 8);
          }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          wb[q][kk][h] = wmine ? *reinterpret_cast<const u32x4*>(wfrag + (size_t)(chunk * 4 + kk) * 512 + h * 256)
                               : u32x4{0u, 0u, 0u, 0u};
    }
    // all of the group's loads are in flight before the first multiply: one
    // memory round trip per group
    gemm::wait_vmcnt<0>();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const bool valid = c0 + q < n_my;
      const uint32_t keep = valid ? 0xffffffffu : 0u;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        // the lane's 8 fp32 weights -> three exact bf16 planes (W' = W0 + W1 + W2)
        bf16x8 w[3];
        {
          u32x4 o[3];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v0 = __uint_as_float(wb[q][kk][i >> 1][2 * (i & 1)] & keep);
            const float v1 = __uint_as_float(wb[q][kk][i >> 1][2 * (i & 1) + 1] & keep);
            float h0, m0, l0, h1, m1, l1;
            split3(v0, h0, m0, l0);
            split3(v1, h1, m1, l1);
            o[0][i] = pack_hi(h0, h1);
            o[1][i] = pack_hi(m0, m1);
            o[2][i] = pack_hi(l0, l1);
          }
#pragma unroll
          for (int p = 0; p < 3; ++p) w[p] = as_bf16x8(o[p]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if constexpr (XF32) {
            float f[8], hi[8], mid[8], lo[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              f[i] = __uint_as_float(xf[q][mt][kk][0][i]);
              f[4 + i] = __uint_as_float(xf[q][mt][kk][1][i]);
            }
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              s = fmaf(f[i], f[i], s);
              split3(f[i], hi[i], mid[i], lo[i]);
            }
            ss[mt] += valid ? s : 0.0f;
            u32x4 xh, xm, xl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              xh[i] = pack_hi(hi[2 * i], hi[2 * i + 1]);
              xm[i] = pack_hi(mid[2 * i], mid[2 * i + 1]);
              xl[i] = pack_hi(lo[2 * i], lo[2 * i + 1]);
            }
            // the products of weight >= 2^-24 relative: (hi, mid, lo) x
            // (W0, W1, W2) with plane indices summing to at most 2
            acc[0][mt] = mfma_bf16(as_bf16x8(xh), w[0], acc[0][mt]);
            acc[1][mt] = mfma_bf16(as_bf16x8(xh), w[1], acc[1][mt]);
            acc[1][mt] = mfma_bf16(as_bf16x8(xm), w[0], acc[1][mt]);
            acc[2][mt] = mfma_bf16(as_bf16x8(xh), w[2], acc[2][mt]);
            acc[2][mt] = mfma_bf16(as_bf16x8(xm), w[1], acc[2][mt]);
            acc[2][mt] = mfma_bf16(as_bf16x8(xl), w[0], acc[2][mt]);
          } else {
            const int r = mt * 16 + m;
            const u32x4 xv = *reinterpret_cast<const u32x4*>(smem + (kh * G + q) * MT * 16 * kChunkRowBytes +
                                                              r * kChunkRowBytes + (((kk * 4 + g) ^ m) * 16));
            ss[mt] += valid ? sumsq8(xv) : 0.0f;
#pragma unroll
            for (int p = 0; p < 3; ++p) acc[p][mt] = mfma_bf16(as_bf16x8(xv), w[p], acc[p][mt]);
          }
        }
      }
    }
  }
  // lanes m, m + 16, m + 32, m + 48 hold parts of row m's sum of squares
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float s = ss[mt];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (g == 0) ssq[kh][mt * 16 + m] = s;
  }
  __syncthreads();  // the x slots are free: their space takes the partial sums
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[kh][mt * 16 + g * 4 + i][m] = (acc[0][mt][i] + acc[1][mt][i]) + acc[2][mt][i];
  __syncthreads();
  // [16 MT tokens x 16 experts]: the eight partial sums in a fixed order, the
  // same for r in every expert tile
  for (int o = tid; o < kRows * 16; o += 64 * kWaves) {
    const int row = o >> 4, n = o & 15;
    float sum = part[0][row][n], tot = ssq[0][row];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      sum += part[w][row][n];
      tot += ssq[w][row];
    }
    const float r = 1.0f / sqrtf(tot / (float)D + a.eps);
    if (t0 + row < a.T && (SPLIT == 1 || (n >> 3) == half)) {
      a.logits[(size_t)(t0 + row) * a.Epad + et * 16 + n] = r * sum + bias_v;  // n == tid % 16
      if (et == 0 && n == 0) a.rnorm[t0 + row] = r;
    }
  }
  // publish: every thread's stores have reached L2 before the counter moves
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const int old = atomicAdd(&a.tile_count[tt], 1);
    is_last = (old == n_eh - 1);
    if (is_last) a.tile_count[tt] = 0;  // ready for the next forward
  }
  __syncthreads();
  if (!is_last) return;
  // Last expert tile of this token tile: the full logit rows come from this
  // XCD's L2 (every writer ran on this XCD and waited for its stores); no
  // workgroup on this CU read these rows earlier in the launch, so its L1
  // holds no stale copy. Wave h takes tokens 4 h .. 4 h + 3 of each 32-token
  // group of the tile, one per 16-lane row.
  for (int tl0 = 4 * kh; tl0 < kRows; tl0 += 4 * kWaves) {
    const int tl = tl0 + (lane >> 4);
    const bool active = t0 + tl < a.T;
    const size_t trow = (size_t)min(t0 + tl, a.T - 1);
    topk_row<NU>(a.logits + trow * a.Epad, active, a.E, a.K, m, a.topk_idx + trow * a.K, a.topk_w + trow * a.K);
  }
}

// Expert input h = x r (1 + gamma_e): one workgroup of 256 threads per token;
// thread i owns the 8-column pieces i, i + 256, ... (up to NP of them:
// d_model <= 2048 NP). All loads of a thread are issued together; one block
// reduction gives r.
template <bool XF32, int NP>
__global__ __launch_bounds__(256) void k_norm(RouterArgs a) {
  __shared__ float wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int D = a.D;
  const int nseg = D / 8;
  const size_t row = (size_t)t * D;
  float f[NP][8];
  float4 ge[NP][2];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int sg = tid + 256 * i;
    if (sg < nseg) {
      if constexpr (XF32) {
        const float4 v0 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + row + sg * 8);
        const float4 v1 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + row + sg * 8 + 4);
        f[i][0] = v0.x; f[i][1] = v0.y; f[i][2] = v0.z; f[i][3] = v0.w;
        f[i][4] = v1.x; f[i][5] = v1.y; f[i][6] = v1.z; f[i][7] = v1.w;
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + row + sg * 8);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f[i][2 * k] = bf16_lo(v[k]);
          f[i][2 * k + 1] = bf16_hi(v[k]);
        }
      }
      ge[i][0] = *reinterpret_cast<const float4*>(a.gamma_e + sg * 8);
      ge[i][1] = *reinterpret_cast<const float4*>(a.gamma_e + sg * 8 + 4);
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < NP; ++i)
    if (tid + 256 * i < nseg)
#pragma unroll
      for (int k = 0; k < 8; ++k) ss = fmaf(f[i][k], f[i][k], ss);
  for (int msk = 32; msk >= 1; msk >>= 1) ss += __shfl_xor(ss, msk);
  if (lane == 0) wsum[wave] = ss;
  __syncthreads();
  const float tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const float r = 1.0f / sqrtf(tot / (float)D + a.eps);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int sg = tid + 256 * i;
    if (sg >= nseg) continue;
    const float g2[8] = {ge[i][0].x, ge[i][0].y, ge[i][0].z, ge[i][0].w, ge[i][1].x, ge[i][1].y, ge[i][1].z, ge[i][1].w};
    u32x4 ho;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float h0 = f[i][2 * k] * r * (1.0f + g2[2 * k]);
      const float h1 = f[i][2 * k + 1] * r * (1.0f + g2[2 * k + 1]);
      ho[k] = a.h_f16 ? pack_f16x2(h0, h1) : pack_bf16x2(h0, h1);
    }
    *reinterpret_cast<u32x4*>(a.h + row + sg * 8) = ho;
  }
}

// Create time: W' = W_r diag(1 + gamma_r) in fp32 (router weight fp32 or
// bf16), split exactly into three bf16 planes, in fragment order: plane p,
// expert tile et, 32-column step s hold one 1 KB block whose lane l = n + 16 g
// has the 8 values of expert 16 et + n at columns 32 s + 8 g .. + 7. Experts
// >= E are zero.
__global__ void k_prep_router_w(const void* __restrict__ w, int w_f32, const float* __restrict__ gamma, int E,
                                int Epad, int D, float* __restrict__ wf) {
  const int nks = D / 32;
  const size_t n_items = (size_t)(Epad / 16) * nks * 64;
  for (size_t it = (size_t)blockIdx.x * blockDim.x + threadIdx.x; it < n_items; it += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(it % 64);
    const size_t blk = it / 64;
    const int s = (int)(blk % nks);
    const int et = (int)(blk / nks);
    const int e = et * 16 + (l & 15);
    const int d0 = s * 32 + (l >> 4) * 8;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float wv = 0.0f;
      if (e < E) {
        const size_t src = (size_t)e * D + d0 + i;
        wv = w_f32 ? static_cast<const float*>(w)[src] : bf16_bits_to_f32(static_cast<const uint16_t*>(w)[src]);
      }
      v[i] = wv * (1.0f + gamma[d0 + i]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<float4*>(wf + blk * 512 + h * 256 + l * 4) =
          make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
  }
}

template <bool XF32, int MT, int G, int SPLIT = 1>
void (*pick_logits(int nu))(RouterArgs) {
  return nu <= 2   ? k_logits<XF32, MT, G, 2, SPLIT>
         : nu <= 4 ? k_logits<XF32, MT, G, 4, SPLIT>
         : nu <= 8 ? k_logits<XF32, MT, G, 8, SPLIT>
                   : k_logits<XF32, MT, G, 16, SPLIT>;
}

}  // namespace

hipError_t launch_norm(const RouterArgs& a, hipStream_t stream, const KernelEvents* ev) {
  void (*kn)(RouterArgs);
  if (a.D <= 2048 * 2)
    kn = a.x_f32 ? k_norm<true, 2> : k_norm<false, 2>;
  else
    kn = a.x_f32 ? k_norm<true, 8> : k_norm<false, 8>;
  return launch_kernel(kn, dim3(a.T), dim3(256), stream, ev, a);
}

hipError_t launch_logits(const RouterArgs& a, hipStream_t stream, const KernelEvents* ev) {
  const int n_et = a.Epad / 16;
  // more m-tiles per workgroup once 16-token tiles would give more than two
  // workgroups per CU: W' is then re-read by fewer workgroups, and the grid
  // fits the chip in one round (T = 2304: 288 workgroups of 64 tokens, 35 us,
  // against 576 of 32 tokens, 38 us)
  const size_t n16 = (size_t)((a.T + 15) / 16) * n_et;
#ifndef DG_LOGITS_MT
  const int mt = n16 <= 512 ? 1 : n16 <= 1024 ? 2 : 4;
#else
  const int mt = DG_LOGITS_MT;
#endif
  const int rows = 16 * (a.x_f32 ? min(mt, 2) : mt);
  const int n_tt = (a.T + rows - 1) / rows;
  // at most 64 workgroups of 16-token tiles: two workgroups per expert tile
  // (T = 32: 128 workgroups of 8 experts, 17.4 against 18.3 us; at T = 256,
  // 256 against 128 workgroups gained nothing)
  const int tiles = kQueues * ((n_tt + kQueues - 1) / kQueues) * n_et;
  const int split = (mt == 1 && tiles <= 64) ? 2 : 1;
  const dim3 grid(tiles * split);
  const int nu = a.Epad / 16;  // 2 .. 16
  void (*k)(RouterArgs);
  if (a.x_f32)  // fp32 x lives in registers: at most two m-tiles
    k = mt == 1 ? (split == 2 ? pick_logits<true, 1, 2, 2>(nu) : pick_logits<true, 1, 2>(nu))
                : pick_logits<true, 2, 1>(nu);
  else
    k = mt == 1   ? (split == 2 ? pick_logits<false, 1, 3, 2>(nu) : pick_logits<false, 1, 3>(nu))
        : mt == 2 ? pick_logits<false, 2, 2>(nu)
                  : pick_logits<false, 4, 1>(nu);
  return launch_kernel(k, grid, dim3(64 * kWaves), stream, ev, a);
}

hipError_t launch_prep_router_w(const void* w, int w_f32, const float* gamma, int E, int Epad, int D,
                                float* wf, hipStream_t stream) {
  k_prep_router_w<<<dim3(512), dim3(256), 0, stream>>>(w, w_f32, gamma, E, Epad, D, wf);
  return hipGetLastError();
}

}  // namespace dg
