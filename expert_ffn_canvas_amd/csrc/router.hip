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
//          Where the expert input has to be materialised (fp32 activations,
//          quantised or borrowed experts), the same kernel also writes
//          h = x r (1 + gamma_e), bf16 (fp16 for int4 and Q8_0 experts): each
//          workgroup of a token tile writes its share of the columns once r is
//          known. Otherwise the gate_up GEMM reads x itself, with (1 + gamma_e)
//          folded into its packed weight and r applied to its sums.
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

constexpr int kWaves = 8;  // waves per workgroup; wave h owns chunks h, h + 8, ... of d_model

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

// The logits of one token for top-k, 16 lanes per token: lane j holds those
// of experts NU j .. NU j + NU - 1, read as whole 16-byte pieces (8 bytes for
// NU = 2). Epad is a multiple of 16, so each lane's range lies either wholly
// inside the row or wholly past it; a lane past it re-reads the row's start
// (those experts are >= E and never picked).
template <int NU>
__device__ __forceinline__ void load_row(const float* row, int j, int Epad, float (&lv)[NU]) {
  j = (NU * j < Epad) ? j : 0;
  if constexpr (NU == 2) {
    const float2 v = *reinterpret_cast<const float2*>(row + 2 * j);
    lv[0] = v.x;
    lv[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < NU / 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(row + NU * j + 4 * i);
      lv[4 * i] = v.x;
      lv[4 * i + 1] = v.y;
      lv[4 * i + 2] = v.z;
      lv[4 * i + 3] = v.w;
    }
  }
}

// Top-k of one token per 16-lane row, from the logits load_row gave lane j.
// Round q takes the largest remaining (logit, lowest id) of the row and
// removes it, so the k rounds produce the selection in slot order (logit
// descending, ties by id). Lane q < k keeps round q's pick and writes slot q
// with its softmax over the k (the shift by the largest logit cancels in the
// renormalisation). A NaN logit ranks below every number; experts >= E are
// never picked.
template <int NU>
__device__ __forceinline__ void topk_row(const float (&lv)[NU], bool active, int E, int K, int j, int32_t* idx_out,
                                         float* w_out) {
  uint32_t key[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const float l = (lv[u] == lv[u]) ? lv[u] : -INFINITY;
    key[u] = (NU * j + u < E) ? float_key(l) : 0u;  // every real expert's key is > 0
  }
  uint32_t my_key = 0, my_id = 0, top = 0;
  for (int q = 0; q < K; ++q) {
    uint32_t bk = key[0], bi = (uint32_t)(NU * j);
#pragma unroll
    for (int u = 1; u < NU; ++u) {
      const bool gt = key[u] > bk;  // strict: on equal keys the lower id stays
      bk = gt ? key[u] : bk;
      bi = gt ? (uint32_t)(NU * j + u) : bi;
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
    const bool own = (int)(bi / NU) == j;
#pragma unroll
    for (int u = 0; u < NU; ++u) key[u] = (own && (int)(bi % NU) == u) ? 0u : key[u];
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

// Top-k of tokens lo .. hi - 1 of the token tile at t0, whose logit rows are
// complete in this XCD's L2. Wave h takes tokens lo + 4 h .. lo + 4 h + 3 of
// each 32-token group, one per 16-lane row; all of a wave's rows are loaded
// before the first selection (one memory round trip). Rows are read at
// clamped indices, so every load is in bounds.
template <int NU, int kPass>
__device__ __forceinline__ void topk_span(const RouterArgs& a, int t0, int lo, int hi, int kh, int lane) {
  const int m = lane & 15;
  float lv[kPass][NU];
#pragma unroll
  for (int it = 0; it < kPass; ++it) {
    const int tl = lo + 4 * kh + 4 * kWaves * it + (lane >> 4);
    if (lo + 4 * kh + 4 * kWaves * it < hi)
      load_row<NU>(a.logits + (size_t)min(t0 + min(tl, hi - 1), a.T - 1) * a.Epad, m, a.Epad, lv[it]);
  }
#pragma unroll
  for (int it = 0; it < kPass; ++it) {
    const int tl = lo + 4 * kh + 4 * kWaves * it + (lane >> 4);
    if (lo + 4 * kh + 4 * kWaves * it >= hi) break;
    const size_t trow = (size_t)min(t0 + min(tl, hi - 1), a.T - 1);
    topk_row<NU>(lv[it], tl < hi && t0 + tl < a.T, a.E, a.K, m, a.topk_idx + trow * a.K, a.topk_w + trow * a.K);
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

// The expert input h = x r (1 + gamma_e) of rows t0 .. t0 + ROWS - 1 (r from
// rs), columns of 8-wide segments [s0, s1): one 16-byte store per segment.
template <bool XF32, int ROWS>
__device__ __forceinline__ void write_h(const RouterArgs& a, const float* rs, int t0, int s0, int s1, int tid,
                                        int nthreads) {
  const int ns = s1 - s0;
  const int D = a.D;
  for (int i = tid; i < ROWS * ns; i += nthreads) {
    const int row = i / ns, sg = s0 + i % ns;
    const int t = t0 + row;
    if (t >= a.T) continue;
    const size_t at = (size_t)t * D + sg * 8;
    float f[8];
    if constexpr (XF32) {
      const float4 v0 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + at);
      const float4 v1 = *reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + at + 4);
      f[0] = v0.x; f[1] = v0.y; f[2] = v0.z; f[3] = v0.w;
      f[4] = v1.x; f[5] = v1.y; f[6] = v1.z; f[7] = v1.w;
    } else {
      const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) + at);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f[2 * k] = bf16_lo(v[k]);
        f[2 * k + 1] = bf16_hi(v[k]);
      }
    }
    const float4 g0 = *reinterpret_cast<const float4*>(a.gamma_e + sg * 8);
    const float4 g1 = *reinterpret_cast<const float4*>(a.gamma_e + sg * 8 + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float r = rs[row];
    u32x4 ho;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float h0 = f[2 * k] * r * (1.0f + g[2 * k]);
      const float h1 = f[2 * k + 1] * r * (1.0f + g[2 * k + 1]);
      ho[k] = a.h_f16 ? pack_f16x2(h0, h1) : pack_bf16x2(h0, h1);
    }
    *reinterpret_cast<u32x4*>(a.h + at) = ho;
  }
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
// (b + c) % 8, c fixed within a launch) and share its L2: each publishes its
// logits with a counter. Either the last to arrive selects the top-k of all
// the tile's tokens, one per 16-lane row, or (a.polls >= 0: tall tiles whose
// launch fits the CUs at once) every workgroup waits, a bounded number of
// polls, for the last arrival and then selects for its own share of the
// tokens: a workgroup that stops waiting marks its share given up, and the
// last arriver, after its own share, takes every share so marked. A share
// is given up before the last arrival or its owner sees that arrival, so
// each share is selected at least once, and twice only with identical
// results. With SPLIT = 2 (few token tiles) each expert tile is shared by two
// workgroups, one per half of its 16 experts: each loads only its half of
// every W' fragment (the other lanes' operands are zero), so the W' bytes a
// CU takes in are halved and twice as many CUs share them.
template <bool XF32, int MT, int G, int NU, int SPLIT, int CH>
__global__ __launch_bounds__(64 * kWaves) void k_logits(RouterArgs a) {
  constexpr int kRows = 16 * MT;
  constexpr int kKK = CH / 32;         // 32-column MFMA steps per chunk
  constexpr int kSeg = CH / 8;         // 16-byte segments per staged row
  constexpr int kRB = CH * 2;          // bytes per staged row
  constexpr int kRPD = 1024 / kRB;     // rows per wave-wide transfer
  static_assert(!XF32 || CH == 128, "fp32 rows are read in 128-column chunks");
  constexpr int kXsBytes = XF32 ? 0 : kWaves * G * MT * 16 * kRB;
  constexpr int kPartBytes = kWaves * kRows * 17 * 4;
  constexpr int kBuf = kXsBytes > kPartBytes ? kXsBytes : kPartBytes;
  __shared__ __attribute__((aligned(16))) char smem[kBuf];
  __shared__ float ssq[kWaves][kRows];
  __shared__ float rs[kRows];  // r of each row
  __shared__ int pick;  // 0: no selection; 1: the whole tile; 2: own share; 3: own share, then those given up
  __shared__ uint32_t given_up;
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
  const int nc = D / CH;
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
    u32x4 wb[G][kKK][2];
    u32x4 xf[XF32 ? G : 1][XF32 ? MT : 1][4][2];
#pragma unroll
    for (int q = 0; q < G; ++q) {
      const int chunk = kh + kWaves * min(c0 + q, n_my - 1);
      const int col = chunk * CH;
      if constexpr (XF32) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float* xr = static_cast<const float*>(a.x) + (size_t)min(t0 + mt * 16 + m, a.T - 1) * D + col + g * 8;
#pragma unroll
          for (int kk = 0; kk < kKK; ++kk) {
            xf[q][mt][kk][0] = *reinterpret_cast<const u32x4*>(xr + kk * 32);
            xf[q][mt][kk][1] = *reinterpret_cast<const u32x4*>(xr + kk * 32 + 4);
          }
        }
      } else {
        const uint32_t base =
            __builtin_amdgcn_readfirstlane(gemm::lds_addr(smem) + (kh * G + q) * MT * 16 * kRB);
        const uint16_t* xb = static_cast<const uint16_t*>(a.x);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 16 / kRPD; ++i) {
            const int r = mt * 16 + kRPD * i + lane / kSeg;
            const int s = (lane % kSeg) ^ (r % kSeg);
            gemm::lds_dma16(base + (mt * 16 + kRPD * i) * kRB, xb + (size_t)min(t0 + r, a.T - 1) * D + col + s * 8);
          }
      }
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          wb[q][kk][h] = wmine ? *reinterpret_cast<const u32x4*>(wfrag + (size_t)(chunk * kKK + kk) * 512 + h * 256)
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
      for (int kk = 0; kk < kKK; ++kk) {
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
            const u32x4 xv = *reinterpret_cast<const u32x4*>(smem + (kh * G + q) * MT * 16 * kRB + r * kRB +
                                                              (((kk * 4 + g) ^ (m % kSeg)) * 16));
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
    if (n == 0) rs[row] = r;
    if (t0 + row < a.T && (SPLIT == 1 || (n >> 3) == half)) {
      a.logits[(size_t)(t0 + row) * a.Epad + et * 16 + n] = r * sum + bias_v;  // n == tid % 16
      if (et == 0 && n == 0) a.rnorm[t0 + row] = r;
    }
  }
  // publish: every thread's stores have reached L2 before the counter moves
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // each arrival also counts under its XCD: the last arriver checks that all
  // of the token tile's workgroups ran on its own (it reads their logits from
  // its L2) and raises DG_DEV_XCD_ROUTER if not. Counters of tile tt: word
  // 16 tt (arrivals) and 16 tt + 1 (shares given up, workgroups done), one
  // 128-byte line per tile, so the tiles' polls and arrivals do not queue on
  // one line.
  const int w = jq % n_eh;  // this workgroup's share: tokens, and columns of h
  unsigned long long* arrive = reinterpret_cast<unsigned long long*>(&a.tile_count[16 * tt]);
  unsigned long long* aux = reinterpret_cast<unsigned long long*>(&a.tile_count[16 * tt + 1]);
  if (tid == 0) {
    const int xcc = xcc_id();
    const unsigned long long mine = 1ull | (1ull << (8 + 6 * xcc));
    const unsigned long long now = atomicAdd(arrive, mine) + mine;
    const bool last = (int)(now & 0xffull) == n_eh;  // n_eh <= 32
    if (last && (int)((now >> (8 + 6 * xcc)) & 63ull) != n_eh) raise_flag(a.dev_flags, DG_DEV_XCD_ROUTER);
    int sel = 0;
    if (a.polls < 0) {
      sel = last ? 1 : 0;
      if (last) *arrive = 0;  // ready for the next forward
    } else if (last) {
      sel = n_eh == 1 ? 1 : 3;
    } else {
      bool seen = false;
      for (int n = 0; n <= a.polls && !seen; ++n) {
        seen = (int)(__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xffull) == n_eh;
        if (!seen && n < a.polls) __builtin_amdgcn_s_sleep(1);
      }
      if (!seen) {
        // give the share up, then look once more: if the last arrival came
        // meanwhile, its arriver may have read the given-up shares already
        atomicOr(aux, 1ull << w);
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        seen = (int)(atomicAdd(arrive, 0ull) & 0xffull) == n_eh;
      }
      sel = seen ? 2 : 0;
    }
    pick = sel;
  }
  __syncthreads();
  const int sel = __builtin_amdgcn_readfirstlane(pick);
  // Selection: the full logit rows come from this XCD's L2 (every writer ran
  // on this XCD and waited for its stores before counting itself); this CU
  // read none of the tile's rows before they were complete, so its L1 holds
  // no stale copy.
  constexpr int kPass = (kRows + 4 * kWaves - 1) / (4 * kWaves);
  if (sel == 1) {
    topk_span<NU, kPass>(a, t0, 0, kRows, kh, lane);
  } else if (sel >= 2) {
    topk_span<NU, kPass>(a, t0, w * kRows / n_eh, (w + 1) * kRows / n_eh, kh, lane);
    if (sel == 3) {
      if (tid == 0) given_up = (uint32_t)atomicAdd(aux, 0ull) & ~(1u << w);  // bits of shares < n_eh <= 16
      __syncthreads();
      for (uint32_t left = __builtin_amdgcn_readfirstlane(given_up); left != 0u; left &= left - 1u) {
        const int sh = __builtin_ctz(left);
        topk_span<NU, kPass>(a, t0, sh * kRows / n_eh, (sh + 1) * kRows / n_eh, kh, lane);
      }
    }
  }
  if (a.polls >= 0 && tid == 0) {
    // the tile's last workgroup to get here, when no other reads the
    // counters any more, clears them for the next forward
    const unsigned long long old = atomicAdd(aux, 1ull << 32);
    if ((int)((old >> 32) & 0xffull) == n_eh - 1) {
      *arrive = 0;
      *aux = 0;
    }
  }
  const int nseg = D / 8;
  if (a.h != nullptr) write_h<XF32, kRows>(a, rs, t0, w * nseg / n_eh, (w + 1) * nseg / n_eh, tid, 64 * kWaves);
}

// Create time: W' = W_r diag(1 + gamma_r) in fp32 (router weight fp32 or
// bf16), in fragment order: expert tile et and 32-column step s hold one 2 KB
// block; lane l = n + 16 g keeps the 8 values of expert 16 et + n at columns
// 32 s + 8 g .. + 7, the first four at floats 4 l .. 4 l + 3 of the block's
// first 1 KB and the last four at the same place in its second 1 KB, so each
// half is one wave-wide 1 KB read. The logits kernel splits each value exactly
// into three bf16 planes in registers as it loads it. Experts >= E are zero.
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

template <bool XF32, int MT, int G, int SPLIT = 1, int CH = 128>
void (*pick_logits(int nu))(RouterArgs) {
  return nu <= 2   ? k_logits<XF32, MT, G, 2, SPLIT, CH>
         : nu <= 4 ? k_logits<XF32, MT, G, 4, SPLIT, CH>
         : nu <= 8 ? k_logits<XF32, MT, G, 8, SPLIT, CH>
                   : k_logits<XF32, MT, G, 16, SPLIT, CH>;
}

}  // namespace

hipError_t launch_logits(const RouterArgs& a, hipStream_t stream, const KernelEvents* ev) {
  const int n_et = a.Epad / 16;
  // Token-tile height, 16 mt rows. A workgroup's time follows the bytes it
  // reads: 16 mt rows of x and 16 rows of W' (fp32, twice a bf16 x row), so
  // it grows as mt + 2 (bf16 x) or mt + 1 (fp32 x); a CU that holds two
  // workgroups takes about twice as long. The launch then takes about
  // ceil(workgroups / CUs) (mt + 2): the height that minimises this, the
  // taller on ties (W' is then re-read by fewer workgroups). T = 2304: 232
  // workgroups of 80 tokens, one round, against 288 of 64 tokens.
#ifndef DG_LOGITS_MT
  static const int kCandBf16[] = {1, 2, 4, 5}, kCandF32[] = {1, 2};
  const int* cand = a.x_f32 ? kCandF32 : kCandBf16;
  const int n_cand = a.x_f32 ? 2 : 4;
  int mt = 1;
  long long best = -1;
  for (int i = 0; i < n_cand; ++i) {
    const long long wgs = (long long)((a.T + 16 * cand[i] - 1) / (16 * cand[i])) * n_et;
    const long long cost = (wgs + a.n_cu - 1) / a.n_cu * (cand[i] + (a.x_f32 ? 1 : 2));
    if (best < 0 || cost <= best) {
      best = cost;
      mt = cand[i];
    }
  }
#else
  const int mt = DG_LOGITS_MT;
#endif
  const int n_tt = (a.T + 16 * mt - 1) / (16 * mt);
  // at most 64 workgroups of 16-token tiles: two workgroups per expert tile
  // (T = 32: 128 workgroups of 8 experts, 17.4 against 18.3 us; at T = 256,
  // 256 against 128 workgroups gained nothing)
  const int tiles = kQueues * ((n_tt + kQueues - 1) / kQueues) * n_et;
  const int split = (mt == 1 && tiles <= 64) ? 2 : 1;
  const dim3 grid(tiles * split);
  // Tiles of 64 or 80 tokens share the top-k out when the whole launch fits
  // the CUs at once (every workgroup of a tile then runs at the same time):
  // up to 64 polls of about a microsecond each before a share is given up.
  RouterArgs ac = a;
  ac.polls = (mt >= 4 && (int)grid.x <= a.n_cu) ? (a.no_wait ? 0 : 64) : -1;
  const int nu = a.Epad / 16;  // 2 .. 16
  void (*k)(RouterArgs);
  if (a.x_f32)  // fp32 x lives in registers: at most two m-tiles
    k = mt == 1 ? (split == 2 ? pick_logits<true, 1, 3, 2>(nu) : pick_logits<true, 1, 3>(nu))
                : pick_logits<true, 2, 1>(nu);
  else  // 16 tokens: one 128-column chunk in flight per wave (32 KB of x stages; with three, 96 KB, the
        // canvas256 router took 12.2 against 10.7 us and the 512-token stack 3 us more per layer: the
        // workgroups of the larger stages started up to 2.7 us apart). From 32 tokens: 64-column chunks,
        // so the x stages take 64 KB (80 KB at 80 tokens)
    k = mt == 1   ? (split == 2 ? pick_logits<false, 1, 1, 2>(nu) : pick_logits<false, 1, 1>(nu))
        : mt == 2 ? pick_logits<false, 2, 2, 1, 64>(nu)
        : mt == 4 ? pick_logits<false, 4, 1, 1, 64>(nu)
                  : pick_logits<false, 5, 1, 1, 64>(nu);
  return launch_kernel(k, grid, dim3(64 * kWaves), stream, ev, ac);
}

hipError_t launch_prep_router_w(const void* w, int w_f32, const float* gamma, int E, int Epad, int D,
                                float* wf, hipStream_t stream) {
  k_prep_router_w<<<dim3(512), dim3(256), 0, stream>>>(w, w_f32, gamma, E, Epad, D, wf);
  return hipGetLastError();
}

}  // namespace dg
