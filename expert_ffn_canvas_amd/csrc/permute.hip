// Token -> expert permutation on gfx950, in one workgroup of 1024 threads:
//  * counts[e]: tokens routed to expert e (their sum is k T);
//  * offsets: exclusive prefix sum of counts (the rows of expert e are
//    offsets[e] .. offsets[e+1]-1 in expert-sorted order);
//  * tiles: each expert's rows cut into ceil(count / 64) tiles of near-equal
//    size. Experts are ranked by count (descending, ties to the lower id) and
//    dealt to the 8 per-XCD queues in snake order (0..7, 7..0, ...), all tiles
//    of one expert into one queue, so every queue gets a similar share of the
//    weight bytes and the tiles of a split expert run on one XCD, where they
//    share that XCD's L2;
//  * the stable scatter: the rows of expert e hold its tokens in increasing
//    token order; sorted_token[row], row_w[row] (that slot's routing weight)
//    and row_of_slot[t k + j].
// Everything stays on the device; the host never reads the counts back.
//
// Source of the per-expert token counts: Quant-Tuner PR "Add DiffusionGemma
// (Gemma-4 MoE block-diffusion) support", "Answers to the motivating
// questions" (MoE entries carry per-expert counts).
#include "dg_common.h"
#include "launch.h"

namespace dg {

namespace {

constexpr int kThreads = 1024;
constexpr int kMaxE = 256;
constexpr int kWords = kThreads / 32;  // bitmap words per expert for one chunk of tokens

__device__ __forceinline__ int snake_queue(int r) {
  const int k = r / kQueues, p = r - k * kQueues;
  return (k & 1) ? (kQueues - 1 - p) : p;
}

__global__ __launch_bounds__(kThreads) void k_permute(PermuteArgs a) {
  __shared__ int cnt[kMaxE];
  __shared__ int base[kMaxE];
  __shared__ int cursor[kMaxE];
  __shared__ int order[kMaxE];
  __shared__ int ntile[kMaxE];
  __shared__ int ctot[kMaxE];
  __shared__ int wsum[kMaxE / 64];
  __shared__ uint32_t bits[kMaxE * kWords];
  __shared__ uint16_t pre[kMaxE * kWords];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, K = a.K, T = a.T;

  // the first chunk of tokens is loaded once and kept for the scatter
  int e[8];
  float w[8];
  {
    const int t = tid;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool v = (t < T) && (j < K);
      e[j] = v ? a.topk_idx[(size_t)t * K + j] : 0;
      w[j] = v ? a.topk_w[(size_t)t * K + j] : 0.0f;
    }
  }

  // --- histogram
  if (tid < kMaxE) cnt[tid] = 0;
  __syncthreads();
  if (tid < T) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < K) atomicAdd(&cnt[e[j]], 1);
  }
  for (int t = tid + kThreads; t < T; t += kThreads) {
    int ee[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ee[j] = (j < K) ? a.topk_idx[(size_t)t * K + j] : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < K) atomicAdd(&cnt[ee[j]], 1);
  }
  __syncthreads();

  // --- exclusive scan of the counts (four waves of 64 experts)
  int c = 0, incl = 0;
  if (tid < kMaxE) {
    c = (tid < E) ? cnt[tid] : 0;
    incl = c;
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
  }
  __syncthreads();
  if (tid < kMaxE) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int excl = before + incl - c;
    base[tid] = excl;
    cursor[tid] = excl;
    if (tid < E) {
      a.offsets[tid] = excl;
      a.counts[tid] = c;
      if (tid == E - 1) a.offsets[E] = excl + c;
      // rank by (count desc, id asc)
      int r = 0;
      for (int e2 = 0; e2 < E; ++e2) {
        const int c2 = cnt[e2];
        r += (c2 > c) || (c2 == c && e2 < tid);
      }
      order[r] = tid;
      ntile[tid] = (c + kTileRows - 1) / kTileRows;
    }
  }
  __syncthreads();

  // --- deal the experts to the queues and write their tiles
  if (tid < E) {
    const int e = order[tid];  // thread tid handles the expert of rank tid
    const int r = tid;
    const int x = snake_queue(r);
    int qoff = 0;
    for (int k = 0; k < r / kQueues; ++k) {
      const int rr = k * kQueues + ((k & 1) ? (kQueues - 1 - x) : x);
      qoff += ntile[order[rr]];
    }
    const int ce = cnt[e], nt = ntile[e];
    for (int i = 0; i < nt; ++i) {
      const int lo = (ce * i) / nt, hi = (ce * (i + 1)) / nt;
      if (qoff + i < a.qmax) {
        Tile tl;
        tl.e = e;
        tl.row0 = base[e] + lo;
        tl.mc = hi - lo;
        tl.pad = 0;
        a.tiles[(size_t)(qoff + i) * kQueues + x] = tl;
      }
    }
  }
  if (tid < kQueues) {
    int len = 0;
    for (int k = 0; k * kQueues < E; ++k) {
      const int rr = k * kQueues + ((k & 1) ? (kQueues - 1 - tid) : tid);
      if (rr < E) len += ntile[order[rr]];
    }
    a.qlen[tid] = min(len, a.qmax);
  }

  // --- stable scatter, kThreads tokens at a time
  for (int c0 = 0; c0 < T; c0 += kThreads) {
    const int t = c0 + tid;
    if (c0 > 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool v = (t < T) && (j < K);
        e[j] = v ? a.topk_idx[(size_t)t * K + j] : 0;
        w[j] = v ? a.topk_w[(size_t)t * K + j] : 0.0f;
      }
    }
    for (int i = tid; i < E * kWords; i += kThreads) bits[i] = 0u;
    __syncthreads();
    const uint32_t my_bit = 1u << (tid & 31);
    const int my_word = tid >> 5;
    if (t < T) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < K) atomicOr(&bits[e[j] * kWords + my_word], my_bit);
    }
    __syncthreads();
    if (tid < E) {
      int run = 0;
      for (int i = 0; i < kWords; ++i) {
        pre[tid * kWords + i] = (uint16_t)run;
        run += __popc(bits[tid * kWords + i]);
      }
      ctot[tid] = run;
    }
    __syncthreads();
    if (t < T) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < K) {
          const int rank = pre[e[j] * kWords + my_word] + __popc(bits[e[j] * kWords + my_word] & (my_bit - 1u));
          const int row = cursor[e[j]] + rank;
          a.sorted_token[row] = t;
          a.row_w[row] = w[j];
          a.row_of_slot[(size_t)t * K + j] = row;
        }
      }
    }
    __syncthreads();
    if (tid < E) cursor[tid] += ctot[tid];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream, const KernelEvents* ev) {
  return launch_kernel(k_permute, dim3(1), dim3(kThreads), stream, ev, a);
}

}  // namespace dg
