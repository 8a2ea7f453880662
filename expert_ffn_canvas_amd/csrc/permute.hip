// Token -> expert permutation on gfx950, in one workgroup of 1024 threads:
//  * counts[e]: tokens routed to expert e (their sum is k T);
//  * offsets: exclusive prefix sum of counts (the rows of expert e are
//    offsets[e] .. offsets[e+1]-1 in expert-sorted order);
//  * the task queues of the two grouped GEMMs. Each expert's rows are cut
//    into ceil(count / 64) tiles of near-equal size; a task is one tile times
//    one column block of the expert's weight. Units (expert, column block),
//    each holding all tiles of that expert for that block, are ranked by
//    expert (count descending, ties to the lower id), then block, and dealt
//    round robin to the 8 per-XCD queues. So the tiles that read the same
//    weight block run together on one XCD and share its L2, and since the
//    unit sizes never grow along the deal, every queue holds the mean load
//    to within one unit;
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

// Number of v in [0, m) with v % kQueues == x (m >= 0, 0 <= x < kQueues).
__device__ __forceinline__ int n_mod(int m, int x) { return m > x ? (m - x + kQueues - 1) / kQueues : 0; }

__global__ __launch_bounds__(kThreads) void k_permute(PermuteArgs a) {
  __shared__ int cnt[kMaxE];
  __shared__ int base[kMaxE];
  __shared__ int cursor[kMaxE];
  __shared__ int order[kMaxE];
  __shared__ int ntile[kMaxE];
  __shared__ int ctot[kMaxE];
  __shared__ int wsum[kMaxE / 64];
  __shared__ int pq[2][kQueues][kMaxE + 1];  // per GEMM and queue: load of the ranks before r
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

  // --- per GEMM g and queue x, the load that the units of experts ranked
  // before r put into x: wave w = 8 g + x scans 4 ranks per lane. Expert rank
  // r owns units r NB .. r NB + NB - 1; unit u goes to queue u % 8 and holds
  // ntile tasks.
  {
    const int g = wave >> 3, x = wave & 7;
    const int NB = a.nb[g];
    int v[4], run = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lane + i;
      v[i] = (r < E) ? ntile[order[r]] * (n_mod((r + 1) * NB, x) - n_mod(r * NB, x)) : 0;
      run += v[i];
    }
    int incl = run;
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    int before = incl - run;
    if (lane == 0) pq[g][x][0] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      before += v[i];
      pq[g][x][4 * lane + i + 1] = before;  // load of ranks 0 .. 4 lane + i
    }
  }
  __syncthreads();
  if (tid < 2 * kQueues) {
    const int g = tid / kQueues, x = tid % kQueues;
    a.qlen[tid] = min(pq[g][x][E], a.qmax[g]);
  }
  // --- the tasks of every unit
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int NB = a.nb[g];
    for (int u = tid; u < E * NB; u += kThreads) {
      const int r = u / NB, nb = u - r * NB;
      const int e = order[r], nt = ntile[e];
      if (nt == 0) continue;
      const int x = u % kQueues;
      const int qoff = pq[g][x][r] + nt * (n_mod(u, x) - n_mod(r * NB, x));
      const int ce = cnt[e];
      for (int i = 0; i < nt; ++i) {
        if (qoff + i >= a.qmax[g]) break;
        const int lo = (ce * i) / nt, hi = (ce * (i + 1)) / nt;
        Tile tl;
        tl.e = e;
        tl.row0 = base[e] + lo;
        tl.mc = hi - lo;
        tl.nb = nb;
        a.tasks[g][(size_t)(qoff + i) * kQueues + x] = tl;
      }
    }
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
