// Token -> expert permutation on gfx950, in one workgroup:
//  * counts[e]: tokens routed to expert e (their sum is k T);
//  * offsets: exclusive prefix sum of counts;
//  * the tile list: each expert's rows cut into tiles of at most BM rows,
//    experts ordered by decreasing count (ties: lower id) so that the
//    heaviest tiles are dispatched first;
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

__global__ __launch_bounds__(kThreads) void k_permute(PermuteArgs a) {
  __shared__ int cnt[kMaxE];
  __shared__ int base[kMaxE];
  __shared__ int order[kMaxE];
  __shared__ int tstart[kMaxE];
  __shared__ int ctot[kMaxE];
  __shared__ uint32_t bits[kMaxE * kWords];
  __shared__ uint16_t pre[kMaxE * kWords];

  const int tid = threadIdx.x;
  const int E = a.E, K = a.K, T = a.T, BM = a.BM;
  const int n_slots = T * K;

  if (tid < kMaxE) cnt[tid] = 0;
  __syncthreads();
  for (int s = tid; s < n_slots; s += kThreads) atomicAdd(&cnt[a.topk_idx[s]], 1);
  __syncthreads();

  if (tid < E) {
    // rank of expert tid by (count desc, id asc)
    const int c = cnt[tid];
    int r = 0;
    for (int e2 = 0; e2 < E; ++e2) {
      const int c2 = cnt[e2];
      r += (c2 > c) || (c2 == c && e2 < tid);
    }
    order[r] = tid;
    a.counts[tid] = c;
  }
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      base[e] = run;
      a.offsets[e] = run;
      run += cnt[e];
    }
    a.offsets[E] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int r = 0; r < E; ++r) {
      const int e = order[r];
      tstart[e] = run;
      run += (cnt[e] + BM - 1) / BM;
    }
    *a.n_tiles = run;
  }
  __syncthreads();
  if (tid < E) {
    const int e = tid, c = cnt[e];
    const int nt = (c + BM - 1) / BM;
    for (int i = 0; i < nt; ++i) {
      Tile tl;
      tl.e = e;
      tl.row0 = base[e] + i * BM;
      tl.mc = min(BM, c - i * BM);
      tl.pad = 0;
      a.tiles[tstart[e] + i] = tl;
    }
  }

  // stable scatter, kThreads tokens at a time
  for (int c0 = 0; c0 < T; c0 += kThreads) {
    for (int w = tid; w < E * kWords; w += kThreads) bits[w] = 0u;
    __syncthreads();
    const int t = c0 + tid;
    const uint32_t my_bit = 1u << (tid & 31);
    const int my_word = tid >> 5;
    if (t < T) {
      for (int j = 0; j < K; ++j) atomicOr(&bits[a.topk_idx[t * K + j] * kWords + my_word], my_bit);
    }
    __syncthreads();
    if (tid < E) {
      int run = 0;
      for (int w = 0; w < kWords; ++w) {
        pre[tid * kWords + w] = (uint16_t)run;
        run += __popc(bits[tid * kWords + w]);
      }
      ctot[tid] = run;
    }
    __syncthreads();
    if (t < T) {
      for (int j = 0; j < K; ++j) {
        const int e = a.topk_idx[t * K + j];
        const int rank = pre[e * kWords + my_word] + __popc(bits[e * kWords + my_word] & (my_bit - 1u));
        const int row = base[e] + rank;
        a.sorted_token[row] = t;
        a.row_w[row] = a.topk_w[t * K + j];
        a.row_of_slot[t * K + j] = row;
      }
    }
    __syncthreads();
    if (tid < E) base[tid] += ctot[tid];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  k_permute<<<dim3(1), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace dg
