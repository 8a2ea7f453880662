// Token -> expert permutation on gfx950, in 17 to 24 workgroups of 1024
// threads on as many CUs at once. Each builds the histogram and the scan;
// then workgroup g 8 + x (g = 0 for gate_up, 1 for down) ranks the experts,
// deals them and writes task queue x of GEMM g (workgroup 0 also counts and
// offsets), and workgroups 16 .. do the stable scatter, each for a range of
// tokens (one per 1024 tokens, at most 8). The outputs:
//  * counts[e]: tokens routed to expert e (their sum is k T);
//  * offsets: exclusive prefix sum of counts (the rows of expert e are
//    offsets[e] .. offsets[e+1]-1 in expert-sorted order);
//  * the task queues of the two grouped GEMMs. Each expert's rows are cut
//    into ceil(count / R) tiles of near-equal size (R = 64, or 128 for the
//    tall-tile GEMMs); a task is one tile times
//    one column block of the expert's weight. Units (expert, column block),
//    each holding all tiles of that expert for that block, are ranked by
//    expert (count descending, ties to the lower id), then block, and dealt
//    round robin to the 8 per-XCD queues. So the tiles that read the same
//    weight block run together on one XCD and share its L2, and since the
//    unit sizes never grow along the deal, every queue holds the mean load
//    to within one unit. With tall tiles the deal is by expert instead (all
//    column blocks of rank r go to queue r % 8): an expert's tiles then share
//    its activation rows, hundreds of them, in one L2. For the fused GEMM
//    whole experts are dealt so that the queues' tile counts balance (the
//    larger experts in snake order, the rest level by level in id order), or
//    with wide tiles their costs (all experts in snake order of cost), the
//    same expert to the same queue in both task lists, each queue laid out in
//    expert id order, and the per-tile counters of that GEMM are zeroed;
//  * the stable scatter: the rows of expert e hold its slots in increasing
//    token order; sorted_slot[row] = t k + j (token t, slot j) and
//    row_of_slot[t k + j] = row.
// Everything stays on the device; the host never reads the counts back.
//
// Each part runs in one workgroup, and a store instruction whose 64 lanes hit
// 64 different cache lines costs 64 line transactions, so the layout of the
// writes is what bounds it: a queue's tasks are contiguous and written by
// position (each lane finds which unit covers its position), and the sorted
// slots are ranked into LDS and written out in order when they fit.
//
// Source of the per-expert token counts: Quant-Tuner PR "Add DiffusionGemma
// (Gemma-4 MoE block-diffusion) support", "Answers to the motivating
// questions" (MoE entries carry per-expert counts).
#include "dg_common.h"
#include "launch.h"

namespace dg {

namespace {

constexpr int kThreads = 1024;
constexpr int kWavesP = kThreads / 64;
constexpr int kMaxE = 256;
constexpr int kStage = 20480;  // sorted slots staged in LDS (k T up to this many)

// floor(a / b) for a >= 0, 1 <= b < 2^24. Below 2^22 a float reciprocal
// estimate is off by at most one and is corrected to the exact quotient;
// larger numerators (a tile boundary of an expert with very many rows) take
// the 64-bit division.
__device__ __forceinline__ int div_small(long long a, int b) {
  if (a < (1 << 22)) {
    const int ai = (int)a;
    int q = (int)((float)ai * __builtin_amdgcn_rcpf((float)b));
    q -= (q * b > ai);
    q += ((q + 1) * b <= ai);
    return q;
  }
  return (int)(a / b);
}

// Number of v in [0, m) with v % kQueues == x (m >= 0, 0 <= x < kQueues).
__device__ __forceinline__ int n_mod(int m, int x) { return m > x ? (m - x + kQueues - 1) / kQueues : 0; }

// The k expert ids of token t (k <= 8; ids past k are 0).
__device__ __forceinline__ void load_ids(const int32_t* idx, int t, int K, int (&e)[8]) {
  if (K == 8) {
    const int4 a = *reinterpret_cast<const int4*>(idx + (size_t)t * 8);
    const int4 b = *reinterpret_cast<const int4*>(idx + (size_t)t * 8 + 4);
    e[0] = a.x; e[1] = a.y; e[2] = a.z; e[3] = a.w;
    e[4] = b.x; e[5] = b.y; e[6] = b.z; e[7] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (j < K) ? idx[(size_t)t * K + j] : 0;
  }
}

// Inclusive scan over the 64 lanes of a wave, for values >= 0 under + or
// max (0 is the identity of both): row shifts by 1, 2, 4 and 8 scan each
// 16-lane row, then row 0's total is broadcast into row 1 and row 2's into
// row 3, and rows 0-1's total into rows 2 and 3 (gfx9 DPP).
template <bool kMax>
__device__ __forceinline__ int wave_scan(int x) {
  auto op = [](int a, int b) { return kMax ? max(a, b) : a + b; };
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true));   // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true));   // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true));   // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true));   // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return x;
}
// The wave's total (+ or max) of values >= 0, in every lane.
template <bool kMax>
__device__ __forceinline__ int wave_total(int x) {
  return __builtin_amdgcn_readlane(wave_scan<kMax>(x), 63);
}

__device__ __forceinline__ int snake(int h) {
  return ((h / kQueues) & 1) ? kQueues - 1 - h % kQueues : h % kQueues;
}

// Balanced deal of whole experts, in one wave: lane l holds experts
// 4 l .. 4 l + 3 (tile counts v, token counts c) and gets their queues in q.
// v1 is the smallest nonzero tile count. The experts with more tiles
// ("larger") are dealt in snake order (queues 0..7, then 7..0, ...) by id;
// the experts of v1 tiles then fill the least loaded queues level by level,
// in id order: with queue x at level L_x = (tiles so far) / v1, the i-th of
// them takes the i-th smallest pair (L_x + k, x), k = 0, 1, ..., so
// consecutive ones go to different queues.
// Dealt by id, the larger experts can pile up on one queue (under a skew that
// tracks the ids they come nearly in order of size, but not in general). So
// if the most loaded queue then exceeds an even share of all tiles by more
// than the largest expert, the larger experts are dealt again in snake order
// of their rank by token count (descending, ties to the lower id; the larger
// experts hold exactly the ranks before all others): dealt in non-increasing
// size, the snake keeps any two queues within the largest tile count of each
// other. Either way the larger experts leave no queue above the even share
// plus the largest count, and the level filling then leaves none above the
// even share plus twice the largest count (a queue that takes some ends
// below the common level plus 2 v1): the queues' capacity. Deterministic, so
// both task lists agree. Experts without rows get queue 0 (and no tasks).
// sh: 16 ints of LDS for this wave alone. The wave runs the deal with no other
// wave working, straight-line code it fetches once per launch, so the code is
// kept short: the eight queue loads are summed by LDS atomics and the eight
// levels divided in eight lanes, not reduced or divided one by one.
__device__ void deal_balanced(const int (&v)[4], const int* cnt, int E, int lane, int (&q)[4], int* sh) {
  int big = 0, sum = 0, mx = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    big = max(big, v[i] > 0 ? 0x7fffffff - v[i] : 0);
    sum += v[i];
    mx = max(mx, v[i]);
  }
  big = wave_total<true>(big);
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = 0;
  if (big == 0) return;  // no expert has rows
  const int v1 = 0x7fffffff - big, total = wave_total<false>(sum), a_max = wave_total<true>(mx);
  int nh = 0, nt = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    nh += v[i] > v1;
    nt += v[i] == v1;
  }
  // position of each larger expert in the deal: its index among them by id
  int h[4];
  {
    int k = wave_scan<false>(nh) - nh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = (v[i] > v1) ? k : -1;
      k += v[i] > v1;
    }
  }
  int load[kQueues];
  // the tiles each queue takes from the larger experts (integer sums: the
  // same in any order), in every lane
  auto deal_loads = [&]() {
    if (lane < kQueues) sh[lane] = 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (h[i] >= 0) atomicAdd(&sh[snake(h[i])], v[i]);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int4 l0 = *reinterpret_cast<const int4*>(sh), l1 = *reinterpret_cast<const int4*>(sh + 4);
    load[0] = l0.x; load[1] = l0.y; load[2] = l0.z; load[3] = l0.w;
    load[4] = l1.x; load[5] = l1.y; load[6] = l1.z; load[7] = l1.w;
  };
  deal_loads();
  int hmax = 0;
#pragma unroll
  for (int x = 0; x < kQueues; ++x) hmax = max(hmax, load[x]);
  if (hmax > (total + kQueues - 1) / kQueues + a_max) {
    // positions by rank of token count instead (count desc, id asc)
    int ce[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ce[i] = (4 * lane + i < E) ? cnt[4 * lane + i] : 0;
      if (h[i] >= 0) h[i] = 0;
    }
    for (int e0 = 0; e0 < E; e0 += 4) {
      const int4 c4 = *reinterpret_cast<const int4*>(&cnt[e0]);  // the same address in every lane
      const int cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          h[i] += (h[i] >= 0 && e0 + k < E && (cc[k] > ce[i] || (cc[k] == ce[i] && e0 + k < 4 * lane + i)));
    }
    deal_loads();
  }
  // levels of the queues after the larger experts, and the level filling:
  // the first tail expert of this lane (index i0 among them by id) takes the
  // largest level lam with C(lam) = sum_x max(0, lam - L_x) <= i0 and the
  // (i0 - C(lam))-th queue (by index) at or below it; each later one the next
  // queue at that level, or the first at the next level.
  // queue x's level, divided in lane x
  if (lane < kQueues) sh[kQueues + lane] = div_small(sh[lane], v1);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int lv[kQueues], lmin = 0x7fffffff;
  {
    const int4 a0 = *reinterpret_cast<const int4*>(sh + kQueues), a1 = *reinterpret_cast<const int4*>(sh + kQueues + 4);
    lv[0] = a0.x; lv[1] = a0.y; lv[2] = a0.z; lv[3] = a0.w;
    lv[4] = a1.x; lv[5] = a1.y; lv[6] = a1.z; lv[7] = a1.w;
  }
#pragma unroll
  for (int x = 0; x < kQueues; ++x) lmin = min(lmin, lv[x]);
  const int i0 = wave_scan<false>(nt) - nt;
  int lo = lmin, hi = lmin + i0;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    int c = 0;
#pragma unroll
    for (int x = 0; x < kQueues; ++x) c += max(0, mid - lv[x]);
    if (c <= i0) lo = mid; else hi = mid - 1;
  }
  int c = 0;
#pragma unroll
  for (int x = 0; x < kQueues; ++x) c += max(0, lo - lv[x]);
  int j = i0 - c;  // index among the queues at or below level lo
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (v[i] > v1) {
      q[i] = snake(h[i]);
    } else if (v[i] == v1) {
      int n = 0, pick = 0;
#pragma unroll
      for (int x = 0; x < kQueues; ++x) {
        if (lv[x] <= lo) {
          if (n == j) pick = x;
          ++n;
        }
      }
      q[i] = pick;
      if (++j == n) {  // the level is used up: on to the next
        ++lo;
        j = 0;
      }
    }
  }
}

// Rank of each expert by (key desc, id asc), four lanes per expert: lane q
// reads the keys 16 i + 4 q .. + 3 (consecutive lanes, consecutive banks)
// and compares against them. Calls rank_out(e, r) for e < E.
template <typename Out>
__device__ __forceinline__ void rank_experts(const int* cnt, int E, int tid, Out rank_out) {
  const int e = tid >> 2, q = tid & 3;
  if (e >= E) return;  // threads past the last expert (an expert's 4 lanes leave together)
  const int ce = cnt[e];
  int r = 0;
#pragma unroll
  for (int i = 0; i < kMaxE / 16; ++i) {
    if (16 * i >= E) break;
    const int4 c4 = *reinterpret_cast<const int4*>(&cnt[16 * i + 4 * q]);
    const int cc[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e2 = 16 * i + 4 * q + k;
      r += (e2 < E) && ((cc[k] > ce) || (cc[k] == ce && e2 < e));
    }
  }
  r += __shfl_xor(r, 1);
  r += __shfl_xor(r, 2);
  if (q == 0) rank_out(e, r);
}

// Workgroups that share the stable scatter: the tokens are split into this
// many contiguous ranges of at least kScatterMin tokens (at most kMaxScatter
// ranges), one per workgroup, each starting from the rows the earlier tokens
// take.
constexpr int kMaxScatter = 8;
constexpr int kScatterMin = 256;
__host__ __device__ inline int scatter_groups(int T) {
  const int n = (T + kScatterMin - 1) / kScatterMin;
  return n < kMaxScatter ? (n > 0 ? n : 1) : kMaxScatter;
}

// The stable scatter of tokens [t0, t1), kThreads at a time: lane masks per
// (wave, expert) give each slot its rank among the chunk's earlier tokens;
// cursor[e] starts at the first row of expert e these tokens take (cstart).
// With `staged`, the slots go to LDS compactly, expert e's run at soff[e],
// each with its expert in the top bits (slot < K T <= 2^23, expert < 256),
// and are written out in order at the end.
__device__ __forceinline__ void scatter(const PermuteArgs& a, int (&ids)[8], int t0, int t1, int* cursor,
                                        const int* cstart, const int* soff, int n_mine,
                                        uint64_t (*masks)[kMaxE], int (*wpre)[kMaxE], int* stage, bool staged,
                                        int tid, int lane, int wave) {
  const int E = a.E, K = a.K;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int c0 = t0; c0 < t1; c0 += kThreads) {
    const int t = c0 + tid;
    if (c0 > 0 && t < t1) load_ids(a.topk_idx, t, K, ids);
    for (int i = lane; i < E; i += 64) masks[wave][i] = 0ull;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (t < t1) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < K) atomicOr(reinterpret_cast<unsigned long long*>(&masks[wave][ids[j]]), 1ull << lane);
    }
    __syncthreads();
    if (tid < E) {
      int run = cursor[tid];
#pragma unroll
      for (int w = 0; w < kWavesP; ++w) {
        wpre[w][tid] = run;
        run += __popcll(masks[w][tid]);
      }
      cursor[tid] = run;
    }
    __syncthreads();
    if (t < t1) {
      int rows[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < K) {
          const int ej = ids[j];
          rows[j] = wpre[wave][ej] + __popcll(masks[wave][ej] & below);
          const int slot = t * K + j;
          if (staged)
            stage[soff[ej] + rows[j] - cstart[ej]] = (ej << 23) | slot;
          else
            a.sorted_slot[rows[j]] = slot;
        } else {
          rows[j] = 0;
        }
      }
      if (K == 8) {
        *reinterpret_cast<int4*>(a.row_of_slot + (size_t)t * 8) = make_int4(rows[0], rows[1], rows[2], rows[3]);
        *reinterpret_cast<int4*>(a.row_of_slot + (size_t)t * 8 + 4) = make_int4(rows[4], rows[5], rows[6], rows[7]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < K) a.row_of_slot[(size_t)t * K + j] = rows[j];
      }
    }
    __syncthreads();
  }
  if (staged) {
    for (int i = tid; i < n_mine; i += kThreads) {
      const int v = stage[i], e = v >> 23;
      a.sorted_slot[cstart[e] + (i - soff[e])] = v & ((1 << 23) - 1);
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_permute(PermuteArgs a) {
  // (16-byte aligned: wave 0 moves four experts per lane at a time)
  __shared__ __attribute__((aligned(16))) int cnt[kMaxE];
  __shared__ __attribute__((aligned(16))) int base[kMaxE];
  __shared__ __attribute__((aligned(16))) int cursor[kMaxE];
  __shared__ __attribute__((aligned(16))) int order[kMaxE];  // expert of each rank (the balanced deal: rank = id)
  __shared__ __attribute__((aligned(16))) int ntile[kMaxE];
  __shared__ __attribute__((aligned(16))) int dcost[kMaxE];  // wide tiles: the deal's cost of each expert
  __shared__ __attribute__((aligned(16))) int qof[kMaxE];    // wide tiles: the queue of each expert
  __shared__ int pq[1][kMaxE + 1];            // this queue: load of the ranks before r
  __shared__ uint64_t masks[kWavesP][kMaxE];  // per wave and expert: lanes whose token has it
  __shared__ int wpre[kWavesP][kMaxE];        // first row of (wave, expert) in the chunk
  __shared__ int stage[kStage];
  __shared__ __attribute__((aligned(16))) int before[kMaxE];  // scatter: slots of expert e in earlier tokens
  __shared__ __attribute__((aligned(16))) int mine[kMaxE];    // scatter: slots of expert e in this range
  __shared__ int soff[kMaxE + 4];                             // scatter: start of expert e's run in the stage
  __shared__ __attribute__((aligned(16))) int dscratch[16];   // the balanced deal's queue loads and levels

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, K = a.K, T = a.T;
  const int role = blockIdx.x;  // 0 .. 15: queue role % 8 of GEMM role / 8; from 16: the scatter
  // a scatter workgroup's token range [t0, t1)
  const bool scat = role >= 2 * kQueues;
  int t0 = 0, t1 = 0;
  if (scat) {
    const int S = scatter_groups(T), s = role - 2 * kQueues;
    t0 = (int)((long)s * T / S);
    t1 = (int)((long)(s + 1) * T / S);
  }
  const bool staged = (size_t)K * (t1 - t0) <= (size_t)kStage;

  // the first chunk of tokens is loaded once and kept for the scatter
  int ids[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (tid < T) load_ids(a.topk_idx, tid, K, ids);

  // --- histogram (a scatter workgroup also counts the slots before its range and in it)
  if (tid < kMaxE) {
    cnt[tid] = 0;
    before[tid] = 0;
    mine[tid] = 0;
  }
  __syncthreads();
  if (tid < T) {
    int* part = (scat && tid < t0) ? before : (scat && tid < t1) ? mine : nullptr;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < K) {
        atomicAdd(&cnt[ids[j]], 1);
        if (part) atomicAdd(&part[ids[j]], 1);
      }
    }
  }
  for (int t = tid + kThreads; t < T; t += kThreads) {
    int ee[8];
    load_ids(a.topk_idx, t, K, ee);
    int* part = (scat && t < t0) ? before : (scat && t < t1) ? mine : nullptr;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < K) {
        atomicAdd(&cnt[ee[j]], 1);
        if (part) atomicAdd(&part[ee[j]], 1);
      }
    }
  }
  __syncthreads();

  // --- exclusive scan of the counts, in wave 0 (lane l: experts 4 l .. 4 l + 3)
  int v[4] = {0, 0, 0, 0};  // wave 0: tile counts of the lane's experts
  if (wave == 0) {
    const int4 c4 = *reinterpret_cast<const int4*>(&cnt[4 * lane]);
    const int c[4] = {c4.x, c4.y, c4.z, c4.w};  // zero for experts >= E
    const int sum = (c[0] + c[1]) + (c[2] + c[3]);
    int run = wave_scan<false>(sum) - sum;
    int b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      b[i] = run;
      v[i] = (c[i] + a.tile_rows - 1) / a.tile_rows;
      if (role == 0 && e < E) {  // counts and offsets: the first task-list workgroup
        a.offsets[e] = run;
        a.counts[e] = c[i];
        if (e == E - 1) a.offsets[E] = run + c[i];
      }
      run += c[i];
    }
    *reinterpret_cast<int4*>(&base[4 * lane]) = make_int4(b[0], b[1], b[2], b[3]);
    *reinterpret_cast<int4*>(&cursor[4 * lane]) = make_int4(b[0], b[1], b[2], b[3]);
    *reinterpret_cast<int4*>(&ntile[4 * lane]) = make_int4(v[0], v[1], v[2], v[3]);
    if (a.deal == kDealBalanced && a.tile_rows == kWideRows) {
      int k4[4];  // the cost of each expert for the deal of wide tiles (0 without rows)
#pragma unroll
      for (int i = 0; i < 4; ++i) k4[i] = v[i] > 0 ? kTileCost * v[i] + c[i] : 0;
      *reinterpret_cast<int4*>(&dcost[4 * lane]) = make_int4(k4[0], k4[1], k4[2], k4[3]);
    }
  }
  if (role == 0 && tid < 2) a.qlen[2 * kQueues + tid] = a.qmax[tid];  // the queue capacities, for inspection
  if (scat) {
    // the range's first row of each expert (kept in base: cursor advances),
    // and the runs of its slots in the stage
    if (wave == 0) {
      const int4 b4 = *reinterpret_cast<const int4*>(&base[4 * lane]);
      const int4 p4 = *reinterpret_cast<const int4*>(&before[4 * lane]);
      const int4 m4 = *reinterpret_cast<const int4*>(&mine[4 * lane]);
      const int4 st = make_int4(b4.x + p4.x, b4.y + p4.y, b4.z + p4.z, b4.w + p4.w);
      *reinterpret_cast<int4*>(&base[4 * lane]) = st;
      *reinterpret_cast<int4*>(&cursor[4 * lane]) = st;
      const int m[4] = {m4.x, m4.y, m4.z, m4.w};
      const int sum = (m[0] + m[1]) + (m[2] + m[3]);
      int run = wave_scan<false>(sum) - sum;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        soff[4 * lane + i] = run;
        run += m[i];
      }
      if (lane == 63) soff[kMaxE] = run;  // experts >= E have no slots: soff[E] is the range's slot count
    }
    __syncthreads();
    scatter(a, ids, t0, t1, cursor, base, soff, soff[kMaxE], masks, wpre, stage, staged, tid, lane, wave);
    return;
  }
  // --- the deal, and queue x of GEMM g: the load that the units of the
  // experts ranked before r put into it (wave 0, 4 ranks per lane). Expert
  // rank r owns units r NB .. r NB + NB - 1; unit u goes to queue u % 8 (or,
  // dealing by expert, all of them to queue r % 8 or, balanced, to the
  // expert's queue) and holds ntile tasks. The unit deal and the deal by
  // expert lay their queues out in the experts' order by count; the balanced
  // deal lays them out in id order.
  const int g = role / kQueues, x = role % kQueues;
  const int NB = a.nb[g];
  int* pre = pq[0];
  int w4[4];
  const bool wide = a.deal == kDealBalanced && a.tile_rows == kWideRows;
  if (a.deal == kDealBalanced && !wide) {
    if (wave == 0) {
      int q[4];
      deal_balanced(v, cnt, E, lane, q, dscratch);
#pragma unroll
      for (int i = 0; i < 4; ++i) w4[i] = (q[i] == x) ? v[i] * NB : 0;
      *reinterpret_cast<int4*>(&order[4 * lane]) = make_int4(4 * lane, 4 * lane + 1, 4 * lane + 2, 4 * lane + 3);
    }
  } else {
    // Experts ranked by count (the unit deal, the deal by expert: their queue
    // order), or with wide tiles by cost, dealt in snake order of that rank
    // (descending, ties to the lower id). A wide tile's tasks take about
    // kTileCost rows' time plus their rows, so balancing the tile counts
    // alone left the queues up to one tile and its rows apart (2304 tokens:
    // 140 tiles over 8 queues, the last ended 35 us after the first; by cost
    // the launch takes 343 against 353 us).
    __syncthreads();
    rank_experts(wide ? dcost : cnt, E, tid, [&](int e, int r) {
      if (wide)
        qof[e] = snake(r);
      else
        order[r] = e;
    });
    __syncthreads();
    if (wave == 0) {
      if (wide) {
        const int4 q4 = *reinterpret_cast<const int4*>(&qof[4 * lane]);
        const int q[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) w4[i] = (v[i] > 0 && q[i] == x) ? v[i] * NB : 0;
        *reinterpret_cast<int4*>(&order[4 * lane]) = make_int4(4 * lane, 4 * lane + 1, 4 * lane + 2, 4 * lane + 3);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * lane + i;
          const int units = a.deal == kDealUnits ? n_mod((r + 1) * NB, x) - n_mod(r * NB, x)
                                                 : ((r % kQueues == x) ? NB : 0);
          w4[i] = (r < E) ? ntile[order[r]] * units : 0;
        }
      }
    }
  }
  if (wave == 0) {
    const int run = (w4[0] + w4[1]) + (w4[2] + w4[3]);
    int before = wave_scan<false>(run) - run;
    if (lane == 0) pre[0] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      before += w4[i];
      pre[4 * lane + i + 1] = before;  // load of ranks 0 .. 4 lane + i
    }
  }
  __syncthreads();
  const int len = min(pre[E], a.qmax[g]);
  if (tid == 0) {
    a.qlen[g * kQueues + x] = len;
    if (pre[E] > a.qmax[g]) raise_flag(a.dev_flags, DG_DEV_QUEUE_OVERFLOW);
  }

  // --- the tasks of the queue, one lane per position p, stored at
  // tasks[x qmax + p] (consecutive lanes, consecutive entries). The lane
  // needs the expert rank r whose units cover p: a table of the rank at every
  // position (one lane per rank fills its positions) for the unit deal, where
  // each rank holds a few; else a binary search on the queue's prefix. Then
  // it finds the unit and the tile inside it.
  Tile* out = a.tasks[g] + (size_t)x * a.qmax[g];
  const bool table = a.deal == kDealUnits && len <= kStage;
  if (table) {
    for (int r = tid; r < E; r += kThreads) {
      const int p1 = min(pre[r + 1], len);
      for (int p = pre[r]; p < p1; ++p) stage[p] = r;
    }
    __syncthreads();
  }
  const bool by_unit = a.deal == kDealUnits;
  for (int p = tid; p < len; p += kThreads) {
    int r;
    if (table) {
      r = stage[p];
    } else {
      int lo = 0, hi = E;  // pre[lo] <= p < pre[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= p) lo = mid; else hi = mid;
      }
      r = lo;
    }
    const int e = order[r], nt = ntile[e];
    const int local = p - pre[r];
    const int m = div_small(local, nt), i = local - m * nt;
    const int nb0 = by_unit ? (x - (r * NB) % kQueues + kQueues) % kQueues : 0;
    const int nb_step = by_unit ? kQueues : 1;
    const int ce = cnt[e];
    Tile tl;
    tl.e = e;
    const int r0 = div_small((long long)ce * i, nt), r1 = div_small((long long)ce * (i + 1), nt);
    tl.row0 = base[e] + r0;
    tl.mc = r1 - r0;
    tl.nb = nb0 + nb_step * m;
    out[p] = tl;
    if (g == 0 && a.tile_done != nullptr && tl.nb == 0) a.tile_done[tl.row0] = 0;
  }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream, const KernelEvents* ev) {
  return launch_kernel(k_permute, dim3(2 * kQueues + scatter_groups(a.T)), dim3(kThreads), stream, ev, a);
}

}  // namespace dg
