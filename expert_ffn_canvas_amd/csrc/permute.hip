// Token -> expert permutation on gfx950, in 17 workgroups of 1024 threads on
// 17 CUs at once. Each builds the histogram and the scan; then workgroup
// g 8 + x (g = 0 for gate_up, 1 for down) ranks the experts, deals them and
// writes task queue x of GEMM g (workgroup 0 also counts and offsets), and
// workgroup 16 does the stable scatter. The outputs:
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
//    larger experts in snake order, the rest level by level in id order), the same
//    expert to the same queue in both task lists, each queue laid out in
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

// Balanced deal of whole experts: qof[e] = queue of expert e. v1 is the
// smallest nonzero tile count. The experts with more tiles ("larger") are
// dealt in snake order (queues 0..7, then 7..0, ...) by id; the experts of v1
// tiles then fill the least loaded queues level by level, in id order: with
// queue q at level Lq = (tiles so far) / v1, the i-th of them takes the i-th
// smallest pair (Lq + k, q), k = 0, 1, ..., found by a binary search on the
// level, so consecutive ones go to different queues.
// Dealt by id, the larger experts can pile up on one queue (under a skew that
// tracks the ids they come nearly in order of size, but not in general). So
// if the most loaded queue then exceeds an even share of all tiles by more
// than the largest expert, the larger experts are dealt again in snake order
// of their rank by count (descending, ties to the lower id; the larger
// experts hold exactly the ranks before all others; rank fills crank): dealt
// in non-increasing size, the snake keeps any two queues within the largest
// tile count of each other. Either way the larger experts leave no queue
// above the even share plus the largest count, and the level filling then
// leaves none above the even share plus twice the largest count (a queue that
// takes some ends below the common level plus 2 v1): the queues' capacity.
// Deterministic, so both task lists agree. Called by every thread of the
// block; expert e is thread e.
template <typename Rank>
__device__ void deal_balanced(const int* ntile, int* crank, int E, int tid, int lane, int wave, int* qof, int* sh,
                              Rank rank) {
  int* load = sh;       // [kQueues] tiles of the larger experts per queue
  int* wmin = sh + 8;   // [4] per wave: smallest nonzero count
  int* hcnt = sh + 12;  // [4] per wave: larger experts
  int* tcnt = sh + 16;  // [4] per wave: experts of v1 tiles
  int* wsum = sh + 20;  // [4] per wave: tiles
  int* wmax = sh + 24;  // [4] per wave: largest count
  const int e = tid;
  const bool mine = wave < kMaxE / 64;
  const int v = (e < E) ? ntile[e] : 0;
  if (tid < kQueues) load[tid] = 0;
  if (mine) {
    int m = v > 0 ? v : 0x7fffffff, sm = v, mx = v;
    for (int d = 32; d >= 1; d >>= 1) {
      m = min(m, __shfl_xor(m, d));
      sm += __shfl_xor(sm, d);
      mx = max(mx, __shfl_xor(mx, d));
    }
    if (lane == 0) {
      wmin[wave] = m;
      wsum[wave] = sm;
      wmax[wave] = mx;
    }
  }
  __syncthreads();
  const int v1 = min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3]));
  if (v1 == 0x7fffffff) return;  // no expert has rows
  const int total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  const int a_max = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const bool heavy = mine && v > v1, tail = mine && v == v1;
  const uint64_t below = (1ull << lane) - 1ull;
  uint64_t hb = 0, tb = 0;
  if (mine) {
    hb = __ballot(heavy);
    tb = __ballot(tail);
    if (lane == 0) {
      hcnt[wave] = __popcll(hb);
      tcnt[wave] = __popcll(tb);
    }
  }
  __syncthreads();
  int hbase = 0, tbase = 0;
  for (int w = 0; w < kMaxE / 64; ++w) {
    hbase += (w < wave) ? hcnt[w] : 0;
    tbase += (w < wave) ? tcnt[w] : 0;
  }
  auto snake = [](int h) { return ((h / kQueues) & 1) ? kQueues - 1 - h % kQueues : h % kQueues; };
  if (heavy) atomicAdd(&load[snake(hbase + __popcll(hb & below))], v);
  __syncthreads();
  int hmax = 0;
#pragma unroll
  for (int q = 0; q < kQueues; ++q) hmax = max(hmax, load[q]);
  if (hmax > (total + kQueues - 1) / kQueues + a_max) {
    // the larger experts again, in order of size (the same decision in every thread)
    rank(crank);
    __syncthreads();
    if (tid < kQueues) load[tid] = 0;
    __syncthreads();
    if (heavy) atomicAdd(&load[snake(crank[e])], v);
    __syncthreads();
  }
  if (heavy) qof[e] = snake(crank[e] >= 0 ? crank[e] : hbase + __popcll(hb & below));
  if (tail) {
    const int i = tbase + __popcll(tb & below);
    int lv[kQueues], lmin = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < kQueues; ++q) {
      lv[q] = div_small(load[q], v1);
      lmin = min(lmin, lv[q]);
    }
    // the largest level lam with C(lam) <= i, C(lam) = sum_q max(0, lam - Lq)
    int lo = lmin, hi = lmin + i;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      int c = 0;
#pragma unroll
      for (int q = 0; q < kQueues; ++q) c += max(0, mid - lv[q]);
      if (c <= i) lo = mid; else hi = mid - 1;
    }
    int c = 0;
#pragma unroll
    for (int q = 0; q < kQueues; ++q) c += max(0, lo - lv[q]);
    int j = i - c, pick = 0;
#pragma unroll
    for (int q = 0; q < kQueues; ++q) {  // the j-th queue (by index) at or below level lo
      if (lv[q] <= lo) {
        if (j == 0) pick = q;
        --j;
      }
    }
    qof[e] = pick;
  }
}

// Rank of each expert by (count desc, id asc), four lanes per expert: lane q
// reads the counts 16 i + 4 q .. + 3 (consecutive lanes, consecutive banks)
// and compares against them. Calls rank_out(e, r) for e < E.
template <typename Out>
__device__ __forceinline__ void rank_experts(const int* cnt, int E, int tid, Out rank_out) {
  const int e = tid >> 2, q = tid & 3;
  const int ce = (e < E) ? cnt[e] : 0;
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
  if (q == 0 && e < E) rank_out(e, r);
}

// The stable scatter, kThreads tokens at a time: lane masks per (wave,
// expert) give each slot its rank among the chunk's earlier tokens.
__device__ __forceinline__ void scatter(const PermuteArgs& a, int (&ids)[8], int* cursor,
                                        uint64_t (*masks)[kMaxE], int (*wpre)[kMaxE], int* stage, bool staged,
                                        int tid, int lane, int wave) {
  const int E = a.E, K = a.K, T = a.T;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < T; c0 += kThreads) {
    const int t = c0 + tid;
    if (c0 > 0 && t < T) load_ids(a.topk_idx, t, K, ids);
    for (int i = lane; i < E; i += 64) masks[wave][i] = 0ull;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (t < T) {
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
    if (t < T) {
      int rows[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < K) {
          const int ej = ids[j];
          rows[j] = wpre[wave][ej] + __popcll(masks[wave][ej] & below);
          const int slot = t * K + j;
          if (staged)
            stage[rows[j]] = slot;
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
    const int n = K * T;
    for (int i = tid; i < n; i += kThreads) a.sorted_slot[i] = stage[i];
  }
}

__global__ __launch_bounds__(kThreads) void k_permute(PermuteArgs a) {
  __shared__ int cnt[kMaxE];
  __shared__ int base[kMaxE];
  __shared__ int cursor[kMaxE];
  __shared__ int order[kMaxE];
  __shared__ int crank[kMaxE];  // kDealBalanced: rank of each expert by (count desc, id asc)
  __shared__ int qof[kMaxE];  // kDealBalanced: queue of each expert (rank = id)
  __shared__ int dshare[32];  // kDealBalanced: queue loads and per-wave counts
  __shared__ int ntile[kMaxE];
  __shared__ int wsum[kMaxE / 64];
  __shared__ int pq[1][kMaxE + 1];            // this queue: load of the ranks before r
  __shared__ uint64_t masks[kWavesP][kMaxE];  // per wave and expert: lanes whose token has it
  __shared__ int wpre[kWavesP][kMaxE];        // first row of (wave, expert) in the chunk
  __shared__ int stage[kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, K = a.K, T = a.T;
  const int role = blockIdx.x;  // 0 .. 15: queue role % 8 of GEMM role / 8; 16: the scatter
  const bool staged = (size_t)K * T <= (size_t)kStage;

  // the first chunk of tokens is loaded once and kept for the scatter
  int ids[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (tid < T) load_ids(a.topk_idx, tid, K, ids);

  // --- histogram
  if (tid < kMaxE) cnt[tid] = 0;
  __syncthreads();
  if (tid < T) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < K) atomicAdd(&cnt[ids[j]], 1);
  }
  for (int t = tid + kThreads; t < T; t += kThreads) {
    int ee[8];
    load_ids(a.topk_idx, t, K, ee);
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
      if (role == 0) {  // counts and offsets: the first task-list workgroup
        a.offsets[tid] = excl;
        a.counts[tid] = c;
        if (tid == E - 1) a.offsets[E] = excl + c;
      }
      ntile[tid] = (c + a.tile_rows - 1) / a.tile_rows;
    }
  }
  if (role == 0 && tid < 2) a.qlen[2 * kQueues + tid] = a.qmax[tid];  // the queue capacities, for inspection
  if (role == 2 * kQueues) {
    scatter(a, ids, cursor, masks, wpre, stage, staged, tid, lane, wave);
    return;
  }
  // --- the deal. The unit deal and the deal by expert lay their queues out in
  // the experts' order by count; the balanced deal lays them out in id order
  // and deals its larger experts by id, which is fast and almost always within
  // the queues' capacity. If it is not (the largest queue, in tasks of either
  // GEMM, over that GEMM's capacity), the larger experts are dealt again in
  // order of size, which provably fits (the capacity's bound). Both task-list
  // workgroups of a queue take the same decision.
  if (a.deal == kDealBalanced) {
    if (tid < kMaxE) {
      order[tid] = tid;
      qof[tid] = 0;
      crank[tid] = -1;  // no rank by size unless the deal by id is set aside
    }
    __syncthreads();
    deal_balanced(ntile, crank, E, tid, lane, wave, qof, dshare,
                  [&](int* cr) { rank_experts(cnt, E, tid, [&](int e, int r) { cr[e] = r; }); });
  } else {
    rank_experts(cnt, E, tid, [&](int e, int r) { order[r] = e; });
  }
  __syncthreads();

  // --- queue x of GEMM g: the load that the units of the experts ranked
  // before r put into it (one wave, 4 ranks per lane). Expert rank r owns
  // units r NB .. r NB + NB - 1; unit u goes to queue u % 8 (or, dealing by
  // expert, all of them to queue r % 8 or qof[r]) and holds ntile tasks.
  const int g = role / kQueues, x = role % kQueues;
  const int NB = a.nb[g];
  int* pre = pq[0];
  if (wave == 0) {
    int v[4], run = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * lane + i;
      const int units = a.deal == kDealUnits     ? n_mod((r + 1) * NB, x) - n_mod(r * NB, x)
                        : a.deal == kDealExperts ? ((r % kQueues == x) ? NB : 0)
                                                 : ((r < E && qof[r] == x) ? NB : 0);
      v[i] = (r < E) ? ntile[order[r]] * units : 0;
      run += v[i];
    }
    int incl2 = run;
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl2, d);
      if (lane >= d) incl2 += o;
    }
    int before = incl2 - run;
    if (lane == 0) pre[0] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      before += v[i];
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
  return launch_kernel(k_permute, dim3(2 * kQueues + 1), dim3(kThreads), stream, ev, a);
}

}  // namespace dg
