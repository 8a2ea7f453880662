// Host-side launchers of the gfx950 kernels (one per kernel family). Each
// enqueues work on `stream` and returns the launch status; none synchronises.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Optional start/stop events of one kernel, stamped by the dispatch itself
// (hipExtLaunchKernel), so they time exactly that kernel.
struct KernelEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Launch of a kernel that takes one argument struct, with optional events.
template <typename Arg>
inline hipError_t launch_kernel(void (*kernel)(Arg), dim3 grid, dim3 block, hipStream_t stream,
                                const KernelEvents* ev, const Arg& arg) {
  void* args[1] = {const_cast<Arg*>(&arg)};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream,
                            ev ? ev->start : nullptr, ev ? ev->stop : nullptr, 0);
}

struct Tile;

// Largest number of rows one tile holds (four 16-row MFMA tiles), and the
// largest of the tall tiles used once experts receive many rows each.
constexpr int kTileRows = 64;
constexpr int kTallRows = 128;
// Wide tiles of 8-wave workgroups (one per CU): every row of an expert up to
// this many in one tile.
constexpr int kWideRows = 160;
constexpr int kWideWaves = 8;
// Tile height of the bf16 GEMMs from the rows per expert on average: 64-row
// tiles below 64, 128-row tiles up to kWideFrom, wide tiles from there.
constexpr int kWideFrom = 96;
inline int bf16_tile_rows(int T, int K, int E) {
  const long rows = (long)T * K;
  return rows >= (long)kWideFrom * E ? kWideRows : rows >= 64L * E ? kTallRows : kTileRows;
}
// Short tiles of the quantised GEMMs (packed int4, Q8_0, MXFP4, MXFP8), used
// while the rows per expert average at most kShortUpTo: nearly every expert
// then fits one tile, and the kernels' smaller sums let one more workgroup
// share a CU (three for int4 and Q8_0, four for MXFP4 and MXFP8).
constexpr int kShortRows = 32;
constexpr int kShortUpTo = 20;
inline int quant_tile_rows(int T, int K, int E) {
  return (long)T * K <= (long)kShortUpTo * E ? kShortRows : kTileRows;
}
// GEMM tasks are spread over this many queues, one per XCD: queue x holds the
// tasks that workgroups with blockIdx % kQueues == x process.
constexpr int kQueues = 8;

// The cost of an expert of t tiles and m rows for the balanced deal of wide
// tiles: each task of a tile streams its weight block whatever its rows, and
// its rows add about as much again per row as that block costs per
// kTileCost rows (task timelines of the fused launch at 2304 tokens: a
// 160-row tile's tasks cost as much as 120 of its rows), so
// cost = kTileCost t + m.
constexpr int kTileCost = 128;

// Upper bound on the length of one task queue of a GEMM with NB column blocks
// for T tokens cut into tiles of at most R rows. The tile count is at most
// K T / R + E (each expert's ceil(M_e / R) exceeds M_e / R by less than one),
// and one expert holds at most ceil(T / R) tiles (a token routes to it once).
//  * round robin over units of non-increasing size (the unit deal, the deal
//    by expert): within one unit of the mean;
//  * the balanced deal by tiles: the experts with more than the smallest tile
//    count v1 are dealt in snake order by id, or, when that leaves a queue
//    more than the largest count above an even share, in snake order of
//    their count, non-increasing (which keeps any two queues within the
//    largest count of each other): either way no queue ends more than the
//    largest count above the even share; the
//    experts of v1 tiles then fill the least loaded levels, after which a
//    queue that took some ends below the common level plus 2 v1, and one that
//    took none is where the snake left it: within twice the largest count of
//    the mean;
//  * the balanced deal by cost (wide tiles): the experts in snake order of
//    cost, non-increasing, keep any two queues within the largest cost
//    c_max <= kTileCost ceil(T / R) + T of each other, so none above the mean
//    cost (kTileCost tiles + K T) / 8 plus c_max; a queue's tiles are at most
//    its cost / kTileCost: tiles / 8 + ceil(T / R) + (K T / 8 + T) / kTileCost.
// The permutation still clamps a queue at this length and raises
// DG_DEV_QUEUE_OVERFLOW if it ever had to.
inline int max_queue_len(int T, int K, int E, int NB, int R) {
  const long max_tiles = ((long)K * T + R - 1) / R + E;
  const long per_expert = (T + R - 1) / R;
  const long by_tiles = ((long)NB * max_tiles + kQueues - 1) / kQueues + 2 * NB * per_expert;
  const long rows_term = ((long)K * T + 8L * T + 8L * kTileCost - 1) / (8L * kTileCost);
  const long by_cost = (long)NB * ((max_tiles + kQueues - 1) / kQueues + per_expert + rows_term + 1);
  return (int)(by_tiles > by_cost ? by_tiles : by_cost);
}

// Column blocks of the two GEMMs: gate_up tasks cover 64 features (their gate
// and up rows), down tasks 128 outputs; with wide tiles 128 and 256 (the last
// block may be partial).
inline int gate_up_blocks(int F, int tile_rows = kTileRows) {
  return tile_rows == kWideRows ? (F + 127) / 128 : F / 64;
}
inline int down_blocks(int D, int tile_rows = kTileRows) {
  return tile_rows == kWideRows ? (D + 255) / 256 : D / 128;
}

struct RouterArgs {
  const void* x;        // [T, D] fp32 or bf16
  int x_f32;
  int T, D, E, Epad, K;
  const float* wr;      // W' = W_r diag(1 + gamma_r), fp32 [Epad][D] in fragment order (see launch_prep_router_w)
  const float* bias;    // [E] or null
  const float* gamma_e;
  float eps;
  int h_f16;            // expert input stored as fp16 (int4 or Q8_0 experts) instead of bf16
  uint16_t* h;          // [T, D] expert input, or null where the GEMM reads x (the norm folded)
  float* rnorm;         // [T] r = 1/sqrt(mean x^2 + eps) of each token
  float* logits;        // [T, Epad]
  uint64_t* tile_count; // [16 ceil(T / 16)] counters of the logits kernel, zero between forwards, one 128-byte
                        // line per token tile tt: word 16 tt holds the arrivals in bits 0..7 and per XCD x
                        // the arrivals from it in bits 8 + 6 x ..; word 16 tt + 1 the shares given up (bit
                        // per workgroup of the tile) and in bits 32..39 the workgroups done
  int32_t* topk_idx;    // [T, K]
  float* topk_w;        // [T, K]
  uint32_t* dev_flags;  // sticky device status word (DG_DEV_* bits of dg_moe.h)
  int n_cu;             // compute units of the device (sets the token-tile height)
  int no_wait;          // no workgroup waits for its token tile's last arrival (the path of a wait that ran out)
  int polls;            // set by launch_logits: < 0, the last arriver of a token tile selects the top-k of all
                        // its tokens; >= 0, each workgroup waits up to this many polls for the last arrival,
                        // then selects for its own share of the tokens
};
// r, logits, top-k and the routing weights, and h = x r (1 + gamma_e) where h
// is not null.
hipError_t launch_logits(const RouterArgs& a, hipStream_t stream, const KernelEvents* ev);
// Create time: W' in fp32 from the router weight (fp32 or bf16 [E, D]) and gamma_r [D].
// Layout: 2 KB block (expert tile et, 32-column step s) holds, for lane
// l = n + 16 g, W'[16 et + n][32 s + 8 g + j] at float 256 (j / 4) + 4 l + j % 4,
// so each half of a lane's 8 values is one 1 KB wave-wide read.
hipError_t launch_prep_router_w(const void* w, int w_f32, const float* gamma_r, int E, int Epad, int D,
                                float* wf, hipStream_t stream);

// How the permutation deals the GEMM tasks to the per-XCD queues:
//  kDealUnits: units (expert, column block) round robin, each GEMM on its own;
//  kDealExperts: whole experts (all their tiles and blocks), rank r to queue r % 8;
//  kDealBalanced: whole experts to balance the queues (their tile counts, or
//    with wide tiles their cost kTileCost per tile plus the rows), the same
//    expert to the same queue in both GEMMs (the fused GEMM needs each tile's
//    gate_up and down tasks on one XCD).
constexpr int kDealUnits = 0, kDealExperts = 1, kDealBalanced = 2;

struct PermuteArgs {
  const int32_t* topk_idx;
  int T, K, E;
  int tile_rows;          // largest rows per tile: kTileRows, kShortRows, kTallRows or kWideRows
  int deal;               // kDealUnits, kDealExperts or kDealBalanced
  uint64_t* tile_done;    // kDealBalanced: [K T], zeroed at the first row of every tile (the fused
                          // GEMM's per-tile counters); else null
  int nb[2];              // column blocks of gate_up and down
  int qmax[2];            // capacity of each queue of gate_up and down
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E + 1]
  Tile* tasks[2];         // [kQueues][qmax] each: task p of queue x at tasks[x * qmax + p]
  int32_t* qlen;          // [2][kQueues] queue lengths, then qmax[0], qmax[1]
  int32_t* sorted_slot;   // [K T] slot t K + j of each expert-sorted row
  int32_t* row_of_slot;   // [K T]
  uint32_t* dev_flags;    // sticky device status word (DG_DEV_* bits of dg_moe.h)
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream, const KernelEvents* ev);

struct GemmArgs {
  const Tile* tiles;       // this GEMM's task queues
  const int32_t* qlen;     // [kQueues] their lengths
  int qmax;                // their capacity
  const int32_t* sorted_slot;  // [K T] slot t K + j of each expert-sorted row
  int K;
  const uint16_t* h;       // [T, D] expert input (bf16, or fp16 for quantised experts); the raw x when rnorm is set
  const float* rnorm;      // [T] r of each token when h is the raw x and (1 + gamma_e) is folded into
                           // w_gate_up: the gate and up sums are scaled by it; else null
  const void* w_gate_up;   // bf16 [E, 2F, D], int4 bytes [E, 2F, D/2], or packed Q8_0 / MX codes
  const void* w_down;      // bf16 [E, D, F], int4 bytes [E, D, F/2], or packed Q8_0 / MX codes
  // scales: fp16 (int4, Q8_0), or E8M0 bytes (MXFP4, MXFP8) read through these pointers
  const uint16_t* s_gate_up;
  const uint16_t* s_down;
  uint16_t* act;           // [K T, F] gelu_tanh(gate) * up, expert-sorted rows
  uint16_t* y;             // [K T, D] bf16 down(act), expert-sorted rows
  int D, F;
  int w_packed;            // weights in the fragment layout of launch_pack_panels / _i4 / _q8
};
// Create-time relayout of bf16 expert weights [E][R][K] (R % 16 == 0,
// K % 32 == 0) into MFMA fragment order: 1 KB block (e, s, p) holds, at lane
// l = n + 16 g, the 8 values W[e][16 p + n][32 s + 8 g .. + 7]; blocks are
// ordered e-major, then the 32-column step s, then the 16-row panel p. A wave
// reading one B-operand fragment of a panel then reads 1 KB contiguously, and
// the workgroups streaming an expert's panels at the same K step read one
// contiguous region. With `gamma` ([K] fp32) each value is first multiplied
// by (1 + gamma[k]) and rounded to bf16 (nearest even).
hipError_t launch_pack_panels(const uint16_t* src, uint16_t* dst, int E, int R, int K, const float* gamma,
                              hipStream_t stream);
// Both bf16 GEMMs in one launch (tasks dealt with kDealBalanced): the gate_up
// tasks of each queue, then its down tasks, each down task waiting for the
// gate_up blocks of its tile through tile_done (zeroed by the permutation).
struct FusedGemmArgs {
  GemmArgs gu, dn;
  uint64_t* tile_done; // [K T] per tile, at its first row: gate_up tasks finished in bits 0..7, and per
                       // XCD x those that ran there in bits 8 + 7 x ..
  int nb_gate_up;      // gate_up column blocks per tile
  uint32_t* dev_flags; // sticky device status word (DG_DEV_* bits of dg_moe.h)
  const int32_t* counts; // [E] rows of each expert (its tile count: whether its weights are shared by tiles)
  int wait_polls;      // polls of a down task for its tile's gate_up tasks before it gives up
                       // (kGemmWaitPolls; 0 with DG_FWD_GEMM_NO_WAIT)
};
// A down task's bounded wait: about a tenth of a second of polls.
constexpr int kGemmWaitPolls = 1 << 17;
hipError_t launch_gemm_fused(const FusedGemmArgs& f, int tile_rows, hipStream_t stream, const KernelEvents* ev);
// Create-time relayout of int4-g128 expert weights (codes [E][R][K/2], scales
// [E][R][ceil(K/128)]) into fragment order: 1 KB of codes per (expert, 16-row
// panel, 128-input group), the short last group padded with code 8 (zero);
// the scales of the two panels one task reads side by side, 16 rows x 2 fp16
// per (expert, panel pair, group). pair_stride: panels between a pair's two
// (gate_up: F / 16, gate panel q with up panel q; down: 1, panels 2q, 2q + 1).
hipError_t launch_pack_i4(const uint8_t* codes, const uint16_t* scales, uint8_t* pcodes, uint16_t* pscales, int E,
                          int R, int K, int pair_stride, hipStream_t stream);
// The two int4 products on the caller's row-major layout (borrow mode).
hipError_t launch_gate_up_i4(const GemmArgs& a, hipStream_t stream, const KernelEvents* ev);
hipError_t launch_down_i4(const GemmArgs& a, hipStream_t stream, const KernelEvents* ev);
// Both products with packed int4 weights in one launch, as launch_gemm_fused,
// for tiles of tile_rows (kTileRows or kShortRows) rows.
hipError_t launch_gemm_fused_i4(const FusedGemmArgs& f, int tile_rows, hipStream_t stream, const KernelEvents* ev);
// Create-time relayout of Q8_0 expert weights (rows of K / 32 blocks of 34
// bytes: fp16 scale, 32 int8 codes) into fragment order: per (expert, 128-input
// step, 16-row panel), 2 KB of codes (lane l = n + 16 g: 32 bytes of row n in
// two halves at 16 l and 1024 + 16 l, 8 per 32-input block, inputs
// 8 g .. 8 g + 7 in the order 0 2 1 3 4 6 5 7) and 64 scales [row][block]; a
// short last step is padded with zero codes and scales.
hipError_t launch_pack_q8(const uint8_t* blocks, uint8_t* pcodes, uint16_t* pscales, int E, int R, int K,
                          hipStream_t stream);
// Both products with packed Q8_0 weights (fp16 expert input and activation)
// in one launch, as launch_gemm_fused.
hipError_t launch_gemm_fused_q8(const FusedGemmArgs& f, int tile_rows, hipStream_t stream, const KernelEvents* ev);
// Create-time relayout of MXFP4 expert weights (rows of K / 32 blocks of 17
// bytes: E8M0 scale byte, 16 bytes of E2M1 codes, input j in the low nibble of
// byte j or the high nibble of byte j - 16) into fragment order: per (expert,
// 128-input step, 16-row panel), 1 KB of codes (lane n + 16 g: 16 bytes of row
// n, one dword per 32-input block holding inputs 8 g .. 8 g + 7, even input in
// the low nibble) and 64 scale bytes [row][block]; a short last step is
// padded with zero codes and scale bytes.
hipError_t launch_pack_mx4(const uint8_t* blocks, uint8_t* pcodes, uint8_t* pscales, int E, int R, int K,
                           hipStream_t stream);
// Both products with packed MXFP4 weights (bf16 expert input and activation)
// in one launch, as launch_gemm_fused.
hipError_t launch_gemm_fused_mx4(const FusedGemmArgs& f, int tile_rows, hipStream_t stream, const KernelEvents* ev);
// Create-time relayout of MXFP8 expert weights (rows of K / 32 blocks of 33
// bytes: E8M0 scale byte, 32 E4M3 codes in input order) into fragment order:
// per (expert, 128-input step, 16-row panel), 2 KB of codes (lane l = n + 16 g:
// 32 bytes of row n in two halves at 16 l and 1024 + 16 l, two dwords per
// 32-input block holding inputs 8 g .. 8 g + 7 in order) and 64 scale bytes
// [row][block]; a short last step is padded with zero codes and scale bytes.
hipError_t launch_pack_mx8(const uint8_t* blocks, uint8_t* pcodes, uint8_t* pscales, int E, int R, int K,
                           hipStream_t stream);
// Both products with packed MXFP8 weights (bf16 expert input and activation)
// in one launch, as launch_gemm_fused.
hipError_t launch_gemm_fused_mx8(const FusedGemmArgs& f, int tile_rows, hipStream_t stream, const KernelEvents* ev);

struct CombineArgs {
  const uint16_t* y;           // [K T, D] bf16 expert outputs, expert-sorted rows
  const float* topk_w;         // [T, K] routing weights
  const int32_t* row_of_slot;
  int T, K, D;
  const void* x;       // residual to add, or null
  const void* addend;  // extra addend, or null
  void* out;
  int act_f32;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream, const KernelEvents* ev);

// Canvas output stage (tied LM head + softmax entropy), all device pointers.
struct HeadArgs {
  const uint16_t* h;    // [T, D] bf16
  const uint16_t* emb;  // [V, D] bf16 row-major
  int n_wg;             // persistent workgroups of the logits kernel (one per CU)
  int T, V, D;
  float beta;           // inverse temperature of the softmax
  float* logits;        // [T, V] fp32 or null
  float* entropy;       // [T]
  int32_t* argmax;      // [T]
  float* mean_entropy;  // [1] or null
  // per (position, vocabulary tile of 256) softmax partials, [T][ceil(V/256)]
  float* part_m;
  float* part_s;
  float* part_u;
  float* part_best;
  int32_t* part_id;
};

// The stage: logits + per-tile partials, the merge per position, the mean
// (skipped when mean_entropy is null). ev, if not null, points at three
// KernelEvents, one per launch.
hipError_t launch_head(const HeadArgs& a, hipStream_t stream, const KernelEvents* ev);

}  // namespace dg
