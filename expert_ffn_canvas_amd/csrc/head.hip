// Canvas output stage on gfx950: the tied LM head and the per-position softmax
// entropy of a canvas.
//
//   logits[t, v] = sum_d h[t, d] emb[v, d]          (bf16 inputs, fp32 sums)
//   entropy[t]   = -sum_v p_v ln p_v, p = softmax(beta logits[t, :])   (nats)
//   argmax[t]    = the lowest v with the largest logit
//   mean_entropy = the mean of entropy[t] over the positions
//
// Sources: the input embedding is tied to the output head (HF card
// "DiffusionGemma-26B-A4B-it - ROCmFP4 / ROCmFPX GGUF", Variants); every
// denoising step yields raw fp32 logits for the whole 256-token canvas and the
// sampler follows the mean canvas entropy (fucina documentation "DiffusionGemma
// 26B-A4B - block text-diffusion", Logit-parity harness; Chat and REPL; Sampler
// knobs); vocabulary 262144 (auto-round PR "Add quantization support for
// DiffusionGemma", test log).
//
// k_head: one workgroup of 8 waves per tile of 256 positions x 256 vocabulary
// rows. Both operands are row-major in HBM ([T, D] and [V, D]); 64-input
// stages of both tiles (32 KB each) are copied by LDS DMA into a two-stage
// ring, each 128-byte row's 16-byte segments XOR-swizzled so the MFMA operand
// reads are free of bank conflicts. Wave w owns positions 128 (w & 1) .. + 127
// and vocabulary rows 64 (w >> 1) .. + 63 of the tile: 8 x 4 accumulator
// tiles of v_mfma_f32_16x16x32_bf16. The epilogue writes the logits (fp32,
// non-temporal) and reduces each position's 256 values to a softmax partial
// (m = max of beta l, s = sum e^(beta l - m), u = sum e^(beta l - m)(beta l - m),
// and the argmax), merged across lanes and waves in a fixed order.
// k_head_merge: one wave per position merges the partials of all vocabulary
// tiles in a fixed order: entropy = ln s - u / s. k_head_mean: one wave sums
// the entropies in a fixed order. Every result is bit-reproducible.
#include "dg_common.h"
#include "gemm_common.h"
#include "launch.h"

namespace dg {

namespace {

constexpr int kHTok = 256;                       // positions per tile
constexpr int kHVoc = 256;                       // vocabulary rows per tile
constexpr int kHK = 64;                          // inputs per stage
constexpr int kHRowBytes = kHK * 2;              // 128
constexpr int kHSegs = kHK / 8;                  // 16-byte segments per row
constexpr int kHWaves = 8;
constexpr int kHThreads = 64 * kHWaves;
constexpr int kHTileBytes = kHTok * kHRowBytes;  // 32 KB (A and B alike)
constexpr int kHStageBytes = 2 * kHTileBytes;    // A then B
constexpr int kHStages = 2;
constexpr int kHRowsPerDma = 1024 / kHRowBytes;  // rows one wave-wide transfer fills (8)
constexpr int kHDmaPerTile = kHTok / (kHRowsPerDma * kHWaves);  // transfers per wave and tile (4)
constexpr int kHDma = 2 * kHDmaPerTile;          // transfers per wave and stage

static_assert(kHTok == kHVoc, "A and B tiles share the transfer pattern");

// 16-byte position of logical segment s of staged row r. Sixteen consecutive
// rows reading one segment hit sixteen distinct 16-byte bank groups of a
// 256-byte line, and any eight consecutive rows eight distinct ones of a
// 128-byte line.
__device__ __forceinline__ int hswz(int r, int s) { return s ^ ((r >> 1) & (kHSegs - 1)); }

// One stage: rows of the position tile (from h) and of the vocabulary tile
// (from emb), inputs k0 .. k0 + 63. Rows past T or V re-read the last row.
__device__ __forceinline__ void head_dma(uint32_t stage, const uint16_t* h, const uint16_t* emb, int t0, int v0,
                                         int T, int V, int D, int k0, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kHDmaPerTile; ++i) {
    const int blk = wave + kHWaves * i;  // 8-row block of the tile
    const int r = blk * kHRowsPerDma + lane / kHSegs;
    const int sg = hswz(r, lane % kHSegs);
    const uint32_t off = __builtin_amdgcn_readfirstlane(stage + blk * 1024);
    gemm::lds_dma16(off, h + (size_t)min(t0 + r, T - 1) * D + k0 + sg * 8);
    gemm::lds_dma16(off + kHTileBytes, emb + (size_t)min(v0 + r, V - 1) * D + k0 + sg * 8);
  }
}

// Softmax partial of a set of values x = beta l: m = max x, s = sum e^(x - m),
// u = sum e^(x - m)(x - m); the argmax of l (value and id, lowest id on ties).
struct SmPart {
  float m, s, u, best;
  int id;
};

__device__ __forceinline__ SmPart sm_empty() { return SmPart{-INFINITY, 0.0f, 0.0f, -INFINITY, 0x7fffffff}; }

// Merge b into a (a's set, then b's): both sets rescaled to the larger max.
__device__ __forceinline__ SmPart sm_merge(const SmPart& a, const SmPart& b) {
  SmPart r;
  if (b.s == 0.0f) {
    r = a;
  } else if (a.s == 0.0f) {
    r = b;
  } else {
    r.m = fmaxf(a.m, b.m);
    const float da = a.m - r.m, db = b.m - r.m;
    const float ea = __expf(da), eb = __expf(db);
    r.s = ea * a.s + eb * b.s;
    r.u = ea * (a.u + da * a.s) + eb * (b.u + db * b.s);
  }
  const bool take = b.best > a.best || (b.best == a.best && b.id < a.id);
  r.best = take ? b.best : a.best;
  r.id = take ? b.id : a.id;
  return r;
}

__device__ __forceinline__ SmPart sm_shfl_xor(const SmPart& p, int mask) {
  SmPart o;
  o.m = __shfl_xor(p.m, mask);
  o.s = __shfl_xor(p.s, mask);
  o.u = __shfl_xor(p.u, mask);
  o.best = __shfl_xor(p.best, mask);
  o.id = __shfl_xor(p.id, mask);
  return o;
}

__global__ __launch_bounds__(kHThreads) void k_head(HeadArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kHStages * kHStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int th = wave & 1, vq = wave >> 1;
  const int ntb = (a.T + kHTok - 1) / kHTok;
  const int vb = blockIdx.x / ntb, tb = blockIdx.x - vb * ntb;
  const int t0 = tb * kHTok, v0 = vb * kHVoc;
  const int D = a.D, nk = D / kHK;
  const uint32_t base = gemm::lds_addr(smem);
  const int m = lane & 15, g = lane >> 4;

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[i][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  head_dma(base, a.h, a.emb, t0, v0, a.T, a.V, D, 0, wave, lane);
  for (int k = 0; k < nk; ++k) {
    gemm::wait_vmcnt<0>();  // this wave's transfers of stage k have landed
    gemm::lds_barrier();    // everyone's have, and everyone is done with stage k - 1
    if (k + 1 < nk)
      head_dma(base + ((k + 1) & 1) * kHStageBytes, a.h, a.emb, t0, v0, a.T, a.V, D, (k + 1) * kHK, wave, lane);
    const char* As = smem + (k & 1) * kHStageBytes;
    const char* Bs = As + kHTileBytes;
#pragma unroll
    for (int kk = 0; kk < kHK / 32; ++kk) {
      const int s = kk * 4 + g;
      bf16x8 b[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = vq * 64 + p * 16 + m;
        b[p] = as_bf16x8(*reinterpret_cast<const u32x4*>(Bs + r * kHRowBytes + hswz(r, s) * 16));
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int r = th * 128 + mt * 16 + m;
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4*>(As + r * kHRowBytes + hswz(r, s) * 16));
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[mt][p] = mfma_bf16(av, b[p], acc[mt][p]);
      }
    }
  }

  // logits: lane (m, g) holds vocabulary row v0 + 64 vq + 16 p + m of
  // positions 128 th + 16 mt + 4 g + i
  if (a.logits != nullptr) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + th * 128 + mt * 16 + g * 4 + i;
        if (t < a.T) {
          float* row = a.logits + (size_t)t * a.V;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int v = v0 + vq * 64 + p * 16 + m;
            if (v < a.V) __builtin_nontemporal_store(acc[mt][p][i], row + v);
          }
        }
      }
  }

  // softmax partials: per position, this lane's 4 values (p ascending, so the
  // lowest id wins a tie), then the 16 lanes of the row group, then the 4
  // vocabulary quarters through LDS in vq order
  __syncthreads();  // the stages are free: their space takes the wave partials
  SmPart* wpart = reinterpret_cast<SmPart*>(smem);  // [vq][256 positions]
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      SmPart q = sm_empty();
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int v = v0 + vq * 64 + p * 16 + m;
        if (v < a.V) {
          const float l = acc[mt][p][i];
          const float x = a.beta * l;
          SmPart one{x, 1.0f, 0.0f, l, v};
          q = sm_merge(q, one);
        }
      }
#pragma unroll
      for (int msk = 1; msk < 16; msk <<= 1) {
        const SmPart o = sm_shfl_xor(q, msk);
        // fixed order: the lower lane's set first
        q = (m & msk) ? sm_merge(o, q) : sm_merge(q, o);
      }
      if (m == 0) wpart[vq * kHTok + th * 128 + mt * 16 + g * 4 + i] = q;
    }
  __syncthreads();
  for (int r = tid; r < kHTok; r += kHThreads) {
    const int t = t0 + r;
    if (t >= a.T) continue;
    SmPart q = wpart[r];
#pragma unroll
    for (int w = 1; w < 4; ++w) q = sm_merge(q, wpart[w * kHTok + r]);
    const size_t o = (size_t)vb * a.T + t;
    a.part_m[o] = q.m;
    a.part_s[o] = q.s;
    a.part_u[o] = q.u;
    a.part_best[o] = q.best;
    a.part_id[o] = q.id;
  }
}

// One wave per position: lane j merges the partials of vocabulary tiles
// j, j + 64, ... in order, then the 64 lanes merge in a fixed butterfly.
__global__ __launch_bounds__(256) void k_head_merge(HeadArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int nvb = (a.V + kHVoc - 1) / kHVoc;
  SmPart q = sm_empty();
  for (int vb = lane; vb < nvb; vb += 64) {
    const size_t o = (size_t)vb * a.T + t;
    const SmPart b{a.part_m[o], a.part_s[o], a.part_u[o], a.part_best[o], a.part_id[o]};
    q = sm_merge(q, b);
  }
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) {
    const SmPart o = sm_shfl_xor(q, msk);
    q = (lane & msk) ? sm_merge(o, q) : sm_merge(q, o);
  }
  if (lane == 0) {
    a.entropy[t] = logf(q.s) - q.u / q.s;
    a.argmax[t] = q.id;
  }
}

// One wave: the mean of entropy[0 .. T-1], lane j summing j, j + 64, ... in
// order, then a fixed butterfly.
__global__ __launch_bounds__(64) void k_head_mean(HeadArgs a) {
  const int lane = threadIdx.x;
  float s = 0.0f;
  for (int t = lane; t < a.T; t += 64) s += a.entropy[t];
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) s += __shfl_xor(s, msk);
  if (lane == 0) a.mean_entropy[0] = s / (float)a.T;
}

}  // namespace

hipError_t launch_head(const HeadArgs& a, hipStream_t stream, const KernelEvents* ev) {
  const int ntb = (a.T + kHTok - 1) / kHTok, nvb = (a.V + kHVoc - 1) / kHVoc;
  hipError_t e = launch_kernel(k_head, dim3(nvb * ntb), dim3(kHThreads), stream, ev, a);
  if (e != hipSuccess) return e;
  e = launch_kernel(k_head_merge, dim3((a.T + 3) / 4), dim3(256), stream, ev ? ev + 1 : nullptr, a);
  if (e != hipSuccess || a.mean_entropy == nullptr) return e;
  return launch_kernel(k_head_mean, dim3(1), dim3(64), stream, ev ? ev + 2 : nullptr, a);
}

}  // namespace dg
