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
// k_head: one workgroup of 8 waves per CU, looping over tiles of 256
// positions x 256 vocabulary rows (persistent). 64-input stages of both tiles
// (32 KB each) are copied by LDS DMA, the positions (read from L2) into a
// two-stage ring and the vocabulary rows (streamed from HBM, the longer wait)
// into a three-stage ring: 160 KB of LDS, two vocabulary stages in flight
// while one is multiplied. Each staged 128-byte row has its 16-byte segments
// XOR-swizzled so the MFMA operand reads are free of bank conflicts. Both
// operands are read row-major ([T, D] and [V, D]) in place. Wave w multiplies
// positions 128 (w & 1) .. + 127 and vocabulary rows 64 (w >> 1) .. + 63 of
// the tile: 8 x 4 accumulator tiles of v_mfma_f32_16x16x32_bf16. The epilogue
// of a tile writes the logits (fp32, non-temporal) and reduces each
// position's 256 values to a softmax partial (m = max of beta l,
// s = sum e^(beta l - m), u = sum e^(beta l - m)(beta l - m), and the argmax),
// first over each 16-lane row by DPP, then over the four vocabulary quarters
// in a fixed order, while the next tile's first stages are already loading.
// k_head_merge: one workgroup per position merges the partials of all
// vocabulary tiles in a fixed order: entropy = ln s - u / s. k_head_mean: one
// wave sums the entropies in a fixed order. Every result is bit-reproducible.
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
constexpr int kHARing = 2;                       // position stages
constexpr int kHBRing = 3;                       // vocabulary stages
constexpr int kHRowsPerDma = 1024 / kHRowBytes;  // rows one wave-wide transfer fills (8)
constexpr int kHDmaPerTile = kHTok / (kHRowsPerDma * kHWaves);  // transfers per wave and tile (4)

static_assert(kHTok == kHVoc, "A and B tiles share the transfer pattern");

// 16-byte position of logical segment s of staged row r. Sixteen consecutive
// rows reading one segment hit sixteen distinct 16-byte bank groups of a
// 256-byte line, and any eight consecutive rows eight distinct ones of a
// 128-byte line.
__device__ __forceinline__ int hswz(int r, int s) { return s ^ ((r >> 1) & (kHSegs - 1)); }

// Stage k0 .. k0 + 63 of the position tile (rows of h; rows past T re-read
// the last one): instruction i of wave w fills the 8-row block w + 8 i.
__device__ __forceinline__ void head_dma_a(uint32_t stage, const uint16_t* h, int t0, int T, int D, int k0, int wave,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < kHDmaPerTile; ++i) {
    const int blk = wave + kHWaves * i;
    const int r = blk * kHRowsPerDma + lane / kHSegs;
    const int sg = hswz(r, lane % kHSegs);
    gemm::lds_dma16(__builtin_amdgcn_readfirstlane(stage + blk * 1024),
                    h + (size_t)min(t0 + r, T - 1) * D + k0 + sg * 8);
  }
}

// Stage k of the vocabulary tile vb (rows of the row-major table; rows past V
// re-read the last one).
__device__ __forceinline__ void head_dma_b(uint32_t stage, const uint16_t* emb, int vb, int V, int D, int k,
                                           int wave, int lane) {
#pragma unroll
  for (int i = 0; i < kHDmaPerTile; ++i) {
    const int blk = wave + kHWaves * i;
    const int r = blk * kHRowsPerDma + lane / kHSegs;
    const int sg = hswz(r, lane % kHSegs);
    gemm::lds_dma16<true>(__builtin_amdgcn_readfirstlane(stage + blk * 1024),
                          emb + (size_t)min(vb * kHVoc + r, V - 1) * D + k * kHK + sg * 8);
  }
}

// Softmax partial of a set of values x = beta l: m = max x, s = sum e^(x - m),
// u = sum e^(x - m)(x - m); the argmax of l (value and id, lowest id on ties).
// An empty set has s = 0.
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

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __uint_as_float(dpp<CTRL>(__float_as_uint(v)));
}

// Max, sum and argmax over the 16 lanes of a row (every lane gets the result;
// a sum is formed in the same grouping in every lane, so it is the same bits).
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppMirror>(v));
}

__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}

template <int CTRL>
__device__ __forceinline__ void argmax_with(float& best, int& id) {
  const float ob = dpp_f<CTRL>(best);
  const int oi = (int)dpp<CTRL>((uint32_t)id);
  const bool take = ob > best || (ob == best && oi < id);
  best = take ? ob : best;
  id = take ? oi : id;
}

__device__ __forceinline__ void row_argmax(float& best, int& id) {
  argmax_with<kDppXor1>(best, id);
  argmax_with<kDppXor2>(best, id);
  argmax_with<kDppHalfMirror>(best, id);
  argmax_with<kDppMirror>(best, id);
}

// Persistent: workgroup b takes tiles b, b + G, b + 2 G, ... (G workgroups,
// one per CU) and runs their stages as one stream, so the first stages of the
// next tile are on their way while this tile's epilogue runs. Stage g of the
// stream is stage g % nk of the workgroup's tile g / nk; it goes to position
// slot g % 2 and vocabulary slot g % 3.
__global__ __launch_bounds__(kHThreads) void k_head(HeadArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[(kHARing + kHBRing) * kHTileBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int th = wave & 1, vq = wave >> 1;
  const int ntb = (a.T + kHTok - 1) / kHTok;
  const int ntiles = ((a.V + kHVoc - 1) / kHVoc) * ntb;
  const int G = gridDim.x;
  if ((int)blockIdx.x >= ntiles) return;
  const int D = a.D, nk = D / kHK;
  const int nstage = ((ntiles - (int)blockIdx.x + G - 1) / G) * nk;
  const uint32_t abase = gemm::lds_addr(smem), bbase = abase + kHARing * kHTileBytes;
  const int m = lane & 15, g = lane >> 4;

  // tile of stream stage q: vocabulary tile and first position
  auto tile_of = [&](int q, int& vb, int& t0) {
    const int tl = (int)blockIdx.x + (q / nk) * G;
    vb = tl / ntb;
    t0 = (tl - vb * ntb) * kHTok;
  };
  auto issue_a = [&](int q) {
    int vb, t0;
    tile_of(q, vb, t0);
    head_dma_a(abase + (q & 1) * kHTileBytes, a.h, t0, a.T, D, (q % nk) * kHK, wave, lane);
  };
  auto issue_b = [&](int q) {
    int vb, t0;
    tile_of(q, vb, t0);
    head_dma_b(bbase + (q % kHBRing) * kHTileBytes, a.emb, vb, a.V, D, q % nk, wave, lane);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p) acc[i][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  // issue order: A0 B0 B1, then per stage q: A(q + 1) B(q + 2); vmcnt retires
  // loads in order, so stage q is in once at most B(q + 1) is outstanding. The
  // stage after a tile's epilogue (which stores) waits for everything.
  issue_a(0);
  issue_b(0);
  if (nstage > 1) issue_b(1);
  bool after_epilogue = false;
  for (int q = 0; q < nstage; ++q) {
    if (q + 1 < nstage && !after_epilogue)
      gemm::wait_vmcnt<kHDmaPerTile>();
    else
      gemm::wait_vmcnt<0>();
    gemm::lds_barrier();  // stage q is in for every wave; everyone is done with stage q - 1
    if (q + 1 < nstage) issue_a(q + 1);
    if (q + 2 < nstage) issue_b(q + 2);
    const char* As = smem + (q & 1) * kHTileBytes;
    const char* Bs = smem + (kHARing + q % kHBRing) * kHTileBytes;
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
    after_epilogue = false;
    if (q % nk != nk - 1) continue;

    // ---- epilogue of the tile: lane (m, g) holds vocabulary row
    // v0 + 64 vq + 16 p + m of positions t0 + 128 th + 16 mt + 4 g + i
    after_epilogue = true;
    int vb, t0;
    tile_of(q, vb, t0);
    const int v0 = vb * kHVoc;
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
    // per position and wave: the max, then the sums against it, then the
    // argmax, each over this lane's 4 values (p ascending) and the row's 16
    // lanes; the wave partials go to the position slot of stage q (every wave
    // is done reading it once all have passed the barrier below)
    gemm::lds_barrier();
    SmPart* wpart = reinterpret_cast<SmPart*>(smem + (q & 1) * kHTileBytes);  // [vq][256 positions]
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x[4];
        bool ok[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          ok[p] = v0 + vq * 64 + p * 16 + m < a.V;
          x[p] = ok[p] ? a.beta * acc[mt][p][i] : -INFINITY;
        }
        const float mx = row_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        float sv = 0.0f, uv = 0.0f, best = -INFINITY;
        int id = 0x7fffffff;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if (ok[p]) {
            const float d = x[p] - mx;
            const float e = __expf(d);
            sv += e;
            uv = fmaf(e, d, uv);
            const float l = acc[mt][p][i];
            if (l > best) {  // strict: the lower id (lower p) stays on a tie
              best = l;
              id = v0 + vq * 64 + p * 16 + m;
            }
          }
        }
        sv = row_sum(sv);
        uv = row_sum(uv);
        row_argmax(best, id);
        if (m == 0) wpart[vq * kHTok + th * 128 + mt * 16 + g * 4 + i] = SmPart{mx, sv, uv, best, id};
      }
    gemm::lds_barrier();
    for (int r = tid; r < kHTok; r += kHThreads) {
      const int t = t0 + r;
      if (t >= a.T) continue;
      SmPart sp = wpart[r];
#pragma unroll
      for (int w = 1; w < 4; ++w) sp = sm_merge(sp, wpart[w * kHTok + r]);
      const size_t o = (size_t)t * ((a.V + kHVoc - 1) / kHVoc) + vb;  // position-major
      a.part_m[o] = sp.m;
      a.part_s[o] = sp.s;
      a.part_u[o] = sp.u;
      a.part_best[o] = sp.best;
      a.part_id[o] = sp.id;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int p = 0; p < 4; ++p) acc[i][p] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// One workgroup of 256 threads per position: thread j merges the partials of
// vocabulary tiles j, j + 256, ... in order (four loads in flight at a time),
// then each wave's lanes merge in a fixed butterfly, then the four waves in
// order.
__global__ __launch_bounds__(256) void k_head_merge(HeadArgs a) {
  __shared__ SmPart wp[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int nvb = (a.V + kHVoc - 1) / kHVoc;
  SmPart q = sm_empty();
  for (int c = tid; c < nvb; c += 4 * 256) {
    SmPart b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vb = c + 256 * u;
      b[u] = sm_empty();
      if (vb < nvb) {
        const size_t o = (size_t)t * nvb + vb;  // consecutive threads read consecutive tiles
        b[u] = SmPart{a.part_m[o], a.part_s[o], a.part_u[o], a.part_best[o], a.part_id[o]};
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) q = sm_merge(q, b[u]);
  }
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) {
    const SmPart o = sm_shfl_xor(q, msk);
    q = (lane & msk) ? sm_merge(o, q) : sm_merge(q, o);  // the lower lane's set first, in both lanes
  }
  if (lane == 0) wp[wave] = q;
  __syncthreads();
  if (tid == 0) {
    SmPart r = wp[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) r = sm_merge(r, wp[w]);
    a.entropy[t] = logf(r.s) - r.u / r.s;
    a.argmax[t] = r.id;
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
  const int grid = min(nvb * ntb, a.n_wg);
  hipError_t e = launch_kernel(k_head, dim3(grid), dim3(kHThreads), stream, ev, a);
  if (e != hipSuccess) return e;
  e = launch_kernel(k_head_merge, dim3(a.T), dim3(256), stream, ev ? ev + 1 : nullptr, a);
  if (e != hipSuccess || a.mean_entropy == nullptr) return e;
  return launch_kernel(k_head_mean, dim3(1), dim3(64), stream, ev ? ev + 2 : nullptr, a);
}

}  // namespace dg
