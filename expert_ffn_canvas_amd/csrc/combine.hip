// Weighted combine back to token order on gfx950:
//   out[t] = sum_j w[t, j] y[row_of_slot[t k + j]]  (+ x[t]) (+ addend[t])
// with w the routing weights and y the expert outputs of the slots (bf16). The k
// slots are accumulated (fused multiply-add, fp32) in their routing order
// (logit descending), always in the same order, so the result is
// bit-reproducible; the output is rounded once (round-to-nearest-even for
// bf16). The expert outputs are read once, with the non-temporal hint.
#include "dg_common.h"
#include "launch.h"

namespace dg {

namespace {

constexpr int kThreads = 256;

constexpr int kCols = kThreads * 4;  // columns per workgroup

// Workgroup (t, chunk): token t, columns chunk * 1024 .. + 1023.
template <bool OUT_F32>
__global__ __launch_bounds__(kThreads) void k_combine(CombineArgs a) {
  const int K = a.K, D = a.D;
  const int n_chunk = (D + kCols - 1) / kCols;
  const int t = blockIdx.x / n_chunk;
  const int c = (blockIdx.x - t * n_chunk) * kCols + threadIdx.x * 4;
  int rows[8];
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = (j < K) ? a.row_of_slot[(size_t)t * K + j] : 0;
    w[j] = (j < K) ? a.topk_w[(size_t)t * K + j] : 0.0f;
  }
  if (c < D) {
    uint2 yv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < K) {
        const uint64_t v = ld_stream(reinterpret_cast<const uint64_t*>(a.y + (size_t)rows[j] * D + c));
        yv[j] = make_uint2((uint32_t)v, (uint32_t)(v >> 32));
      }
    float4 s = make_float4(w[0] * bf16_lo(yv[0].x), w[0] * bf16_hi(yv[0].x), w[0] * bf16_lo(yv[0].y),
                           w[0] * bf16_hi(yv[0].y));
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      if (j < K) {
        s.x = fmaf(w[j], bf16_lo(yv[j].x), s.x);
        s.y = fmaf(w[j], bf16_hi(yv[j].x), s.y);
        s.z = fmaf(w[j], bf16_lo(yv[j].y), s.z);
        s.w = fmaf(w[j], bf16_hi(yv[j].y), s.w);
      }
    }
    const void* extra[2] = {a.x, a.addend};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (extra[q] == nullptr) continue;
      if (OUT_F32) {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(extra[q]) + (size_t)t * D + c);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(extra[q]) + (size_t)t * D + c);
        s.x += bf16_lo(v.x); s.y += bf16_hi(v.x); s.z += bf16_lo(v.y); s.w += bf16_hi(v.y);
      }
    }
    if (OUT_F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + (size_t)t * D + c) = s;
    } else {
      uint2 o;
      o.x = pack_bf16x2(s.x, s.y);
      o.y = pack_bf16x2(s.z, s.w);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + (size_t)t * D + c) = o;
    }
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream, const KernelEvents* ev) {
  const dim3 grid(a.T * ((a.D + kCols - 1) / kCols));
  return launch_kernel(a.act_f32 ? k_combine<true> : k_combine<false>, grid, dim3(kThreads), stream, ev, a);
}

}  // namespace dg
