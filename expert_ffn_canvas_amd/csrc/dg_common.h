// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_moe.h"

namespace dg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One task of a grouped GEMM: rows row0 .. row0+mc-1 of the expert-sorted
// order (all routed to expert e, mc <= 64) times column block nb of that
// expert's weight.
struct Tile {
  int e;
  int row0;
  int mc;
  int nb;
};

constexpr int kWave = 64;

// Load with the non-temporal hint, for the expert weights (and the embedding
// table): each launch reads them once, so they stream past the caches
// instead of displacing the activations, gated rows and routing tables that
// the launch and the kernels after it re-read from L2 and the memory-side
// cache (canvas 256: the layer 204 -> 195 us).
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two bf16 bit patterns packed little-endian in one dword -> floats.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// GELU, tanh form. 0.5 z (1 + tanh(y)) equals z / (1 + exp(-2y)), with
// y = sqrt(2/pi) (z + 0.044715 z^3); the exponential saturates cleanly at
// both ends (z -> 0 for very negative z, z -> z for very positive z).
__device__ __forceinline__ float gelu_tanh(float z) {
  const float two_c = 1.5957691216057308f;  // 2 sqrt(2/pi)
  const float y2 = two_c * (z + 0.044715f * z * z * z);
  return z / (1.0f + __expf(-y2));
}

// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] B[32x16].
// Lane l supplies A row (l % 16) and B column (l % 16), each with 8
// consecutive k values from the k-group (l / 16); it receives D column
// (l % 16), rows 4 (l / 16) .. 4 (l / 16) + 3.
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Lane exchange inside a 16-lane row by DPP (no LDS traffic): the value of the
// partner lane that pattern CTRL names.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
// Patterns inside a 16-lane row: swap neighbours, swap pairs, mirror each
// half row, mirror the row. Combining with the partner after each of the four
// in turn leaves every lane with the combination of all sixteen (every step
// joins two disjoint groups, the same two in both partners).
constexpr int kDppXor1 = 0xb1, kDppXor2 = 0x4e, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ f16x8 as_f16x8(const u32x4& v) { return __builtin_bit_cast(f16x8, v); }

// Index of the XCD (accelerator complex die) this wave runs on, from the
// hardware register that holds it (HW_REG_XCC_ID, bits 3:0); 0..7 on MI355X.
__device__ __forceinline__ int xcc_id() { return (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7u); }

// Sets bits of a sticky device status word (a vector atomic in global memory).
__device__ __forceinline__ void raise_flag(uint32_t* flags, uint32_t bits) {
  if (flags != nullptr) atomicOr(flags, bits);
}

}  // namespace dg
