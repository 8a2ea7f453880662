// CPU oracle for the DiffusionGemma 26B-A4B mixture-of-experts feed-forward layer.
//
// TEST INFRASTRUCTURE ONLY. This file is the slow, plain reference that the GPU
// library is checked against. Only the tests, the smoke check and the CPU
// baseline leg of the benchmark load it. The GPU library never links, loads or
// calls it, and it shares no code with the GPU sources.
//
// What the layer computes (sources, cited by page title and section):
//  * 128 experts, 8 active per token: Quant-Tuner PR "Add DiffusionGemma
//    (Gemma-4 MoE block-diffusion) support", Summary; HF card
//    "DiffusionGemma-26B-A4B-it - ROCmFP4 / ROCmFPX GGUF", introduction.
//  * Per expert: gate_proj and up_proj are Linear(2816 -> 704), down_proj is
//    Linear(704 -> 2816), all without bias; the activation is GELUTanh:
//    auto-round PR "Add quantization support for DiffusionGemma",
//    transformers backend test log, the DiffusionGemmaTextExperts module dumps
//    before and after replacement.
//  * The expert input goes through pre_feedforward_layernorm_2, a (1+gamma)
//    RMSNorm whose only consumer is the fused 3D gate_up projection; the
//    router reads the raw residual through a norm of its own: Quant-Tuner PR,
//    "Answers to the motivating questions", AWQ answer.
//  * int4 weights: bits 4, group_size 128, symmetric, integer data type:
//    auto-round PR, test log, quantization_config.
//  * Q8_0 weights: the Q8 GGUF builds the pages measure (HF card
//    "DiffusionGemma-26B-A4B-it - ROCmFP4 / ROCmFPX GGUF", Variants); the
//    pages do not spell the format out, so it is read as the public ggml
//    block of 32 consecutive inputs: an fp16 scale d followed by 32 int8
//    codes q, standing for q * d.
//  * MXFP4 weights: the FP4 builds the same card compares (its finding that
//    4-bit loses on gfx1151 turns on FP4 having no hardware path there). The
//    pages do not define the format; it is read as the OCP Microscaling MXFP4
//    format: blocks of 32 consecutive inputs sharing an E8M0 scale 2^(e-127)
//    (e = 255: NaN), each input an E2M1 code (sign bit, two exponent bits with
//    bias 1, one mantissa bit), stored per block as the scale byte and then 16
//    code bytes, input j of the block in the low nibble of byte j for j < 16
//    and in the high nibble of byte j - 16 for j >= 16 (the GGUF block
//    arrangement).
//  * MXFP8 weights: the FP8 builds of the same card (its credits name FP4 and
//    FP8 tensor types) are not defined on the pages either; they are read as
//    the OCP Microscaling MXFP8 format with E4M3 elements: blocks of 32
//    consecutive inputs sharing an E8M0 scale, each input an E4M3 code (sign
//    bit, four exponent bits with bias 7, three mantissa bits; exponent field
//    0 is subnormal, the all-ones pattern with mantissa 7 is NaN, there are no
//    infinities), stored per block as the scale byte and then 32 code bytes,
//    input j of the block in byte j.
//
// Readings where the pages are silent (each one is listed with its reason in
// the design notes): router norm = the same (1+gamma) RMSNorm form as the
// expert norm; eps is a parameter; the router bias is added to the logits
// before the softmax; the 8 experts are the 8 largest logits, ties going to
// the lower expert id; weights are the softmax renormalised over those 8;
// fused gate_up rows 0..F-1 are gate and F..2F-1 are up; the int4 code q is
// dequantised as (q - 8) * s with s an fp16 scale per (output row, 128-wide
// group along the input dimension), the last group of a row taking whatever
// remains (64 wide for K = 704).
//
// Precision: router in fp64, experts in fp32 (plain sequential sums over the
// input dimension), combine in fp32. Inputs stored as bf16 or fp16 are widened
// exactly before use.
//
// Pins: every function here is pinned by the CPU tests against brute force,
// library routines (numpy / torch fp64), closed forms and invariants; the
// full-shape layer result has no printed value on the pages ("parity
// unpinned" beyond those pins, see the oracle pin tests).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#include <algorithm>
#include <omp.h>

namespace {

enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2, OR_I4G128 = 3, OR_Q8_0 = 4, OR_MXFP4 = 5, OR_MXFP8 = 6 };

// E2M1 code (4 bits) -> value: exponent field 0 is subnormal (0 or 0.5),
// otherwise 2^(exponent - 1) (1 + mantissa / 2); bit 3 is the sign.
inline float e2m1_value(int code) {
  const int ex = (code >> 1) & 3, m = code & 1;
  const float mag = ex == 0 ? 0.5f * static_cast<float>(m) : std::ldexp(1.0f + 0.5f * static_cast<float>(m), ex - 1);
  return (code & 8) ? -mag : mag;
}

// E4M3 code (8 bits) -> value: exponent field 0 is subnormal, m 2^-9;
// otherwise 2^(exponent - 7) (1 + mantissa / 8); exponent 15 with mantissa 7
// is NaN; bit 7 is the sign.
inline float e4m3_value(int code) {
  const int ex = (code >> 3) & 15, m = code & 7;
  if (ex == 15 && m == 7) return NAN;
  const float mag = ex == 0 ? std::ldexp(static_cast<float>(m), -9) : std::ldexp(1.0f + 0.125f * static_cast<float>(m), ex - 7);
  return (code & 0x80) ? -mag : mag;
}

// E8M0 scale byte -> 2^(e - 127); 255 encodes NaN.
inline float e8m0_value(int e) { return e == 255 ? NAN : std::ldexp(1.0f, e - 127); }

// bf16 -> fp32: a bf16 value is the upper 16 bits of an fp32 value.
inline float bf16_bits_to_float(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// IEEE binary16 -> fp32, written from the format definition
// (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits).
inline float half_bits_to_float(uint16_t h) {
  const uint32_t sign = static_cast<uint32_t>(h >> 15) << 31;
  const uint32_t expo = (h >> 10) & 0x1f;
  const uint32_t frac = h & 0x3ff;
  uint32_t u;
  if (expo == 0) {
    // zero or subnormal: frac * 2^-24, exact in fp32
    float v = static_cast<float>(frac) * 5.9604644775390625e-8f;
    std::memcpy(&u, &v, 4);
    u |= sign;
  } else if (expo == 31) {
    u = sign | 0x7f800000u | (frac << 13);  // inf or NaN
  } else {
    u = sign | ((expo - 15 + 127) << 23) | (frac << 13);
  }
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// fp32 -> bf16 with round-to-nearest-even on the dropped 16 bits.
inline uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
    return static_cast<uint16_t>((u >> 16) | 0x40);  // keep NaN a NaN
  }
  const uint32_t lower = u & 0xffffu;
  uint32_t upper = u >> 16;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
  return static_cast<uint16_t>(upper);
}

inline float load_elem(const void* p, int dtype, size_t i) {
  switch (dtype) {
    case OR_F32: return static_cast<const float*>(p)[i];
    case OR_BF16: return bf16_bits_to_float(static_cast<const uint16_t*>(p)[i]);
    case OR_F16: return half_bits_to_float(static_cast<const uint16_t*>(p)[i]);
    default: return NAN;
  }
}

// Weight element (row, k) of one expert matrix with K inputs per row.
// bf16: dense [rows, K]. int4: bytes [rows, ceil(K/2)], element k in the low
// nibble of byte k/2 when k is even and in the high nibble when k is odd;
// scales fp16 [rows, ceil(K/128)]. Q8_0: K/32 blocks of 34 bytes per row,
// block b = (fp16 scale d, little endian; int8 codes of inputs 32 b .. 32 b + 31).
// MXFP4: K/32 blocks of 17 bytes per row (E8M0 scale byte, 16 code bytes).
// MXFP8: K/32 blocks of 33 bytes per row (E8M0 scale byte, 32 code bytes).
// Element (row, k) of a matrix stored in 32-input blocks (Q8_0, MXFP4, MXFP8).
// Kept out of line so that the bf16 and int4 reads stay small.
__attribute__((noinline)) float block_weight(int dtype, const void* data, int K, size_t row, int k) {
  if (dtype == OR_Q8_0) {
    const uint8_t* blk = static_cast<const uint8_t*>(data) + (row * static_cast<size_t>(K / 32) + k / 32) * 34;
    const uint16_t d = static_cast<uint16_t>(blk[0] | (blk[1] << 8));
    const int q = static_cast<int8_t>(blk[2 + k % 32]);
    return static_cast<float>(q) * half_bits_to_float(d);  // exact in fp32
  }
  if (dtype == OR_MXFP8) {
    const uint8_t* blk = static_cast<const uint8_t*>(data) + (row * static_cast<size_t>(K / 32) + k / 32) * 33;
    return e4m3_value(blk[1 + k % 32]) * e8m0_value(blk[0]);  // exact in fp32 (four significant bits times 2^n; inf past fp32 range)
  }
  const uint8_t* blk = static_cast<const uint8_t*>(data) + (row * static_cast<size_t>(K / 32) + k / 32) * 17;
  const int j = k % 32;
  const uint8_t byte = blk[1 + (j & 15)];
  const int code = j < 16 ? (byte & 0x0f) : (byte >> 4);
  return e2m1_value(code) * e8m0_value(blk[0]);  // exact in fp32 (two significant bits times a power of two)
}

struct WeightView {
  int dtype;
  const void* data;
  const uint16_t* scales;
  int K;
  float at(size_t row, int k) const {
    if (dtype == OR_BF16) {
      return bf16_bits_to_float(static_cast<const uint16_t*>(data)[row * K + k]);
    }
    if (dtype == OR_Q8_0 || dtype == OR_MXFP4 || dtype == OR_MXFP8) return block_weight(dtype, data, K, row, k);
    const size_t row_bytes = (static_cast<size_t>(K) + 1) / 2;
    const uint8_t byte = static_cast<const uint8_t*>(data)[row * row_bytes + k / 2];
    const int q = (k & 1) ? (byte >> 4) : (byte & 0x0f);
    const size_t n_groups = (static_cast<size_t>(K) + 127) / 128;
    const float s = half_bits_to_float(scales[row * n_groups + k / 128]);
    return static_cast<float>(q - 8) * s;  // exact in fp32
  }
};

// GELU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
inline float gelu_tanh_f32(float z) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  const float inner = c * (z + 0.044715f * z * z * z);
  return 0.5f * z * (1.0f + std::tanh(inner));
}

inline double gelu_tanh_f64(double z) {
  const double c = std::sqrt(2.0 / M_PI);
  return 0.5 * z * (1.0 + std::tanh(c * (z + 0.044715 * z * z * z)));
}

struct Layer {
  int T, D, F, E, K;
  double eps;
  int x_dtype;
  const void* x;
  int rw_dtype;
  const void* router_w;
  const float* router_gamma;
  const float* router_bias;  // may be null
  const float* ffn_gamma;
  int ew_dtype;
  const void* w_gate_up;
  const void* w_down;
  const uint16_t* s_gate_up;
  const uint16_t* s_down;
};

// Router for one token: fp64 RMS statistic, fp64 logits of the normalised
// residual, order by (logit desc, id asc), keep the first K, softmax weights
// over the kept K (equal to the full softmax renormalised over them).
// If `forced` is non-null the kept set is that list instead (weights from the
// same fp64 logits), ordered the same way.
void route_token(const Layer& L, int t, const int32_t* forced, int32_t* idx_out, double* w_out,
                 double* logit_out, double* gap_out, double* r_out) {
  const int D = L.D, E = L.E, K = L.K;
  double ss = 0.0;
  for (int d = 0; d < D; ++d) {
    const double v = load_elem(L.x, L.x_dtype, static_cast<size_t>(t) * D + d);
    ss += v * v;
  }
  const double r = 1.0 / std::sqrt(ss / D + L.eps);
  if (r_out) *r_out = r;

  std::vector<double> z(D);
  for (int d = 0; d < D; ++d) {
    const double v = load_elem(L.x, L.x_dtype, static_cast<size_t>(t) * D + d);
    z[d] = v * r * (1.0 + static_cast<double>(L.router_gamma[d]));
  }
  std::vector<double> logit(E);
  for (int e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) {
      acc += z[d] * static_cast<double>(load_elem(L.router_w, L.rw_dtype, static_cast<size_t>(e) * D + d));
    }
    logit[e] = acc + (L.router_bias ? static_cast<double>(L.router_bias[e]) : 0.0);
  }
  if (logit_out) {
    for (int e = 0; e < E; ++e) logit_out[e] = logit[e];
  }

  std::vector<int> order(E);
  for (int e = 0; e < E; ++e) order[e] = e;
  auto before = [&](int a, int b) {
    if (logit[a] != logit[b]) return logit[a] > logit[b];
    return a < b;
  };
  std::sort(order.begin(), order.end(), before);
  if (gap_out) *gap_out = (K < E) ? logit[order[K - 1]] - logit[order[K]] : INFINITY;

  std::vector<int> chosen(K);
  if (forced) {
    for (int j = 0; j < K; ++j) chosen[j] = forced[j];
    std::sort(chosen.begin(), chosen.end(), before);
  } else {
    for (int j = 0; j < K; ++j) chosen[j] = order[j];
  }
  double lmax = logit[chosen[0]];
  for (int j = 1; j < K; ++j) lmax = std::max(lmax, logit[chosen[j]]);
  double denom = 0.0;
  for (int j = 0; j < K; ++j) denom += std::exp(logit[chosen[j]] - lmax);
  for (int j = 0; j < K; ++j) {
    idx_out[j] = chosen[j];
    w_out[j] = std::exp(logit[chosen[j]] - lmax) / denom;
  }
}

// One expert FFN on one fp32 input row h[D] -> y[D] (fp32):
// g = W_gate h, u = W_up h, a = gelu_tanh(g) * u, y = W_down a.
void expert_ffn(const Layer& L, int e, const float* h, float* y, std::vector<float>& a) {
  const int D = L.D, F = L.F;
  const size_t e_gu = static_cast<size_t>(e) * 2 * F;  // first row of expert e in [E*2F, D]
  const size_t e_dn = static_cast<size_t>(e) * D;      // first row of expert e in [E*D, F]
  WeightView wgu{L.ew_dtype, L.w_gate_up, L.s_gate_up, D};
  WeightView wdn{L.ew_dtype, L.w_down, L.s_down, F};
  for (int f = 0; f < F; ++f) {
    float g = 0.0f, u = 0.0f;
    for (int d = 0; d < D; ++d) g += h[d] * wgu.at(e_gu + f, d);
    for (int d = 0; d < D; ++d) u += h[d] * wgu.at(e_gu + F + f, d);
    a[f] = gelu_tanh_f32(g) * u;
  }
  for (int o = 0; o < D; ++o) {
    float acc = 0.0f;
    for (int f = 0; f < F; ++f) acc += a[f] * wdn.at(e_dn + o, f);
    y[o] = acc;
  }
}

}  // namespace

extern "C" {

// Scalar helpers exposed for the pin tests.
float oracle_gelu_tanh_f32(float z) { return gelu_tanh_f32(z); }
double oracle_gelu_tanh_f64(double z) { return gelu_tanh_f64(z); }
float oracle_half_to_float(uint16_t h) { return half_bits_to_float(h); }
uint16_t oracle_float_to_bf16(float f) { return float_to_bf16_rne(f); }

// Dequantise rows of an int4-g128 matrix with K inputs per row into fp32 [rows, K].
void oracle_dequant_i4(const uint8_t* q, const uint16_t* s, int64_t rows, int K, float* out) {
  WeightView v{OR_I4G128, q, s, K};
  for (int64_t r = 0; r < rows; ++r)
    for (int k = 0; k < K; ++k) out[r * K + k] = v.at(static_cast<size_t>(r), k);
}

// MXFP4 blocks [rows, K/32, 17 bytes] -> fp32 [rows, K].
void oracle_dequant_mxfp4(const uint8_t* blocks, int64_t rows, int K, float* out) {
  WeightView v{OR_MXFP4, blocks, nullptr, K};
  for (int64_t r = 0; r < rows; ++r)
    for (int k = 0; k < K; ++k) out[r * K + k] = v.at(static_cast<size_t>(r), k);
}

// MXFP8 blocks [rows, K/32, 33 bytes] -> fp32 [rows, K].
void oracle_dequant_mxfp8(const uint8_t* blocks, int64_t rows, int K, float* out) {
  WeightView v{OR_MXFP8, blocks, nullptr, K};
  for (int64_t r = 0; r < rows; ++r)
    for (int k = 0; k < K; ++k) out[r * K + k] = v.at(static_cast<size_t>(r), k);
}

// Q8_0 blocks [rows, K/32, 34 bytes] -> fp32 [rows, K].
void oracle_dequant_q8_0(const uint8_t* blocks, int64_t rows, int K, float* out) {
  WeightView v{OR_Q8_0, blocks, nullptr, K};
  for (int64_t r = 0; r < rows; ++r)
    for (int k = 0; k < K; ++k) out[r * K + k] = v.at(static_cast<size_t>(r), k);
}

// Router only, for all T tokens. idx [T,K] int32, w [T,K] fp64, logits [T,E]
// fp64 (nullable), gap [T] fp64 = 8th-largest minus 9th-largest logit
// (nullable), r [T] fp64 (nullable). forced [T,K] (nullable) replaces the
// selection. Returns 0, or -1 on a bad argument.
int oracle_route(int T, int D, int E, int K, double eps, int x_dtype, const void* x, int rw_dtype,
                 const void* router_w, const float* router_gamma, const float* router_bias,
                 const int32_t* forced, int32_t* idx, double* w, double* logits, double* gap,
                 double* r, int n_threads) {
  if (T < 0 || D <= 0 || E <= 0 || K <= 0 || K > E) return -1;
  Layer L{};
  L.T = T; L.D = D; L.E = E; L.K = K; L.eps = eps;
  L.x_dtype = x_dtype; L.x = x; L.rw_dtype = rw_dtype; L.router_w = router_w;
  L.router_gamma = router_gamma; L.router_bias = router_bias;
  if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    route_token(L, t, forced ? forced + static_cast<size_t>(t) * K : nullptr, idx + static_cast<size_t>(t) * K,
                w + static_cast<size_t>(t) * K, logits ? logits + static_cast<size_t>(t) * E : nullptr,
                gap ? gap + t : nullptr, r ? r + t : nullptr);
  }
  return 0;
}

// Token -> expert permutation defined from the routing alone:
// counts[e] = number of (t, j) with idx[t,j] == e; offsets = exclusive prefix
// sum of counts ([E+1]); the rows of expert e are offsets[e] .. offsets[e+1]-1
// and hold its tokens in increasing token order; sorted_token[row] is the
// token of a row and row_of_slot[t*K + j] the row of slot (t, j).
int oracle_permute(int T, int K, int E, const int32_t* idx, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_token, int32_t* row_of_slot) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t s = 0; s < static_cast<int64_t>(T) * K; ++s) {
    if (idx[s] < 0 || idx[s] >= E) return -1;
    counts[idx[s]] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> fill(offsets, offsets + E);
  for (int t = 0; t < T; ++t) {
    for (int j = 0; j < K; ++j) {
      const int e = idx[static_cast<size_t>(t) * K + j];
      const int row = fill[e]++;
      sorted_token[row] = t;
      row_of_slot[static_cast<size_t>(t) * K + j] = row;
    }
  }
  return 0;
}

// The whole layer. For each token t in `tokens` (all T if null):
//   route (fp64), h = fp32(x r (1 + gamma_ffn)), y_j = FFN_{e_j}(h) in fp32,
//   out = sum_j fp32(w_j) * y_j in slot order (fp32),
//   then, if add_input, out += fp32(x); if addend, out += fp32(addend).
// out32 [n_tok, D] fp32 (before any output rounding). idx/w/gap per computed
// token (nullable). dtypes: x/addend 0=f32 1=bf16; router_w 0=f32 1=bf16;
// expert weights 1=bf16 3=int4-g128 4=Q8_0 5=MXFP4 6=MXFP8. Returns 0 or -1 on a bad argument.
int oracle_moe_forward(int T, int D, int F, int E, int K, double eps, int x_dtype, const void* x,
                       int rw_dtype, const void* router_w, const float* router_gamma,
                       const float* router_bias, const float* ffn_gamma, int ew_dtype,
                       const void* w_gate_up, const void* w_down, const uint16_t* s_gate_up,
                       const uint16_t* s_down, const int32_t* forced, const int32_t* tokens,
                       int n_tok, int add_input, const void* addend, float* out32, int32_t* idx_out,
                       double* w_out, double* gap_out, int n_threads) {
  if (T < 0 || D <= 0 || F <= 0 || E <= 0 || K <= 0 || K > E) return -1;
  if (ew_dtype != OR_BF16 && ew_dtype != OR_I4G128 && ew_dtype != OR_Q8_0 && ew_dtype != OR_MXFP4 &&
      ew_dtype != OR_MXFP8)
    return -1;
  if (ew_dtype == OR_I4G128 && (!s_gate_up || !s_down)) return -1;
  if ((ew_dtype == OR_Q8_0 || ew_dtype == OR_MXFP4 || ew_dtype == OR_MXFP8) && (D % 32 || F % 32)) return -1;
  Layer L{T, D, F, E, K, eps, x_dtype, x, rw_dtype, router_w, router_gamma, router_bias, ffn_gamma,
          ew_dtype, w_gate_up, w_down, s_gate_up, s_down};
  const int n = tokens ? n_tok : T;
  for (int i = 0; i < n; ++i) {
    const int t = tokens ? tokens[i] : i;
    if (t < 0 || t >= T) return -1;
  }
  if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel
  {
    std::vector<float> h(D), y(D), a(F);
    std::vector<int32_t> idx(K);
    std::vector<double> w(K);
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < n; ++i) {
      const int t = tokens ? tokens[i] : i;
      double gap = 0.0, r = 0.0;
      route_token(L, t, forced ? forced + static_cast<size_t>(t) * K : nullptr, idx.data(), w.data(),
                  nullptr, &gap, &r);
      for (int d = 0; d < D; ++d) {
        const double v = load_elem(x, x_dtype, static_cast<size_t>(t) * D + d);
        h[d] = static_cast<float>(v * r * (1.0 + static_cast<double>(ffn_gamma[d])));
      }
      float* o = out32 + static_cast<size_t>(i) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.0f;
      for (int j = 0; j < K; ++j) {
        expert_ffn(L, idx[j], h.data(), y.data(), a);
        const float wj = static_cast<float>(w[j]);
        for (int d = 0; d < D; ++d) o[d] += wj * y[d];
      }
      if (add_input) {
        for (int d = 0; d < D; ++d) o[d] += load_elem(x, x_dtype, static_cast<size_t>(t) * D + d);
      }
      if (addend) {
        for (int d = 0; d < D; ++d) o[d] += load_elem(addend, x_dtype, static_cast<size_t>(t) * D + d);
      }
      for (int j = 0; j < K; ++j) {
        if (idx_out) idx_out[static_cast<size_t>(i) * K + j] = idx[j];
        if (w_out) w_out[static_cast<size_t>(i) * K + j] = w[j];
      }
      if (gap_out) gap_out[i] = gap;
    }
  }
  return 0;
}

// One expert FFN on given fp32 rows (for the closed-form pins): h [n, D] -> y [n, D].
int oracle_expert_ffn(int D, int F, int E, int e, int ew_dtype, const void* w_gate_up,
                      const void* w_down, const uint16_t* s_gate_up, const uint16_t* s_down,
                      const float* h, int n, float* y) {
  if (e < 0 || e >= E) return -1;
  Layer L{};
  L.D = D; L.F = F; L.E = E; L.ew_dtype = ew_dtype; L.w_gate_up = w_gate_up; L.w_down = w_down;
  L.s_gate_up = s_gate_up; L.s_down = s_down;
  std::vector<float> a(F);
  for (int i = 0; i < n; ++i) expert_ffn(L, e, h + static_cast<size_t>(i) * D, y + static_cast<size_t>(i) * D, a);
  return 0;
}

// fp32 -> bf16 (RNE) for an array; used by the stacked-layer reference.
void oracle_round_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = float_to_bf16_rne(in[i]);
}

}  // extern "C"
