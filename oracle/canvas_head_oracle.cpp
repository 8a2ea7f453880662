// CPU oracle for the canvas output stage of DiffusionGemma 26B-A4B: the tied
// LM head over the 256-position canvas and the per-position softmax entropy.
//
// TEST INFRASTRUCTURE ONLY. This is the slow, plain reference that the GPU
// library's output stage is checked against. Only the tests, the smoke check
// and the CPU baseline leg of the benchmark load it. The GPU library never
// links, loads or calls it, and it shares no code with the GPU sources.
//
// What the stage computes (sources, cited by page title and section):
//  * The model's input embedding is tied to its output head (HF card
//    "DiffusionGemma-26B-A4B-it - ROCmFP4 / ROCmFPX GGUF", Variants:
//    tie_word_embeddings), so the logits of a canvas position are the dot
//    products of its final hidden state with every row of the embedding table
//    [vocab, d_model] (vocab 262144: auto-round PR "Add quantization support for
//    DiffusionGemma", test log, tokenizer line; the same log's
//    quantization_config keeps the decoder's token embedding at 16 bits;
//    d_model 2816).
//  * Each denoising step turns the whole 256-token canvas into raw fp32 logits
//    [256, vocab] (fucina documentation "DiffusionGemma 26B-A4B - block
//    text-diffusion", Logit-parity harness) and the sampler tracks the mean
//    canvas entropy H-bar (same page, Chat and REPL; Sampler knobs, adaptive
//    stop).
//
// Readings where the pages are silent (each listed with its reason in the
// design notes): the stage's input is the canvas hidden state after the
// model's final norm (the pages print no norm or logit cap for the head);
// entropy in nats of softmax(beta * logits) per position, beta an inverse
// temperature (1 for the plain softmax); H-bar the plain mean over the
// positions; the argmax ties go to the lower token id.
//
// Precision: logits are fp64 sums, in input order, of the exact products of
// the bf16 inputs; the softmax and the entropy are fp64, written from their
// definitions (two passes: the maximum, then the normalised probabilities).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#include <omp.h>

namespace {

inline double bf16_to_double(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

}  // namespace

extern "C" {

// Output stage for the positions `tokens` (all T if null), n = n_tok or T.
//   logits[t, v] = sum_d h[t, d] emb[v, d]                       (fp64)
//   p_v = exp(beta l_v - max) / sum_u exp(beta l_u - max)        (softmax)
//   entropy[t] = -sum_v p_v ln p_v (p_v = 0 contributes 0)       (nats)
//   argmax[t] = the lowest v with the largest logit; gap[t] = the largest
//   logit minus the largest over the other ids (0 on an exact tie).
// h [T, D] and emb [V, D] are bf16 bit patterns. logits_out [n, V] may be
// null. Returns 0, or -1 on a bad argument.
int oracle_canvas_head(int T, int V, int D, const uint16_t* h, const uint16_t* emb, double beta,
                       const int32_t* tokens, int n_tok, double* logits_out, double* entropy_out,
                       int32_t* argmax_out, double* gap_out, int n_threads) {
  if (T < 0 || V < 1 || D < 1 || !h || !emb || !(beta > 0.0)) return -1;
  const int n = tokens ? n_tok : T;
  for (int i = 0; i < n; ++i) {
    const int t = tokens ? tokens[i] : i;
    if (t < 0 || t >= T) return -1;
  }
  if (n_threads > 0) omp_set_num_threads(n_threads);
  std::vector<double> lg(static_cast<size_t>(V));
  for (int i = 0; i < n; ++i) {
    const int t = tokens ? tokens[i] : i;
    const uint16_t* hr = h + static_cast<size_t>(t) * D;
#pragma omp parallel for schedule(static)
    for (int v = 0; v < V; ++v) {
      const uint16_t* er = emb + static_cast<size_t>(v) * D;
      double s = 0.0;
      for (int d = 0; d < D; ++d) s += bf16_to_double(hr[d]) * bf16_to_double(er[d]);
      lg[v] = s;
    }
    int best = 0;
    for (int v = 1; v < V; ++v)
      if (lg[v] > lg[best]) best = v;  // strict: the lower id stays on a tie
    double second = -INFINITY;
    for (int v = 0; v < V; ++v)
      if (v != best && lg[v] > second) second = lg[v];
    double z = 0.0;
    for (int v = 0; v < V; ++v) z += std::exp(beta * (lg[v] - lg[best]));
    double H = 0.0;
    for (int v = 0; v < V; ++v) {
      const double p = std::exp(beta * (lg[v] - lg[best])) / z;
      if (p > 0.0) H -= p * std::log(p);
    }
    if (logits_out) std::memcpy(logits_out + static_cast<size_t>(i) * V, lg.data(), sizeof(double) * V);
    if (entropy_out) entropy_out[i] = H;
    if (argmax_out) argmax_out[i] = best;
    if (gap_out) gap_out[i] = V > 1 ? lg[best] - second : INFINITY;
  }
  return 0;
}

}  // extern "C"
