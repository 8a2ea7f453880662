/* C ABI of the canvas output stage of DiffusionGemma 26B-A4B on gfx950: the
 * tied LM head over a canvas and the per-position softmax entropy.
 *
 * What it computes, for positions t = 0 .. T-1 of a canvas (T = 256 for one
 * canvas) and vocabulary ids v = 0 .. V-1:
 *   logits[t, v]  = sum_d h[t, d] emb[v, d]   (bf16 inputs, fp32 sums)
 *   entropy[t]    = -sum_v p_v ln p_v, with p = softmax(beta logits[t, :])
 *                   (nats; beta > 0 is an inverse temperature, 1 for the
 *                   plain softmax)
 *   argmax[t]     = the lowest v with the largest logit
 *   mean_entropy  = (1/T) sum_t entropy[t]
 * Sources: the input embedding is tied to the output head (HF card
 * "DiffusionGemma-26B-A4B-it - ROCmFP4 / ROCmFPX GGUF", Variants:
 * tie_word_embeddings), so emb is the model's token embedding table [V, D]
 * (V = 262144, auto-round PR "Add quantization support for DiffusionGemma",
 * test log, tokenizer; kept at 16 bits there); each denoising step produces
 * raw fp32 logits [256, vocab] for the whole canvas, and the sampler's status
 * and adaptive stop use the mean canvas entropy H-bar (fucina documentation
 * "DiffusionGemma 26B-A4B - block text-diffusion", Logit-parity harness; Chat
 * and REPL; Sampler knobs). h is the canvas's final hidden state after the
 * model's last norm (the pages print no norm or logit cap for the head, so the
 * stage applies none). The sampler's acceptance rule itself is not part of
 * this stage.
 *
 * Conventions as in dg_moe.h: every entry point returns a dg_status, argument
 * errors are found on the host before anything is enqueued, detail text is
 * in dg_moe_last_error(), tensor pointers are device pointers, row-major and
 * densely packed. */
#ifndef DG_HEAD_H
#define DG_HEAD_H

#include <stdint.h>

#include "dg_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dg_head_config {
  uint32_t struct_size; /* = sizeof(dg_head_config)                               */
  int32_t vocab;        /* V, 1 .. 2^24 (262144 for the model)                     */
  int32_t d_model;      /* D, multiple of 64, <= 16384 (2816)                      */
  int32_t max_tokens;   /* largest T a forward may take; sizes the workspace       */
  int32_t h_dtype;      /* hidden states: DG_BF16                                  */
  int32_t emb_dtype;    /* embedding table: DG_BF16                                */
  uint32_t flags;       /* none defined: 0                                         */
} dg_head_config;

typedef struct dg_head_s* dg_head_handle;

/* Create an output-stage handle for the embedding table emb [V, D] (device,
 * bf16, 16-byte aligned). The table is borrowed and read in place: it must
 * stay valid and unmodified for the handle's lifetime (it is the model's input
 * embedding as well). Allocates the workspace for config->max_tokens (the per-tile
 * softmax partials, 20 bytes per position and 256 vocabulary rows), so
 * dg_head_forward never allocates. Errors: DG_ERR_INVALID_ARG (null
 * cfg/emb/out, wrong struct_size, unknown flag), DG_ERR_SHAPE, DG_ERR_DTYPE,
 * DG_ERR_ALIGN, DG_ERR_OOM, DG_ERR_HIP, DG_ERR_UNSUPPORTED (current device is
 * not gfx950). *out is NULL on any error. */
dg_status dg_head_create(const dg_head_config* cfg, const void* emb, dg_head_handle* out);

/* For the T positions of h [T, D] (bf16, 16-byte aligned): logits [T, V] fp32
 * (written only if not NULL), entropy [T] fp32, argmax [T] int32 and, if not
 * NULL, mean_entropy [1] fp32, as defined above. beta must be finite and > 0.
 * Asynchronous on `stream`; T = 0 returns DG_OK and launches nothing. Outputs
 * must not overlap h or each other. One handle must not run two forwards at
 * the same time (they share the workspace). Every output is bit-reproducible
 * (fixed reduction orders). Errors: DG_ERR_INVALID_ARG (null handle/h/
 * entropy/argmax, beta not finite and > 0, overlapping buffers), DG_ERR_SHAPE
 * (T < 0 or T > max_tokens), DG_ERR_ALIGN (h not 16-byte aligned, outputs not
 * 4-byte aligned), DG_ERR_HIP (launch failure). */
dg_status dg_head_forward(dg_head_handle hd, const void* h, int32_t T, float beta, float* logits, float* entropy,
                          int32_t* argmax, float* mean_entropy, void* stream);

/* Measurement entry point: dg_head_forward whose kernel launches also stamp
 * six caller-created hipEvent_t (passed as void*): events[2 i] at the start and
 * events[2 i + 1] at the end of kernel i, in launch order: the logits and
 * per-tile softmax partials, the merge of the partials per position, and the
 * mean (its two events are recorded back to back when mean_entropy is NULL).
 * T must be > 0 and every event non-NULL (else DG_ERR_INVALID_ARG, nothing
 * launched). */
dg_status dg_head_forward_profiled(dg_head_handle hd, const void* h, int32_t T, float beta, float* logits,
                                   float* entropy, int32_t* argmax, float* mean_entropy, void* const* events,
                                   void* stream);

/* Release the handle and its workspace (not the borrowed table). NULL is a
 * no-op. Not stream ordered: the caller makes sure no
 * forward on it is still running. */
dg_status dg_head_destroy(dg_head_handle hd);

/* Bytes of device workspace a handle with this configuration allocates; 0 if
 * the configuration is invalid. */
uint64_t dg_head_workspace_bytes(const dg_head_config* cfg);

/* Size of the library-owned device scratch of dg_head_forward_noalloc. */
#define DG_HEAD_NOALLOC_SCRATCH_BYTES (8u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the stage of
 * dg_head_forward without a handle, for the table emb [V, D] (bf16, 16-byte
 * aligned, read in place) and the sizes in cfg (validated as for
 * dg_head_create; T <= cfg->max_tokens). It allocates nothing: the per-tile
 * softmax partials go to a library-owned device array of
 * DG_HEAD_NOALLOC_SCRATCH_BYTES (8 MiB), one copy per device, set up on the
 * device's first call and held until the process ends. Five arrays of
 * T * ceil(V / 256) 4-byte partials, each rounded up to 256 bytes, must fit
 * in it (T <= 409 positions at V = 262144), else DG_ERR_SHAPE and nothing is
 * launched. Every call on a device shares that device's array: calls that
 * overlap in time on one device (two streams, two threads) race and give
 * wrong results; issue them on one stream. Each call writes every partial it
 * reads, so nothing needs clearing between calls. The outputs, their meaning,
 * the other argument rules and errors are those of dg_head_forward, and the
 * results are bit-identical to it. Errors: as dg_head_create and
 * dg_head_forward. */
dg_status dg_head_forward_noalloc(const dg_head_config* cfg, const void* emb, const void* h, int32_t T, float beta,
                                  float* logits, float* entropy, int32_t* argmax, float* mean_entropy, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DG_HEAD_H */
