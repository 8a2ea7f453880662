/*
 * dg_moe.h - C ABI of the MI355X (gfx950) mixture-of-experts feed-forward layer
 * of DiffusionGemma 26B-A4B.
 *
 * The layer (per token t, residual x_t of width d_model):
 *
 *   r_t      = 1 / sqrt(mean_d x_t[d]^2 + eps)
 *   logits   = W_r (x_t r_t (1 + gamma_r)) + b                 router with its own norm
 *   S_t      = the top_k largest logits (ties: lower expert id)
 *   w_{t,e}  = softmax(logits)_e / sum_{e' in S_t} softmax(logits)_{e'}
 *   h_t      = x_t r_t (1 + gamma_e)                           pre_feedforward_layernorm_2
 *   FFN_e(h) = W_down[e] (gelu_tanh(W_gate[e] h) * (W_up[e] h))
 *   MoE(x)_t = sum_{e in S_t} w_{t,e} FFN_e(h_t)
 *
 * Sources (page title, section):
 *  - 128 experts with 8 active: Quant-Tuner PR "Add DiffusionGemma (Gemma-4 MoE
 *    block-diffusion) support", Summary.
 *  - Expert linears gate_proj/up_proj 2816->704 and down_proj 704->2816, no
 *    bias, GELUTanh activation: auto-round PR "Add quantization support for
 *    DiffusionGemma", transformers backend test log, expert module dumps.
 *  - (1+gamma) RMSNorm pre_feedforward_layernorm_2 feeding only the fused 3D
 *    gate_up projection; the router reading the raw residual through its own
 *    norm: Quant-Tuner PR, "Answers to the motivating questions" (AWQ answer).
 *  - int4, group size 128, symmetric: auto-round PR, quantization_config.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (hipMalloc or torch CUDA memory),
 *    row-major and densely packed; 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *  - Every call returns a dg_status. Arguments are checked on the host before
 *    anything is enqueued; on an error nothing is launched and
 *    dg_moe_last_error() holds a message (thread-local). No C++ exception
 *    crosses this boundary. Faults during asynchronous execution surface at
 *    the caller's next synchronisation.
 *  - The library never synchronises the device inside dg_moe_forward and never
 *    reads device data back to the host there.
 */
#ifndef DG_MOE_H
#define DG_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_MOE_ABI_VERSION 2

/* Element types. DG_I4G128: 4-bit codes q in [0,15] standing for (q - 8) * s,
 * two codes per byte (even input index in the low nibble), with one fp16
 * scale s per (output row, group of 128 consecutive inputs); the last group
 * of a row holds whatever remains (64 inputs when the row is 704 long).
 * DG_Q8_0: the ggml Q8_0 block, read from the Q8 GGUF builds of the HF card
 * "DiffusionGemma-26B-A4B-it - ROCmFP4 / ROCmFPX GGUF" (Variants): each run of
 * 32 consecutive inputs of a row is 34 bytes, an fp16 scale d (little endian)
 * then 32 int8 codes q, each standing for q * d.
 * DG_MXFP4: OCP Microscaling MXFP4, read for the FP4 builds the same card
 * compares (introduction; "The 4-bit is NOT the fastest here"): each run of 32
 * consecutive inputs of a row is 17 bytes, an E8M0 scale byte e (2^(e - 127);
 * 255 is NaN) then 16 bytes of E2M1 codes (sign, two exponent bits with bias 1,
 * one mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6), input j in the low nibble of
 * byte j for j < 16 and in the high nibble of byte j - 16 otherwise; each code
 * stands for its value times the block scale.
 * DG_MXFP8: OCP Microscaling MXFP8 with E4M3 elements, read for the FP8 builds
 * of the same card (Credits: FP4 and FP8 tensor types): each run of 32
 * consecutive inputs of a row is 33 bytes, an E8M0 scale byte e (as above)
 * then 32 E4M3 codes in input order (sign, four exponent bits with bias 7,
 * three mantissa bits; exponent field 0 is subnormal, m 2^-9; 0x7f and 0xff
 * are NaN; 448 the largest); each code stands for its value times the block
 * scale. Scale bytes below 3 can put the smallest codes under bf16's smallest
 * subnormal (2^-133); the GPU then rounds those weights to it. */
typedef enum dg_dtype {
  DG_F32 = 0,
  DG_BF16 = 1,
  DG_F16 = 2,
  DG_I4G128 = 3,
  DG_Q8_0 = 4,
  DG_MXFP4 = 5,
  DG_MXFP8 = 6
} dg_dtype;

typedef enum dg_status {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = -1, /* null pointer, bad handle, bad flag            */
  DG_ERR_SHAPE = -2,       /* a size out of the supported range            */
  DG_ERR_DTYPE = -3,       /* unsupported element type or combination      */
  DG_ERR_ALIGN = -4,       /* a pointer not 16-byte aligned                */
  DG_ERR_OOM = -5,         /* device allocation failed in dg_moe_create    */
  DG_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed   */
  DG_ERR_UNSUPPORTED = -7  /* no GPU of the supported architecture         */
} dg_status;

/* dg_moe_config.flags */
#define DG_MOE_PACK_WEIGHTS 0x1u /* copy the expert weights into handle-owned
                                    memory at create (else borrow the caller's),
                                    rearranged into the matrix-core fragment order,
                                    which the GEMMs stream faster. With bf16 experts
                                    and bf16 activations the gate_up copy also
                                    carries the expert norm's scale: each value is
                                    multiplied by (1 + ffn_gamma[input]) and rounded
                                    to bf16, and the forward scales the gate and up
                                    sums by r instead of forming h */

/* dg_moe_forward flags */
#define DG_FWD_ADD_INPUT 0x1u /* out = x + MoE(x) (+ addend) */
/* For tests: where the router's workgroups of one token tile would wait for
 * the last of them and share out the top-k selection, each looks for that
 * arrival only once and otherwise leaves its share to the last arriver (the
 * path taken when such a wait runs out). The results are bit-identical;
 * only the timing differs. */
#define DG_FWD_ROUTER_NO_WAIT 0x2u
/* For tests of the failure path: the down tasks of the fused GEMM launch do
 * not wait for their tile's gate_up tasks at all, so every one of them takes
 * the path of a wait that ran out: it writes NaN for its outputs and raises
 * DG_DEV_WAIT_TIMEOUT in the handle's device status word (which stays set).
 * Every kernel still ends normally. Ignored where the GEMMs run as two
 * launches (int4 experts read in place). */
#define DG_FWD_GEMM_NO_WAIT 0x4u

typedef struct dg_moe_config {
  uint32_t struct_size;   /* = sizeof(dg_moe_config)                                  */
  int32_t n_experts;      /* E, 1..256 (128 for the model)                             */
  int32_t top_k;          /* k, 1..min(E, 8) (8 for the model)                         */
  int32_t d_model;        /* D, multiple of 128, <= 16384 (2816)                       */
  int32_t d_ff;           /* F, multiple of 64, <= 4096 (704)                          */
  int32_t max_tokens;     /* largest T a forward may take; sizes the workspace         */
  float rms_eps;          /* eps of both RMSNorms (> 0)                                */
  int32_t act_dtype;      /* x / out / addend: DG_F32 or DG_BF16                       */
  int32_t router_w_dtype; /* router weight: DG_F32 or DG_BF16                          */
  int32_t expert_w_dtype; /* expert weights: DG_BF16, DG_I4G128, DG_Q8_0, DG_MXFP4 or
                             DG_MXFP8 (the last three need DG_MOE_PACK_WEIGHTS,
                             else DG_ERR_DTYPE)                                       */
  uint32_t flags;         /* DG_MOE_PACK_WEIGHTS                                       */
} dg_moe_config;

/* Weights of one layer; device pointers. */
typedef struct dg_moe_weights {
  const void* router_w;       /* [E, D] router_w_dtype                                      */
  const float* router_gamma;  /* [D] fp32; the router norm multiplies by (1 + gamma)        */
  const float* router_bias;   /* [E] fp32 added to the logits before the softmax, or NULL   */
  const float* ffn_gamma;     /* [D] fp32; the expert-input norm multiplies by (1 + gamma)  */
  const void* w_gate_up;      /* bf16 [E, 2F, D]: rows 0..F-1 gate, F..2F-1 up;
                                 int4: uint8 [E, 2F, D/2]; Q8_0: uint8 [E, 2F, D/32, 34];
                                 MXFP4: uint8 [E, 2F, D/32, 17]; MXFP8: [E, 2F, D/32, 33]  */
  const void* w_down;         /* bf16 [E, D, F]; int4: uint8 [E, D, F/2];
                                 Q8_0: uint8 [E, D, F/32, 34]; MXFP4: uint8 [E, D, F/32, 17];
                                 MXFP8: uint8 [E, D, F/32, 33]                             */
  const uint16_t* s_gate_up;  /* int4 only: fp16 [E, 2F, D/128]                            */
  const uint16_t* s_down;     /* int4 only: fp16 [E, D, ceil(F/128)]                       */
} dg_moe_weights;

/* Bits of the handle's device status word: each is set by a kernel that finds
 * a condition the layer's design rules out, and stays set for the handle's
 * lifetime. dg_moe_forward_debug copies the word out. None of them is set by
 * a correct run; a set bit means that the output of some forward may be wrong.
 *  DG_DEV_QUEUE_OVERFLOW: a GEMM task queue needed more entries than its
 *    capacity; the permutation dropped the excess tasks.
 *  DG_DEV_XCD_ROUTER, DG_DEV_XCD_GEMM: the router workgroups of one token
 *    tile, or the fused-GEMM tasks of one tile, did not all run on one XCD.
 *    They pass data through that XCD's L2 and rely on workgroups b and b + 8
 *    of a launch sharing an XCD (the dispatcher deals workgroups to the 8
 *    XCDs round robin, from an XCD that may differ between launches).
 *  DG_DEV_WAIT_TIMEOUT: a down task of the fused GEMM launch gave up waiting
 *    for its tile's gate_up tasks and wrote NaN for its outputs. */
#define DG_DEV_QUEUE_OVERFLOW 0x1u
#define DG_DEV_XCD_ROUTER 0x2u
#define DG_DEV_XCD_GEMM 0x4u
#define DG_DEV_WAIT_TIMEOUT 0x8u

/* Optional routing outputs of dg_moe_forward_debug; any member may be NULL. */
typedef struct dg_moe_debug {
  int32_t* topk_idx;     /* [T, k] selected experts, by logit descending then id     */
  float* topk_w;         /* [T, k] their renormalised softmax weights                */
  int32_t* counts;       /* [E] tokens routed to each expert                         */
  int32_t* offsets;      /* [E + 1] exclusive prefix sum of counts                   */
  int32_t* sorted_slot;  /* [k T] slot t k + j of each expert-sorted row (increasing
                            token order inside an expert)                            */
  int32_t* row_of_slot;  /* [k T] expert-sorted row of slot (t, j)                   */
  int32_t* queue_len;    /* [2, 8] tasks in each per-XCD queue of the gate_up GEMM,
                            then of the down GEMM, and their common capacity:
                            queue_len[16] (gate_up), queue_len[17] (down): 18 ints   */
  uint32_t* dev_flags;   /* [1] the handle's device status word (DG_DEV_* bits)      */
} dg_moe_debug;

typedef struct dg_moe_s* dg_moe_handle;

/* Create a layer handle: validates the configuration, allocates the whole
 * workspace for config->max_tokens (so dg_moe_forward never allocates), and
 * prepares the router weight. In borrow mode (default) the expert weight
 * pointers are kept and must stay valid and unmodified for the handle's
 * lifetime; with DG_MOE_PACK_WEIGHTS they are copied (in 1 KB fragment
 * blocks of 16 rows x 32 inputs, or 16 rows x 128 int4 inputs, or 2 KB of
 * 16 rows x 128 Q8_0 codes plus their 64 scales, or 1 KB (MXFP4) or 2 KB
 * (MXFP8) of 16 rows x 128 codes plus their 64 scale bytes), after which
 * the caller's expert buffers are no longer read. router_gamma is folded into the handle's copy of the router
 * weight (W_r diag(1 + router_gamma), in fp32 precision); router_bias and
 * ffn_gamma are always copied. Work is enqueued on `stream` and the call
 * synchronises that stream before returning.
 * Errors: DG_ERR_INVALID_ARG (null cfg/weights/out, wrong struct_size),
 * DG_ERR_SHAPE, DG_ERR_DTYPE, DG_ERR_ALIGN, DG_ERR_OOM, DG_ERR_HIP,
 * DG_ERR_UNSUPPORTED (current device is not gfx950). *out is set to NULL on
 * any error. */
dg_status dg_moe_create(const dg_moe_config* cfg, const dg_moe_weights* weights, void* stream,
                        dg_moe_handle* out);

/* out[T, D] (act_dtype) = MoE(x[T, D]) (+ x if DG_FWD_ADD_INPUT) (+ addend if not
 * NULL), summed in fp32 and rounded once (round-to-nearest-even for bf16).
 * Asynchronous on `stream`. T = 0 returns DG_OK and launches nothing.
 * `out` must not overlap `x` or `addend`. One handle must not run two
 * forwards at the same time (they share the workspace): use one handle per
 * stream. Errors: DG_ERR_INVALID_ARG (null handle/x/out, unknown flag,
 * out overlapping an input), DG_ERR_SHAPE (T < 0 or T > max_tokens),
 * DG_ERR_ALIGN, DG_ERR_HIP (launch failure). */
dg_status dg_moe_forward(dg_moe_handle h, const void* x, void* out, int32_t T, const void* addend,
                         uint32_t flags, void* stream);

/* dg_moe_forward plus copies of the routing and permutation (device memory,
 * filled asynchronously on `stream`). For tests and inspection. */
dg_status dg_moe_forward_debug(dg_moe_handle h, const void* x, void* out, int32_t T,
                               const dg_moe_debug* dbg, void* stream);

/* Measurement entry point: dg_moe_forward whose kernel launches also stamp
 * twelve caller-created hipEvent_t (passed as void*): events[2 i] at the
 * start and events[2 i + 1] at the end of kernel i, in launch order: the
 * expert-input norm, the router (r, logits, top-k), the permutation, the
 * gate_up GEMM, the down GEMM and the combine. The events are recorded by the
 * kernel dispatches themselves (hipExtLaunchKernel), so
 * hipEventElapsedTime(events[2 i], events[2 i + 1]) is that kernel's own
 * duration. No kernel of its own runs the expert-input norm (the router
 * writes h where it is materialised, and where the norm is folded into the
 * packed gate_up weight h is never formed): events 0 and 1 are recorded back
 * to back. One launch runs both GEMMs
 * (except for int4 experts in borrow mode): events 6 and 7 time it, and events
 * 8 and 9 are recorded back to back after it. T must be > 0; every event must
 * be non-NULL (else DG_ERR_INVALID_ARG, nothing launched). */
dg_status dg_moe_forward_profiled(dg_moe_handle h, const void* x, void* out, int32_t T, const void* addend,
                                  uint32_t flags, void* const* events, void* stream);

/* Release the handle and everything it allocated. NULL is a no-op. Not stream
 * ordered: the caller makes sure no forward on it is still running. */
dg_status dg_moe_destroy(dg_moe_handle h);

/* Static text for a status code. */
const char* dg_moe_status_string(dg_status s);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* dg_moe_last_error(void);

/* DG_MOE_ABI_VERSION of the loaded library. */
int32_t dg_moe_abi_version(void);

/* Bytes of device workspace a handle with this configuration allocates
 * (excluding packed weights); 0 if the configuration is invalid. */
uint64_t dg_moe_workspace_bytes(const dg_moe_config* cfg);

#ifdef __cplusplus
}
#endif

#endif /* DG_MOE_H */
