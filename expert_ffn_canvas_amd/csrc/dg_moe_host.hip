// Host side of the C ABI in include/dg_moe.h: argument validation, the
// workspace allocated once at create time, router-weight preparation, and the
// asynchronous launch sequence of one forward:
//
//   router (r + logits + top-k + weights, and the expert input where it is
//   materialised)
//   -> permutation (counts, offsets, tile list, stable scatter)
//   -> gate_up grouped GEMM (+ GELU-tanh gating)
//   -> down grouped GEMM (x routing weight)
//   -> combine back to token order.
//
// It also holds the host side of include/dg_head.h, the canvas output stage
// (tied LM head and softmax entropy): validation, its workspace, its launches.
//
// Nothing in a forward allocates, synchronises or reads device data back.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <mutex>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "dg_common.h"
#include "dg_head.h"
#include "dg_moe.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

dg_status fail(dg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

dg_status ok() {
  g_last_error.clear();
  return DG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t act_elem_bytes(int dt) { return dt == DG_F32 ? 4 : 2; }

// Sub-buffer layout of the workspace (byte offsets from the base).
struct Layout {
  size_t h, rnorm, logits, tile_count, topk_idx, topk_w, counts, offsets, tasks[2], qlen, sorted_slot, row_of_slot, act,
      y, tile_done, dev_flags;
  size_t wr, bias, gamma_e;
  size_t total;
  int Epad, nb[2], qmax[2];  // per GEMM (gate_up, down): column blocks, queue capacity
  // bf16 activations with packed bf16 experts: (1 + gamma_e) is folded into
  // the packed gate_up weight, the gate_up GEMM reads x and scales its sums by
  // r, and the expert input h is never materialised
  bool fold;
};

// Both GEMMs run in one launch (gate_up tasks, then each tile's down tasks once
// its gate_up blocks are done), except for int4 experts read in place.
bool fuses_gemms(const dg_moe_config& c) {
  return c.expert_w_dtype != DG_I4G128 || (c.flags & DG_MOE_PACK_WEIGHTS);
}

bool folds_expert_norm(const dg_moe_config& c) {
  return (c.flags & DG_MOE_PACK_WEIGHTS) && c.expert_w_dtype == DG_BF16 && c.act_dtype == DG_BF16;
}

Layout plan(const dg_moe_config& c) {
  Layout L{};
  const size_t T = (size_t)c.max_tokens, D = (size_t)c.d_model, F = (size_t)c.d_ff;
  const size_t E = (size_t)c.n_experts, K = (size_t)c.top_k;
  L.Epad = (int)round_up(E, 32);
  L.fold = folds_expert_norm(c);
  L.nb[0] = dg::gate_up_blocks((int)F);
  L.nb[1] = dg::down_blocks((int)D);
  // the shortest tiles give the longest queues
  // (bf16 experts and int4 read in place never take short tiles)
  const int min_rows =
      (c.expert_w_dtype == DG_BF16 || (c.expert_w_dtype == DG_I4G128 && !(c.flags & DG_MOE_PACK_WEIGHTS)))
          ? dg::kTileRows
          : dg::kShortRows;
  for (int g = 0; g < 2; ++g) L.qmax[g] = dg::max_queue_len((int)T, (int)K, (int)E, L.nb[g], min_rows);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = round_up(off + bytes, 256);
    return at;
  };
  L.h = take(L.fold ? 0 : T * D * 2);
  L.rnorm = take(T * 4);
  L.logits = take(T * (size_t)L.Epad * 4);
  L.tile_count = take((T + 15) / 16 * 128);
  L.topk_idx = take(T * K * 4);
  L.topk_w = take(T * K * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  for (int g = 0; g < 2; ++g) L.tasks[g] = take((size_t)L.qmax[g] * dg::kQueues * sizeof(dg::Tile));
  L.qlen = take((2 * dg::kQueues + 2) * 4);  // the queue lengths, then the two capacities
  L.sorted_slot = take(K * T * 4);
  L.row_of_slot = take(K * T * 4);
  L.act = take(K * T * F * 2);
  L.y = take(K * T * D * 2);
  L.tile_done = take(fuses_gemms(c) ? K * T * 8 : 0);
  L.dev_flags = take(4);
  L.wr = take((size_t)L.Epad * D * 4);
  L.bias = take(E * 4);
  L.gamma_e = take(D * 4);
  L.total = off;
  return L;
}

dg_status check_config(const dg_moe_config* c) {
  if (!c) return fail(DG_ERR_INVALID_ARG, "config is NULL");
  if (c->struct_size != sizeof(dg_moe_config))
    return fail(DG_ERR_INVALID_ARG, "config struct_size %u != %zu", c->struct_size, sizeof(dg_moe_config));
  if (c->n_experts < 1 || c->n_experts > 256) return fail(DG_ERR_SHAPE, "n_experts %d not in [1, 256]", c->n_experts);
  if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_experts)
    return fail(DG_ERR_SHAPE, "top_k %d not in [1, min(n_experts, 8)]", c->top_k);
  if (c->d_model < 128 || c->d_model > 16384 || c->d_model % 128)
    return fail(DG_ERR_SHAPE, "d_model %d must be a multiple of 128 in [128, 16384]", c->d_model);
  if (c->d_ff < 64 || c->d_ff > 4096 || c->d_ff % 64)
    return fail(DG_ERR_SHAPE, "d_ff %d must be a multiple of 64 in [64, 4096]", c->d_ff);
  if (c->max_tokens < 1 || c->max_tokens > (1 << 20))
    return fail(DG_ERR_SHAPE, "max_tokens %d not in [1, 2^20]", c->max_tokens);
  if (!(c->rms_eps > 0.0f) || !std::isfinite(c->rms_eps)) return fail(DG_ERR_INVALID_ARG, "rms_eps must be finite and > 0");
  if (c->act_dtype != DG_F32 && c->act_dtype != DG_BF16)
    return fail(DG_ERR_DTYPE, "act_dtype %d: only DG_F32 or DG_BF16", c->act_dtype);
  if (c->router_w_dtype != DG_F32 && c->router_w_dtype != DG_BF16)
    return fail(DG_ERR_DTYPE, "router_w_dtype %d: only DG_F32 or DG_BF16", c->router_w_dtype);
  if (c->expert_w_dtype != DG_BF16 && c->expert_w_dtype != DG_I4G128 && c->expert_w_dtype != DG_Q8_0 &&
      c->expert_w_dtype != DG_MXFP4 && c->expert_w_dtype != DG_MXFP8)
    return fail(DG_ERR_DTYPE, "expert_w_dtype %d: only DG_BF16, DG_I4G128, DG_Q8_0, DG_MXFP4 or DG_MXFP8",
                c->expert_w_dtype);
  if (c->flags & ~DG_MOE_PACK_WEIGHTS) return fail(DG_ERR_INVALID_ARG, "unknown config flags 0x%x", c->flags);
  if ((c->expert_w_dtype == DG_Q8_0 || c->expert_w_dtype == DG_MXFP4 || c->expert_w_dtype == DG_MXFP8) &&
      !(c->flags & DG_MOE_PACK_WEIGHTS))
    return fail(DG_ERR_DTYPE,
                "DG_Q8_0, DG_MXFP4 and DG_MXFP8 experts are read from the packed copy only: set DG_MOE_PACK_WEIGHTS");
  return DG_OK;
}

}  // namespace

struct dg_moe_s {
  dg_moe_config cfg;
  Layout L;
  int device;
  int n_cu;           // compute units of the device
  char* ws;           // workspace + prepared router parameters
  void* packed;       // expert weights copied at create (pack mode), else null
  int w_packed = 0;   // expert weights in the fragment layout of their packing kernel
  const void* w_gate_up;
  const void* w_down;
  const uint16_t* s_gate_up;
  const uint16_t* s_down;
  bool has_bias;

  template <typename P>
  P* at(size_t off) const { return reinterpret_cast<P*>(ws + off); }
};

namespace {

struct ExpertBytes {
  size_t gu, dn, sgu, sdn;
};

ExpertBytes expert_bytes(const dg_moe_config& c) {
  const size_t E = c.n_experts, D = c.d_model, F = c.d_ff;
  ExpertBytes b{};
  if (c.expert_w_dtype == DG_BF16) {
    b.gu = E * 2 * F * D * 2;
    b.dn = E * D * F * 2;
  } else if (c.expert_w_dtype == DG_Q8_0) {  // packed only: 128 codes and 4 scales per (row, 128-input step)
    const size_t nks_d = (D + 127) / 128, nks_f = (F + 127) / 128;
    b.gu = E * 2 * F * nks_d * 128;
    b.dn = E * D * nks_f * 128;
    b.sgu = E * 2 * F * nks_d * 4 * 2;
    b.sdn = E * D * nks_f * 4 * 2;
  } else if (c.expert_w_dtype == DG_MXFP4 || c.expert_w_dtype == DG_MXFP8) {
    // packed only: 64 (MXFP4) or 128 (MXFP8) code bytes and 4 scale bytes per (row, 128-input step)
    const size_t nks_d = (D + 127) / 128, nks_f = (F + 127) / 128;
    const size_t cb = c.expert_w_dtype == DG_MXFP4 ? 64 : 128;
    b.gu = E * 2 * F * nks_d * cb;
    b.dn = E * D * nks_f * cb;
    b.sgu = E * 2 * F * nks_d * 4;
    b.sdn = E * D * nks_f * 4;
  } else {
    b.gu = E * 2 * F * (D / 2);
    b.dn = E * D * (F / 2);
    b.sgu = E * 2 * F * (D / 128) * 2;
    b.sdn = E * D * ((F + 127) / 128) * 2;
  }
  return b;
}

dg_status hip_fail(hipError_t e, const char* what) {
  return fail(DG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int32_t dg_moe_abi_version(void) { return DG_MOE_ABI_VERSION; }

const char* dg_moe_status_string(dg_status s) {
  switch (s) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID_ARG: return "invalid argument";
    case DG_ERR_SHAPE: return "unsupported shape";
    case DG_ERR_DTYPE: return "unsupported dtype";
    case DG_ERR_ALIGN: return "pointer not 16-byte aligned";
    case DG_ERR_OOM: return "device out of memory";
    case DG_ERR_HIP: return "HIP runtime error";
    case DG_ERR_UNSUPPORTED: return "unsupported device";
  }
  return "unknown status";
}

const char* dg_moe_last_error(void) { return g_last_error.c_str(); }

uint64_t dg_moe_workspace_bytes(const dg_moe_config* cfg) {
  if (check_config(cfg) != DG_OK) return 0;
  return (uint64_t)plan(*cfg).total;
}

dg_status dg_moe_create(const dg_moe_config* cfg, const dg_moe_weights* w, void* stream_v, dg_moe_handle* out) {
  if (out) *out = nullptr;
  dg_status st = check_config(cfg);
  if (st != DG_OK) return st;
  if (!w || !out) return fail(DG_ERR_INVALID_ARG, "weights or out is NULL");
  const bool i4 = cfg->expert_w_dtype == DG_I4G128;
  const bool q8 = cfg->expert_w_dtype == DG_Q8_0;
  const bool mx4 = cfg->expert_w_dtype == DG_MXFP4;
  const bool mx8 = cfg->expert_w_dtype == DG_MXFP8;
  if (!w->router_w || !w->router_gamma || !w->ffn_gamma || !w->w_gate_up || !w->w_down)
    return fail(DG_ERR_INVALID_ARG, "a required weight pointer is NULL");
  if (i4 && (!w->s_gate_up || !w->s_down)) return fail(DG_ERR_INVALID_ARG, "int4 weights need both scale tensors");
  const void* ptrs[] = {w->router_w, w->router_gamma, w->router_bias, w->ffn_gamma,
                        w->w_gate_up, w->w_down, w->s_gate_up, w->s_down};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(DG_ERR_ALIGN, "weight pointer %p is not 16-byte aligned", p);

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(DG_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);

  dg_moe_s* hd = new (std::nothrow) dg_moe_s();
  if (!hd) return fail(DG_ERR_OOM, "host allocation failed");
  hd->cfg = *cfg;
  hd->L = plan(*cfg);
  hd->device = dev;
  hd->n_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  hipStream_t stream = static_cast<hipStream_t>(stream_v);

  e = hipMalloc(reinterpret_cast<void**>(&hd->ws), hd->L.total);
  if (e != hipSuccess) {
    delete hd;
    (void)hipGetLastError();
    return fail(DG_ERR_OOM, "workspace of %zu bytes: %s", hd->L.total, hipGetErrorString(e));
  }
  ExpertBytes eb = expert_bytes(*cfg);
  if (cfg->flags & DG_MOE_PACK_WEIGHTS) {
    if (i4) {  // packed int4 codes: a full 128-input group per (row, group), the short last one padded
      const size_t E = cfg->n_experts, D = cfg->d_model, F = cfg->d_ff;
      eb.gu = E * 2 * F * ((D + 127) / 128) * 64;
      eb.dn = E * D * ((F + 127) / 128) * 64;
    }
    const size_t total = round_up(eb.gu, 256) + round_up(eb.dn, 256) + round_up(eb.sgu, 256) + round_up(eb.sdn, 256);
    e = hipMalloc(&hd->packed, total);
    if (e != hipSuccess) {
      (void)hipFree(hd->ws);
      delete hd;
      (void)hipGetLastError();
      return fail(DG_ERR_OOM, "packed weights of %zu bytes: %s", total, hipGetErrorString(e));
    }
    char* p = static_cast<char*>(hd->packed);
    hd->w_gate_up = p;
    hd->w_down = p + round_up(eb.gu, 256);
    const bool scaled = i4 || q8 || mx4 || mx8;
    hd->s_gate_up =
        scaled ? reinterpret_cast<const uint16_t*>(p + round_up(eb.gu, 256) + round_up(eb.dn, 256)) : nullptr;
    hd->s_down = scaled ? reinterpret_cast<const uint16_t*>(p + round_up(eb.gu, 256) + round_up(eb.dn, 256) +
                                                            round_up(eb.sgu, 256))
                        : nullptr;
    hipError_t c1, c2, c3 = hipSuccess, c4 = hipSuccess;
    if (mx4 || mx8) {  // MXFP4 / MXFP8: codes and scale bytes in fragment order, per 128-input step
      auto pack = mx4 ? dg::launch_pack_mx4 : dg::launch_pack_mx8;
      c1 = pack(static_cast<const uint8_t*>(w->w_gate_up), static_cast<uint8_t*>(const_cast<void*>(hd->w_gate_up)),
                reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(hd->s_gate_up)), cfg->n_experts, 2 * cfg->d_ff,
                cfg->d_model, stream);
      c2 = pack(static_cast<const uint8_t*>(w->w_down), static_cast<uint8_t*>(const_cast<void*>(hd->w_down)),
                reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(hd->s_down)), cfg->n_experts, cfg->d_model,
                cfg->d_ff, stream);
      hd->w_packed = 1;
    } else if (q8) {  // Q8_0: codes and scales in fragment order, per 128-input step
      c1 = dg::launch_pack_q8(static_cast<const uint8_t*>(w->w_gate_up),
                              static_cast<uint8_t*>(const_cast<void*>(hd->w_gate_up)),
                              const_cast<uint16_t*>(hd->s_gate_up), cfg->n_experts, 2 * cfg->d_ff, cfg->d_model,
                              stream);
      c2 = dg::launch_pack_q8(static_cast<const uint8_t*>(w->w_down),
                              static_cast<uint8_t*>(const_cast<void*>(hd->w_down)), const_cast<uint16_t*>(hd->s_down),
                              cfg->n_experts, cfg->d_model, cfg->d_ff, stream);
      hd->w_packed = 1;
    } else if (i4) {  // int4: codes and scales in fragment order
      c1 = dg::launch_pack_i4(static_cast<const uint8_t*>(w->w_gate_up), w->s_gate_up,
                              static_cast<uint8_t*>(const_cast<void*>(hd->w_gate_up)),
                              const_cast<uint16_t*>(hd->s_gate_up), cfg->n_experts, 2 * cfg->d_ff, cfg->d_model,
                              cfg->d_ff / 16, stream);
      c2 = dg::launch_pack_i4(static_cast<const uint8_t*>(w->w_down), w->s_down,
                              static_cast<uint8_t*>(const_cast<void*>(hd->w_down)), const_cast<uint16_t*>(hd->s_down),
                              cfg->n_experts, cfg->d_model, cfg->d_ff, 1, stream);
      hd->w_packed = 1;
    } else {  // bf16: MFMA fragment order, 1 KB per wave-wide read
      c1 = dg::launch_pack_panels(static_cast<const uint16_t*>(w->w_gate_up),
                                  static_cast<uint16_t*>(const_cast<void*>(hd->w_gate_up)), cfg->n_experts,
                                  2 * cfg->d_ff, cfg->d_model, hd->L.fold ? w->ffn_gamma : nullptr, stream);
      c2 = dg::launch_pack_panels(static_cast<const uint16_t*>(w->w_down),
                                  static_cast<uint16_t*>(const_cast<void*>(hd->w_down)), cfg->n_experts,
                                  cfg->d_model, cfg->d_ff, nullptr, stream);
      hd->w_packed = 1;
    }
    if (c1 != hipSuccess || c2 != hipSuccess || c3 != hipSuccess || c4 != hipSuccess) {
      dg_moe_destroy(hd);
      return fail(DG_ERR_HIP, "copying expert weights failed");
    }
  } else {
    hd->w_gate_up = w->w_gate_up;
    hd->w_down = w->w_down;
    hd->s_gate_up = w->s_gate_up;
    hd->s_down = w->s_down;
  }
  hd->has_bias = w->router_bias != nullptr;
  const size_t D = cfg->d_model, E = cfg->n_experts;
  hipError_t c[3];
  c[0] = hipMemcpyAsync(hd->ws + hd->L.gamma_e, w->ffn_gamma, D * 4, hipMemcpyDeviceToDevice, stream);
  c[1] = hd->has_bias ? hipMemcpyAsync(hd->ws + hd->L.bias, w->router_bias, E * 4, hipMemcpyDeviceToDevice, stream)
                      : hipSuccess;
  c[2] = dg::launch_prep_router_w(w->router_w, cfg->router_w_dtype == DG_F32, w->router_gamma, (int)E, hd->L.Epad,
                                  (int)D, hd->at<float>(hd->L.wr), stream);
  for (hipError_t ci : c) {
    if (ci != hipSuccess) {
      dg_moe_destroy(hd);
      return hip_fail(ci, "preparing router parameters");
    }
  }
  e = hipMemsetAsync(hd->ws + hd->L.tile_count, 0, ((size_t)cfg->max_tokens + 15) / 16 * 128, stream);
  if (e == hipSuccess) e = hipMemsetAsync(hd->ws + hd->L.dev_flags, 0, 4, stream);
  if (e != hipSuccess) {
    dg_moe_destroy(hd);
    return hip_fail(e, "create: clearing the arrival counters and the status word");
  }
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    dg_moe_destroy(hd);
    return hip_fail(e, "create: stream synchronize");
  }
  *out = hd;
  return ok();
}

static dg_status run_forward(dg_moe_handle hd, const void* x, void* out, int32_t T, const void* addend,
                             uint32_t flags, const dg_moe_debug* dbg, void* const* events, void* stream_v) {
  if (!hd) return fail(DG_ERR_INVALID_ARG, "handle is NULL");
  if (flags & ~(DG_FWD_ADD_INPUT | DG_FWD_ROUTER_NO_WAIT | DG_FWD_GEMM_NO_WAIT))
    return fail(DG_ERR_INVALID_ARG, "unknown forward flags 0x%x", flags);
  const dg_moe_config& c = hd->cfg;
  if (T < 0 || T > c.max_tokens) return fail(DG_ERR_SHAPE, "T = %d not in [0, max_tokens = %d]", T, c.max_tokens);
  if (T == 0) return ok();
  if (!x || !out) return fail(DG_ERR_INVALID_ARG, "x or out is NULL");
  if (!aligned16(x) || !aligned16(out) || (addend && !aligned16(addend)))
    return fail(DG_ERR_ALIGN, "x, out and addend must be 16-byte aligned");
  const size_t bytes = (size_t)T * c.d_model * act_elem_bytes(c.act_dtype);
  auto overlap = [bytes](const void* p, const void* q) {
    const char* a = static_cast<const char*>(p);
    const char* b = static_cast<const char*>(q);
    return a < b + bytes && b < a + bytes;
  };
  if (overlap(out, x) || (addend && overlap(out, addend)))
    return fail(DG_ERR_INVALID_ARG, "out overlaps x or addend");

  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  const Layout& L = hd->L;
  const bool i4 = c.expert_w_dtype == DG_I4G128;
  const bool q8 = c.expert_w_dtype == DG_Q8_0;
  const bool mx4 = c.expert_w_dtype == DG_MXFP4;
  const bool mx8 = c.expert_w_dtype == DG_MXFP8;
  // per-kernel start/stop events: norm, logits, permute, gate_up, down, combine
  dg::KernelEvents kev[6];
  if (events)
    for (int i = 0; i < 6; ++i) {
      kev[i].start = static_cast<hipEvent_t>(events[2 * i]);
      kev[i].stop = static_cast<hipEvent_t>(events[2 * i + 1]);
    }
  auto ev = [&](int i) -> const dg::KernelEvents* { return events ? &kev[i] : nullptr; };

  dg::RouterArgs ra{};
  ra.x = x;
  ra.x_f32 = c.act_dtype == DG_F32;
  ra.T = T;
  ra.D = c.d_model;
  ra.E = c.n_experts;
  ra.Epad = L.Epad;
  ra.K = c.top_k;
  ra.wr = hd->at<float>(L.wr);
  ra.bias = hd->has_bias ? hd->at<float>(L.bias) : nullptr;
  ra.gamma_e = hd->at<float>(L.gamma_e);
  ra.eps = c.rms_eps;
  ra.n_cu = hd->n_cu;
  ra.no_wait = (flags & DG_FWD_ROUTER_NO_WAIT) ? 1 : 0;
  ra.h_f16 = (i4 || q8) ? 1 : 0;  // MXFP4 / MXFP8 widen to bf16 (their block scales need bf16's exponent range)
  ra.h = L.fold ? nullptr : hd->at<uint16_t>(L.h);
  ra.rnorm = hd->at<float>(L.rnorm);
  ra.logits = hd->at<float>(L.logits);
  ra.tile_count = hd->at<uint64_t>(L.tile_count);
  ra.topk_idx = hd->at<int32_t>(L.topk_idx);
  ra.topk_w = hd->at<float>(L.topk_w);
  ra.dev_flags = hd->at<uint32_t>(L.dev_flags);
  hipError_t e = hipSuccess;
  if (events) {  // the router writes the expert input: the norm's two events mark the same point
    e = hipEventRecord(kev[0].start, stream);
    if (e == hipSuccess) e = hipEventRecord(kev[0].stop, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "event record");
  e = dg::launch_logits(ra, stream, ev(1));
  if (e != hipSuccess) return hip_fail(e, "router launch");

  dg::PermuteArgs pa{};
  pa.topk_idx = ra.topk_idx;
  pa.T = T;
  pa.K = c.top_k;
  pa.E = c.n_experts;
  const bool fused = fuses_gemms(c);
  const int tile_rows = c.expert_w_dtype == DG_BF16 ? dg::bf16_tile_rows(T, c.top_k, c.n_experts)
                        : (i4 && !fused)            ? dg::kTileRows
                                                    : dg::quant_tile_rows(T, c.top_k, c.n_experts);
  const bool tall = tile_rows > dg::kTileRows;
  pa.tile_rows = tile_rows;
  pa.deal = fused ? dg::kDealBalanced : tall ? dg::kDealExperts : dg::kDealUnits;
  pa.tile_done = fused ? hd->at<uint64_t>(L.tile_done) : nullptr;
  pa.nb[0] = dg::gate_up_blocks(c.d_ff, tile_rows);
  pa.nb[1] = dg::down_blocks(c.d_model, tile_rows);
  for (int g = 0; g < 2; ++g) {
    pa.qmax[g] = dg::max_queue_len(T, c.top_k, c.n_experts, pa.nb[g], pa.tile_rows);
    pa.tasks[g] = hd->at<dg::Tile>(L.tasks[g]);
  }
  pa.counts = hd->at<int32_t>(L.counts);
  pa.offsets = hd->at<int32_t>(L.offsets);
  pa.qlen = hd->at<int32_t>(L.qlen);
  pa.sorted_slot = hd->at<int32_t>(L.sorted_slot);
  pa.row_of_slot = hd->at<int32_t>(L.row_of_slot);
  pa.dev_flags = ra.dev_flags;
  e = dg::launch_permute(pa, stream, ev(2));
  if (e != hipSuccess) return hip_fail(e, "permute launch");

  dg::GemmArgs ga{};
  ga.tiles = pa.tasks[0];
  ga.qlen = pa.qlen;
  ga.qmax = pa.qmax[0];
  ga.sorted_slot = pa.sorted_slot;
  ga.K = c.top_k;
  ga.h = L.fold ? static_cast<const uint16_t*>(x) : ra.h;
  ga.rnorm = L.fold ? ra.rnorm : nullptr;
  ga.w_gate_up = hd->w_gate_up;
  ga.w_down = hd->w_down;
  ga.w_packed = hd->w_packed;
  ga.s_gate_up = hd->s_gate_up;
  ga.s_down = hd->s_down;
  ga.act = hd->at<uint16_t>(L.act);
  ga.y = hd->at<uint16_t>(L.y);
  ga.D = c.d_model;
  ga.F = c.d_ff;
  if (fused) {
    dg::FusedGemmArgs fa{};
    fa.gu = ga;
    fa.dn = ga;
    fa.dn.tiles = pa.tasks[1];
    fa.dn.qlen = pa.qlen + dg::kQueues;
    fa.dn.qmax = pa.qmax[1];
    fa.tile_done = pa.tile_done;
    fa.nb_gate_up = pa.nb[0];
    fa.dev_flags = ra.dev_flags;
    fa.wait_polls = (flags & DG_FWD_GEMM_NO_WAIT) ? 0 : dg::kGemmWaitPolls;
    fa.counts = pa.counts;
    e = mx4  ? dg::launch_gemm_fused_mx4(fa, tile_rows, stream, ev(3))
        : mx8 ? dg::launch_gemm_fused_mx8(fa, tile_rows, stream, ev(3))
        : q8 ? dg::launch_gemm_fused_q8(fa, tile_rows, stream, ev(3))
        : i4 ? dg::launch_gemm_fused_i4(fa, tile_rows, stream, ev(3))
             : dg::launch_gemm_fused(fa, tile_rows, stream, ev(3));
    if (e != hipSuccess) return hip_fail(e, "GEMM launch");
    if (events) {  // one launch for both GEMMs: the down events mark the point after it
      e = hipEventRecord(kev[4].start, stream);
      if (e == hipSuccess) e = hipEventRecord(kev[4].stop, stream);
      if (e != hipSuccess) return hip_fail(e, "event record");
    }
  } else {
    // int4 experts read in place (row-major codes): two launches
    e = dg::launch_gate_up_i4(ga, stream, ev(3));
    if (e != hipSuccess) return hip_fail(e, "gate_up launch");
    ga.tiles = pa.tasks[1];
    ga.qlen = pa.qlen + dg::kQueues;
    ga.qmax = pa.qmax[1];
    e = dg::launch_down_i4(ga, stream, ev(4));
    if (e != hipSuccess) return hip_fail(e, "down launch");
  }

  dg::CombineArgs ca{};
  ca.y = ga.y;
  ca.topk_w = ra.topk_w;
  ca.row_of_slot = pa.row_of_slot;
  ca.T = T;
  ca.K = c.top_k;
  ca.D = c.d_model;
  ca.x = (flags & DG_FWD_ADD_INPUT) ? x : nullptr;
  ca.addend = addend;
  ca.out = out;
  ca.act_f32 = c.act_dtype == DG_F32;
  e = dg::launch_combine(ca, stream, ev(5));
  if (e != hipSuccess) return hip_fail(e, "combine launch");

  if (dbg) {
    const size_t tk = (size_t)T * c.top_k;
    struct Cp {
      void* dst;
      size_t off;
      size_t bytes;
    } cps[] = {{dbg->topk_idx, L.topk_idx, tk * 4},
               {dbg->topk_w, L.topk_w, tk * 4},
               {dbg->counts, L.counts, (size_t)c.n_experts * 4},
               {dbg->offsets, L.offsets, (size_t)(c.n_experts + 1) * 4},
               {dbg->sorted_slot, L.sorted_slot, tk * 4},
               {dbg->row_of_slot, L.row_of_slot, tk * 4},
               {dbg->queue_len, L.qlen, (2 * dg::kQueues + 2) * 4},
               {dbg->dev_flags, L.dev_flags, 4}};
    for (const Cp& cp : cps) {
      if (!cp.dst) continue;
      e = hipMemcpyAsync(cp.dst, hd->ws + cp.off, cp.bytes, hipMemcpyDeviceToDevice, stream);
      if (e != hipSuccess) return hip_fail(e, "debug copy");
    }
  }
  return ok();
}

dg_status dg_moe_forward(dg_moe_handle hd, const void* x, void* out, int32_t T, const void* addend, uint32_t flags,
                         void* stream) {
  return run_forward(hd, x, out, T, addend, flags, nullptr, nullptr, stream);
}

dg_status dg_moe_forward_profiled(dg_moe_handle hd, const void* x, void* out, int32_t T, const void* addend,
                                  uint32_t flags, void* const* events, void* stream) {
  if (!events) return fail(DG_ERR_INVALID_ARG, "events is NULL");
  for (int i = 0; i < 12; ++i)
    if (!events[i]) return fail(DG_ERR_INVALID_ARG, "events[%d] is NULL", i);
  if (T <= 0) return fail(DG_ERR_SHAPE, "profiled forward needs T > 0");
  return run_forward(hd, x, out, T, addend, flags, nullptr, events, stream);
}

dg_status dg_moe_forward_debug(dg_moe_handle hd, const void* x, void* out, int32_t T, const dg_moe_debug* dbg,
                               void* stream) {
  if (!dbg) return fail(DG_ERR_INVALID_ARG, "debug struct is NULL");
  return run_forward(hd, x, out, T, nullptr, 0, dbg, nullptr, stream);
}

dg_status dg_moe_destroy(dg_moe_handle hd) {
  if (!hd) return ok();
  hipError_t e1 = hd->ws ? hipFree(hd->ws) : hipSuccess;
  hipError_t e2 = hd->packed ? hipFree(hd->packed) : hipSuccess;
  delete hd;
  if (e1 != hipSuccess) return hip_fail(e1, "hipFree(workspace)");
  if (e2 != hipSuccess) return hip_fail(e2, "hipFree(packed weights)");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Canvas output stage

struct dg_head_s {
  dg_head_config cfg;
  int n_cu;             // compute units of the device (persistent workgroups)
  const uint16_t* emb;  // the borrowed table
  char* ws;
  size_t nvb;  // vocabulary tiles of 256
};

namespace {

constexpr int kHeadVocabTile = 256;

dg_status check_head_config(const dg_head_config* c) {
  if (!c) return fail(DG_ERR_INVALID_ARG, "config is NULL");
  if (c->struct_size != sizeof(dg_head_config))
    return fail(DG_ERR_INVALID_ARG, "struct_size %u != %zu", c->struct_size, sizeof(dg_head_config));
  if (c->vocab < 1 || c->vocab > (1 << 24)) return fail(DG_ERR_SHAPE, "vocab %d not in [1, 2^24]", c->vocab);
  if (c->d_model < 64 || c->d_model > 16384 || c->d_model % 64)
    return fail(DG_ERR_SHAPE, "d_model %d must be a multiple of 64 in [64, 16384]", c->d_model);
  if (c->max_tokens < 1 || c->max_tokens > (1 << 20))
    return fail(DG_ERR_SHAPE, "max_tokens %d not in [1, 2^20]", c->max_tokens);
  if (c->h_dtype != DG_BF16) return fail(DG_ERR_DTYPE, "h_dtype %d: only DG_BF16", c->h_dtype);
  if (c->emb_dtype != DG_BF16) return fail(DG_ERR_DTYPE, "emb_dtype %d: only DG_BF16", c->emb_dtype);
  if (c->flags != 0) return fail(DG_ERR_INVALID_ARG, "unknown config flags 0x%x", c->flags);
  return DG_OK;
}

size_t head_nvb(const dg_head_config& c) { return ((size_t)c.vocab + kHeadVocabTile - 1) / kHeadVocabTile; }

// Five arrays of nvb x max_tokens 4-byte partials, each 256-byte aligned.
size_t head_part_bytes(const dg_head_config& c) { return round_up(head_nvb(c) * c.max_tokens * 4, 256); }

bool spans_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Checks the arguments of one call of the stage (config c, T positions); DG_OK or the error.
dg_status head_check_call(const dg_head_config& c, const void* h, int32_t T, float beta, float* logits,
                          float* entropy, int32_t* argmax, float* mean_entropy, void* const* events) {
  if (!h || !entropy || !argmax) return fail(DG_ERR_INVALID_ARG, "h, entropy or argmax is NULL");
  if (!(beta > 0.0f) || !std::isfinite(beta)) return fail(DG_ERR_INVALID_ARG, "beta must be finite and > 0");
  if (T < 0 || T > c.max_tokens) return fail(DG_ERR_SHAPE, "T = %d not in [0, max_tokens = %d]", T, c.max_tokens);
  if (!aligned16(h)) return fail(DG_ERR_ALIGN, "h is not 16-byte aligned");
  const void* outs[] = {logits, entropy, argmax, mean_entropy};
  for (const void* p : outs)
    if (p && (reinterpret_cast<uintptr_t>(p) & 3u)) return fail(DG_ERR_ALIGN, "output %p is not 4-byte aligned", p);
  const size_t nh = (size_t)T * c.d_model * 2;
  const size_t sizes[] = {(size_t)T * c.vocab * 4, (size_t)T * 4, (size_t)T * 4, 4};
  for (int i = 0; i < 4; ++i) {
    if (spans_overlap(outs[i], sizes[i], h, nh)) return fail(DG_ERR_INVALID_ARG, "an output overlaps h");
    for (int j = i + 1; j < 4; ++j)
      if (spans_overlap(outs[i], sizes[i], outs[j], sizes[j])) return fail(DG_ERR_INVALID_ARG, "outputs overlap");
  }
  if (events) {
    if (T == 0) return fail(DG_ERR_INVALID_ARG, "a profiled forward needs T > 0");
    for (int i = 0; i < 6; ++i)
      if (!events[i]) return fail(DG_ERR_INVALID_ARG, "event %d is NULL", i);
  }
  return DG_OK;
}

// Enqueues the stage (arguments already checked, T > 0) with the per-tile
// partials in five arrays of `pb` bytes from `ws` (each laid out [T][nvb]).
dg_status head_enqueue(const dg_head_config& c, const void* emb, int n_cu, char* ws, size_t pb, const void* h,
                       int32_t T, float beta, float* logits, float* entropy, int32_t* argmax, float* mean_entropy,
                       void* const* events, void* stream_v) {
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  dg::HeadArgs a{};
  a.h = static_cast<const uint16_t*>(h);
  a.emb = static_cast<const uint16_t*>(emb);
  a.n_wg = n_cu;
  a.T = T;
  a.V = c.vocab;
  a.D = c.d_model;
  a.beta = beta;
  a.logits = logits;
  a.entropy = entropy;
  a.argmax = argmax;
  a.mean_entropy = mean_entropy;
  a.part_m = reinterpret_cast<float*>(ws);
  a.part_s = reinterpret_cast<float*>(ws + pb);
  a.part_u = reinterpret_cast<float*>(ws + 2 * pb);
  a.part_best = reinterpret_cast<float*>(ws + 3 * pb);
  a.part_id = reinterpret_cast<int32_t*>(ws + 4 * pb);
  dg::KernelEvents kev[3];
  if (events)
    for (int i = 0; i < 3; ++i) {
      kev[i].start = static_cast<hipEvent_t>(events[2 * i]);
      kev[i].stop = static_cast<hipEvent_t>(events[2 * i + 1]);
    }
  hipError_t e = dg::launch_head(a, stream, events ? kev : nullptr);
  if (e != hipSuccess) return hip_fail(e, "output stage launch");
  if (events && !mean_entropy) {
    e = hipEventRecord(kev[2].start, stream);
    if (e == hipSuccess) e = hipEventRecord(kev[2].stop, stream);
    if (e != hipSuccess) return hip_fail(e, "event record");
  }
  return ok();
}

dg_status head_launch(dg_head_handle hd, const void* h, int32_t T, float beta, float* logits, float* entropy,
                      int32_t* argmax, float* mean_entropy, void* const* events, void* stream) {
  if (!hd) return fail(DG_ERR_INVALID_ARG, "handle is NULL");
  const dg_status st = head_check_call(hd->cfg, h, T, beta, logits, entropy, argmax, mean_entropy, events);
  if (st != DG_OK) return st;
  if (T == 0) return ok();
  // partials laid out [T][nvb] (a prefix of each array sized for max_tokens)
  return head_enqueue(hd->cfg, hd->emb, hd->n_cu, hd->ws, head_part_bytes(hd->cfg), h, T, beta, logits, entropy,
                      argmax, mean_entropy, events, stream);
}

// ---------------------------------------------------------------------------
// The stage without a handle, for callers that cannot allocate: its partials
// live in this library-owned device array (one copy per device, held until the
// process ends). Host code never passes the array's name to a kernel or a copy:
// the name is a host-side stand-in; the device address of each device's copy
// comes from hipGetSymbolAddress, taken once per device with it current.
constexpr size_t kHeadScratchBytes = DG_HEAD_NOALLOC_SCRATCH_BYTES;

}  // namespace

static __device__ __align__(256) char scratch[DG_HEAD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
struct DeviceScratch {
  void* ptr = nullptr;  // this device's copy of `scratch`
  int n_cu = 0;
  bool ready = false;
};
std::mutex g_scratch_mu;
DeviceScratch g_scratch[kMaxDevices];

// The device address of the current device's scratch copy and its compute
// units, set up on the device's first call.
dg_status device_scratch(int* dev_out, DeviceScratch* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DG_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  DeviceScratch& d = g_scratch[dev];
  if (!d.ready) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return fail(DG_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    d.ptr = p;
    d.n_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
    d.ready = true;
  }
  *dev_out = dev;
  *out = d;
  return DG_OK;
}

}  // namespace

extern "C" {

dg_status dg_head_forward_noalloc(const dg_head_config* cfg, const void* emb, const void* h, int32_t T, float beta,
                                  float* logits, float* entropy, int32_t* argmax, float* mean_entropy, void* stream) {
  dg_status st = check_head_config(cfg);
  if (st != DG_OK) return st;
  if (!emb) return fail(DG_ERR_INVALID_ARG, "emb is NULL");
  if (!aligned16(emb)) return fail(DG_ERR_ALIGN, "emb is not 16-byte aligned");
  st = head_check_call(*cfg, h, T, beta, logits, entropy, argmax, mean_entropy, nullptr);
  if (st != DG_OK) return st;
  const size_t pb = round_up(head_nvb(*cfg) * (size_t)T * 4, 256);
  if (5 * pb > kHeadScratchBytes)
    return fail(DG_ERR_SHAPE, "T = %d positions over %d vocabulary rows need %zu bytes of partials; the static "
                "scratch holds %zu (T * ceil(V / 256) * 20 bytes, each of the five arrays rounded to 256)",
                T, cfg->vocab, 5 * pb, kHeadScratchBytes);
  if (T == 0) return ok();
  int dev = 0;
  DeviceScratch d;
  st = device_scratch(&dev, &d);
  if (st != DG_OK) return st;
  return head_enqueue(*cfg, emb, d.n_cu, static_cast<char*>(d.ptr), pb, h, T, beta, logits, entropy, argmax,
                      mean_entropy, nullptr, stream);
}

uint64_t dg_head_workspace_bytes(const dg_head_config* cfg) {
  if (check_head_config(cfg) != DG_OK) return 0;
  return 5 * (uint64_t)head_part_bytes(*cfg);
}

dg_status dg_head_create(const dg_head_config* cfg, const void* emb, dg_head_handle* out) {
  if (out) *out = nullptr;
  dg_status st = check_head_config(cfg);
  if (st != DG_OK) return st;
  if (!emb || !out) return fail(DG_ERR_INVALID_ARG, "emb or out is NULL");
  if (!aligned16(emb)) return fail(DG_ERR_ALIGN, "emb is not 16-byte aligned");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(DG_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
  dg_head_s* hd = new (std::nothrow) dg_head_s();
  if (!hd) return fail(DG_ERR_OOM, "host allocation failed");
  hd->cfg = *cfg;
  hd->n_cu = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  hd->emb = static_cast<const uint16_t*>(emb);
  hd->nvb = head_nvb(*cfg);
  const size_t bytes = 5 * head_part_bytes(*cfg);
  e = hipMalloc(reinterpret_cast<void**>(&hd->ws), bytes);
  if (e != hipSuccess) {
    delete hd;
    (void)hipGetLastError();
    return fail(DG_ERR_OOM, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
  }
  *out = hd;
  return ok();
}

dg_status dg_head_forward(dg_head_handle hd, const void* h, int32_t T, float beta, float* logits, float* entropy,
                          int32_t* argmax, float* mean_entropy, void* stream) {
  return head_launch(hd, h, T, beta, logits, entropy, argmax, mean_entropy, nullptr, stream);
}

dg_status dg_head_forward_profiled(dg_head_handle hd, const void* h, int32_t T, float beta, float* logits,
                                   float* entropy, int32_t* argmax, float* mean_entropy, void* const* events,
                                   void* stream) {
  if (!events) return fail(DG_ERR_INVALID_ARG, "events is NULL");
  return head_launch(hd, h, T, beta, logits, entropy, argmax, mean_entropy, events, stream);
}

dg_status dg_head_destroy(dg_head_handle hd) {
  if (!hd) return ok();
  hipError_t e = hd->ws ? hipFree(hd->ws) : hipSuccess;
  delete hd;
  if (e != hipSuccess) return hip_fail(e, "hipFree");
  return ok();
}

}  // extern "C"
