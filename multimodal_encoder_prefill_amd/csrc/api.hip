// C ABI of libmhe (declared in include/mhe.h): argument checks, workspace
// carving and the launch sequence of one decoder layer and of the whole
// prefill. Every check runs on the host before the first launch of a call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mhe.h"
#include "internal.h"

using mhe::bf16_t;

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return MHE_OK;
  return fail(MHE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxSeq = 1 << 17;
// Activation buffers that feed a GEMM as its A operand get this many extra
// elements per row: row strides that are multiples of 2 KB make the 128-byte
// row pieces a GEMM k-step loads collide in the same L2 channels.
constexpr int kActPad = 128;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int32_t check_config(const mhe_config* c) {
  if (!c) return fail(MHE_ERR_NULL, "config is NULL");
  if (c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->intermediate <= 0)
    return fail(MHE_ERR_SHAPE, "config sizes must be positive");
  if (c->n_heads % c->n_kv_heads != 0)
    return fail(MHE_ERR_SHAPE, "n_heads (%d) is not a multiple of n_kv_heads (%d)", c->n_heads,
                c->n_kv_heads);
  if (c->head_dim % 2 != 0) return fail(MHE_ERR_SHAPE, "head_dim must be even");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps))
    return fail(MHE_ERR_SHAPE, "rms_eps must be finite and >= 0");
  if (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta))
    return fail(MHE_ERR_SHAPE, "rope_theta must be finite and > 0");
  for (int i = 0; i < 3; ++i)
    if (c->mrope_section[i] < 0) return fail(MHE_ERR_SHAPE, "mrope_section must be >= 0");
  if (!mhe::attention_supported(c->n_heads, c->n_kv_heads, c->head_dim))
    return fail(MHE_ERR_UNSUPPORTED,
                "attention built for head_dim 64/128 and 1, 2, 4 or 8 query heads per kv head "
                "(got head_dim %d, %d/%d heads)",
                c->head_dim, c->n_heads, c->n_kv_heads);
  if (!mhe::rmsnorm_supported(c->hidden))
    return fail(MHE_ERR_UNSUPPORTED, "hidden %d: must be a multiple of 8 and <= 8192", c->hidden);
  const int qw = c->n_heads * c->head_dim;
  const int qkvw = (c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
  if (!mhe::gemm_supported(qkvw, c->hidden) || !mhe::gemm_supported(c->hidden, qw) ||
      !mhe::gemm_supported(c->intermediate, c->hidden) ||
      !mhe::gemm_supported(c->hidden, c->intermediate))
    return fail(MHE_ERR_UNSUPPORTED,
                "GEMM needs hidden, n_heads*head_dim and intermediate to be multiples of 64");
  return MHE_OK;
}

// The FP8 layer's GEMMs need k % 128 == 0 for all four projections.
int32_t check_config_fp8(const mhe_config* c) {
  int32_t rc;
  if ((rc = check_config(c))) return rc;
  const int qw = c->n_heads * c->head_dim;
  const int qkvw = (c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
  if (!mhe::gemm_fp8_supported(qkvw, c->hidden) || !mhe::gemm_fp8_supported(c->hidden, qw) ||
      !mhe::gemm_fp8_supported(c->intermediate, c->hidden) ||
      !mhe::gemm_fp8_supported(c->hidden, c->intermediate))
    return fail(MHE_ERR_UNSUPPORTED,
                "FP8 GEMM needs hidden, n_heads*head_dim and intermediate to be multiples of 128");
  return MHE_OK;
}

struct Workspace {
  int ld_h, ld_o, ld_i;  // row strides of hn, ao, act
  bf16_t* hn;    // [S, H] with row stride ld_h
  bf16_t* qkv;   // [S, (Hq + 2 Hkv) D]
  bf16_t* kn;    // [Hkv, Sp, D]
  bf16_t* vt;    // [Hkv, D, Sp]
  bf16_t* ao;    // [S, Hq D] with row stride ld_o
  bf16_t* act;   // [S, I] with row stride ld_i, aliases qkv..ao (used after attention)
  int32_t* vis;  // [S]
  int32_t* cnt;  // [1]
  float2* rope;  // [S][D/2] rotary cos/sin, formed once per call
  float* partial;  // split-K partial tiles of the GEMMs' last wave
  size_t partial_bytes;
  // FP8 layers only: E4M3 copy of the current GEMM input (row strides in
  // bytes ld8_h / ld8_o / ld8_i by the input), its four per-call scales and
  // the partial maxima of the quantisation
  uint8_t* q8;
  int ld8_h, ld8_o, ld8_i;
  float* scales;   // [4]: the per-call scales of the four GEMM inputs
  float* factors;  // [4]: 448 / max|input|
  float* amax;     // partial maxima of the input being quantised
  size_t total;
};

Workspace carve(const mhe_config& c, int seq, char* base, bool fp8 = false) {
  const size_t S = static_cast<size_t>(seq);
  const size_t sp = static_cast<size_t>(mhe::seq_pad(seq));
  const size_t D = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads;
  Workspace w{};
  w.ld_h = c.hidden + kActPad;
  w.ld_o = c.n_heads * c.head_dim + kActPad;
  w.ld_i = c.intermediate + kActPad;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  w.hn = reinterpret_cast<bf16_t*>(take(S * w.ld_h * 2));
  const size_t region_start = off;
  w.qkv = reinterpret_cast<bf16_t*>(take(S * (Hq + 2 * Hkv) * D * 2));
  w.kn = reinterpret_cast<bf16_t*>(take(Hkv * sp * D * 2));
  w.vt = reinterpret_cast<bf16_t*>(take(Hkv * D * sp * 2));
  w.ao = reinterpret_cast<bf16_t*>(take(S * w.ld_o * 2));
  const size_t attn_bytes = off - region_start;
  const size_t act_bytes = align_up(S * w.ld_i * 2);
  w.act = reinterpret_cast<bf16_t*>(base ? base + region_start : nullptr);
  if (act_bytes > attn_bytes) off = region_start + act_bytes;
  w.vis = reinterpret_cast<int32_t*>(take(S * 4));
  w.cnt = reinterpret_cast<int32_t*>(take(4));
  w.rope = reinterpret_cast<float2*>(take(S * (D / 2) * sizeof(float2)));
  w.partial_bytes = mhe::gemm_partial_bytes();
  w.partial = reinterpret_cast<float*>(take(w.partial_bytes));
  if (fp8) {
    w.ld8_h = c.hidden + kActPad;
    w.ld8_o = c.n_heads * c.head_dim + kActPad;
    w.ld8_i = c.intermediate + kActPad;
    w.q8 = reinterpret_cast<uint8_t*>(take(S * std::max({w.ld8_h, w.ld8_o, w.ld8_i})));
    w.scales = reinterpret_cast<float*>(take(4 * sizeof(float)));
    w.factors = reinterpret_cast<float*>(take(4 * sizeof(float)));
    const int parts = std::max({mhe::kAmaxParts, mhe::rmsnorm_fp8_parts(seq),
                                mhe::gemm_amax_parts(seq, c.intermediate),
                                mhe::attention_amax_parts(seq, c.n_kv_heads)});
    w.amax = reinterpret_cast<float*>(take(static_cast<size_t>(parts) * sizeof(float)));
  }
  w.total = off;
  return w;
}

// The kernels move tensors in 16-byte vectors (and 16-byte LDS-DMA loads),
// so every tensor starts on a 16-byte boundary; scales are single floats.
bool misaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int32_t check_weights_fp8(const mhe_layer_weights_fp8* w, int layer) {
  if (!w) return fail(MHE_ERR_NULL, "layer %d weights table is NULL", layer);
  const void* p[] = {w->ln_in, w->w_qkv, w->s_qkv, w->q_norm, w->k_norm, w->w_o, w->s_o,
                     w->ln_post, w->w_gate_up, w->s_gate_up, w->w_down, w->s_down};
  const char* names[] = {"ln_in", "w_qkv", "s_qkv", "q_norm", "k_norm", "w_o", "s_o",
                         "ln_post", "w_gate_up", "s_gate_up", "w_down", "s_down"};
  const bool is_scale[] = {false, false, true, false, false, false, true, false, false, true, false, true};
  for (int i = 0; i < 12; ++i) {
    if (!p[i]) return fail(MHE_ERR_NULL, "layer %d: %s is NULL", layer, names[i]);
    if (!is_scale[i] && misaligned16(p[i]))
      return fail(MHE_ERR_SHAPE, "layer %d: %s is not 16-byte aligned", layer, names[i]);
  }
  return MHE_OK;
}

int32_t check_weights(const mhe_layer_weights* w, int layer) {
  if (!w) return fail(MHE_ERR_NULL, "layer %d weights table is NULL", layer);
  const void* p[] = {w->ln_in, w->w_q, w->w_k, w->w_v, w->q_norm, w->k_norm,
                     w->w_o, w->ln_post, w->w_gate, w->w_up, w->w_down};
  const char* names[] = {"ln_in", "w_q", "w_k", "w_v", "q_norm", "k_norm",
                         "w_o", "ln_post", "w_gate", "w_up", "w_down"};
  for (int i = 0; i < 11; ++i) {
    if (!p[i]) return fail(MHE_ERR_NULL, "layer %d: %s is NULL", layer, names[i]);
    if (misaligned16(p[i])) return fail(MHE_ERR_SHAPE, "layer %d: %s is not 16-byte aligned", layer, names[i]);
  }
  return MHE_OK;
}

int32_t check_seq(int32_t seq) {
  if (seq <= 0 || seq > kMaxSeq) return fail(MHE_ERR_SHAPE, "seq %d out of range [1, %d]", seq, kMaxSeq);
  return MHE_OK;
}

int32_t check_ws(const void* ws, size_t have, size_t need) {
  if (!ws) return fail(MHE_ERR_NULL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
    return fail(MHE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(MHE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  return MHE_OK;
}

// ---- opt-in launch timing: event pairs around the launches of chosen steps ----
struct EventPair {
  hipEvent_t start, stop;
};
struct StepTrace {
  std::vector<EventPair> pending;
  double done_ms = 0.0;
  int64_t launches = 0;
};
std::atomic<uint32_t> g_trace_mask{0};
std::mutex g_trace_mu;
StepTrace g_trace[MHE_STEP_COUNT];
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pooled_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (returning hipError_t); when the step is traced, brackets it
// with two events recorded on `st`.
template <typename F>
int32_t traced(int step, hipStream_t st, const char* what, F&& launch) {
  if (!(g_trace_mask.load(std::memory_order_relaxed) & (1u << step))) return hip_check(launch(), what);
  EventPair ev{nullptr, nullptr};
  {
    std::lock_guard<std::mutex> lk(g_trace_mu);
    ev.start = pooled_event();
    ev.stop = pooled_event();
  }
  if (!ev.start || !ev.stop) return fail(MHE_ERR_HIP, "%s: could not create trace events", what);
  int32_t rc;
  if ((rc = hip_check(hipEventRecord(ev.start, st), "trace event"))) return rc;
  if ((rc = hip_check(launch(), what))) return rc;
  if ((rc = hip_check(hipEventRecord(ev.stop, st), "trace event"))) return rc;
  std::lock_guard<std::mutex> lk(g_trace_mu);
  g_trace[step].pending.push_back(ev);
  return MHE_OK;
}

// The launch sequence of one decoder layer (arguments already checked).
int32_t run_layer(const mhe_config& c, const mhe_layer_weights& w, bf16_t* x, const int32_t* pos,
                  int seq, const Workspace& ws, hipStream_t st) {
  const int H = c.hidden, D = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads;
  const int qw = Hq * D, kvw = Hkv * D;
  int32_t rc;
  if ((rc = traced(MHE_STEP_INPUT_NORM, st, "input rmsnorm", [&] {
         return mhe::launch_rmsnorm(x, static_cast<const bf16_t*>(w.ln_in), ws.hn, ws.ld_h, seq, H,
                                    c.rms_eps, st);
       })))
    return rc;
  // q | k | v projections in one launch
  const mhe::BSegments qkv{{static_cast<const bf16_t*>(w.w_q), static_cast<const bf16_t*>(w.w_k),
                            static_cast<const bf16_t*>(w.w_v)},
                           {qw, kvw, kvw},
                           3};
  if ((rc = traced(MHE_STEP_QKV, st, "qkv projection", [&] {
         return mhe::launch_gemm(mhe::Epilogue::kStore, ws.hn, ws.ld_h, qkv, H, ws.qkv, qw + 2 * kvw, nullptr, seq, qw + 2 * kvw, H,
                                ws.partial, ws.partial_bytes, st);
       })))
    return rc;
  // k norm + rotary, K and V relayout; q norm + rotary inside the attention
  const mhe::RopeParams rp{Hq, Hkv, D, c.rms_eps, c.rope_theta,
                           {c.mrope_section[0], c.mrope_section[1], c.mrope_section[2]}};
  if ((rc = traced(MHE_STEP_QK_ROPE, st, "k norm + rotary", [&] {
         return mhe::launch_k_norm_rope(rp, ws.qkv, static_cast<const bf16_t*>(w.k_norm), pos, seq, ws.kn,
                                        ws.vt, st, ws.rope);
       })))
    return rc;
  if ((rc = traced(MHE_STEP_ATTENTION, st, "attention", [&] {
         return mhe::launch_attention_qnorm(ws.qkv, qw + 2 * kvw, static_cast<const bf16_t*>(w.q_norm), ws.rope,
                                            c.rms_eps, ws.kn, ws.vt, ws.ao, ws.ld_o, seq, Hq, Hkv, D, st);
       })))
    return rc;
  // O projection + residual, in place on x
  const mhe::BSegments wo{{static_cast<const bf16_t*>(w.w_o), nullptr, nullptr}, {H, 0, 0}, 1};
  if ((rc = traced(MHE_STEP_O_PROJ, st, "o projection", [&] {
         return mhe::launch_gemm(mhe::Epilogue::kResidual, ws.ao, ws.ld_o, wo, qw, x, H, x, seq, H, qw, ws.partial,
                                ws.partial_bytes, st);
       })))
    return rc;
  if ((rc = traced(MHE_STEP_POST_NORM, st, "post-attention rmsnorm", [&] {
         return mhe::launch_rmsnorm(x, static_cast<const bf16_t*>(w.ln_post), ws.hn, ws.ld_h, seq, H,
                                    c.rms_eps, st);
       })))
    return rc;
  const mhe::BSegments gu{{static_cast<const bf16_t*>(w.w_gate), static_cast<const bf16_t*>(w.w_up), nullptr},
                          {c.intermediate, c.intermediate, 0},
                          2};
  if ((rc = traced(MHE_STEP_GATE_UP, st, "gate/up projection", [&] {
         return mhe::launch_gemm(mhe::Epilogue::kSwiGLU, ws.hn, ws.ld_h, gu, H, ws.act, ws.ld_i, nullptr, seq, c.intermediate, H,
                                ws.partial, ws.partial_bytes, st);
       })))
    return rc;
  const mhe::BSegments wd{{static_cast<const bf16_t*>(w.w_down), nullptr, nullptr}, {H, 0, 0}, 1};
  return traced(MHE_STEP_DOWN, st, "down projection", [&] {
    return mhe::launch_gemm(mhe::Epilogue::kResidual, ws.act, ws.ld_i, wd, c.intermediate, x, H, x, seq, H, c.intermediate,
                            ws.partial, ws.partial_bytes, st);
  });
}

// Per-tensor E4M3 copy of x [seq, cols] (row stride ldx) into ws.q8 (row
// stride ldq bytes) with its scale in ws.scales[slot]. `parts` partial maxima
// of |x| are already in ws.amax when parts > 0; otherwise they are taken here.
int32_t quantize_input(const bf16_t* x, int ldx, int seq, int cols, int ldq, int slot, int parts,
                       const Workspace& ws, hipStream_t st) {
  return traced(MHE_STEP_QUANTIZE, st, "fp8 quantize", [&] {
    hipError_t e;
    if (parts <= 0) {
      parts = mhe::amax_parts(seq);
      if ((e = mhe::launch_amax(x, ldx, seq, cols, ws.amax, parts, st)) != hipSuccess) return e;
    }
    if ((e = mhe::launch_amax_finalize(ws.amax, parts, ws.scales + slot, ws.factors + slot, st)) != hipSuccess)
      return e;
    return mhe::launch_quantize_fp8(x, ldx, seq, cols, ws.factors + slot, ws.q8, ldq, st);
  });
}

// The decoder layer with its four linears in FP8 (weights quantised
// beforehand, activations here): the launch sequence of run_layer with each
// GEMM input quantised per tensor. The RMSNorm outputs go straight to E4M3
// (the codes of the bf16 rows the bf16 layer would write); the attention and
// gate/up kernels emit the partial maxima of their outputs, so no input
// needs a separate maximum sweep.
int32_t run_layer(const mhe_config& c, const mhe_layer_weights_fp8& w, bf16_t* x, const int32_t* pos,
                  int seq, const Workspace& ws, hipStream_t st) {
  const int H = c.hidden, D = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads, I = c.intermediate;
  const int qw = Hq * D, qkvw = qw + 2 * Hkv * D;
  const uint8_t* wgu = static_cast<const uint8_t*>(w.w_gate_up);
  int32_t rc;
  if ((rc = traced(MHE_STEP_INPUT_NORM, st, "input rmsnorm", [&] {
         return mhe::launch_rmsnorm_fp8(x, static_cast<const bf16_t*>(w.ln_in), seq, H, c.rms_eps, ws.amax,
                                        ws.scales + 0, ws.factors + 0, ws.q8, ws.ld8_h, st);
       })))
    return rc;
  const mhe::F8Segments qkv{{static_cast<const uint8_t*>(w.w_qkv), nullptr, nullptr}, {qkvw, 0, 0},
                            {w.s_qkv, nullptr, nullptr}, 1};
  if ((rc = traced(MHE_STEP_QKV, st, "qkv projection", [&] {
         return mhe::launch_gemm_fp8(mhe::Epilogue::kStore, ws.q8, ws.ld8_h, ws.scales + 0, qkv, H, ws.qkv,
                                     qkvw, nullptr, seq, qkvw, H, ws.partial, ws.partial_bytes, st);
       })))
    return rc;
  const mhe::RopeParams rp{Hq, Hkv, D, c.rms_eps, c.rope_theta,
                           {c.mrope_section[0], c.mrope_section[1], c.mrope_section[2]}};
  if ((rc = traced(MHE_STEP_QK_ROPE, st, "k norm + rotary", [&] {
         return mhe::launch_k_norm_rope(rp, ws.qkv, static_cast<const bf16_t*>(w.k_norm), pos, seq, ws.kn,
                                        ws.vt, st, ws.rope);
       })))
    return rc;
  if ((rc = traced(MHE_STEP_ATTENTION, st, "attention", [&] {
         return mhe::launch_attention_qnorm(ws.qkv, qkvw, static_cast<const bf16_t*>(w.q_norm), ws.rope,
                                            c.rms_eps, ws.kn, ws.vt, ws.ao, ws.ld_o, seq, Hq, Hkv, D, st,
                                            ws.amax);
       })))
    return rc;
  if ((rc = quantize_input(ws.ao, ws.ld_o, seq, qw, ws.ld8_o, 1, mhe::attention_amax_parts(seq, Hkv), ws, st)))
    return rc;
  const mhe::F8Segments wo{{static_cast<const uint8_t*>(w.w_o), nullptr, nullptr}, {H, 0, 0},
                           {w.s_o, nullptr, nullptr}, 1};
  if ((rc = traced(MHE_STEP_O_PROJ, st, "o projection", [&] {
         return mhe::launch_gemm_fp8(mhe::Epilogue::kResidual, ws.q8, ws.ld8_o, ws.scales + 1, wo, qw, x, H,
                                     x, seq, H, qw, ws.partial, ws.partial_bytes, st);
       })))
    return rc;
  if ((rc = traced(MHE_STEP_POST_NORM, st, "post-attention rmsnorm", [&] {
         return mhe::launch_rmsnorm_fp8(x, static_cast<const bf16_t*>(w.ln_post), seq, H, c.rms_eps, ws.amax,
                                        ws.scales + 2, ws.factors + 2, ws.q8, ws.ld8_h, st);
       })))
    return rc;
  const mhe::F8Segments gu{{wgu, wgu + static_cast<size_t>(I) * H, nullptr}, {I, I, 0},
                           {w.s_gate_up, w.s_gate_up, nullptr}, 2};
  int act_parts = 0;
  if ((rc = traced(MHE_STEP_GATE_UP, st, "gate/up projection", [&] {
         return mhe::launch_gemm_fp8(mhe::Epilogue::kSwiGLU, ws.q8, ws.ld8_h, ws.scales + 2, gu, H, ws.act,
                                     ws.ld_i, nullptr, seq, I, H, ws.partial, ws.partial_bytes, st, ws.amax,
                                     &act_parts);
       })))
    return rc;
  if (act_parts <= 0) return fail(MHE_ERR_HIP, "gate/up projection wrote no partial maxima");
  if ((rc = quantize_input(ws.act, ws.ld_i, seq, I, ws.ld8_i, 3, act_parts, ws, st))) return rc;
  const mhe::F8Segments wd{{static_cast<const uint8_t*>(w.w_down), nullptr, nullptr}, {H, 0, 0},
                           {w.s_down, nullptr, nullptr}, 1};
  return traced(MHE_STEP_DOWN, st, "down projection", [&] {
    return mhe::launch_gemm_fp8(mhe::Epilogue::kResidual, ws.q8, ws.ld8_i, ws.scales + 3, wd, I, x, H, x,
                                seq, H, I, ws.partial, ws.partial_bytes, st);
  });
}

int32_t check_weights(const mhe_layer_weights_fp8* w, int layer) { return check_weights_fp8(w, layer); }
int32_t check_config_for(const mhe_layer_weights*, const mhe_config* c) { return check_config(c); }
int32_t check_config_for(const mhe_layer_weights_fp8*, const mhe_config* c) { return check_config_fp8(c); }
constexpr bool is_fp8(const mhe_layer_weights*) { return false; }
constexpr bool is_fp8(const mhe_layer_weights_fp8*) { return true; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + bn && pb < pa + an;
}

// The rotary cos/sin of every (token, slot), shared by all layers of a call.
int32_t rope_table(const mhe_config& c, const int32_t* pos, int seq, const Workspace& ws, hipStream_t st) {
  const mhe::RopeParams rp{c.n_heads, c.n_kv_heads, c.head_dim, c.rms_eps, c.rope_theta,
                           {c.mrope_section[0], c.mrope_section[1], c.mrope_section[2]}};
  return traced(MHE_STEP_QK_ROPE, st, "rotary table",
                [&] { return mhe::launch_rope_table(rp, pos, seq, ws.rope, st); });
}

// mhe_layer_forward / mhe_layer_forward_fp8.
template <class W>
int32_t layer_forward_impl(const mhe_config* cfg, const W* w, void* hidden, const int32_t* positions,
                           int32_t seq, void* workspace, size_t workspace_bytes, void* stream) {
  constexpr bool fp8 = is_fp8(static_cast<const W*>(nullptr));
  int32_t rc;
  if ((rc = check_config_for(w, cfg))) return rc;
  if ((rc = check_weights(w, 0))) return rc;
  if (!hidden) return fail(MHE_ERR_NULL, "hidden is NULL");
  if (!positions) return fail(MHE_ERR_NULL, "positions is NULL");
  if (misaligned16(hidden)) return fail(MHE_ERR_SHAPE, "hidden is not 16-byte aligned");
  if ((rc = check_seq(seq))) return rc;
  const Workspace need = carve(*cfg, seq, nullptr, fp8);
  if ((rc = check_ws(workspace, workspace_bytes, need.total))) return rc;
  const Workspace ws = carve(*cfg, seq, static_cast<char*>(workspace), fp8);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = rope_table(*cfg, positions, seq, ws, st))) return rc;
  return run_layer(*cfg, *w, static_cast<bf16_t*>(hidden), positions, seq, ws, st);
}

// mhe_encode / mhe_encode_fp8 (W: the layer weight table type).
template <class W>
int32_t encode_impl(const mhe_config* cfg, const W* layers, int32_t n_layers,
                    const void* inputs_embeds, const int32_t* positions,
                    const uint8_t* visual_mask, int32_t n_vis, const void* const* deepstack,
                    int32_t n_ds, int32_t seq, void* out, void* workspace, size_t workspace_bytes,
                    void* stream) {
  constexpr bool fp8 = is_fp8(static_cast<const W*>(nullptr));
  int32_t rc;
  if ((rc = check_config_for(layers, cfg))) return rc;
  if ((rc = check_seq(seq))) return rc;
  if (n_layers < 0) return fail(MHE_ERR_SHAPE, "n_layers %d < 0", n_layers);
  if (n_ds < 0) return fail(MHE_ERR_SHAPE, "n_ds %d < 0", n_ds);
  if (n_vis < 0 || n_vis > seq) return fail(MHE_ERR_SHAPE, "n_vis %d out of range [0, %d]", n_vis, seq);
  if (!inputs_embeds || !out) return fail(MHE_ERR_NULL, "inputs_embeds and out are required");
  if (!positions) return fail(MHE_ERR_NULL, "positions is NULL");
  if (misaligned16(inputs_embeds) || misaligned16(out))
    return fail(MHE_ERR_SHAPE, "inputs_embeds and out must be 16-byte aligned");
  if (n_layers > 0 && !layers) return fail(MHE_ERR_NULL, "layers is NULL");
  for (int l = 0; l < n_layers; ++l)
    if ((rc = check_weights(&layers[l], l))) return rc;
  const int used_ds = (n_vis > 0) ? (n_ds < n_layers ? n_ds : n_layers) : 0;
  if (used_ds > 0) {
    if (!visual_mask) return fail(MHE_ERR_NULL, "visual_mask is NULL with DeepStack levels");
    if (!deepstack) return fail(MHE_ERR_NULL, "deepstack table is NULL");
    for (int l = 0; l < used_ds; ++l) {
      if (!deepstack[l]) return fail(MHE_ERR_NULL, "deepstack[%d] is NULL", l);
      if (misaligned16(deepstack[l])) return fail(MHE_ERR_SHAPE, "deepstack[%d] is not 16-byte aligned", l);
    }
  }
  const size_t act_bytes = static_cast<size_t>(seq) * cfg->hidden * 2;
  if (overlaps(out, act_bytes, inputs_embeds, act_bytes))
    return fail(MHE_ERR_SHAPE, "out overlaps inputs_embeds");
  const Workspace need = carve(*cfg, seq, nullptr, fp8);
  if ((rc = check_ws(workspace, workspace_bytes, need.total))) return rc;
  if (overlaps(out, act_bytes, workspace, need.total))
    return fail(MHE_ERR_SHAPE, "out overlaps the workspace");

  const Workspace ws = carve(*cfg, seq, static_cast<char*>(workspace), fp8);
  hipStream_t st = static_cast<hipStream_t>(stream);
  bf16_t* x = static_cast<bf16_t*>(out);
  if ((rc = hip_check(hipMemcpyAsync(x, inputs_embeds, act_bytes, hipMemcpyDeviceToDevice, st),
                      "copy inputs_embeds")))
    return rc;
  if (used_ds > 0 &&
      (rc = hip_check(mhe::launch_visual_index(visual_mask, seq, n_vis, ws.vis, ws.cnt, st),
                      "visual index")))
    return rc;
  if (n_layers > 0 && (rc = rope_table(*cfg, positions, seq, ws, st))) return rc;
  for (int l = 0; l < n_layers; ++l) {
    if ((rc = run_layer(*cfg, layers[l], x, positions, seq, ws, st))) return rc;
    if (l < used_ds && (rc = traced(MHE_STEP_DEEPSTACK, st, "deepstack add", [&] {
                          return mhe::launch_deepstack_add(x, cfg->hidden, ws.vis, n_vis,
                                                           static_cast<const bf16_t*>(deepstack[l]), st);
                        })))
      return rc;
  }
  return MHE_OK;
}

}  // namespace

extern "C" {

int32_t mhe_abi_version(void) { return MHE_ABI_VERSION; }

const char* mhe_status_string(int32_t s) {
  switch (s) {
    case MHE_OK: return "ok";
    case MHE_ERR_NULL: return "null pointer";
    case MHE_ERR_SHAPE: return "invalid shape";
    case MHE_ERR_MISMATCH: return "token / grid count mismatch";
    case MHE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MHE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MHE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mhe_last_error(void) { return g_last_error.c_str(); }

int32_t mhe_trace_enable(uint32_t step_mask) {
  if (step_mask >> MHE_STEP_COUNT) return fail(MHE_ERR_SHAPE, "trace mask 0x%x has unknown step bits", step_mask);
  g_trace_mask.store(step_mask);
  return MHE_OK;
}

int32_t mhe_trace_read(int32_t step, double* total_ms, int64_t* launches) {
  if (step < 0 || step >= MHE_STEP_COUNT) return fail(MHE_ERR_SHAPE, "unknown step %d", step);
  if (!total_ms || !launches) return fail(MHE_ERR_NULL, "total_ms and launches are required");
  std::lock_guard<std::mutex> lk(g_trace_mu);
  StepTrace& t = g_trace[step];
  int32_t rc = MHE_OK;
  for (const EventPair& ev : t.pending) {
    float ms = 0.f;
    if (rc == MHE_OK) {
      rc = hip_check(hipEventSynchronize(ev.stop), "trace event synchronize");
      if (rc == MHE_OK) rc = hip_check(hipEventElapsedTime(&ms, ev.start, ev.stop), "trace elapsed time");
      if (rc == MHE_OK) {
        t.done_ms += ms;
        t.launches += 1;
      }
    }
    g_event_pool.push_back(ev.start);
    g_event_pool.push_back(ev.stop);
  }
  t.pending.clear();
  *total_ms = t.done_ms;
  *launches = t.launches;
  t.done_ms = 0.0;
  t.launches = 0;
  return rc;
}

size_t mhe_workspace_bytes(const mhe_config* cfg, int32_t seq) {
  if (check_config(cfg) || check_seq(seq)) return 0;
  return carve(*cfg, seq, nullptr).total;
}

int32_t mhe_layer_forward(const mhe_config* cfg, const mhe_layer_weights* w, void* hidden,
                          const int32_t* positions, int32_t seq, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return layer_forward_impl(cfg, w, hidden, positions, seq, workspace, workspace_bytes, stream);
}

size_t mhe_workspace_bytes_fp8(const mhe_config* cfg, int32_t seq) {
  if (check_config_fp8(cfg) || check_seq(seq)) return 0;
  return carve(*cfg, seq, nullptr, true).total;
}

int32_t mhe_layer_forward_fp8(const mhe_config* cfg, const mhe_layer_weights_fp8* w, void* hidden,
                              const int32_t* positions, int32_t seq, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return layer_forward_impl(cfg, w, hidden, positions, seq, workspace, workspace_bytes, stream);
}

int32_t mhe_deepstack_inject(void* hidden, int32_t seq, int32_t hidden_dim,
                             const uint8_t* visual_mask, int32_t n_vis, const void* feature,
                             void* workspace, size_t workspace_bytes, void* stream) {
  int32_t rc;
  if ((rc = check_seq(seq))) return rc;
  if (hidden_dim <= 0 || hidden_dim % 8 != 0)
    return fail(MHE_ERR_SHAPE, "hidden_dim %d must be a positive multiple of 8", hidden_dim);
  if (n_vis < 0 || n_vis > seq) return fail(MHE_ERR_SHAPE, "n_vis %d out of range [0, %d]", n_vis, seq);
  if (n_vis == 0) return MHE_OK;
  if (!hidden || !visual_mask || !feature) return fail(MHE_ERR_NULL, "hidden, visual_mask and feature are required");
  if ((rc = check_ws(workspace, workspace_bytes, align_up(static_cast<size_t>(seq) * 4) + 256))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* idx = static_cast<int32_t*>(workspace);
  int32_t* cnt = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align_up(static_cast<size_t>(seq) * 4));
  if ((rc = hip_check(mhe::launch_visual_index(visual_mask, seq, n_vis, idx, cnt, st), "visual index")))
    return rc;
  return hip_check(mhe::launch_deepstack_add(static_cast<bf16_t*>(hidden), hidden_dim, idx, n_vis,
                                             static_cast<const bf16_t*>(feature), st),
                   "deepstack add");
}

int32_t mhe_deepstack_inject_noalloc(void* hidden, int32_t seq, int32_t hidden_dim,
                                     const uint8_t* visual_mask, int32_t n_vis, const void* feature,
                                     void* stream) {
  static_assert(kMaxSeq <= mhe::kStaticIndexRows, "the static index scratch covers every seq");
  if (seq <= 0) return fail(MHE_ERR_SHAPE, "seq %d must be > 0", seq);
  if (seq > mhe::kStaticIndexRows)
    return fail(MHE_ERR_SHAPE, "seq %d exceeds the %d tokens the library's static scratch holds", seq,
                mhe::kStaticIndexRows);
  if (hidden_dim <= 0 || hidden_dim % 8 != 0)
    return fail(MHE_ERR_SHAPE, "hidden_dim %d must be a positive multiple of 8", hidden_dim);
  if (n_vis < 0 || n_vis > seq) return fail(MHE_ERR_SHAPE, "n_vis %d out of range [0, %d]", n_vis, seq);
  if (n_vis == 0) return MHE_OK;
  if (!hidden || !visual_mask || !feature) return fail(MHE_ERR_NULL, "hidden, visual_mask and feature are required");
  int32_t *idx = nullptr, *cnt = nullptr;
  int32_t rc;
  if ((rc = hip_check(mhe::static_index_scratch(&idx, &cnt), "static scratch address"))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = hip_check(mhe::launch_visual_index(visual_mask, seq, n_vis, idx, cnt, st), "visual index")))
    return rc;
  return hip_check(mhe::launch_deepstack_add(static_cast<bf16_t*>(hidden), hidden_dim, idx, n_vis,
                                             static_cast<const bf16_t*>(feature), st),
                   "deepstack add");
}

int32_t mhe_encode(const mhe_config* cfg, const mhe_layer_weights* layers, int32_t n_layers,
                   const void* inputs_embeds, const int32_t* positions,
                   const uint8_t* visual_mask, int32_t n_vis, const void* const* deepstack,
                   int32_t n_ds, int32_t seq, void* out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return encode_impl(cfg, layers, n_layers, inputs_embeds, positions, visual_mask, n_vis, deepstack,
                     n_ds, seq, out, workspace, workspace_bytes, stream);
}

int32_t mhe_encode_fp8(const mhe_config* cfg, const mhe_layer_weights_fp8* layers, int32_t n_layers,
                       const void* inputs_embeds, const int32_t* positions,
                       const uint8_t* visual_mask, int32_t n_vis, const void* const* deepstack,
                       int32_t n_ds, int32_t seq, void* out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return encode_impl(cfg, layers, n_layers, inputs_embeds, positions, visual_mask, n_vis, deepstack,
                     n_ds, seq, out, workspace, workspace_bytes, stream);
}

int32_t mhe_count_visual(const uint8_t* visual_mask, int32_t seq, int32_t* count_host,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int32_t rc;
  if ((rc = check_seq(seq))) return rc;
  if (!visual_mask || !count_host) return fail(MHE_ERR_NULL, "visual_mask and count_host are required");
  if ((rc = check_ws(workspace, workspace_bytes, align_up(static_cast<size_t>(seq) * 4) + 256))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* idx = static_cast<int32_t*>(workspace);
  int32_t* cnt = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align_up(static_cast<size_t>(seq) * 4));
  if ((rc = hip_check(mhe::launch_visual_index(visual_mask, seq, 0, idx, cnt, st), "visual index")))
    return rc;
  if ((rc = hip_check(hipMemcpyAsync(count_host, cnt, 4, hipMemcpyDeviceToHost, st), "count copy")))
    return rc;
  return hip_check(hipStreamSynchronize(st), "stream synchronize");
}

int32_t mhe_rms_norm(const void* x, const void* gamma, void* y, int32_t rows, int32_t dim,
                     float eps, void* stream) {
  if (!x || !gamma || !y) return fail(MHE_ERR_NULL, "x, gamma and y are required");
  if (rows <= 0) return fail(MHE_ERR_SHAPE, "rows %d must be > 0", rows);
  if (!mhe::rmsnorm_supported(dim)) return fail(MHE_ERR_UNSUPPORTED, "dim %d: multiple of 8, <= 8192", dim);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(MHE_ERR_SHAPE, "eps must be finite and >= 0");
  return hip_check(mhe::launch_rmsnorm(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(gamma),
                                       static_cast<bf16_t*>(y), dim, rows, dim, eps,
                                       static_cast<hipStream_t>(stream)),
                   "rmsnorm");
}

size_t mhe_linear_workspace_bytes(void) { return mhe::gemm_partial_bytes(); }

static int32_t check_gemm_ws(const void* ws, size_t ws_bytes) {
  if (!ws) return MHE_OK;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
    return fail(MHE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return MHE_OK;
}

int32_t mhe_linear(const void* a, const void* w, void* c, const void* residual, int32_t m,
                   int32_t n, int32_t k, void* workspace, size_t workspace_bytes, void* stream) {
  if (!a || !w || !c) return fail(MHE_ERR_NULL, "a, w and c are required");
  if (m <= 0 || n <= 0 || k <= 0) return fail(MHE_ERR_SHAPE, "m, n, k must be > 0");
  if (!mhe::gemm_supported(n, k)) return fail(MHE_ERR_UNSUPPORTED, "needs n %% 32 == 0 and k %% 64 == 0 (n=%d, k=%d)", n, k);
  const size_t cb = static_cast<size_t>(m) * n * 2;
  if (overlaps(c, cb, a, static_cast<size_t>(m) * k * 2) || overlaps(c, cb, w, static_cast<size_t>(n) * k * 2))
    return fail(MHE_ERR_SHAPE, "c overlaps an operand");
  if (residual && residual != c && overlaps(c, cb, residual, cb))
    return fail(MHE_ERR_SHAPE, "residual partially overlaps c");
  int32_t rc;
  if ((rc = check_gemm_ws(workspace, workspace_bytes))) return rc;
  if (workspace && (overlaps(workspace, workspace_bytes, c, cb) || overlaps(workspace, workspace_bytes, a, static_cast<size_t>(m) * k * 2)))
    return fail(MHE_ERR_SHAPE, "workspace overlaps an operand");
  mhe::BSegments b{{static_cast<const bf16_t*>(w), nullptr, nullptr}, {n, 0, 0}, 1};
  return hip_check(mhe::launch_gemm(residual ? mhe::Epilogue::kResidual : mhe::Epilogue::kStore,
                                    static_cast<const bf16_t*>(a), k, b, k, static_cast<bf16_t*>(c), n,
                                    static_cast<const bf16_t*>(residual), m, n, k,
                                    static_cast<float*>(workspace), workspace ? workspace_bytes : 0,
                                    static_cast<hipStream_t>(stream)),
                   "linear");
}

int32_t mhe_linear_swiglu(const void* a, const void* w_gate, const void* w_up, void* c,
                          int32_t m, int32_t n, int32_t k, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!a || !w_gate || !w_up || !c) return fail(MHE_ERR_NULL, "a, w_gate, w_up and c are required");
  if (m <= 0 || n <= 0 || k <= 0) return fail(MHE_ERR_SHAPE, "m, n, k must be > 0");
  if (!mhe::gemm_supported(n, k)) return fail(MHE_ERR_UNSUPPORTED, "needs n %% 32 == 0 and k %% 64 == 0 (n=%d, k=%d)", n, k);
  const size_t cb = static_cast<size_t>(m) * n * 2;
  if (overlaps(c, cb, a, static_cast<size_t>(m) * k * 2))
    return fail(MHE_ERR_SHAPE, "c overlaps a");
  int32_t rc;
  if ((rc = check_gemm_ws(workspace, workspace_bytes))) return rc;
  if (workspace && overlaps(workspace, workspace_bytes, c, cb))
    return fail(MHE_ERR_SHAPE, "workspace overlaps c");
  mhe::BSegments b{{static_cast<const bf16_t*>(w_gate), static_cast<const bf16_t*>(w_up), nullptr},
                   {n, n, 0},
                   2};
  return hip_check(mhe::launch_gemm(mhe::Epilogue::kSwiGLU, static_cast<const bf16_t*>(a), k, b, k,
                                    static_cast<bf16_t*>(c), n, nullptr, m, n, k,
                                    static_cast<float*>(workspace), workspace ? workspace_bytes : 0,
                                    static_cast<hipStream_t>(stream)),
                   "linear_swiglu");
}

size_t mhe_quantize_fp8_workspace_bytes(void) { return (mhe::kAmaxParts + 64) * sizeof(float); }

int32_t mhe_quantize_fp8(const void* const* parts, const int32_t* part_rows, int32_t n_parts,
                         int32_t cols, void* q, float* scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!parts || !part_rows || !q || !scale) return fail(MHE_ERR_NULL, "parts, part_rows, q and scale are required");
  if (n_parts < 1 || n_parts > 8) return fail(MHE_ERR_SHAPE, "n_parts %d out of range [1, 8]", n_parts);
  if (cols <= 0 || cols % 8 != 0) return fail(MHE_ERR_SHAPE, "cols %d must be a positive multiple of 8", cols);
  int64_t rows = 0;
  for (int i = 0; i < n_parts; ++i) {
    if (!parts[i]) return fail(MHE_ERR_NULL, "parts[%d] is NULL", i);
    if (part_rows[i] <= 0) return fail(MHE_ERR_SHAPE, "part_rows[%d] = %d must be > 0", i, part_rows[i]);
    rows += part_rows[i];
  }
  if (rows * cols > (int64_t(1) << 40)) return fail(MHE_ERR_SHAPE, "tensor too large");
  int32_t rc;
  if ((rc = check_ws(workspace, workspace_bytes, mhe_quantize_fp8_workspace_bytes()))) return rc;
  for (int i = 0; i < n_parts; ++i)
    if (overlaps(q, static_cast<size_t>(rows) * cols, parts[i], static_cast<size_t>(part_rows[i]) * cols * 2))
      return fail(MHE_ERR_SHAPE, "q overlaps parts[%d]", i);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* partial = static_cast<float*>(workspace);
  float* factor = partial + mhe::kAmaxParts;
  // every part gets its share of the partial maxima; one scale over all parts
  int offs[9] = {0};
  for (int i = 0; i < n_parts; ++i)
    offs[i + 1] = offs[i] + std::max(1, std::min(mhe::amax_parts(part_rows[i]), mhe::kAmaxParts / n_parts));
  for (int i = 0; i < n_parts; ++i)
    if ((rc = hip_check(mhe::launch_amax(static_cast<const bf16_t*>(parts[i]), cols, part_rows[i], cols,
                                         partial + offs[i], offs[i + 1] - offs[i], st),
                        "fp8 amax")))
      return rc;
  if ((rc = hip_check(mhe::launch_amax_finalize(partial, offs[n_parts], scale, factor, st), "fp8 scale")))
    return rc;
  uint8_t* dst = static_cast<uint8_t*>(q);
  for (int i = 0; i < n_parts; ++i) {
    if ((rc = hip_check(mhe::launch_quantize_fp8(static_cast<const bf16_t*>(parts[i]), cols, part_rows[i],
                                                 cols, factor, dst, cols, st),
                        "fp8 quantize")))
      return rc;
    dst += static_cast<size_t>(part_rows[i]) * cols;
  }
  return MHE_OK;
}

int32_t mhe_linear_fp8(const void* a, const float* scale_a, const void* w, const float* scale_w,
                       void* c, const void* residual, int32_t m, int32_t n, int32_t k,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!a || !scale_a || !w || !scale_w || !c) return fail(MHE_ERR_NULL, "a, scale_a, w, scale_w and c are required");
  if (m <= 0 || n <= 0 || k <= 0) return fail(MHE_ERR_SHAPE, "m, n, k must be > 0");
  if (!mhe::gemm_fp8_supported(n, k))
    return fail(MHE_ERR_UNSUPPORTED, "needs n %% 32 == 0 and k %% 128 == 0 (n=%d, k=%d)", n, k);
  const size_t cb = static_cast<size_t>(m) * n * 2;
  if (overlaps(c, cb, a, static_cast<size_t>(m) * k) || overlaps(c, cb, w, static_cast<size_t>(n) * k))
    return fail(MHE_ERR_SHAPE, "c overlaps an operand");
  if (residual && residual != c && overlaps(c, cb, residual, cb))
    return fail(MHE_ERR_SHAPE, "residual partially overlaps c");
  int32_t rc;
  if ((rc = check_gemm_ws(workspace, workspace_bytes))) return rc;
  if (workspace && (overlaps(workspace, workspace_bytes, c, cb) || overlaps(workspace, workspace_bytes, a, static_cast<size_t>(m) * k)))
    return fail(MHE_ERR_SHAPE, "workspace overlaps an operand");
  mhe::F8Segments b{{static_cast<const uint8_t*>(w), nullptr, nullptr}, {n, 0, 0}, {scale_w, nullptr, nullptr}, 1};
  return hip_check(mhe::launch_gemm_fp8(residual ? mhe::Epilogue::kResidual : mhe::Epilogue::kStore,
                                        static_cast<const uint8_t*>(a), k, scale_a, b, k,
                                        static_cast<bf16_t*>(c), n, static_cast<const bf16_t*>(residual), m,
                                        n, k, static_cast<float*>(workspace), workspace ? workspace_bytes : 0,
                                        static_cast<hipStream_t>(stream)),
                   "linear_fp8");
}

int32_t mhe_linear_swiglu_fp8(const void* a, const float* scale_a, const void* w_gate_up,
                              const float* scale_w, void* c, int32_t m, int32_t n, int32_t k,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!a || !scale_a || !w_gate_up || !scale_w || !c)
    return fail(MHE_ERR_NULL, "a, scale_a, w_gate_up, scale_w and c are required");
  if (m <= 0 || n <= 0 || k <= 0) return fail(MHE_ERR_SHAPE, "m, n, k must be > 0");
  if (!mhe::gemm_fp8_supported(n, k))
    return fail(MHE_ERR_UNSUPPORTED, "needs n %% 32 == 0 and k %% 128 == 0 (n=%d, k=%d)", n, k);
  const size_t cb = static_cast<size_t>(m) * n * 2;
  if (overlaps(c, cb, a, static_cast<size_t>(m) * k)) return fail(MHE_ERR_SHAPE, "c overlaps a");
  int32_t rc;
  if ((rc = check_gemm_ws(workspace, workspace_bytes))) return rc;
  if (workspace && overlaps(workspace, workspace_bytes, c, cb))
    return fail(MHE_ERR_SHAPE, "workspace overlaps c");
  const uint8_t* wg = static_cast<const uint8_t*>(w_gate_up);
  mhe::F8Segments b{{wg, wg + static_cast<size_t>(n) * k, nullptr}, {n, n, 0}, {scale_w, scale_w, nullptr}, 2};
  return hip_check(mhe::launch_gemm_fp8(mhe::Epilogue::kSwiGLU, static_cast<const uint8_t*>(a), k, scale_a,
                                        b, k, static_cast<bf16_t*>(c), n, nullptr, m, n, k,
                                        static_cast<float*>(workspace), workspace ? workspace_bytes : 0,
                                        static_cast<hipStream_t>(stream)),
                   "linear_swiglu_fp8");
}

int32_t mhe_qk_norm_rope(const mhe_config* cfg, const void* qkv, const void* q_norm,
                         const void* k_norm, const int32_t* positions, int32_t seq, void* q_out,
                         void* k_out, void* vt_out, void* stream) {
  int32_t rc;
  if ((rc = check_config(cfg))) return rc;
  if ((rc = check_seq(seq))) return rc;
  if (!qkv || !q_norm || !k_norm || !positions || !q_out || !k_out || !vt_out)
    return fail(MHE_ERR_NULL, "all buffers are required");
  mhe::RopeParams rp{cfg->n_heads, cfg->n_kv_heads, cfg->head_dim, cfg->rms_eps, cfg->rope_theta,
                     {cfg->mrope_section[0], cfg->mrope_section[1], cfg->mrope_section[2]}};
  return hip_check(mhe::launch_qk_norm_rope(rp, static_cast<const bf16_t*>(qkv),
                                            static_cast<const bf16_t*>(q_norm),
                                            static_cast<const bf16_t*>(k_norm), positions, seq,
                                            static_cast<bf16_t*>(q_out), static_cast<bf16_t*>(k_out),
                                            static_cast<bf16_t*>(vt_out),
                                            static_cast<hipStream_t>(stream)),
                   "q/k norm + rotary");
}

int32_t mhe_attention(const void* q, const void* k, const void* vt, void* o, int32_t seq,
                      int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, void* stream) {
  int32_t rc;
  if ((rc = check_seq(seq))) return rc;
  if (!q || !k || !vt || !o) return fail(MHE_ERR_NULL, "q, k, vt and o are required");
  if (n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads != 0)
    return fail(MHE_ERR_SHAPE, "n_heads must be a positive multiple of n_kv_heads");
  if (!mhe::attention_supported(n_heads, n_kv_heads, head_dim))
    return fail(MHE_ERR_UNSUPPORTED, "head_dim 64/128 and 1, 2, 4 or 8 query heads per kv head");
  return hip_check(mhe::launch_attention(static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                                         static_cast<const bf16_t*>(vt), static_cast<bf16_t*>(o), n_heads * head_dim, seq,
                                         n_heads, n_kv_heads, head_dim,
                                         static_cast<hipStream_t>(stream)),
                   "attention");
}

size_t mhe_qnorm_attention_workspace_bytes(const mhe_config* cfg, int32_t seq) {
  if (!cfg || seq <= 0 || cfg->head_dim <= 0) return 0;
  return align_up(static_cast<size_t>(seq) * (cfg->head_dim / 2) * sizeof(float2));
}

int32_t mhe_qnorm_attention(const mhe_config* cfg, const void* qkv, const void* q_norm,
                            const int32_t* positions, const void* k, const void* vt, void* o,
                            int32_t seq, void* workspace, size_t workspace_bytes, void* stream) {
  int32_t rc;
  if ((rc = check_config(cfg))) return rc;
  if ((rc = check_seq(seq))) return rc;
  if (!qkv || !q_norm || !positions || !k || !vt || !o) return fail(MHE_ERR_NULL, "all buffers are required");
  for (const void* p : {qkv, q_norm, k, vt, static_cast<const void*>(o)})
    if (misaligned16(p)) return fail(MHE_ERR_SHAPE, "qkv, q_norm, k, vt and o must be 16-byte aligned");
  const int D = cfg->head_dim, Hq = cfg->n_heads, Hkv = cfg->n_kv_heads;
  if (!mhe::attention_supported(Hq, Hkv, D))
    return fail(MHE_ERR_UNSUPPORTED, "head_dim 64/128 and 1, 2, 4 or 8 query heads per kv head");
  if ((rc = check_ws(workspace, workspace_bytes, mhe_qnorm_attention_workspace_bytes(cfg, seq)))) return rc;
  const mhe::RopeParams rp{Hq, Hkv, D, cfg->rms_eps, cfg->rope_theta,
                           {cfg->mrope_section[0], cfg->mrope_section[1], cfg->mrope_section[2]}};
  hipStream_t st = static_cast<hipStream_t>(stream);
  float2* table = static_cast<float2*>(workspace);
  if ((rc = hip_check(mhe::launch_rope_table(rp, positions, seq, table, st), "rotary table"))) return rc;
  return hip_check(mhe::launch_attention_qnorm(static_cast<const bf16_t*>(qkv), (Hq + 2 * Hkv) * D,
                                               static_cast<const bf16_t*>(q_norm), table, cfg->rms_eps,
                                               static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(vt),
                                               static_cast<bf16_t*>(o), Hq * D, seq, Hq, Hkv, D, st),
                   "attention with q norm + rotary");
}

// ---- token-level front end ----

int32_t mhe_rope_index(const int32_t* ids, int32_t seq, int32_t image_token_id,
                       int32_t video_token_id, const int32_t* image_grid_thw, int32_t n_images,
                       const int32_t* video_grid_thw, int32_t n_videos, int32_t spatial_merge,
                       int32_t* positions, uint8_t* image_mask, uint8_t* video_mask,
                       uint8_t* visual_mask, int32_t* delta) {
  int32_t rc;
  if ((rc = check_seq(seq))) return rc;
  if (!ids || !positions) return fail(MHE_ERR_NULL, "ids and positions are required");
  if (n_images < 0 || n_videos < 0) return fail(MHE_ERR_SHAPE, "negative grid count");
  if ((n_images > 0 && !image_grid_thw) || (n_videos > 0 && !video_grid_thw))
    return fail(MHE_ERR_NULL, "grid array is NULL");
  if (spatial_merge <= 0) return fail(MHE_ERR_SHAPE, "spatial_merge %d must be > 0", spatial_merge);
  if (image_token_id == video_token_id)
    return fail(MHE_ERR_SHAPE, "image and video token ids must differ");
  for (int i = 0; i < n_videos; ++i)
    if (video_grid_thw[3 * i] <= 0 || video_grid_thw[3 * i] > kMaxSeq)
      return fail(MHE_ERR_SHAPE, "video %d has %d frames", i, video_grid_thw[3 * i]);
  std::string err;
  rc = mhe::rope_index_host(ids, seq, image_token_id, video_token_id, image_grid_thw, n_images,
                            video_grid_thw, n_videos, spatial_merge, positions, image_mask,
                            video_mask, visual_mask, delta, &err);
  if (rc != MHE_OK) return fail(rc, "%s", err.c_str());
  return MHE_OK;
}

int32_t mhe_embed_tokens(const int32_t* ids, int32_t seq, const void* table, int32_t row_begin,
                         int32_t rows, int32_t hidden_dim, void* out, int32_t* n_outside,
                         void* stream) {
  int32_t rc;
  if ((rc = check_seq(seq))) return rc;
  if (!ids || !table || !out) return fail(MHE_ERR_NULL, "ids, table and out are required");
  if (rows <= 0 || row_begin < 0)
    return fail(MHE_ERR_SHAPE, "table rows [%d, %d + %d) out of range", row_begin, row_begin, rows);
  if (hidden_dim <= 0 || hidden_dim % 8 != 0)
    return fail(MHE_ERR_SHAPE, "hidden_dim %d must be a positive multiple of 8", hidden_dim);
  return hip_check(mhe::launch_embed_gather(ids, seq, static_cast<const bf16_t*>(table), row_begin,
                                            rows, hidden_dim, static_cast<bf16_t*>(out), n_outside,
                                            static_cast<hipStream_t>(stream)),
                   "embedding gather");
}

int32_t mhe_scatter_visual(void* hidden, int32_t seq, int32_t hidden_dim, const uint8_t* mask,
                           int32_t n, const void* feature, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int32_t rc;
  if ((rc = check_seq(seq))) return rc;
  if (hidden_dim <= 0 || hidden_dim % 8 != 0)
    return fail(MHE_ERR_SHAPE, "hidden_dim %d must be a positive multiple of 8", hidden_dim);
  if (n < 0 || n > seq) return fail(MHE_ERR_SHAPE, "n %d out of range [0, %d]", n, seq);
  if (n == 0) return MHE_OK;
  if (!hidden || !mask || !feature) return fail(MHE_ERR_NULL, "hidden, mask and feature are required");
  if ((rc = check_ws(workspace, workspace_bytes, align_up(static_cast<size_t>(seq) * 4) + 256))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* idx = static_cast<int32_t*>(workspace);
  int32_t* cnt = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align_up(static_cast<size_t>(seq) * 4));
  if ((rc = hip_check(mhe::launch_visual_index(mask, seq, n, idx, cnt, st), "visual index"))) return rc;
  return hip_check(mhe::launch_row_scatter(static_cast<bf16_t*>(hidden), hidden_dim, idx, n,
                                           static_cast<const bf16_t*>(feature), st),
                   "placeholder scatter");
}

size_t mhe_join_visual_workspace_bytes(int32_t seq) {
  if (seq <= 0 || seq > kMaxSeq) return 0;
  return 3 * align_up(static_cast<size_t>(seq) * 4) + 256;
}

int32_t mhe_join_visual(const uint8_t* image_mask, const uint8_t* video_mask, int32_t seq,
                        int32_t hidden_dim, const void* image_feature, int32_t n_image,
                        const void* video_feature, int32_t n_video, void* joint, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int32_t rc;
  if ((rc = check_seq(seq))) return rc;
  if (hidden_dim <= 0 || hidden_dim % 8 != 0)
    return fail(MHE_ERR_SHAPE, "hidden_dim %d must be a positive multiple of 8", hidden_dim);
  if (n_image < 0 || n_video < 0 || static_cast<int64_t>(n_image) + n_video > seq)
    return fail(MHE_ERR_SHAPE, "n_image %d + n_video %d out of range [0, %d]", n_image, n_video, seq);
  if (n_image + n_video == 0) return MHE_OK;
  if (!image_mask || !video_mask || !joint)
    return fail(MHE_ERR_NULL, "image_mask, video_mask and joint are required");
  if ((n_image > 0 && !image_feature) || (n_video > 0 && !video_feature))
    return fail(MHE_ERR_NULL, "feature array is NULL");
  if ((rc = check_ws(workspace, workspace_bytes, mhe_join_visual_workspace_bytes(seq)))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_check(mhe::launch_join_visual(image_mask, video_mask, seq, n_image,
                                           static_cast<const bf16_t*>(image_feature), n_video,
                                           static_cast<const bf16_t*>(video_feature), hidden_dim,
                                           static_cast<int32_t*>(workspace), static_cast<bf16_t*>(joint), st),
                   "visual join");
}

}  // extern "C"

// ---- vision tower ----

namespace {

int32_t check_vision_config(const mhe_vision_config* c) {
  if (!c) return fail(MHE_ERR_NULL, "vision config is NULL");
  if (c->hidden <= 0 || c->n_heads <= 0 || c->intermediate <= 0 || c->depth < 0 ||
      c->patch_dim <= 0 || c->merge <= 0 || c->out_hidden <= 0 || c->pos_side <= 0)
    return fail(MHE_ERR_SHAPE, "vision config sizes must be positive");
  if (c->hidden % c->n_heads != 0) return fail(MHE_ERR_SHAPE, "hidden %% n_heads != 0");
  const int dh = c->hidden / c->n_heads;
  if (dh % 4 != 0 || dh > 128)
    return fail(MHE_ERR_UNSUPPORTED, "vision head_dim %d must be a multiple of 4 and <= 128", dh);
  const int mh = c->merge * c->merge * c->hidden;
  if (c->hidden % 64 || c->intermediate % 64 || c->patch_dim % 64 || mh % 64 || c->out_hidden % 32)
    return fail(MHE_ERR_UNSUPPORTED,
                "vision GEMMs need hidden, intermediate, patch_dim, merge^2*hidden multiples of 64 "
                "and out_hidden a multiple of 32");
  if (!mhe::rmsnorm_supported(mh) || !mhe::rmsnorm_supported(c->hidden))
    return fail(MHE_ERR_UNSUPPORTED, "merge^2 * hidden %d must be <= 8192", mh);
  if (c->n_deepstack < 0 || c->n_deepstack > 8)
    return fail(MHE_ERR_SHAPE, "n_deepstack %d out of range [0, 8]", c->n_deepstack);
  for (int i = 0; i < c->n_deepstack; ++i)
    if (c->deepstack_index[i] < 0 || c->deepstack_index[i] >= c->depth)
      return fail(MHE_ERR_SHAPE, "deepstack_index[%d] = %d not a block", i, c->deepstack_index[i]);
  return MHE_OK;
}

// Grid list -> kernel argument; checks the grids and that they hold n patches.
int32_t make_grids(const mhe_vision_config& c, const int32_t* thw, int n_grids, int n,
                   mhe::VisionGrids* g) {
  if (!thw) return fail(MHE_ERR_NULL, "grid_thw is NULL");
  if (n_grids <= 0 || n_grids > mhe::kMaxVisionGrids)
    return fail(MHE_ERR_SHAPE, "n_grids %d out of range [1, %d]", n_grids, mhe::kMaxVisionGrids);
  int64_t total = 0;
  g->count = n_grids;
  g->merge = c.merge;
  for (int i = 0; i < n_grids; ++i) {
    const int t = thw[3 * i], h = thw[3 * i + 1], w = thw[3 * i + 2];
    if (t <= 0 || h <= 0 || w <= 0 || h % c.merge || w % c.merge)
      return fail(MHE_ERR_SHAPE, "grid %d (%d, %d, %d): positive, h and w multiples of %d", i, t,
                  h, w, c.merge);
    g->t[i] = t;
    g->h[i] = h;
    g->w[i] = w;
    total += static_cast<int64_t>(t) * h * w;
  }
  if (total != n)
    return fail(MHE_ERR_MISMATCH, "grids hold %lld patches, %d given", static_cast<long long>(total), n);
  return MHE_OK;
}

struct VisionWs {
  int ld_u, ld_o, ld_i, ld_m;
  mhe::PatchInfo* info;
  float2* rope;  // [n][head_dim/2] rotary cos/sin
  bf16_t* x;    // [n, H] hidden state of mhe_vision_forward
  bf16_t* u;    // [n, ld_u] norm output (dense [n, H] / [n/m^2, M] for the mergers)
  bf16_t* qkv;  // [n, 3H]
  bf16_t* q;    // [n, heads, 128]
  bf16_t* k;    // [heads, n_pad, 128]
  bf16_t* vt;   // [heads, 128, n_pad]
  bf16_t* ao;   // [n, ld_o]
  bf16_t* act;  // [n, ld_i], aliases qkv..ao
  bf16_t* m1;   // [n/m^2, ld_m], aliases qkv..ao
  float* partial;
  size_t partial_bytes;
  size_t total;
};

VisionWs vision_carve(const mhe_vision_config& c, int n, char* base) {
  const size_t N = n, np = mhe::seq_pad(n), H = c.hidden, heads = c.n_heads;
  const size_t mh = static_cast<size_t>(c.merge) * c.merge * H, nm = N / (c.merge * c.merge);
  VisionWs w{};
  w.ld_u = c.hidden + kActPad;
  w.ld_o = c.hidden + kActPad;
  w.ld_i = c.intermediate + kActPad;
  w.ld_m = static_cast<int>(mh) + kActPad;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  w.info = reinterpret_cast<mhe::PatchInfo*>(take(N * sizeof(mhe::PatchInfo)));
  w.rope = reinterpret_cast<float2*>(take(N * (H / heads / 2) * sizeof(float2)));
  w.x = reinterpret_cast<bf16_t*>(take(N * H * 2));
  w.u = reinterpret_cast<bf16_t*>(take(N * w.ld_u * 2));
  const size_t region = off;
  w.qkv = reinterpret_cast<bf16_t*>(take(N * 3 * H * 2));
  w.q = reinterpret_cast<bf16_t*>(take(N * heads * 128 * 2));
  w.k = reinterpret_cast<bf16_t*>(take(heads * np * 128 * 2));
  w.vt = reinterpret_cast<bf16_t*>(take(heads * 128 * np * 2));
  w.ao = reinterpret_cast<bf16_t*>(take(N * w.ld_o * 2));
  const size_t attn_end = off;
  const size_t need_act = align_up(N * w.ld_i * 2), need_m1 = align_up(nm * w.ld_m * 2);
  w.act = reinterpret_cast<bf16_t*>(base ? base + region : nullptr);
  w.m1 = reinterpret_cast<bf16_t*>(base ? base + region : nullptr);
  off = std::max(attn_end, region + std::max(need_act, need_m1));
  w.partial_bytes = mhe::gemm_partial_bytes();
  w.partial = reinterpret_cast<float*>(take(w.partial_bytes));
  w.total = off;
  (void)mh;
  return w;
}

int32_t vision_gemm(mhe::Epilogue epi, const bf16_t* a, int lda, const void* wt, const void* bias,
                    bf16_t* c, int ldc, const bf16_t* r, int m, int n, int k, const VisionWs& ws,
                    hipStream_t st, const char* what) {
  if (!wt || !bias) return fail(MHE_ERR_NULL, "%s: weight or bias is NULL", what);
  mhe::BSegments b{{static_cast<const bf16_t*>(wt), nullptr, nullptr}, {n, 0, 0}, 1};
  return hip_check(mhe::launch_gemm(epi, a, lda, b, k, c, ldc, r, m, n, k, ws.partial,
                                    ws.partial_bytes, st, static_cast<const bf16_t*>(bias)),
                   what);
}

int32_t run_vision_block(const mhe_vision_config& c, const mhe_vision_block_weights& p, bf16_t* h,
                         int n, const VisionWs& ws, hipStream_t st) {
  const int H = c.hidden, dh = H / c.n_heads;
  int32_t rc;
  if (!p.norm1_w || !p.norm1_b || !p.norm2_w || !p.norm2_b)
    return fail(MHE_ERR_NULL, "vision block norm weights are NULL");
  if ((rc = hip_check(mhe::launch_layernorm(h, H, static_cast<const bf16_t*>(p.norm1_w),
                                            static_cast<const bf16_t*>(p.norm1_b), ws.u, ws.ld_u, n,
                                            H, 1e-6f, st), "layer norm 1")))
    return rc;
  if ((rc = vision_gemm(mhe::Epilogue::kBias, ws.u, ws.ld_u, p.qkv_w, p.qkv_b, ws.qkv, 3 * H,
                        nullptr, n, 3 * H, H, ws, st, "qkv")))
    return rc;
  if ((rc = hip_check(mhe::launch_vision_rope(ws.qkv, 3 * H, n, c.n_heads, dh, ws.rope, ws.q, ws.k,
                                              ws.vt, st), "vision rotary")))
    return rc;
  if ((rc = hip_check(mhe::launch_segment_attention(ws.q, ws.k, ws.vt, ws.ao, ws.ld_o, n, c.n_heads,
                                                    dh, ws.info, st), "vision attention")))
    return rc;
  if ((rc = vision_gemm(mhe::Epilogue::kBiasResidual, ws.ao, ws.ld_o, p.proj_w, p.proj_b, h, H, h,
                        n, H, H, ws, st, "proj")))
    return rc;
  if ((rc = hip_check(mhe::launch_layernorm(h, H, static_cast<const bf16_t*>(p.norm2_w),
                                            static_cast<const bf16_t*>(p.norm2_b), ws.u, ws.ld_u, n,
                                            H, 1e-6f, st), "layer norm 2")))
    return rc;
  if ((rc = vision_gemm(mhe::Epilogue::kBiasGeluTanh, ws.u, ws.ld_u, p.fc1_w, p.fc1_b, ws.act,
                        ws.ld_i, nullptr, n, c.intermediate, H, ws, st, "fc1")))
    return rc;
  return vision_gemm(mhe::Epilogue::kBiasResidual, ws.act, ws.ld_i, p.fc2_w, p.fc2_b, h, H, h, n, H,
                     c.intermediate, ws, st, "fc2");
}

int32_t run_vision_merge(const mhe_vision_config& c, const mhe_vision_merger_weights& p, bool post,
                         const bf16_t* h, int n, bf16_t* out, const VisionWs& ws, hipStream_t st) {
  const int H = c.hidden, mh = c.merge * c.merge * H, nm = n / (c.merge * c.merge);
  int32_t rc;
  if (!p.norm_w || !p.norm_b) return fail(MHE_ERR_NULL, "merger norm weights are NULL");
  // main merger: normalise tokens, then view merge^2 consecutive rows as one;
  // DeepStack merger: view first, normalise the merged rows
  hipError_t e = post ? mhe::launch_layernorm(h, mh, static_cast<const bf16_t*>(p.norm_w),
                                              static_cast<const bf16_t*>(p.norm_b), ws.u, mh, nm,
                                              mh, 1e-6f, st)
                      : mhe::launch_layernorm(h, H, static_cast<const bf16_t*>(p.norm_w),
                                              static_cast<const bf16_t*>(p.norm_b), ws.u, H, n, H,
                                              1e-6f, st);
  if ((rc = hip_check(e, "merger norm"))) return rc;
  if ((rc = vision_gemm(mhe::Epilogue::kBiasGeluErf, ws.u, mh, p.fc1_w, p.fc1_b, ws.m1, ws.ld_m,
                        nullptr, nm, mh, mh, ws, st, "merger fc1")))
    return rc;
  return vision_gemm(mhe::Epilogue::kBias, ws.m1, ws.ld_m, p.fc2_w, p.fc2_b, out, c.out_hidden,
                     nullptr, nm, c.out_hidden, mh, ws, st, "merger fc2");
}

int32_t vision_prelude(const mhe_vision_config* cfg, int n, const int32_t* thw, int n_grids,
                       void* workspace, size_t workspace_bytes, mhe::VisionGrids* g, VisionWs* ws,
                       hipStream_t st) {
  int32_t rc;
  if ((rc = check_vision_config(cfg))) return rc;
  if ((rc = make_grids(*cfg, thw, n_grids, n, g))) return rc;
  if ((rc = check_seq(n))) return rc;
  const VisionWs need = vision_carve(*cfg, n, nullptr);
  if ((rc = check_ws(workspace, workspace_bytes, need.total))) return rc;
  *ws = vision_carve(*cfg, n, static_cast<char*>(workspace));
  if ((rc = hip_check(mhe::launch_patch_info(*g, n, ws->info, st), "patch info"))) return rc;
  return hip_check(mhe::launch_vision_rope_table(ws->info, n, cfg->hidden / cfg->n_heads, ws->rope, st),
                   "vision rotary table");
}

// Patches the grids hold (0 when the list is unusable; make_grids reports why).
int grid_patches(const int32_t* thw, int n_grids) {
  if (!thw || n_grids <= 0 || n_grids > mhe::kMaxVisionGrids) return 0;
  int64_t n = 0;
  for (int i = 0; i < n_grids; ++i) {
    const int64_t p = static_cast<int64_t>(thw[3 * i]) * thw[3 * i + 1] * thw[3 * i + 2];
    if (thw[3 * i] <= 0 || thw[3 * i + 1] <= 0 || thw[3 * i + 2] <= 0) return 0;
    n += p;
    if (n > kMaxSeq) return 0;
  }
  return static_cast<int>(n);
}

int32_t check_blocks(const mhe_vision_weights* w, int first, int count, int depth) {
  if (!w) return fail(MHE_ERR_NULL, "vision weights are NULL");
  if (count > 0 && !w->blocks) return fail(MHE_ERR_NULL, "vision blocks table is NULL");
  if (first < 0 || count < 0 || first + count > depth)
    return fail(MHE_ERR_SHAPE, "blocks [%d, %d) outside [0, %d)", first, first + count, depth);
  return MHE_OK;
}

}  // namespace

extern "C" {

size_t mhe_vision_workspace_bytes(const mhe_vision_config* cfg, int32_t n_patches) {
  if (check_vision_config(cfg) || check_seq(n_patches)) return 0;
  return vision_carve(*cfg, n_patches, nullptr).total;
}

int32_t mhe_vision_embed(const mhe_vision_config* cfg, const mhe_vision_weights* w,
                         const void* pixels, const int32_t* grid_thw, int32_t n_grids,
                         void* hidden, void* workspace, size_t workspace_bytes, void* stream) {
  int32_t rc;
  if (!w || !pixels || !hidden) return fail(MHE_ERR_NULL, "weights, pixels and hidden are required");
  if (!w->patch_w || !w->patch_b || !w->pos_table) return fail(MHE_ERR_NULL, "patch / position weights are NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int n = grid_patches(grid_thw, n_grids);
  mhe::VisionGrids g;
  VisionWs ws;
  if ((rc = vision_prelude(cfg, n, grid_thw, n_grids, workspace, workspace_bytes, &g, &ws, st))) return rc;
  bf16_t* h = static_cast<bf16_t*>(hidden);
  if ((rc = vision_gemm(mhe::Epilogue::kBias, static_cast<const bf16_t*>(pixels), cfg->patch_dim,
                        w->patch_w, w->patch_b, h, cfg->hidden, nullptr, n, cfg->hidden,
                        cfg->patch_dim, ws, st, "patch embed")))
    return rc;
  return hip_check(mhe::launch_pos_embed(h, cfg->hidden, n, cfg->hidden,
                                         static_cast<const bf16_t*>(w->pos_table), cfg->pos_side,
                                         ws.info, st), "position embedding");
}

int32_t mhe_vision_blocks(const mhe_vision_config* cfg, const mhe_vision_weights* w,
                          int32_t first, int32_t count, void* hidden, const int32_t* grid_thw,
                          int32_t n_grids, void* workspace, size_t workspace_bytes, void* stream) {
  int32_t rc;
  if (!hidden) return fail(MHE_ERR_NULL, "hidden is NULL");
  if (cfg && (rc = check_blocks(w, first, count, cfg->depth))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int n = grid_patches(grid_thw, n_grids);
  mhe::VisionGrids g;
  VisionWs ws;
  if ((rc = vision_prelude(cfg, n, grid_thw, n_grids, workspace, workspace_bytes, &g, &ws, st))) return rc;
  for (int b = first; b < first + count; ++b)
    if ((rc = run_vision_block(*cfg, w->blocks[b], static_cast<bf16_t*>(hidden), n, ws, st))) return rc;
  return MHE_OK;
}

int32_t mhe_vision_merge(const mhe_vision_config* cfg, const mhe_vision_merger_weights* m,
                         int32_t postshuffle, const void* hidden, int32_t n_patches, void* out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  int32_t rc;
  if ((rc = check_vision_config(cfg))) return rc;
  if ((rc = check_seq(n_patches))) return rc;
  if (!m || !hidden || !out) return fail(MHE_ERR_NULL, "merger weights, hidden and out are required");
  if (n_patches % (cfg->merge * cfg->merge))
    return fail(MHE_ERR_SHAPE, "n_patches %d is not a multiple of merge^2", n_patches);
  const VisionWs need = vision_carve(*cfg, n_patches, nullptr);
  if ((rc = check_ws(workspace, workspace_bytes, need.total))) return rc;
  const VisionWs ws = vision_carve(*cfg, n_patches, static_cast<char*>(workspace));
  return run_vision_merge(*cfg, *m, postshuffle != 0, static_cast<const bf16_t*>(hidden), n_patches,
                          static_cast<bf16_t*>(out), ws, static_cast<hipStream_t>(stream));
}

int32_t mhe_vision_forward(const mhe_vision_config* cfg, const mhe_vision_weights* w,
                           const void* pixels, const int32_t* grid_thw, int32_t n_grids,
                           void* merged, void* const* deepstack, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int32_t rc;
  if (!w || !pixels || !merged) return fail(MHE_ERR_NULL, "weights, pixels and merged are required");
  if (!w->patch_w || !w->patch_b || !w->pos_table) return fail(MHE_ERR_NULL, "patch / position weights are NULL");
  if (cfg && (rc = check_blocks(w, 0, cfg->depth, cfg->depth))) return rc;
  if (cfg && cfg->n_deepstack > 0) {
    if (!deepstack || !w->deepstack) return fail(MHE_ERR_NULL, "DeepStack outputs or mergers are NULL");
    for (int l = 0; l < cfg->n_deepstack; ++l)
      if (!deepstack[l]) return fail(MHE_ERR_NULL, "deepstack[%d] is NULL", l);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int n = grid_patches(grid_thw, n_grids);
  mhe::VisionGrids g;
  VisionWs ws;
  if ((rc = vision_prelude(cfg, n, grid_thw, n_grids, workspace, workspace_bytes, &g, &ws, st))) return rc;
  const mhe_vision_config& c = *cfg;
  if ((rc = vision_gemm(mhe::Epilogue::kBias, static_cast<const bf16_t*>(pixels), c.patch_dim,
                        w->patch_w, w->patch_b, ws.x, c.hidden, nullptr, n, c.hidden, c.patch_dim,
                        ws, st, "patch embed")))
    return rc;
  if ((rc = hip_check(mhe::launch_pos_embed(ws.x, c.hidden, n, c.hidden,
                                            static_cast<const bf16_t*>(w->pos_table), c.pos_side,
                                            ws.info, st), "position embedding")))
    return rc;
  for (int b = 0; b < c.depth; ++b) {
    if ((rc = run_vision_block(c, w->blocks[b], ws.x, n, ws, st))) return rc;
    for (int l = 0; l < c.n_deepstack; ++l)
      if (c.deepstack_index[l] == b &&
          (rc = run_vision_merge(c, w->deepstack[l], true, ws.x, n, static_cast<bf16_t*>(deepstack[l]),
                                 ws, st)))
        return rc;
  }
  return run_vision_merge(c, w->merger, false, ws.x, n, static_cast<bf16_t*>(merged), ws, st);
}

size_t mhe_vision_attention_workspace_bytes(int32_t n_patches) {
  if (check_seq(n_patches)) return 0;
  return align_up(static_cast<size_t>(n_patches) * sizeof(mhe::PatchInfo));
}

int32_t mhe_vision_attention(const void* q, const void* k, const void* vt, void* o,
                             int32_t n_patches, int32_t n_heads, int32_t head_dim,
                             const int32_t* grid_thw, int32_t n_grids, int32_t merge,
                             void* workspace, size_t workspace_bytes, void* stream) {
  int32_t rc;
  if ((rc = check_seq(n_patches))) return rc;
  if (!q || !k || !vt || !o) return fail(MHE_ERR_NULL, "q, k, vt and o are required");
  if (n_heads <= 0 || head_dim <= 0) return fail(MHE_ERR_SHAPE, "n_heads and head_dim must be > 0");
  if (head_dim > 128 || head_dim % 4 != 0)
    return fail(MHE_ERR_UNSUPPORTED, "vision head_dim %d must be a multiple of 4 and <= 128", head_dim);
  if (merge <= 0) return fail(MHE_ERR_SHAPE, "merge %d must be > 0", merge);
  mhe_vision_config c{};
  c.merge = merge;
  mhe::VisionGrids g;
  if ((rc = make_grids(c, grid_thw, n_grids, n_patches, &g))) return rc;
  if ((rc = check_ws(workspace, workspace_bytes, mhe_vision_attention_workspace_bytes(n_patches)))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  mhe::PatchInfo* info = static_cast<mhe::PatchInfo*>(workspace);
  if ((rc = hip_check(mhe::launch_patch_info(g, n_patches, info, st), "patch info"))) return rc;
  return hip_check(mhe::launch_segment_attention(static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                                                 static_cast<const bf16_t*>(vt), static_cast<bf16_t*>(o),
                                                 n_heads * head_dim, n_patches, n_heads, head_dim, info, st),
                   "vision attention");
}

int32_t mhe_layer_norm(const void* x, const void* w, const void* b, void* y, int32_t rows,
                       int32_t dim, float eps, void* stream) {
  if (!x || !w || !b || !y) return fail(MHE_ERR_NULL, "x, w, b and y are required");
  if (rows <= 0) return fail(MHE_ERR_SHAPE, "rows must be > 0");
  if (!mhe::rmsnorm_supported(dim)) return fail(MHE_ERR_UNSUPPORTED, "dim %d: multiple of 8, <= 8192", dim);
  if (!(eps >= 0.f)) return fail(MHE_ERR_SHAPE, "eps must be >= 0");
  return hip_check(mhe::launch_layernorm(static_cast<const bf16_t*>(x), dim, static_cast<const bf16_t*>(w),
                                         static_cast<const bf16_t*>(b), static_cast<bf16_t*>(y), dim,
                                         rows, dim, eps, static_cast<hipStream_t>(stream)),
                   "layer norm");
}

int32_t mhe_linear_bias(const void* a, const void* w, const void* bias, void* c,
                        const void* residual, int32_t m, int32_t n, int32_t k, int32_t act,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!a || !w || !bias || !c) return fail(MHE_ERR_NULL, "a, w, bias and c are required");
  if (m <= 0 || n <= 0 || k <= 0) return fail(MHE_ERR_SHAPE, "m, n, k must be > 0");
  if (act < 0 || act > 2) return fail(MHE_ERR_SHAPE, "act %d not in {0, 1, 2}", act);
  if (act != 0 && residual) return fail(MHE_ERR_SHAPE, "a residual goes with act 0 only");
  if (!mhe::gemm_supported(n, k)) return fail(MHE_ERR_UNSUPPORTED, "needs n %% 32 == 0 and k %% 64 == 0 (n=%d, k=%d)", n, k);
  const size_t cb = static_cast<size_t>(m) * n * 2;
  if (overlaps(c, cb, a, static_cast<size_t>(m) * k * 2) || overlaps(c, cb, w, static_cast<size_t>(n) * k * 2))
    return fail(MHE_ERR_SHAPE, "c overlaps an operand");
  if (residual && residual != c && overlaps(c, cb, residual, cb))
    return fail(MHE_ERR_SHAPE, "residual partially overlaps c");
  int32_t rc;
  if ((rc = check_gemm_ws(workspace, workspace_bytes))) return rc;
  const mhe::Epilogue epi = act == 1 ? mhe::Epilogue::kBiasGeluTanh
                          : act == 2 ? mhe::Epilogue::kBiasGeluErf
                          : residual ? mhe::Epilogue::kBiasResidual : mhe::Epilogue::kBias;
  mhe::BSegments b{{static_cast<const bf16_t*>(w), nullptr, nullptr}, {n, 0, 0}, 1};
  return hip_check(mhe::launch_gemm(epi, static_cast<const bf16_t*>(a), k, b, k, static_cast<bf16_t*>(c), n,
                                    static_cast<const bf16_t*>(residual), m, n, k,
                                    static_cast<float*>(workspace), workspace ? workspace_bytes : 0,
                                    static_cast<hipStream_t>(stream), static_cast<const bf16_t*>(bias)),
                   "linear bias");
}

}  // extern "C"
