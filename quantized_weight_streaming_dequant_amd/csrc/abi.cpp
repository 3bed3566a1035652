// C ABI of libnt.so: argument checks, workspace layout, launch sequencing and the
// double-buffered layer streamer.  Declarations and contracts: include/nt.h.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <errno.h>
#include <sys/stat.h>
#include <unistd.h>

#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/nt.h"
#include "attn.h"
#include "common.h"
#include "gemv.h"
#include "layer_k.h"
#include "small.h"

using namespace nt;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(NT_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool fmt_ok(int f) { return f >= NT_Q8_0 && f <= NT_Q5_KT; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ------------------------------------------------------------ timing hook
struct Timing {
  std::mutex mu;
  int kclass = -1;
  int max_launches = 0;
  std::vector<hipEvent_t> ev;  // begin/end pairs
} g_timing;

struct TimedLaunch {
  hipStream_t s;
  bool on = false;
  TimedLaunch(int kclass, hipStream_t st) : s(st) {
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.kclass == kclass && (int)g_timing.ev.size() < 2 * g_timing.max_launches) {
      hipEvent_t b, e;
      if (hipEventCreate(&b) == hipSuccess && hipEventCreate(&e) == hipSuccess) {
        (void)hipEventRecord(b, s);
        g_timing.ev.push_back(b);
        g_timing.ev.push_back(e);
        on = true;
      }
    }
  }
  ~TimedLaunch() {
    if (on) {
      std::lock_guard<std::mutex> lk(g_timing.mu);
      (void)hipEventRecord(g_timing.ev.back(), s);
    }
  }
};

// ------------------------------------------------------------ workspace layout
struct LayerWs {
  size_t q, o, h1, a, part, key, total;
};

LayerWs layer_ws(const nt_layer_shape& s) {
  LayerWs w;
  size_t off = 0;
  const size_t nq = (size_t)s.n_q_heads * s.head_dim;
  w.q = off; off = align256(off + 4 * nq);
  w.o = off; off = align256(off + 4 * nq);
  w.h1 = off; off = align256(off + 4 * (size_t)s.dim);
  w.a = off; off = align256(off + 4 * (size_t)s.ffn_dim);
  w.part = off; off = align256(off + 4 * attn_part_floats(s.n_q_heads, s.max_ctx));
  w.key = off; off = align256(off + 8);
  w.total = off;
  return w;
}

// Workspace of the k-token layer: normalised rows, q, k, v, attention output, h1, gate, up,
// SwiGLU output (each [k][...] fp32) and the attention partials of every token.
struct LayerKWs {
  size_t xn, q, kk, vv, o, h1, g, u, a, part, total;
  size_t part_stride;  // floats of partials per token
};

LayerKWs layer_k_ws(const nt_layer_shape& s, int k) {
  LayerKWs w;
  size_t off = 0;
  const size_t nq = (size_t)s.n_q_heads * s.head_dim, nkv = (size_t)s.n_kv_heads * s.head_dim;
  const size_t kk = (size_t)k;
  w.xn = off; off = align256(off + 4 * kk * (size_t)s.dim);
  w.q = off; off = align256(off + 4 * kk * nq);
  w.kk = off; off = align256(off + 4 * kk * nkv);
  w.vv = off; off = align256(off + 4 * kk * nkv);
  w.o = off; off = align256(off + 4 * kk * nq);
  w.h1 = off; off = align256(off + 4 * kk * (size_t)s.dim);
  w.g = off; off = align256(off + 4 * kk * (size_t)s.ffn_dim);
  w.u = off; off = align256(off + 4 * kk * (size_t)s.ffn_dim);
  w.a = off; off = align256(off + 4 * kk * (size_t)s.ffn_dim);
  w.part_stride = (attn_part_floats(s.n_q_heads, s.max_ctx) + 63) & ~(size_t)63;
  w.part = off; off = align256(off + 4 * kk * w.part_stride);
  w.total = off;
  return w;
}

int check_shape(const nt_layer_shape* s) {
  if (!s) return fail(NT_EINVAL, "shape is null");
  if (s->head_dim != 128) return fail(NT_ESHAPE, "head_dim must be 128 (got %d)", s->head_dim);
  if (s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->n_q_heads % s->n_kv_heads)
    return fail(NT_ESHAPE, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", s->n_q_heads, s->n_kv_heads);
  const int grp = s->n_q_heads / s->n_kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8 && grp != 16)
    return fail(NT_ESHAPE, "query heads per KV head must be 1, 2, 4, 8 or 16 (got %d)", grp);
  const int nq = s->n_q_heads * s->head_dim;
  if (s->dim <= 0 || s->dim % 256 || s->dim > NT_GEMV_MAX_COLS)
    return fail(NT_ESHAPE, "dim must be a positive multiple of 256 up to %d (got %d)", NT_GEMV_MAX_COLS, s->dim);
  if (nq % 256 || nq > NT_GEMV_MAX_COLS) return fail(NT_ESHAPE, "n_q_heads*head_dim must be a multiple of 256 up to %d", NT_GEMV_MAX_COLS);
  if (s->ffn_dim <= 0 || s->ffn_dim % 256 || s->ffn_dim > NT_GEMV_MAX_COLS)
    return fail(NT_ESHAPE, "ffn_dim must be a positive multiple of 256 up to %d (got %d)", NT_GEMV_MAX_COLS, s->ffn_dim);
  if (s->max_ctx <= 0 || s->max_ctx % 8 || s->max_ctx > ATTN_MAX_CTX)
    return fail(NT_ESHAPE, "max_ctx must be a positive multiple of 8 up to %d (got %d)", ATTN_MAX_CTX, s->max_ctx);
  if (!(s->eps >= 0.f)) return fail(NT_EINVAL, "eps must be >= 0");
  if (!(s->rope_theta > 0.f)) return fail(NT_EINVAL, "rope_theta must be > 0");
  return NT_OK;
}

int check_weights(const nt_layer_weights* w) {
  if (!w) return fail(NT_EINVAL, "weights are null");
  for (int i = 0; i < NT_W_COUNT; ++i) {
    if (!fmt_ok(w->fmt[i])) return fail(NT_EFORMAT, "unknown format %d for matrix %d", w->fmt[i], i);
    if (!w->w[i]) return fail(NT_EINVAL, "matrix %d pointer is null", i);
    if (!aligned(w->w[i], 16)) return fail(NT_EALIGN, "matrix %d must be 16-byte aligned", i);
  }
  if (w->fmt[NT_W_GATE] != w->fmt[NT_W_UP]) return fail(NT_EFORMAT, "gate and up must share a format");
  if (!w->attn_norm || !w->ffn_norm) return fail(NT_EINVAL, "norm gains are null");
  if (!aligned(w->attn_norm, 16) || !aligned(w->ffn_norm, 16)) return fail(NT_EALIGN, "norm gains must be 16-byte aligned");
  return NT_OK;
}

GemvSeg make_seg(const void* w, int fmt, int rows, int cols, int grp0) {
  GemvSeg g;
  g.w = reinterpret_cast<const uint8_t*>(w);
  g.fmt = fmt;
  g.rows = rows;
  g.row_bytes = (int64_t)(cols / block_elems(fmt)) * block_bytes(fmt);
  g.grp0 = grp0;
  return g;
}

GemvArgs blank_args() {
  GemvArgs a;
  memset(&a, 0, sizeof(a));
  return a;
}

// Enqueue the FFN input half of a layer: a = SwiGLU(Wg n, Wu n), n = RMSNorm(h, ffn_norm).
static hipError_t ffn_up_launch(const nt_layer_weights& w, const nt_layer_shape& s, const float* h, float* out,
                                hipStream_t st) {
  const GemvPlan p = gemv_plan(EPI_SWIGLU, s.dim, 1 << w.fmt[NT_W_GATE]);
  GemvArgs a = blank_args();
  a.x = h; a.gain = w.ffn_norm; a.eps = s.eps; a.cols = s.dim; a.nseg = 2;
  a.seg[0] = make_seg(w.w[NT_W_GATE], w.fmt[NT_W_GATE], s.ffn_dim, s.dim, 0);
  a.seg[1] = make_seg(w.w[NT_W_UP], w.fmt[NT_W_UP], s.ffn_dim, s.dim, 1 << 30);
  a.y = out;
  TimedLaunch tl(NT_K_FFN_UP, st);
  return gemv_launch(1 << w.fmt[NT_W_GATE], EPI_SWIGLU, p, gemv_groups(p, s.ffn_dim), a, st);
}

// Enqueue the greedy head: logits = W_out RMSNorm(h, gain); the fused argmax folds into *key
// (reset first), and *token takes the index it holds.
static int lm_head_enqueue(int fmt, int64_t n_vocab, int dim, const void* output, const float* gain, float eps,
                           const float* h, float* logits, unsigned long long* key, int32_t* token, bool reset,
                           hipStream_t st) {
  hipError_t e;
  if (reset && (e = key_reset_launch(key, 1, st)) != hipSuccess) return hip_fail(e, "key reset launch");
  {
    const GemvPlan p = gemv_plan(EPI_LOGITS, dim, 1 << fmt, (int)n_vocab);
    GemvArgs a = blank_args();
    a.x = h; a.gain = gain; a.eps = eps; a.cols = dim; a.nseg = 1;
    a.seg[0] = make_seg(output, fmt, (int)n_vocab, dim, 0);
    a.y = logits; a.amax = key;
    TimedLaunch tl(NT_K_LM_HEAD, st);
    if ((e = gemv_launch(1 << fmt, EPI_LOGITS, p, gemv_groups(p, (int)n_vocab), a, st)) != hipSuccess)
      return hip_fail(e, "lm head launch");
  }
  if ((e = token_from_key_launch(key, token, st)) != hipSuccess) return hip_fail(e, "token launch");
  return NT_OK;
}

// Enqueue one decode layer (arguments already checked).
int run_layer(const nt_layer_weights& w, const nt_layer_shape& s, int pos, float* h, uint16_t* kc, uint16_t* vc,
              uint8_t* ws, hipStream_t st) {
  const LayerWs L = layer_ws(s);
  float* wq = reinterpret_cast<float*>(ws + L.q);
  float* wo = reinterpret_cast<float*>(ws + L.o);
  float* wh1 = reinterpret_cast<float*>(ws + L.h1);
  float* wa = reinterpret_cast<float*>(ws + L.a);
  const int nq = s.n_q_heads * s.head_dim, nkv = s.n_kv_heads * s.head_dim;
  hipError_t e;

  {  // a1-a3: RMSNorm prologue, q/k/v GEMV, RoPE + fp16 cache append epilogue
    const int mask = (1 << w.fmt[NT_W_Q]) | (1 << w.fmt[NT_W_K]) | (1 << w.fmt[NT_W_V]);
    const GemvPlan p = gemv_plan(EPI_QKV, s.dim, mask);
    GemvArgs a = blank_args();
    a.x = h; a.gain = w.attn_norm; a.eps = s.eps; a.cols = s.dim;
    a.nseg = 3;
    int t = 0;
    a.seg[0] = make_seg(w.w[NT_W_Q], w.fmt[NT_W_Q], nq, s.dim, t); t += gemv_groups(p, nq);
    a.seg[1] = make_seg(w.w[NT_W_K], w.fmt[NT_W_K], nkv, s.dim, t); t += gemv_groups(p, nkv);
    a.seg[2] = make_seg(w.w[NT_W_V], w.fmt[NT_W_V], nkv, s.dim, t); t += gemv_groups(p, nkv);
    a.q_out = wq; a.k_cache = kc; a.v_cache = vc; a.pos = pos; a.max_ctx = s.max_ctx; a.rope_theta = s.rope_theta;
    TimedLaunch tl(NT_K_ATTN_IN, st);
    if ((e = gemv_launch(mask, EPI_QKV, p, t, a, st)) != hipSuccess) return hip_fail(e, "attn_in launch");
  }
  {  // a4: GQA attention over slots [0, pos]
    AttnArgs a;
    a.q = wq; a.k_cache = kc; a.v_cache = vc; a.out = wo;
    a.part = reinterpret_cast<float*>(ws + L.part);
    a.n_kv = s.n_kv_heads; a.n_ctx = pos + 1; a.max_ctx = s.max_ctx;
    a.n_split = attn_n_split(a.n_ctx);
    TimedLaunch tl(NT_K_ATTN, st);
    if ((e = attn_launch(a, s.n_q_heads / s.n_kv_heads, st)) != hipSuccess) return hip_fail(e, "attention launch");
  }
  {  // a5: O GEMV + residual (h1 also kept in the workspace)
    const GemvPlan p = gemv_plan(EPI_RESID, nq, 1 << w.fmt[NT_W_O], s.dim);
    GemvArgs a = blank_args();
    a.x = wo; a.cols = nq; a.nseg = 1;
    a.seg[0] = make_seg(w.w[NT_W_O], w.fmt[NT_W_O], s.dim, nq, 0);
    a.y = h; a.resid = h; a.y2 = wh1;
    TimedLaunch tl(NT_K_O, st);
    if ((e = gemv_launch(1 << w.fmt[NT_W_O], EPI_RESID, p, gemv_groups(p, s.dim), a, st)) != hipSuccess)
      return hip_fail(e, "o launch");
  }
  // a6-a8: RMSNorm prologue, paired gate/up GEMV, SwiGLU epilogue
  if ((e = ffn_up_launch(w, s, h, wa, st)) != hipSuccess) return hip_fail(e, "gate/up launch");
  {  // a9: down GEMV + residual
    const GemvPlan p = gemv_plan(EPI_RESID, s.ffn_dim, 1 << w.fmt[NT_W_DOWN], s.dim);
    GemvArgs a = blank_args();
    a.x = wa; a.cols = s.ffn_dim; a.nseg = 1;
    a.seg[0] = make_seg(w.w[NT_W_DOWN], w.fmt[NT_W_DOWN], s.dim, s.ffn_dim, 0);
    a.y = h; a.resid = h;
    TimedLaunch tl(NT_K_FFN_DOWN, st);
    if ((e = gemv_launch(1 << w.fmt[NT_W_DOWN], EPI_RESID, p, gemv_groups(p, s.dim), a, st)) != hipSuccess)
      return hip_fail(e, "down launch");
  }
  return NT_OK;
}

// Enqueue one decode layer for k tokens at positions pos .. pos + k - 1 (arguments already
// checked): h [k][dim] in/out.  The GEMMs read each weight once for all k tokens; the residual
// adds are the GEMMs accumulating into h; token t attends over slots [0, pos + t].
int run_layer(const nt_layer_weights& w, const nt_layer_shape& s, int pos, float* h, uint16_t* kc, uint16_t* vc,
              uint8_t* ws, hipStream_t st);

int run_layer_k(const nt_layer_weights& w, const nt_layer_shape& s, int pos, int k, float* h, uint16_t* kc,
                uint16_t* vc, uint8_t* ws, hipStream_t st) {
  // one token: the single-token layer's fused launches (its workspace layout fits in this one)
  if (k == 1) return run_layer(w, s, pos, h, kc, vc, ws, st);
  const LayerKWs L = layer_k_ws(s, k);
  float* xn = reinterpret_cast<float*>(ws + L.xn);
  float* q = reinterpret_cast<float*>(ws + L.q);
  float* kk = reinterpret_cast<float*>(ws + L.kk);
  float* vv = reinterpret_cast<float*>(ws + L.vv);
  float* o = reinterpret_cast<float*>(ws + L.o);
  float* h1 = reinterpret_cast<float*>(ws + L.h1);
  float* g = reinterpret_cast<float*>(ws + L.g);
  float* u = reinterpret_cast<float*>(ws + L.u);
  float* a = reinterpret_cast<float*>(ws + L.a);
  const int nq = s.n_q_heads * s.head_dim, nkv = s.n_kv_heads * s.head_dim;
  auto W = [&](int i) { return reinterpret_cast<const uint8_t*>(w.w[i]); };
  hipError_t e;
  // a1: n1 = RMSNorm(h)
  if ((e = rmsnorm_rows_launch(k, s.dim, h, w.attn_norm, s.eps, xn, nullptr, st)) != hipSuccess)
    return hip_fail(e, "rmsnorm launch");
  {  // a2: q, k, v for every token
    TimedLaunch tl(NT_K_ATTN_IN, st);
    if ((e = gemm_launch(w.fmt[NT_W_Q], W(NT_W_Q), nq, s.dim, k, xn, q, st)) != hipSuccess ||
        (e = gemm_launch(w.fmt[NT_W_K], W(NT_W_K), nkv, s.dim, k, xn, kk, st)) != hipSuccess ||
        (e = gemm_launch(w.fmt[NT_W_V], W(NT_W_V), nkv, s.dim, k, xn, vv, st)) != hipSuccess)
      return hip_fail(e, "q/k/v gemm launch");
  }
  // a3: RoPE at pos + t, fp16 k and v into slot pos + t
  if ((e = rope_append_launch(k, s.n_q_heads, s.n_kv_heads, pos, s.rope_theta, q, kk, vv, kc, vc, s.max_ctx, st)) !=
      hipSuccess)
    return hip_fail(e, "rope/append launch");
  {  // a4: token t attends over slots [0, pos + t]
    AttnArgs at;
    at.q = q; at.k_cache = kc; at.v_cache = vc; at.out = o;
    at.part = reinterpret_cast<float*>(ws + L.part);
    at.n_kv = s.n_kv_heads; at.n_ctx = pos + 1; at.max_ctx = s.max_ctx;
    at.n_tok = k; at.q_stride = nq; at.out_stride = nq; at.part_stride = (int64_t)L.part_stride;
    at.n_split = attn_n_split(pos + k);
    TimedLaunch tl(NT_K_ATTN, st);
    if ((e = attn_launch(at, s.n_q_heads / s.n_kv_heads, st)) != hipSuccess) return hip_fail(e, "attention launch");
  }
  {  // a5: h1 = h + Wo o
    TimedLaunch tl(NT_K_O, st);
    if ((e = gemm_launch(w.fmt[NT_W_O], W(NT_W_O), s.dim, nq, k, o, h, st, true)) != hipSuccess)
      return hip_fail(e, "o gemm launch");
  }
  // a6: n2 = RMSNorm(h1), h1 kept in the workspace
  if ((e = rmsnorm_rows_launch(k, s.dim, h, w.ffn_norm, s.eps, xn, h1, st)) != hipSuccess)
    return hip_fail(e, "rmsnorm launch");
  {  // a7, a8: a = SwiGLU(Wg n2, Wu n2)
    TimedLaunch tl(NT_K_FFN_UP, st);
    if ((e = gemm_launch(w.fmt[NT_W_GATE], W(NT_W_GATE), s.ffn_dim, s.dim, k, xn, g, st)) != hipSuccess ||
        (e = gemm_launch(w.fmt[NT_W_UP], W(NT_W_UP), s.ffn_dim, s.dim, k, xn, u, st)) != hipSuccess ||
        (e = swiglu_launch((int64_t)k * s.ffn_dim, g, u, a, st)) != hipSuccess)
      return hip_fail(e, "gate/up launch");
  }
  {  // a9: h2 = h1 + Wd a
    TimedLaunch tl(NT_K_FFN_DOWN, st);
    if ((e = gemm_launch(w.fmt[NT_W_DOWN], W(NT_W_DOWN), s.dim, s.ffn_dim, k, a, h, st, true)) != hipSuccess)
      return hip_fail(e, "down gemm launch");
  }
  return NT_OK;
}

nt_layer_weights weights_in_blob(const uint8_t* blob, const nt_layer_layout& lay) {
  nt_layer_weights w;
  for (int i = 0; i < NT_W_COUNT; ++i) {
    w.fmt[i] = lay.fmt[i];
    w.w[i] = blob + lay.offset[i];
  }
  w.attn_norm = reinterpret_cast<const float*>(blob + lay.offset[NT_W_COUNT]);
  w.ffn_norm = reinterpret_cast<const float*>(blob + lay.offset[NT_W_COUNT + 1]);
  return w;
}

int check_layout(const nt_layer_shape& s, const nt_layer_layout& lay) {
  const int nq = s.n_q_heads * s.head_dim, nkv = s.n_kv_heads * s.head_dim;
  const int64_t rows[NT_W_COUNT] = {nq, nkv, nkv, s.dim, s.ffn_dim, s.ffn_dim, s.dim};
  const int64_t cols[NT_W_COUNT] = {s.dim, s.dim, s.dim, nq, s.dim, s.dim, s.ffn_dim};
  for (int i = 0; i < NT_W_COUNT; ++i) {
    if (!fmt_ok(lay.fmt[i])) return fail(NT_EFORMAT, "layout: unknown format %d for matrix %d", lay.fmt[i], i);
    const int64_t nb = nt_matrix_bytes(lay.fmt[i], rows[i], cols[i]);
    if (lay.offset[i] < 0 || lay.offset[i] % 256 || lay.offset[i] + nb > lay.blob_bytes)
      return fail(NT_ESHAPE, "layout: matrix %d offset %lld (size %lld) is not 256-aligned inside the blob", i,
                  (long long)lay.offset[i], (long long)nb);
  }
  for (int i = NT_W_COUNT; i < NT_W_COUNT + 2; ++i)
    if (lay.offset[i] < 0 || lay.offset[i] % 256 || lay.offset[i] + 4 * (int64_t)s.dim > lay.blob_bytes)
      return fail(NT_ESHAPE, "layout: gain %d offset is not 256-aligned inside the blob", i - NT_W_COUNT);
  if (lay.fmt[NT_W_GATE] != lay.fmt[NT_W_UP]) return fail(NT_EFORMAT, "layout: gate and up must share a format");
  return NT_OK;
}

}  // namespace

namespace nt {
// The thread-local error message of nt_last_error(), for entry points in other files.
int set_error(int code, const char* msg) { return fail(code, "%s", msg); }
}  // namespace nt

// ====================================================================== C ABI

struct nt_streamer {
  uint8_t* staging[2];
  size_t bytes;
  hipEvent_t ready[2], freed[2];
  bool freed_recorded[2];
  uint8_t* bounce[2];       // page-locked host buffers for file-tier layers (null: none)
  size_t bounce_bytes;
  int n_threads;            // readers per blob
  hipEvent_t bounce_free[2];  // recorded after the H2D copy out of bounce[b]
  bool bounce_recorded[2];
  const void* plan_layers;  // identity of the plan the sequence counters belong to
  std::vector<int> streamed;  // and its streamed, unskipped layers
  // what each staging buffer's last copy was issued from (blob, or file and offset), so that a
  // prefetch made from entries the caller has since changed is not used
  struct Src {
    const void* blob;
    int tier, fd;
    int64_t off;
    bool operator==(const Src& o) const { return blob == o.blob && tier == o.tier && fd == o.fd && off == o.off; }
  } src[2];
  int64_t c_run;    // next streamed-layer sequence number to run
  int64_t c_issue;  // next streamed-layer sequence number to copy
};

extern "C" {

const char* nt_last_error(void) { return g_err.c_str(); }
const char* nt_version(void) { return "nt 0.1 (gfx950)"; }

int nt_block_elems(int fmt) { return fmt_ok(fmt) ? block_elems(fmt) : fail(NT_EFORMAT, "unknown format %d", fmt); }
int nt_block_bytes(int fmt) { return fmt_ok(fmt) ? block_bytes(fmt) : fail(NT_EFORMAT, "unknown format %d", fmt); }

int64_t nt_matrix_bytes(int fmt, int64_t rows, int64_t cols) {
  if (!fmt_ok(fmt)) return fail(NT_EFORMAT, "unknown format %d", fmt);
  if (rows <= 0 || cols <= 0 || cols % block_elems(fmt)) return fail(NT_ESHAPE, "bad shape %lld x %lld", (long long)rows, (long long)cols);
  return rows * (cols / block_elems(fmt)) * block_bytes(fmt);
}

int nt_dequant(int fmt, int64_t rows, int64_t cols, const void* blocks, float* w, void* stream) {
  if (!fmt_ok(fmt)) return fail(NT_EFORMAT, "unknown format %d", fmt);
  if (rows <= 0 || cols <= 0 || cols % col_unit(fmt)) return fail(NT_ESHAPE, "cols must be a positive multiple of %d", col_unit(fmt));
  if (!blocks || !w) return fail(NT_EINVAL, "null pointer");
  if (!aligned(blocks, 4) || !aligned(w, 4)) return fail(NT_EALIGN, "blocks and w must be 4-byte aligned");
  hipError_t e = dequant_launch(fmt, rows, cols, blocks, w, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "dequant launch");
}

int nt_repack(int fmt, int64_t rows, int64_t cols, const void* src, void* dst, void* stream) {
  if (fmt != NT_Q4_KT && fmt != NT_Q8_0T && fmt != NT_Q5_KT)
    return fail(NT_EFORMAT, "repack: the target layout must be NT_Q4_KT, NT_Q8_0T or NT_Q5_KT (got %d)", fmt);
  if (rows <= 0 || rows > NT_MAX_ROWS || cols <= 0 || cols % 256 || cols > (1 << 24))
    return fail(NT_ESHAPE, "repack: need 0 < rows <= 2^30 and cols a positive multiple of 256 up to 2^24 (got %lld x %lld)",
                (long long)rows, (long long)cols);
  if (!src || !dst) return fail(NT_EINVAL, "null pointer");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(NT_EALIGN, "src and dst must be 16-byte aligned");
  const uintptr_t bytes = (uintptr_t)(fmt == NT_Q4_KT ? rows * (cols / 256) * 144
                                      : fmt == NT_Q5_KT ? rows * (cols / 256) * 176 : rows * (cols / 32) * 34);
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return fail(NT_EINVAL, "repack: src and dst overlap");
  hipError_t e = fmt == NT_Q4_KT   ? repack_q4kt_launch(rows, cols, src, dst, (hipStream_t)stream)
                 : fmt == NT_Q5_KT ? repack_q5kt_launch(rows, cols, src, dst, (hipStream_t)stream)
                                   : repack_q8t_launch(rows, cols, src, dst, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "repack launch");
}

int nt_gemv_q(int fmt, int64_t rows, int64_t cols, const void* blocks, const float* x, float* y, void* stream) {
  if (!fmt_ok(fmt)) return fail(NT_EFORMAT, "unknown format %d", fmt);
  if (rows <= 0 || rows > NT_MAX_ROWS || cols <= 0 || cols % col_unit(fmt) || cols > NT_GEMV_MAX_COLS)
    return fail(NT_ESHAPE, "need 0 < rows <= 2^30 and cols a positive multiple of %d up to %d (got %lld x %lld)",
                col_unit(fmt), NT_GEMV_MAX_COLS, (long long)rows, (long long)cols);
  if (!blocks || !x || !y) return fail(NT_EINVAL, "null pointer");
  if (!aligned(blocks, 16) || !aligned(x, 16) || !aligned(y, 4)) return fail(NT_EALIGN, "blocks and x must be 16-byte aligned, y 4-byte");
  const GemvPlan p = gemv_plan(EPI_STORE, (int)cols, 1 << fmt, (int)rows);
  GemvArgs a = blank_args();
  a.x = x; a.cols = (int)cols; a.nseg = 1;
  a.seg[0] = make_seg(blocks, fmt, (int)rows, (int)cols, 0);
  a.y = y;
  TimedLaunch tl(NT_K_GEMV, (hipStream_t)stream);
  hipError_t e = gemv_launch(1 << fmt, EPI_STORE, p, gemv_groups(p, (int)rows), a, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "gemv launch");
}

int nt_gemm_q(int fmt, int64_t rows, int64_t cols, int n_tok, const void* blocks, const float* x, float* y,
              void* stream) {
  if (!fmt_ok(fmt)) return fail(NT_EFORMAT, "unknown format %d", fmt);
  if (rows <= 0 || rows > NT_MAX_ROWS || cols <= 0 || cols > NT_MAX_ROWS || cols % col_unit(fmt))
    return fail(NT_ESHAPE, "need 0 < rows, cols <= 2^30 and cols a multiple of %d (got %lld x %lld)", col_unit(fmt),
                (long long)rows, (long long)cols);
  if (n_tok < 1 || n_tok > NT_GEMM_MAX_TOK) return fail(NT_ESHAPE, "n_tok must be in [1, %d]", NT_GEMM_MAX_TOK);
  if (!blocks || !x || !y) return fail(NT_EINVAL, "null pointer");
  if (!aligned(blocks, 16) || !aligned(x, 16) || !aligned(y, 4)) return fail(NT_EALIGN, "blocks and x must be 16-byte aligned, y 4-byte");
  TimedLaunch tl(NT_K_GEMM, (hipStream_t)stream);
  hipError_t e = gemm_launch(fmt, reinterpret_cast<const uint8_t*>(blocks), rows, cols, n_tok, x, y, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "gemm launch");
}

int nt_rmsnorm(int64_t n, const float* x, const float* gain, float eps, float* y, void* stream) {
  if (n <= 0 || n > (1 << 24)) return fail(NT_ESHAPE, "n must be in [1, 2^24]");
  if (!x || !gain || !y) return fail(NT_EINVAL, "null pointer");
  if (!(eps >= 0.f)) return fail(NT_EINVAL, "eps must be >= 0");
  hipError_t e = rmsnorm_launch(n, x, gain, eps, y, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "rmsnorm launch");
}

int nt_rope(int n_heads, int head_dim, int pos, float theta, float* qk, void* stream) {
  if (n_heads <= 0 || head_dim <= 0 || head_dim % 2 || head_dim > 1024) return fail(NT_ESHAPE, "bad head shape");
  if (pos < 0) return fail(NT_EINVAL, "pos must be >= 0");
  if (!(theta > 0.f)) return fail(NT_EINVAL, "theta must be > 0");
  if (!qk) return fail(NT_EINVAL, "null pointer");
  hipError_t e = rope_launch(n_heads, head_dim, pos, theta, qk, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "rope launch");
}

size_t nt_attn_decode_ws_bytes(int n_q_heads, int n_kv_heads, int head_dim, int max_ctx) {
  (void)head_dim;
  if (n_q_heads <= 0 || n_kv_heads <= 0 || max_ctx <= 0) return 0;
  return align256(4 * attn_part_floats(n_q_heads, max_ctx));
}

int nt_attn_decode(int n_q_heads, int n_kv_heads, int head_dim, int n_ctx, int max_ctx, const float* q,
                   const uint16_t* k_cache, const uint16_t* v_cache, float* out, void* ws, size_t ws_bytes,
                   void* stream) {
  if (head_dim != 128) return fail(NT_ESHAPE, "head_dim must be 128");
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads) return fail(NT_ESHAPE, "n_q_heads must be a multiple of n_kv_heads");
  const int grp = n_q_heads / n_kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8 && grp != 16) return fail(NT_ESHAPE, "group size must be 1, 2, 4, 8 or 16");
  if (max_ctx <= 0 || max_ctx % 8 || max_ctx > ATTN_MAX_CTX)
    return fail(NT_ESHAPE, "max_ctx must be a positive multiple of 8 up to %d (got %d)", ATTN_MAX_CTX, max_ctx);
  if (n_ctx < 1 || n_ctx > max_ctx) return fail(NT_ESHAPE, "need 1 <= n_ctx <= max_ctx");
  if (!q || !k_cache || !v_cache || !out || !ws) return fail(NT_EINVAL, "null pointer");
  if (!aligned(ws, 256) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(q, 16))
    return fail(NT_EALIGN, "ws must be 256-byte aligned; q and caches 16-byte aligned");
  if (ws_bytes < nt_attn_decode_ws_bytes(n_q_heads, n_kv_heads, head_dim, max_ctx)) return fail(NT_EINVAL, "workspace too small");
  AttnArgs a;
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.out = out;
  a.part = reinterpret_cast<float*>(ws);
  a.n_kv = n_kv_heads; a.n_ctx = n_ctx; a.max_ctx = max_ctx;
  a.n_split = attn_n_split(n_ctx);
  hipError_t e;
  {
    TimedLaunch tl(NT_K_ATTN, (hipStream_t)stream);
    e = attn_launch(a, grp, (hipStream_t)stream);
  }
  return e == hipSuccess ? NT_OK : hip_fail(e, "attention launch");
}

int nt_swiglu(int64_t n, const float* gate, const float* up, float* out, void* stream) {
  if (n <= 0) return fail(NT_ESHAPE, "n must be positive");
  if (!gate || !up || !out) return fail(NT_EINVAL, "null pointer");
  hipError_t e = swiglu_launch(n, gate, up, out, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "swiglu launch");
}

size_t nt_decode_layer_ws_bytes(const nt_layer_shape* shp) {
  if (!shp || shp->head_dim != 128 || shp->n_q_heads <= 0 || shp->n_kv_heads <= 0) return 0;
  return layer_ws(*shp).total;
}

int nt_decode_layer_ws_offsets(const nt_layer_shape* shp, int64_t* off) {
  int rc = check_shape(shp);
  if (rc) return rc;
  if (!off) return fail(NT_EINVAL, "null pointer");
  const LayerWs L = layer_ws(*shp);
  off[0] = (int64_t)L.q; off[1] = (int64_t)L.o; off[2] = (int64_t)L.h1; off[3] = (int64_t)L.a; off[4] = (int64_t)L.part;
  return NT_OK;
}

int nt_decode_layer(const nt_layer_weights* w, const nt_layer_shape* shp, int pos, float* h, uint16_t* k_cache,
                    uint16_t* v_cache, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shp);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (pos < 0 || pos >= shp->max_ctx) return fail(NT_ESHAPE, "pos %d outside [0, max_ctx)", pos);
  if (!h || !k_cache || !v_cache || !ws) return fail(NT_EINVAL, "null pointer");
  if (!aligned(h, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(ws, 256))
    return fail(NT_EALIGN, "h and caches must be 16-byte aligned, ws 256-byte");
  if (ws_bytes < layer_ws(*shp).total) return fail(NT_EINVAL, "workspace too small (%zu < %zu)", ws_bytes, layer_ws(*shp).total);
  return run_layer(*w, *shp, pos, h, k_cache, v_cache, reinterpret_cast<uint8_t*>(ws), (hipStream_t)stream);
}

int nt_ffn_up(const nt_layer_weights* w, const nt_layer_shape* shp, const float* h, float* a, void* stream) {
  int rc;
  if ((rc = check_shape(shp))) return rc;
  if ((rc = check_weights(w))) return rc;
  if (!h || !a) return fail(NT_EINVAL, "null pointer");
  if (!aligned(h, 16) || !aligned(a, 4)) return fail(NT_EALIGN, "h must be 16-byte aligned, a 4-byte");
  const hipError_t e = ffn_up_launch(*w, *shp, h, a, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "gate/up launch");
}

int nt_embed_row(int fmt, int64_t n_vocab, int64_t dim, const void* table, const int32_t* token, float* h,
                 void* stream) {
  if (!fmt_ok(fmt)) return fail(NT_EFORMAT, "unknown format %d", fmt);
  if (n_vocab <= 0 || dim <= 0 || dim % col_unit(fmt)) return fail(NT_ESHAPE, "bad embedding shape");
  if (!table || !token || !h) return fail(NT_EINVAL, "null pointer");
  if (!aligned(table, 4)) return fail(NT_EALIGN, "table must be 4-byte aligned");
  hipError_t e = embed_launch(fmt, n_vocab, dim, table, token, h, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "embed launch");
}

int nt_argmax(int64_t n, const float* v, int32_t* out_index, void* stream) {
  if (n <= 0 || n > 0x7FFFFFFF) return fail(NT_ESHAPE, "n must be in [1, 2^31)");
  if (!v || !out_index) return fail(NT_EINVAL, "null pointer");
  hipError_t e = argmax_launch(n, v, out_index, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "argmax launch");
}

int nt_layer_cosine(int64_t n, const float* a, const float* b, float* out, void* stream) {
  if (n <= 0 || n > (1 << 24)) return fail(NT_ESHAPE, "n must be in [1, 2^24]");
  if (!a || !b || !out) return fail(NT_EINVAL, "null pointer");
  if (!aligned(a, 4) || !aligned(b, 4) || !aligned(out, 4)) return fail(NT_EALIGN, "a, b and out must be 4-byte aligned");
  hipError_t e = cosine_launch(n, a, b, out, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "cosine launch");
}

int64_t nt_set_stream_min_weights(int64_t min_weights) { return gemv_set_stream_min_weights(min_weights); }

int nt_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes <= 0 || bytes % 16) return fail(NT_ESHAPE, "bytes must be a positive multiple of 16");
  if (!buf || !sink) return fail(NT_EINVAL, "null pointer");
  if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(NT_EALIGN, "buf must be 16-byte aligned, sink 4-byte");
  hipError_t e = read_probe_launch(buf, bytes, sink, (hipStream_t)stream);
  return e == hipSuccess ? NT_OK : hip_fail(e, "read probe launch");
}

int nt_stream_create(void* staging0, void* staging1, size_t staging_bytes, nt_streamer** out) {
  if (!out) return fail(NT_EINVAL, "out is null");
  *out = nullptr;
  if (!staging0 || !staging1 || staging0 == staging1) return fail(NT_EINVAL, "need two distinct staging buffers");
  if (!aligned(staging0, 256) || !aligned(staging1, 256)) return fail(NT_EALIGN, "staging buffers must be 256-byte aligned");
  if (staging_bytes == 0) return fail(NT_EINVAL, "staging_bytes is 0");
  nt_streamer* st = new nt_streamer();
  st->staging[0] = reinterpret_cast<uint8_t*>(staging0);
  st->staging[1] = reinterpret_cast<uint8_t*>(staging1);
  st->bytes = staging_bytes;
  for (int b = 0; b < 2; ++b) {
    hipError_t e;
    if ((e = hipEventCreateWithFlags(&st->ready[b], hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&st->freed[b], hipEventDisableTiming)) != hipSuccess) {
      delete st;
      return hip_fail(e, "hipEventCreate");
    }
    st->freed_recorded[b] = false;
  }
  st->bounce[0] = st->bounce[1] = nullptr;
  st->bounce_bytes = 0;
  st->n_threads = 1;
  st->bounce_recorded[0] = st->bounce_recorded[1] = false;
  st->plan_layers = nullptr;
  st->c_run = st->c_issue = 0;
  *out = st;
  return NT_OK;
}

int nt_stream_set_bounce(nt_streamer* st, void* bounce0, void* bounce1, size_t bounce_bytes, int n_threads) {
  if (!st) return fail(NT_EINVAL, "null streamer");
  if (!bounce0 || !bounce1 || bounce0 == bounce1) return fail(NT_EINVAL, "need two distinct bounce buffers");
  if (!aligned(bounce0, 4096) || !aligned(bounce1, 4096)) return fail(NT_EALIGN, "bounce buffers must be 4096-byte aligned");
  if (bounce_bytes == 0) return fail(NT_EINVAL, "bounce_bytes is 0");
  if (n_threads < 1 || n_threads > 64) return fail(NT_EINVAL, "n_threads must be in [1, 64]");
  for (void* p : {bounce0, bounce1}) {
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof(attr));
    hipError_t he = hipPointerGetAttributes(&attr, p);
    if (he != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return fail(NT_EHOSTMEM, "bounce buffers must be page-locked host memory");
    }
  }
  if (!st->bounce[0]) {
    for (int b = 0; b < 2; ++b) {
      hipError_t e = hipEventCreateWithFlags(&st->bounce_free[b], hipEventDisableTiming);
      if (e != hipSuccess) {
        if (b == 1) (void)hipEventDestroy(st->bounce_free[0]);
        return hip_fail(e, "hipEventCreate");
      }
    }
  } else {
    for (int b = 0; b < 2; ++b)
      if (st->bounce_recorded[b]) (void)hipEventSynchronize(st->bounce_free[b]);  // the old buffers' copies are done
  }
  st->bounce[0] = reinterpret_cast<uint8_t*>(bounce0);
  st->bounce[1] = reinterpret_cast<uint8_t*>(bounce1);
  st->bounce_bytes = bounce_bytes;
  st->n_threads = n_threads;
  st->bounce_recorded[0] = st->bounce_recorded[1] = false;
  return NT_OK;
}

void nt_stream_destroy(nt_streamer* st) {
  if (!st) return;
  for (int b = 0; b < 2; ++b) {
    (void)hipEventSynchronize(st->ready[b]);
    (void)hipEventSynchronize(st->freed[b]);
    (void)hipEventDestroy(st->ready[b]);
    (void)hipEventDestroy(st->freed[b]);
  }
  if (st->bounce[0]) {
    for (int b = 0; b < 2; ++b) {
      (void)hipEventSynchronize(st->bounce_free[b]);
      (void)hipEventDestroy(st->bounce_free[b]);
    }
  }
  delete st;
}

static int check_plan(const nt_model_plan* plan, const nt_streamer* st) {
  if (!plan || !plan->layers || plan->n_layers <= 0) return fail(NT_EINVAL, "empty plan");
  int rc = check_shape(&plan->shape);
  if (rc) return rc;
  if ((rc = check_layout(plan->shape, plan->layout))) return rc;
  for (int l = 0; l < plan->n_layers; ++l) {
    const nt_layer_entry& e = plan->layers[l];
    if (e.resident != NT_TIER_PINNED && e.resident != NT_TIER_RESIDENT && e.resident != NT_TIER_FILE)
      return fail(NT_EINVAL, "layer %d has an unknown tier %d", l, e.resident);
    if (e.skip) continue;  // never read: its blob, caches and tier need nothing
    if (!e.k_cache || !e.v_cache) return fail(NT_EINVAL, "layer %d has a null cache pointer", l);
    if (e.resident != NT_TIER_RESIDENT && !st)
      return fail(NT_EINVAL, "layer %d is not resident and no streamer was given", l);
    if (e.resident == NT_TIER_FILE) {
      if (e.fd < 0 || e.file_offset < 0) return fail(NT_EINVAL, "layer %d: bad file descriptor or offset", l);
      if (!st->bounce[0]) return fail(NT_EINVAL, "layer %d is read from a file but the streamer has no bounce buffers", l);
      if ((size_t)plan->layout.blob_bytes > st->bounce_bytes)
        return fail(NT_EINVAL, "layer blob larger than the bounce buffers");
      // the whole blob must lie inside the file now, so that a short read cannot stop the call
      // after earlier layers were enqueued (only an I/O error or a file shrinking meanwhile can)
      struct stat sb;
      if (fstat(e.fd, &sb) != 0) return fail(NT_EHOSTMEM, "layer %d: fstat of its file failed (errno %d)", l, errno);
      if (e.file_offset + plan->layout.blob_bytes > (int64_t)sb.st_size)
        return fail(NT_EHOSTMEM, "layer %d: blob at offset %lld runs past the end of its file (%lld bytes)", l,
                    (long long)e.file_offset, (long long)sb.st_size);
      continue;
    }
    if (!e.blob) return fail(NT_EINVAL, "layer %d has a null blob", l);
    if (!aligned(e.blob, 256)) return fail(NT_EALIGN, "layer %d blob must be 256-byte aligned", l);
    if (e.resident == NT_TIER_PINNED) {
      hipPointerAttribute_t attr;
      memset(&attr, 0, sizeof(attr));
      hipError_t he = hipPointerGetAttributes(&attr, e.blob);
      if (he != hipSuccess || attr.type != hipMemoryTypeHost) {
        (void)hipGetLastError();  // clear a sticky error left by the query on pageable memory
        return fail(NT_EHOSTMEM, "layer %d blob is not page-locked host memory", l);
      }
    }
  }
  return NT_OK;
}

// Read n bytes at offset off of fd into dst with t threads, each taking one contiguous piece
// (a multiple of 4096 bytes but the last) and repeating pread until it is done.  False on a
// read error or an early end of file.
static bool read_blob(int fd, int64_t off, uint8_t* dst, size_t n, int t) {
  auto piece = [fd, off, dst](size_t a, size_t b, bool* ok) {
    while (a < b) {
      const ssize_t r = pread(fd, dst + a, b - a, (off_t)(off + (int64_t)a));
      if (r < 0 && errno == EINTR) continue;
      if (r <= 0) {
        *ok = false;
        return;
      }
      a += (size_t)r;
    }
    *ok = true;
  };
  const size_t step = ((n + (size_t)t - 1) / (size_t)t + 4095) & ~(size_t)4095;
  std::vector<std::thread> th;
  bool ok[64];
  int k = 0;
  for (size_t a = 0; a < n; a += step, ++k) {
    const size_t b = a + step < n ? a + step : n;
    bool spawned = false;
    if (a + step < n) {
      try {
        th.emplace_back(piece, a, b, &ok[k]);
        spawned = true;
      } catch (...) {
        // no thread to be had: read this piece here
      }
    }
    if (!spawned) piece(a, b, &ok[k]);  // the last piece (or one no thread took) on this thread
  }
  for (auto& x : th) x.join();
  for (int i = 0; i < k; ++i)
    if (!ok[i]) return false;
  return true;
}

static nt_streamer::Src entry_src(const nt_layer_entry& e) {
  nt_streamer::Src r;
  r.tier = e.resident;
  r.blob = e.resident == NT_TIER_FILE ? nullptr : e.blob;
  r.fd = e.resident == NT_TIER_FILE ? e.fd : -1;
  r.off = e.resident == NT_TIER_FILE ? e.file_offset : 0;
  return r;
}

static int stream_issue(nt_streamer* st, const nt_model_plan* plan, const std::vector<int>& streamed, hipStream_t copy,
                        nt_stream_stats* stats) {
  const int64_t q = st->c_issue;
  const int b = (int)(q & 1);
  const int layer = streamed[(size_t)(q % (int64_t)streamed.size())];
  const nt_layer_entry& ent = plan->layers[layer];
  st->src[b] = entry_src(ent);
  const size_t nbytes = (size_t)plan->layout.blob_bytes;
  hipError_t e;
  const void* src = ent.blob;
  if (ent.resident == NT_TIER_FILE) {
    // the bounce buffer's previous copy (two issues ago) must be done before it is refilled
    if (st->bounce_recorded[b] && (e = hipEventSynchronize(st->bounce_free[b])) != hipSuccess)
      return hip_fail(e, "hipEventSynchronize(bounce)");
    if (!read_blob(ent.fd, ent.file_offset, st->bounce[b], nbytes, st->n_threads))
      return fail(NT_EHOSTMEM, "layer %d: short or failed read of %zu bytes at offset %lld", layer, nbytes,
                  (long long)ent.file_offset);
    src = st->bounce[b];
  }
  if (st->freed_recorded[b] && (e = hipStreamWaitEvent(copy, st->freed[b], 0)) != hipSuccess)
    return hip_fail(e, "hipStreamWaitEvent(copy)");
  if ((e = hipMemcpyAsync(st->staging[b], src, nbytes, hipMemcpyHostToDevice, copy)) != hipSuccess)
    return hip_fail(e, "hipMemcpyAsync");
  if (ent.resident == NT_TIER_FILE) {
    if ((e = hipEventRecord(st->bounce_free[b], copy)) != hipSuccess) return hip_fail(e, "hipEventRecord(bounce)");
    st->bounce_recorded[b] = true;
  }
  if ((e = hipEventRecord(st->ready[b], copy)) != hipSuccess) return hip_fail(e, "hipEventRecord(ready)");
  if (stats) stats->h2d_bytes += (int64_t)nbytes;
  st->c_issue = q + 1;
  return NT_OK;
}

// n_tok 0: the single-token layer (nt_decode_layer's launches); n_tok >= 1: the k-token layer.
static int stream_layers_impl(nt_streamer* st, const nt_model_plan* plan, int pos, float* h, uint8_t* ws,
                              hipStream_t compute, hipStream_t copy, nt_stream_stats* stats, int n_tok = 0) {
  auto layer = [&](const nt_layer_weights& w, const nt_layer_entry& ent) {
    return n_tok == 0 ? run_layer(w, plan->shape, pos, h, ent.k_cache, ent.v_cache, ws, compute)
                      : run_layer_k(w, plan->shape, pos, n_tok, h, ent.k_cache, ent.v_cache, ws, compute);
  };
  std::vector<int> streamed;  // the layers copied through the staging buffers, in order
  for (int l = 0; l < plan->n_layers; ++l)
    if (plan->layers[l].resident != NT_TIER_RESIDENT && !plan->layers[l].skip) streamed.push_back(l);
  if (st && !streamed.empty()) {
    // the copies in flight from the previous call (sequence numbers c_run .. c_issue - 1) must
    // come from the entries as they are now
    bool same = st->plan_layers == (const void*)plan->layers && st->streamed == streamed;
    for (int64_t q = st->c_run; same && q < st->c_issue; ++q) {
      const int layer = streamed[(size_t)(q % (int64_t)streamed.size())];
      same = st->src[q & 1] == entry_src(plan->layers[layer]);
    }
    if (!same) {
      // a new plan: drain what the streamer had in flight, then restart its sequence
      for (int b = 0; b < 2; ++b) {
        (void)hipEventSynchronize(st->ready[b]);
        (void)hipEventSynchronize(st->freed[b]);
        st->freed_recorded[b] = false;
      }
      st->plan_layers = plan->layers;
      st->streamed = streamed;
      st->c_run = st->c_issue = 0;
    }
  }
  int rc;
  if (st && !streamed.empty())
    while (st->c_issue < st->c_run + 2)
      if ((rc = stream_issue(st, plan, streamed, copy, stats))) return rc;
  for (int l = 0; l < plan->n_layers; ++l) {
    const nt_layer_entry& ent = plan->layers[l];
    if (ent.skip) continue;
    if (ent.resident == NT_TIER_RESIDENT) {
      const nt_layer_weights w = weights_in_blob(reinterpret_cast<const uint8_t*>(ent.blob), plan->layout);
      if ((rc = layer(w, ent))) return rc;
      continue;
    }
    const int64_t q = st->c_run;
    const int b = (int)(q & 1);
    while (st->c_issue <= q)
      if ((rc = stream_issue(st, plan, streamed, copy, stats))) return rc;
    hipError_t e;
    if ((e = hipStreamWaitEvent(compute, st->ready[b], 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(compute)");
    const nt_layer_weights w = weights_in_blob(st->staging[b], plan->layout);
    if ((rc = layer(w, ent))) return rc;
    if ((e = hipEventRecord(st->freed[b], compute)) != hipSuccess) return hip_fail(e, "hipEventRecord(freed)");
    st->freed_recorded[b] = true;
    st->c_run = q + 1;
    if (stats) stats->layers_streamed += 1;
    while (st->c_issue < st->c_run + 2)
      if ((rc = stream_issue(st, plan, streamed, copy, stats))) return rc;
  }
  return NT_OK;
}

int nt_stream_layers(nt_streamer* st, const nt_model_plan* plan, int pos, float* h, void* ws, size_t ws_bytes,
                     void* compute, void* copy, nt_stream_stats* stats) {
  if (stats) stats->layers_streamed = stats->h2d_bytes = 0;
  int rc = check_plan(plan, st);
  if (rc) return rc;
  if (pos < 0 || pos >= plan->shape.max_ctx) return fail(NT_ESHAPE, "pos %d outside [0, max_ctx)", pos);
  if (!h || !ws) return fail(NT_EINVAL, "null pointer");
  if (!aligned(h, 16) || !aligned(ws, 256)) return fail(NT_EALIGN, "h must be 16-byte aligned, ws 256-byte");
  if (ws_bytes < layer_ws(plan->shape).total) return fail(NT_EINVAL, "workspace too small");
  if (st) {
    if ((size_t)plan->layout.blob_bytes > st->bytes) return fail(NT_EINVAL, "layer blob larger than the staging buffers");
    if (compute == copy) return fail(NT_EINVAL, "compute and copy streams must differ");
  }
  return stream_layers_impl(st, plan, pos, h, reinterpret_cast<uint8_t*>(ws), (hipStream_t)compute, (hipStream_t)copy,
                            stats);
}

size_t nt_decode_token_ws_bytes(const nt_layer_shape* shp) { return nt_decode_layer_ws_bytes(shp); }

int nt_decode_token(nt_streamer* st, const nt_model_plan* plan, const nt_model_head* head, int pos, int32_t* token,
                    float* logits, float* h, void* ws, size_t ws_bytes, void* compute, void* copy,
                    nt_stream_stats* stats) {
  if (stats) stats->layers_streamed = stats->h2d_bytes = 0;
  int rc = check_plan(plan, st);
  if (rc) return rc;
  if (!head || !head->token_embd || !head->output_norm || !head->output || !token || !logits || !h || !ws)
    return fail(NT_EINVAL, "null pointer");
  if (!fmt_ok(head->embd_fmt) || !fmt_ok(head->out_fmt)) return fail(NT_EFORMAT, "unknown head format");
  if (head->n_vocab <= 0 || head->n_vocab > NT_MAX_ROWS) return fail(NT_ESHAPE, "vocabulary size must be in [1, 2^30]");
  if (!aligned(head->output, 16) || !aligned(head->token_embd, 4) || !aligned(head->output_norm, 16) || !aligned(h, 16) ||
      !aligned(ws, 256))
    return fail(NT_EALIGN, "misaligned head, h or ws pointer");
  if (pos < 0 || pos >= plan->shape.max_ctx) return fail(NT_ESHAPE, "pos %d outside [0, max_ctx)", pos);
  const LayerWs L = layer_ws(plan->shape);
  if (ws_bytes < L.total) return fail(NT_EINVAL, "workspace too small");
  if (st) {
    if ((size_t)plan->layout.blob_bytes > st->bytes) return fail(NT_EINVAL, "layer blob larger than the staging buffers");
    if (compute == copy) return fail(NT_EINVAL, "compute and copy streams must differ");
  }
  hipStream_t cs = (hipStream_t)compute;
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  unsigned long long* key = reinterpret_cast<unsigned long long*>(wsb + L.key);
  hipError_t e;
  if ((e = embed_launch(head->embd_fmt, head->n_vocab, plan->shape.dim, head->token_embd, token, h, key, cs)) != hipSuccess)
    return hip_fail(e, "embed launch");
  if ((rc = stream_layers_impl(st, plan, pos, h, wsb, cs, (hipStream_t)copy, stats))) return rc;
  // the embedding launch reset the key
  return lm_head_enqueue(head->out_fmt, head->n_vocab, plan->shape.dim, head->output, head->output_norm,
                         plan->shape.eps, h, logits, key, token, false, cs);
}

int nt_lm_head(int fmt, int64_t n_vocab, int64_t dim, const void* output, const float* output_norm, float eps,
               const float* h, float* logits, int32_t* token, void* ws, size_t ws_bytes, void* stream) {
  if (!fmt_ok(fmt)) return fail(NT_EFORMAT, "unknown format %d", fmt);
  if (n_vocab <= 0 || n_vocab > NT_MAX_ROWS) return fail(NT_ESHAPE, "n_vocab must be in [1, %d]", NT_MAX_ROWS);
  if (dim <= 0 || dim % 256 || dim > NT_GEMV_MAX_COLS)
    return fail(NT_ESHAPE, "dim must be a positive multiple of 256 up to %d", NT_GEMV_MAX_COLS);
  if (!output || !output_norm || !h || !logits || !token || !ws) return fail(NT_EINVAL, "null pointer");
  if (!(eps >= 0.f)) return fail(NT_EINVAL, "eps must be >= 0");
  if (!aligned(output, 16) || !aligned(output_norm, 16) || !aligned(h, 16) || !aligned(logits, 4) ||
      !aligned(token, 4) || !aligned(ws, 256))
    return fail(NT_EALIGN, "output, output_norm and h must be 16-byte aligned, logits and token 4-byte, ws 256-byte");
  if (ws_bytes < NT_LM_HEAD_WS_BYTES) return fail(NT_EINVAL, "workspace too small (%zu < %d)", ws_bytes, NT_LM_HEAD_WS_BYTES);
  return lm_head_enqueue(fmt, n_vocab, (int)dim, output, output_norm, eps, h, logits,
                         reinterpret_cast<unsigned long long*>(ws), token, true, (hipStream_t)stream);
}

size_t nt_decode_layer_k_ws_bytes(const nt_layer_shape* shp, int n_tok) {
  if (!shp || shp->head_dim != 128 || shp->n_q_heads <= 0 || shp->n_kv_heads <= 0 || shp->max_ctx <= 0 ||
      n_tok < 1 || n_tok > NT_GEMM_MAX_TOK)
    return 0;
  return layer_k_ws(*shp, n_tok).total;
}

int nt_decode_layer_k_ws_offsets(const nt_layer_shape* shp, int n_tok, int64_t* off) {
  int rc = check_shape(shp);
  if (rc) return rc;
  if (n_tok < 1 || n_tok > NT_GEMM_MAX_TOK) return fail(NT_ESHAPE, "n_tok must be in [1, %d]", NT_GEMM_MAX_TOK);
  if (!off) return fail(NT_EINVAL, "null pointer");
  if (n_tok == 1) {  // the single-token layer's workspace layout
    const LayerWs L1 = layer_ws(*shp);
    off[0] = (int64_t)L1.q; off[1] = (int64_t)L1.o; off[2] = (int64_t)L1.h1; off[3] = (int64_t)L1.a;
    return NT_OK;
  }
  const LayerKWs L = layer_k_ws(*shp, n_tok);
  off[0] = (int64_t)L.q; off[1] = (int64_t)L.o; off[2] = (int64_t)L.h1; off[3] = (int64_t)L.a;
  return NT_OK;
}

int nt_decode_layer_k(const nt_layer_weights* w, const nt_layer_shape* shp, int pos, int n_tok, float* h,
                      uint16_t* k_cache, uint16_t* v_cache, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(shp);
  if (rc) return rc;
  if ((rc = check_weights(w))) return rc;
  if (n_tok < 1 || n_tok > NT_GEMM_MAX_TOK) return fail(NT_ESHAPE, "n_tok must be in [1, %d]", NT_GEMM_MAX_TOK);
  if (pos < 0 || pos + n_tok > shp->max_ctx)
    return fail(NT_ESHAPE, "positions %d .. %d outside [0, max_ctx)", pos, pos + n_tok - 1);
  if (!h || !k_cache || !v_cache || !ws) return fail(NT_EINVAL, "null pointer");
  if (!aligned(h, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(ws, 256))
    return fail(NT_EALIGN, "h and caches must be 16-byte aligned, ws 256-byte");
  const size_t need = layer_k_ws(*shp, n_tok).total;
  if (ws_bytes < need) return fail(NT_EINVAL, "workspace too small (%zu < %zu)", ws_bytes, need);
  return run_layer_k(*w, *shp, pos, n_tok, h, k_cache, v_cache, reinterpret_cast<uint8_t*>(ws), (hipStream_t)stream);
}

size_t nt_verify_tokens_ws_bytes(const nt_layer_shape* shp, int n_tok) { return nt_decode_layer_k_ws_bytes(shp, n_tok); }

int nt_verify_tokens(nt_streamer* st, const nt_model_plan* plan, const nt_model_head* head, int pos, int n_tok,
                     const int32_t* tokens, int32_t* next, float* logits, float* h, void* ws, size_t ws_bytes,
                     void* compute, void* copy, nt_stream_stats* stats) {
  if (stats) stats->layers_streamed = stats->h2d_bytes = 0;
  int rc = check_plan(plan, st);
  if (rc) return rc;
  if (n_tok < 1 || n_tok > NT_GEMM_MAX_TOK) return fail(NT_ESHAPE, "n_tok must be in [1, %d]", NT_GEMM_MAX_TOK);
  if (!head || !head->token_embd || !head->output_norm || !head->output || !tokens || !next || !logits || !h || !ws)
    return fail(NT_EINVAL, "null pointer");
  if (!fmt_ok(head->embd_fmt) || !fmt_ok(head->out_fmt)) return fail(NT_EFORMAT, "unknown head format");
  if (head->n_vocab <= 0 || head->n_vocab > NT_MAX_ROWS) return fail(NT_ESHAPE, "vocabulary size must be in [1, 2^30]");
  if (!aligned(head->output, 16) || !aligned(head->token_embd, 4) || !aligned(head->output_norm, 16) || !aligned(h, 16) ||
      !aligned(logits, 4) || !aligned(ws, 256))
    return fail(NT_EALIGN, "misaligned head, h, logits or ws pointer");
  if (pos < 0 || pos + n_tok > plan->shape.max_ctx)
    return fail(NT_ESHAPE, "positions %d .. %d outside [0, max_ctx)", pos, pos + n_tok - 1);
  const LayerKWs L = layer_k_ws(plan->shape, n_tok);
  if (ws_bytes < L.total) return fail(NT_EINVAL, "workspace too small (%zu < %zu)", ws_bytes, L.total);
  if (st) {
    if ((size_t)plan->layout.blob_bytes > st->bytes) return fail(NT_EINVAL, "layer blob larger than the staging buffers");
    if (compute == copy) return fail(NT_EINVAL, "compute and copy streams must differ");
  }
  hipStream_t cs = (hipStream_t)compute;
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  const int dim = plan->shape.dim;
  hipError_t e;
  if ((e = embed_launch(head->embd_fmt, head->n_vocab, dim, head->token_embd, tokens, h, nullptr, cs, n_tok)) != hipSuccess)
    return hip_fail(e, "embed launch");
  if ((rc = stream_layers_impl(st, plan, pos, h, wsb, cs, (hipStream_t)copy, stats, n_tok == 1 ? 0 : n_tok))) return rc;
  if (n_tok == 1)  // the single-token head: RMSNorm prologue, GEMV and fused argmax in one launch
    return lm_head_enqueue(head->out_fmt, head->n_vocab, dim, head->output, head->output_norm, plan->shape.eps, h,
                           logits, reinterpret_cast<unsigned long long*>(wsb + layer_ws(plan->shape).key), next, true,
                           cs);
  float* xn = reinterpret_cast<float*>(wsb + L.xn);
  if ((e = rmsnorm_rows_launch(n_tok, dim, h, head->output_norm, plan->shape.eps, xn, nullptr, cs)) != hipSuccess)
    return hip_fail(e, "rmsnorm launch");
  {
    TimedLaunch tl(NT_K_LM_HEAD, cs);
    if ((e = gemm_launch(head->out_fmt, reinterpret_cast<const uint8_t*>(head->output), head->n_vocab, dim, n_tok, xn,
                         logits, cs)) != hipSuccess)
      return hip_fail(e, "lm head gemm launch");
  }
  if ((e = argmax_launch(head->n_vocab, logits, next, cs, n_tok)) != hipSuccess) return hip_fail(e, "argmax launch");
  return NT_OK;
}

int nt_timing_begin(int kclass, int max_launches) {
  if (kclass < 0 || kclass >= NT_K_COUNT || max_launches <= 0) return fail(NT_EINVAL, "bad timing request");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (hipEvent_t ev : g_timing.ev) (void)hipEventDestroy(ev);
  g_timing.ev.clear();
  g_timing.kclass = kclass;
  g_timing.max_launches = max_launches;
  return NT_OK;
}

int nt_timing_end(int* n_launches, double* total_ms) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  double tot = 0.0;
  int n = 0;
  int rc = NT_OK;
  for (size_t i = 0; i + 1 < g_timing.ev.size(); i += 2) {
    if (hipEventSynchronize(g_timing.ev[i + 1]) != hipSuccess) { rc = fail(NT_EHIP, "event sync failed"); break; }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_timing.ev[i], g_timing.ev[i + 1]) != hipSuccess) { rc = fail(NT_EHIP, "elapsed time failed"); break; }
    tot += ms;
    ++n;
  }
  for (hipEvent_t ev : g_timing.ev) (void)hipEventDestroy(ev);
  g_timing.ev.clear();
  g_timing.kclass = -1;
  if (n_launches) *n_launches = n;
  if (total_ms) *total_ms = tot;
  return rc;
}

}  // extern "C"
