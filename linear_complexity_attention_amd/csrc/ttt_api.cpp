// C ABI of the TTT-layer library: validation, workspace carving and the
// scheduler that enqueues the kernels of one forward pass.
//
// Schedule of one ttt_forward (ViT3 summary page, section 02: forward on the
// keys, hand backward, update, readout; LaCT analysis page, "Order of
// operations": causal chunks read before they update):
//   key statistics (optional)  ->  for every update batch c (one in full-batch
//   mode, ceil(N/C) in causal mode): gradient partials at W_c, then
//   W_{c+1} = W_c - sum(partials) [+ re-norm]  ->  readout of every token at the
//   state its mode assigns (full: W_1; causal chunk c: W_c).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/ttt.h"
#include "ttt_internal.h"

using namespace ttt;

struct ttt_handle {
  ttt_config cfg;
  std::string err;
  hipEvent_t events[8] = {};
  bool timing = false;
  // second stream for the independent head ranges of one request (the ViT3
  // block), with its fork and join events; created on first use on device
  // side_dev, default priority
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  int side_dev = -1;
};

namespace ttt {
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace ttt

namespace {

thread_local std::string g_create_err;

int vfail(ttt_handle* h, int code, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  if (h) h->err = buf; else g_create_err = buf;
  return code;
}

int fail(ttt_handle* h, int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int r = vfail(h, code, fmt, ap);
  va_end(ap);
  return r;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// token tensors are read and written with 16-byte vector accesses
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// matrices the caller passes for a request (ttt_weights.w entries)
int n_mats(int inner) {
  switch (inner) {
    case TTT_INNER_LINEAR: case TTT_INNER_DWCONV: return 1;
    case TTT_INNER_SWIGLU: case TTT_INNER_VIT3: return 3;
    default: return 2;   // MLP, GLU
  }
}

bool env_log() {
  const char* e = std::getenv("TTT_LOG");
  return e && e[0] == '1';
}

// One head range of a request and the inner model its heads run: every
// request is one range, except the ViT3 block, whose head 0 runs the depthwise
// convolution and whose other heads run the GLU (ViT3 page, section 04).
// slot[i] is the caller's weight entry that holds matrix i of the model.
struct Range {
  int model, h0, hc, nm;
  int slot[3];
};

int ranges_of(const ttt_config& c, int inner, Range* r) {
  switch (inner) {
    case TTT_INNER_VIT3:
      r[0] = Range{INNER_DWCONV, 0, 1, 1, {2, 0, 0}};
      if (c.H == 1) return 1;
      r[1] = Range{INNER_GLU, 1, c.H - 1, 2, {0, 1, 0}};
      return 2;
    case TTT_INNER_LINEAR: r[0] = Range{INNER_LINEAR, 0, c.H, 1, {0, 0, 0}}; return 1;
    case TTT_INNER_MLP_GELU: r[0] = Range{INNER_MLP, 0, c.H, 2, {0, 1, 0}}; return 1;
    case TTT_INNER_SWIGLU: r[0] = Range{INNER_SWIGLU, 0, c.H, 3, {0, 1, 2}}; return 1;
    case TTT_INNER_GLU: r[0] = Range{INNER_GLU, 0, c.H, 2, {0, 1, 0}}; return 1;
    default: r[0] = Range{INNER_DWCONV, 0, c.H, 1, {0, 0, 0}}; return 1;
  }
}

// the request's update mask restricted to a range, in the range's numbering
unsigned range_mask(unsigned mask, const Range& r) {
  unsigned m = 0;
  for (int i = 0; i < r.nm; ++i) m |= ((mask >> r.slot[i]) & 1u) << i;
  return m;
}

// Where every buffer of one range lives inside its part of the workspace.
struct Plan {
  // problem
  int P, nm, hid, nb, chunk, span;   // span: tokens of the longest update batch
  long long msz, wsz;                // elements per matrix / per pair
  // choices
  bool mfma_grad, mfma_query;        // GELU-MLP MFMA kernels
  bool lact_grad, lact_query;        // SwiGLU MFMA kernels
  bool dwconv;                       // depthwise-convolution kernels
  bool glu_grad, glu_query;          // GLU MFMA kernels
  bool step_mfma;                    // fp32 GELU-MLP step on the matrix cores (else k_gen_*)
  bool mfma_direct;                  // the MFMA gradient kernel applies the step to every whole pair
  bool mfma_one_round;               // ... with one workgroup per pair
  bool mfma_split;                   // ... and some pair is split (the update kernel finishes those)
  bool mfma_fused_q;                 // ... no pair is split: the gradient kernel also reads every pair out
  int S_stats, S_grad;               // S_grad: partial slots of the gradient kernel
  int S_step;                        // token slices of the fp32 matrix-core step
  int sk_G, sk_J;                    // stream-K geometry (MFMA gradient kernel)
  // byte offsets
  size_t off_stats_part, off_stats, off_states, off_part, off_gbuf, off_mom, off_muon, off_flag, total;
  size_t off_step[6];                // X, Z, A, dZ, F, G of the fp32 matrix-core step
  long long state_stride;            // floats between consecutive states
};

int choose_splits(long long other_blocks, int tokens, int per_block_min, int target) {
  long long s = (target + other_blocks - 1) / other_blocks;
  long long maxs = (tokens + per_block_min - 1) / per_block_min;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

int stats_splits(long long pairs, int tokens) {
  long long s = 4LL * device_cu_count() / pairs;
  const long long maxs = (tokens + 63) / 64;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

// ttt_options with the defaults filled in
struct Opts {
  int epochs = 1;
  unsigned mask = 0;
  bool causal = false;              // chunk > 0 and TTT_ORDER_CAUSAL
  const unsigned char* chunk_update = nullptr;
  int rule = RULE_GD;
  float beta = 0.f, muon_scale = 1.f;
  int ns_steps = 5;
};

bool is_conv(int inner) { return inner == TTT_INNER_DWCONV || inner == TTT_INNER_VIT3; }

int check_request(ttt_handle* h, int loss, int inner, int chunk, const ttt_options* o, Opts* out) {
  const ttt_config& c = h->cfg;
  if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_DOT) return fail(h, TTT_ERR_INVALID, "unknown loss %d", loss);
  if (inner < TTT_INNER_LINEAR || inner > TTT_INNER_VIT3) return fail(h, TTT_ERR_INVALID, "unknown inner model %d", inner);
  if (chunk < 0) return fail(h, TTT_ERR_INVALID, "chunk must be >= 0 (got %d)", chunk);
  Opts op;
  const int nm = n_mats(inner);
  op.mask = (1u << nm) - 1;
  if (o) {
    if (o->epochs < 0) return fail(h, TTT_ERR_INVALID, "epochs must be >= 0 (got %d)", o->epochs);
    if (o->epochs > 1) op.epochs = o->epochs;
    if (o->update_mask & ~op.mask)
      return fail(h, TTT_ERR_INVALID, "update_mask 0x%x names matrices the inner model does not have (%d)",
                  o->update_mask, nm);
    if (o->update_mask) op.mask = o->update_mask;
    if (o->order != TTT_ORDER_CAUSAL && o->order != TTT_ORDER_WRITE_THEN_QUERY)
      return fail(h, TTT_ERR_INVALID, "unknown order %d", o->order);
    op.causal = chunk > 0 && o->order == TTT_ORDER_CAUSAL;
    op.chunk_update = o->chunk_update;
    if (o->rule != TTT_RULE_GD && o->rule != TTT_RULE_MOMENTUM && o->rule != TTT_RULE_MUON)
      return fail(h, TTT_ERR_INVALID, "unknown update rule %d", o->rule);
    op.rule = o->rule == TTT_RULE_GD ? RULE_GD : o->rule == TTT_RULE_MOMENTUM ? RULE_MOMENTUM : RULE_MUON;
    if (!std::isfinite(o->beta)) return fail(h, TTT_ERR_INVALID, "beta must be finite");
    op.beta = o->beta;
    if (op.rule == RULE_MUON && !std::isfinite(o->muon_scale))
      return fail(h, TTT_ERR_INVALID, "muon_scale must be finite");
    op.muon_scale = o->muon_scale;
    if (o->ns_steps < 0 || o->ns_steps > 64) return fail(h, TTT_ERR_INVALID, "ns_steps must be in 0..64");
    if (o->ns_steps) op.ns_steps = o->ns_steps;
  } else {
    op.causal = chunk > 0;
  }
  if (op.causal && c.key_norm)
    return fail(h, TTT_ERR_UNSUPPORTED,
                "key_norm with causal chunks: whole-sequence key statistics would read future keys");
  if ((inner == TTT_INNER_MLP_GELU || inner == TTT_INNER_SWIGLU) && (c.hidden < 1 || c.hidden > 512))
    return fail(h, TTT_ERR_UNSUPPORTED, "hidden must be in 1..512 (got %d)", c.hidden);
  if (is_conv(inner)) {
    if ((long long)c.grid_h * c.grid_w != c.N || c.grid_h < 1)
      return fail(h, TTT_ERR_INVALID, "the convolution needs grid_h * grid_w == N (%d x %d vs %d)", c.grid_h,
                  c.grid_w, c.N);
    if (c.conv_k != 1 && c.conv_k != 3 && c.conv_k != 5 && c.conv_k != 7)
      return fail(h, TTT_ERR_UNSUPPORTED, "conv_k must be 1, 3, 5 or 7 (got %d)", c.conv_k);
    if (chunk > 0 && chunk < c.N)
      return fail(h, TTT_ERR_UNSUPPORTED, "the convolution inner model is full batch only (chunk 0)");
    if (op.rule == RULE_MUON || c.renorm)
      return fail(h, TTT_ERR_UNSUPPORTED, "Muon and the column re-norm are defined for matrices, not convolution "
                                          "kernels");
  }
  const long long nb = chunk ? (c.N + (long long)chunk - 1) / chunk : 1;
  if (nb > 65535) return fail(h, TTT_ERR_UNSUPPORTED, "too many chunks (%lld > 65535)", nb);
  if (nb * op.epochs > (1LL << 20)) return fail(h, TTT_ERR_UNSUPPORTED, "too many updates (%lld)", nb * op.epochs);
  if (out) *out = op;
  return TTT_OK;
}

Problem make_problem(const ttt_handle* h, int loss, const Range& r) {
  const ttt_config& c = h->cfg;
  Problem pb{};
  pb.B = c.B; pb.H = r.hc; pb.N = c.N; pb.d = c.d;
  pb.Hs = c.H; pb.h0 = r.h0;
  pb.inner = r.model;
  pb.hid = (r.model == INNER_MLP || r.model == INNER_SWIGLU) ? c.hidden : c.d;
  pb.loss = loss == TTT_LOSS_MSE ? LOSS_MSE : LOSS_DOT;
  pb.nm = r.nm;
  pb.bf16 = c.dtype == TTT_BF16;
  pb.gh = c.grid_h; pb.gw = c.grid_w; pb.ck = c.conv_k;
  pb.msz = r.model == INNER_DWCONV ? (long long)c.d * c.conv_k * c.conv_k : (long long)c.d * pb.hid;
  return pb;
}

Plan make_plan(const ttt_handle* h, const Problem& pb, int chunk, const Opts& op) {
  const ttt_config& c = h->cfg;
  Plan pl{};
  pl.P = pb.B * pb.H;
  pl.nm = pb.nm;
  pl.hid = pb.hid;
  pl.chunk = chunk;
  pl.nb = chunk ? (c.N + chunk - 1) / chunk : 1;
  pl.span = chunk ? (chunk < c.N ? chunk : c.N) : c.N;
  pl.msz = pb.msz;
  pl.wsz = pb.msz * pb.nm;
  const bool generic_only = (c.flags & TTT_FLAG_FORCE_GENERIC) != 0;
  // The MFMA and LaCT kernels address every head of the tensors: a range of
  // the ViT3 split takes the generic and convolution kernels.  A chain of
  // several updates feeds each step's rounding into the next (the recurrence
  // amplifies weight perturbations), so bf16 weight operands are used for a
  // single update only; multi-step MLP gradients stay in fp32.
  const bool fast = !generic_only && pb.full_heads();
  pl.dwconv = pb.inner == INNER_DWCONV;
  pl.mfma_grad = fast && mfma_full_supported(pb) && pl.nb == 1 && op.epochs == 1;
  pl.mfma_query = fast && mfma_query_supported(pb);
  // a plain gradient step of every matrix with many pairs: the gradient
  // kernel takes whole pairs and applies the step itself (no partials, no
  // update kernel)
  if (pl.mfma_grad && op.rule == RULE_GD && !c.renorm && (op.mask & 3u) == 3u) {
    pl.mfma_one_round = mfma_grad_direct_fits(pb);
    const long long split = pl.mfma_one_round ? 0 : mfma_grad_split_pairs(pb, pl.span);
    pl.mfma_direct = split < pl.P;     // some pair is whole
    pl.mfma_split = split > 0;
    // the finite check reads the final state, which the fused readout does not write
    pl.mfma_fused_q = pl.mfma_direct && !pl.mfma_split && pl.mfma_query && !(c.flags & TTT_FLAG_CHECK_FINITE);
  }
  pl.lact_grad = fast && !c.key_norm && lact_supported(pb);
  pl.lact_query = fast && lact_readout_supported(pb);
  // the GLU kernels address pairs through Problem::row, so they also serve a
  // head range of the ViT3 split; their readout reads one state (full batch
  // or write-then-query)
  pl.glu_grad = !generic_only && glu_supported(pb) && pl.nb == 1 && op.epochs == 1;
  pl.glu_query = !generic_only && glu_supported(pb) && !op.causal;
  // key-stat slices: at most 4 workgroups per CU in total, so that all of them
  // run in one round (a partial second round would idle most of the chip)
  pl.S_stats = c.key_norm ? stats_splits(pl.P, c.N) : 0;
  if (pl.dwconv) {
    pl.S_grad = dwconv_grad_splits(pb);
  } else if (pl.glu_grad) {
    pl.S_grad = glu_grad_splits(pb, pl.span);
  } else if (pl.lact_grad) {
    pl.S_grad = lact_grad_splits(pb, pl.span);
  } else if (pl.mfma_grad) {
    int tpp_unused;
    mfma_grad_geometry(pb, pl.span, &pl.sk_G, &pl.sk_J, &tpp_unused);
    pl.S_grad = pl.sk_G * pl.sk_J;   // partial slots
    if (pl.mfma_one_round && pl.S_grad < pl.P) pl.S_grad = pl.P;   // one slot per pair
  } else {
    pl.S_grad = choose_splits((long long)pl.P * ((pb.hid + 31) / 32), pl.span, 16, 1024);
  }
  // the GELU MLP off the fused bf16 kernel (several steps, fp32 tensors):
  // the fp32 matrix-core step, or the generic kernels when the weights are not
  // 16-byte aligned (known only at the call, so both get workspace)
  pl.step_mfma = !generic_only && !pl.mfma_grad && step_mfma_shape(pb);
  pl.S_step = pl.step_mfma ? step_mfma_splits(pb, pl.span) : 0;
  size_t off = 0;
  pl.off_stats_part = off;
  if (c.key_norm) off = align256(off + sizeof(float) * (size_t)pl.P * pl.S_stats * 3 * c.d);
  pl.off_stats = off;
  if (c.key_norm) off = align256(off + sizeof(float) * (size_t)pl.P * c.d * 2);
  pl.off_states = off;
  pl.state_stride = (long long)pl.P * pl.wsz;
  off = align256(off + sizeof(float) * (size_t)pl.nb * pl.state_stride);
  pl.off_part = off;
  off = align256(off + sizeof(float) * (size_t)std::max(pl.S_grad, pl.S_step) * (pl.mfma_grad ? 1 : pl.P) * pl.wsz);
  if (pl.step_mfma) {
    const size_t td = sizeof(float) * (size_t)pl.P * pl.span * c.d, th = sizeof(float) * (size_t)pl.P * pl.span * pb.hid;
    const size_t sz[6] = {td, th, th, th, td, td};
    for (int i = 0; i < 6; ++i) {
      pl.off_step[i] = off;
      off = align256(off + sz[i]);
    }
  }
  pl.off_gbuf = off;
  if (!pl.mfma_grad && !pl.lact_grad && !pl.dwconv && !pl.glu_grad)
    off = align256(off + sizeof(float) * (size_t)pl.P * pl.span * c.d);
  pl.off_mom = off;
  if (op.rule != RULE_GD) off = align256(off + sizeof(float) * (size_t)pl.P * pl.wsz);
  pl.off_muon = off;
  if (op.rule == RULE_MUON) off = align256(off + sizeof(float) * muon_scratch_floats(pb));
  pl.off_flag = off;
  off = align256(off + 64);
  pl.total = off;
  return pl;
}

// every range's problem and plan, and the workspace they need together
struct Layout {
  int n;
  Range r[2];
  Problem pb[2];
  Plan pl[2];
  size_t base[2], total;
};

Layout make_layout(const ttt_handle* h, int loss, int inner, int chunk, const Opts& op) {
  Layout L{};
  L.n = ranges_of(h->cfg, inner, L.r);
  size_t off = 0;
  for (int i = 0; i < L.n; ++i) {
    L.pb[i] = make_problem(h, loss, L.r[i]);
    L.pl[i] = make_plan(h, L.pb[i], chunk, op);
    L.base[i] = off;
    off = align256(off + L.pl[i].total);
  }
  L.total = off;
  return L;
}

int hip_fail(ttt_handle* h, hipError_t e, const char* what) {
  return fail(h, TTT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace ttt {
int set_error(ttt_handle* h, int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int r = vfail(h, code, fmt, ap);
  va_end(ap);
  return r;
}
}  // namespace ttt

extern "C" {

int ttt_version(void) { return TTT_ABI_VERSION; }

const char* ttt_status_string(int s) {
  switch (s) {
    case TTT_OK: return "ok";
    case TTT_ERR_INVALID: return "invalid argument";
    case TTT_ERR_UNSUPPORTED: return "unsupported request";
    case TTT_ERR_HIP: return "HIP runtime error";
    case TTT_ERR_NONFINITE: return "non-finite output";
    case TTT_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int ttt_create(const ttt_config* cfg, ttt_handle** out) {
  g_create_err.clear();
  if (!out) return fail(nullptr, TTT_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(nullptr, TTT_ERR_INVALID, "cfg is NULL");
  const ttt_config& c = *cfg;
  if (c.B < 1 || c.H < 1 || c.N < 1) return fail(nullptr, TTT_ERR_INVALID, "B, H, N must be >= 1 (got %d, %d, %d)", c.B, c.H, c.N);
  if (c.d < 1 || c.d > 128) return fail(nullptr, TTT_ERR_UNSUPPORTED, "d must be in 1..128 (got %d)", c.d);
  if (c.hidden < 0) return fail(nullptr, TTT_ERR_INVALID, "hidden must be >= 0 (got %d)", c.hidden);
  if (c.grid_h < 0 || c.grid_w < 0 || c.conv_k < 0)
    return fail(nullptr, TTT_ERR_INVALID, "grid_h, grid_w and conv_k must be >= 0");
  if (c.dtype != TTT_F32 && c.dtype != TTT_BF16) return fail(nullptr, TTT_ERR_INVALID, "unknown dtype %d", c.dtype);
  if (!(c.eps >= 0.f) || !std::isfinite(c.eps)) return fail(nullptr, TTT_ERR_INVALID, "eps must be finite and >= 0");
  if (c.flags & ~(TTT_FLAG_CHECK_FINITE | TTT_FLAG_FORCE_GENERIC | TTT_FLAG_LOG))
    return fail(nullptr, TTT_ERR_INVALID, "unknown flag bits 0x%x", c.flags);
  if ((long long)c.B * c.H > 65535) return fail(nullptr, TTT_ERR_UNSUPPORTED, "B*H must be <= 65535");
  if ((long long)c.B * c.H * c.N * c.d > (1LL << 40)) return fail(nullptr, TTT_ERR_UNSUPPORTED, "tensor too large");
  ttt_handle* h = new (std::nothrow) ttt_handle;
  if (!h) return fail(nullptr, TTT_ERR_INVALID, "out of host memory");
  h->cfg = c;
  *out = h;
  return TTT_OK;
}

int ttt_set_timing_events(ttt_handle* h, void* const* events, int n_events) {
  if (!h) return fail(nullptr, TTT_ERR_INVALID, "handle is NULL");
  if (!events || n_events == 0) { h->timing = false; return TTT_OK; }
  if (n_events != 8) return fail(h, TTT_ERR_INVALID, "n_events must be 8 (got %d)", n_events);
  for (int i = 0; i < 8; ++i) h->events[i] = reinterpret_cast<hipEvent_t>(events[i]);   // NULL: skipped
  h->timing = true;
  return TTT_OK;
}

int ttt_destroy(ttt_handle* h) {
  if (h && h->side) {
    // pending work on the side stream finishes before its resources go
    (void)hipEventDestroy(h->ev_fork);
    (void)hipEventDestroy(h->ev_join);
    (void)hipStreamDestroy(h->side);
  }
  delete h;
  return TTT_OK;
}

const char* ttt_last_error(const ttt_handle* h) { return h ? h->err.c_str() : g_create_err.c_str(); }

int ttt_workspace_bytes_ex(const ttt_handle* hc, int loss, int inner, int chunk, const ttt_options* opt,
                           size_t* bytes) {
  ttt_handle* h = const_cast<ttt_handle*>(hc);
  if (!h) return fail(nullptr, TTT_ERR_INVALID, "handle is NULL");
  if (!bytes) return fail(h, TTT_ERR_INVALID, "bytes is NULL");
  Opts op;
  int rc = check_request(h, loss, inner, chunk, opt, &op);
  if (rc) return rc;
  *bytes = make_layout(h, loss, inner, chunk, op).total;
  return TTT_OK;
}

int ttt_workspace_bytes(const ttt_handle* h, int loss, int inner, int chunk, size_t* bytes) {
  return ttt_workspace_bytes_ex(h, loss, inner, chunk, nullptr, bytes);
}

const char* ttt_path_name_ex(const ttt_handle* hc, int loss, int inner, int chunk, const ttt_options* opt) {
  ttt_handle* h = const_cast<ttt_handle*>(hc);
  Opts op;
  if (!h || check_request(h, loss, inner, chunk, opt, &op)) return nullptr;
  const Layout L = make_layout(h, loss, inner, chunk, op);
  if (inner == TTT_INNER_VIT3)
    return L.n > 1 && L.pl[1].glu_grad && L.pl[1].glu_query ? "dwconv+mfma_glu" : "dwconv+generic";
  const Plan& pl = L.pl[0];
  if (pl.dwconv) return "dwconv";
  if (pl.glu_grad && pl.glu_query) return "mfma_glu";
  if (pl.glu_query) return "generic_grad+mfma_glu_query";
  if (pl.mfma_fused_q) return "mfma_fused";   // the gradient kernel also reads every pair out
  if (pl.mfma_grad && pl.mfma_query) return "mfma";
  if (pl.step_mfma) return pl.mfma_query ? "mfma_f32_grad+mfma_query" : "mfma_f32_grad";
  if (pl.mfma_query) return "generic_grad+mfma_query";
  if (pl.lact_grad && pl.lact_query) return "mfma_swiglu";
  if (pl.lact_query) return "generic_grad+mfma_swiglu_query";
  return "generic";
}

const char* ttt_path_name(const ttt_handle* h, int loss, int inner, int chunk) {
  return ttt_path_name_ex(h, loss, inner, chunk, nullptr);
}

}  // extern "C"

namespace {

struct Call {
  const void *q, *k, *v;
  void* o;
  const ttt_weights* W0;
  const ttt_eta* eta;
  const ttt_weights_out* W_out;
  int chunk;
  hipStream_t st;
};

// Enqueue every kernel of one head range:
//   key statistics (optional) -> for every update batch b (one in full-batch
//   mode, ceil(N/C) with chunks) and every epoch: gradient partials at the
//   current weights, then W_{b+1} = rule(W_b, sum of partials) [+ re-norm]
//   -> readout of every token at the state its order assigns (causal chunk c:
//   W_c; otherwise the final state).
void enqueue_range(ttt_handle* h, const Range& r, Problem pb, const Plan& pl, const Opts& op0, char* ws,
                   const Call& cl, bool timed) {
  const ttt_config& c = h->cfg;
  hipStream_t st = cl.st;
  const int chunk = cl.chunk;
  float* stats_part = reinterpret_cast<float*>(ws + pl.off_stats_part);
  float* stats = reinterpret_cast<float*>(ws + pl.off_stats);
  float* states = reinterpret_cast<float*>(ws + pl.off_states);
  float* part = reinterpret_cast<float*>(ws + pl.off_part);
  float* gbuf = reinterpret_cast<float*>(ws + pl.off_gbuf);
  float* mom = reinterpret_cast<float*>(ws + pl.off_mom);
  float* muon = reinterpret_cast<float*>(ws + pl.off_muon);
  Opts op = op0;
  op.mask = range_mask(op0.mask, r);

  pb.q = cl.q; pb.k = cl.k; pb.v = cl.v; pb.o = cl.o;
  pb.eta_scale = cl.eta->scale;
  pb.eta_tok = cl.eta->per_token;
  pb.stats = c.key_norm ? stats : nullptr;
  const int nm = r.nm;

  // the caller's W0 entries of this range's matrices, from its first head on
  WRef w0{};
  for (int i = 0; i < 3; ++i) w0.m[i] = cl.W0->w[r.slot[i < nm ? i : 0]] + (long long)r.h0 * pb.msz;
  w0.sb = cl.W0->batch_stride;
  w0.sh = pb.msz;
  float* wout[3] = {nullptr, nullptr, nullptr};
  if (cl.W_out)
    for (int i = 0; i < nm; ++i) wout[i] = cl.W_out->w[r.slot[i]];

  auto state_ref = [&](int s) -> WRef {   // s >= 1
    WRef rr{};
    float* base = states + (long long)(s - 1) * pl.state_stride;
    for (int i = 0; i < 3; ++i) rr.m[i] = base + (long long)(i < nm ? i : 0) * pb.msz;
    rr.sb = (long long)pb.H * pl.wsz;
    rr.sh = pl.wsz;
    return rr;
  };
  auto mark = [&](int i) {
    if (timed && h->timing && h->events[i]) (void)hipEventRecord(h->events[i], st);
  };
  mark(0);
  if (c.key_norm) {
    launch_stats_partial(pb, pl.S_stats, stats_part, st);
    // the MFMA and GLU gradient kernels merge the slices themselves; the
    // generic and convolution kernels read finished (mu, rstd) pairs
    if (!pl.mfma_grad && !pl.glu_grad) launch_stats_final(pb, pl.S_stats, stats_part, c.eps, stats, st);
  }
  if (op.rule != RULE_GD)      // the momentum starts at zero: a fill kernel (graph-capture safe)
    launch_fill_zero(mom, (long long)pl.P * pl.wsz, st);
  mark(1);

  // update batches in order; state b + 1 holds the weights after batch b
  bool first_step = true;
  for (int b = 0; b < pl.nb; ++b) {
    const int t0 = chunk ? b * chunk : 0;
    const int nt = chunk ? std::min(chunk, c.N - t0) : c.N;
    const WRef cur = b == 0 ? w0 : state_ref(b);
    float* next = states + (long long)b * pl.state_stride;
    const bool last_batch = b == pl.nb - 1;
    UpdateArgs ua{};
    ua.w0 = w0;
    ua.next = next;
    ua.mask = op.mask;
    ua.renorm = c.renorm;
    ua.rule = op.rule;
    ua.beta = op.beta;
    ua.mom = mom;
    ua.part_pair_stride = (long long)pl.P * pl.wsz;
    if (op.chunk_update && !op.chunk_update[b]) {
      // read-only batch: W_{b+1} = W_b (an update with no partials)
      ua.cur = cur;
      ua.part = part;
      ua.part_mode = PART_SPLITS;
      ua.S = 0;
      ua.rule = RULE_GD;
      ua.renorm = 0;
      for (int i = 0; i < 3; ++i) ua.out[i] = last_batch ? wout[i] : nullptr;
      launch_update(pb, ua, st);
      continue;
    }
    for (int e = 0; e < op.epochs; ++e) {
      // later epochs of a batch read and rewrite state b + 1 in place
      const WRef src = e == 0 ? cur : state_ref(b + 1);
      if (first_step) mark(2);
      int S_used = pl.S_grad;
      if (pl.dwconv) {
        launch_dwconv_grad(pb, src, pl.S_grad, part, st);
      } else if (pl.glu_grad) {
        launch_glu_grad(pb, src, t0, nt, pl.S_grad, c.key_norm ? stats_part : nullptr, pl.S_stats, c.eps, part, st);
      } else if (pl.lact_grad) {
        launch_lact_grad(pb, src, t0, nt, pl.S_grad, cl.eta->scale, part, st);
      } else if (pl.mfma_grad) {
        // the kernel accumulates eta_n-weighted (V_hat - V) or -eta_n V; the
        // scalar eta and the MSE constant 2/(n_b d) are applied to its partials
        const float scale = pb.loss == LOSS_MSE ? cl.eta->scale * 2.0f / ((float)nt * (float)c.d) : cl.eta->scale;
        const GradDirect gd{next, {wout[0], wout[1]}, pl.mfma_fused_q ? 1 : 0};
        launch_mfma_full_grad(pb, src, t0, nt, scale, c.key_norm ? stats_part : nullptr, pl.S_stats, c.eps, part,
                              pl.mfma_direct ? &gd : nullptr, pl.mfma_one_round, st);
      } else if (pl.step_mfma && step_mfma_aligned(src)) {
        auto sbuf = [&](int i) { return reinterpret_cast<float*>(ws + pl.off_step[i]); };
        launch_step_mfma(pb, src, t0, nt, StepMfmaBufs{sbuf(0), sbuf(1), sbuf(2), nullptr, sbuf(3), sbuf(4), sbuf(5)},
                         part, pl.S_step, st);
        S_used = pl.S_step;
      } else {
        launch_gen_grad_out(pb, src, t0, nt, gbuf, st);
        launch_gen_dW(pb, src, t0, nt, gbuf, pl.S_grad, part, st);
      }
      if (first_step) mark(3);
      if (pl.mfma_direct && !pl.mfma_split) {   // the gradient kernel has written W* (and W_out)
        if (first_step) { mark(4); mark(5); }
        first_step = false;
        continue;
      }
      ua.cur = src;
      ua.part = part;
      ua.part_mode = pl.mfma_grad ? PART_STREAMK : PART_SPLITS;
      ua.S = S_used;
      if (pl.mfma_grad) mfma_grad_geometry(pb, nt, &ua.sk_G, &ua.sk_J, &ua.sk_tpp);
      ua.sk_direct = pl.mfma_direct;
      const bool last = last_batch && e == op.epochs - 1;
      for (int i = 0; i < 3; ++i) ua.out[i] = last ? wout[i] : nullptr;
      ua.mom_only = op.rule == RULE_MUON;
      if (first_step) mark(4);
      launch_update(pb, ua, st);
      if (op.rule == RULE_MUON) {
        // W_{b+1} = W_b - s NS(M) (next already holds W_b), then the re-norm
        float* mout[3] = {nullptr, nullptr, nullptr};
        if (!c.renorm)
          for (int i = 0; i < 3; ++i) mout[i] = ua.out[i];
        launch_muon(pb, mom, next, mout, op.mask, op.muon_scale, op.ns_steps, muon, st);
        if (c.renorm) launch_renorm(pb, ua, st);
      }
      if (first_step) mark(5);
      first_step = false;
    }
  }

  mark(6);
  // causal chunks read the state their chunk starts from; otherwise every
  // query reads the final state (write-then-query)
  const float* rstates = op.causal ? states : states + (long long)(pl.nb - 1) * pl.state_stride;
  const int rchunk = op.causal ? chunk : 0;
  const int rn = op.causal ? pl.nb : 1;
  if (pl.mfma_fused_q) {
    // the gradient kernel has read every pair out
  } else if (pl.dwconv) {
    launch_dwconv_query(pb, rstates, st);
  } else if (pl.glu_query) {
    launch_glu_query(pb, rstates, st);
  } else if (pl.mfma_query) {
    launch_mfma_query(pb, w0, rstates, pl.state_stride, rn, rchunk, st);
  } else if (pl.lact_query) {
    launch_lact_readout(pb, w0, rstates, pl.state_stride, rn, rchunk, st);
  } else {
    launch_gen_query(pb, w0, rstates, pl.state_stride, rn, rchunk, st);
  }
  mark(7);
}

}  // namespace

extern "C" {

// the handle's second stream on the current device, created here when
// may_create (never from the no-alloc entry point); null: run serially
static hipStream_t side_stream(ttt_handle* h, bool may_create) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  if (h->side) return h->side_dev == dev ? h->side : nullptr;
  if (!may_create) return nullptr;
  hipStream_t s = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return nullptr;
  if (hipEventCreateWithFlags(&a, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&b, hipEventDisableTiming) != hipSuccess) {
    if (a) (void)hipEventDestroy(a);
    (void)hipStreamDestroy(s);
    return nullptr;
  }
  h->side = s;
  h->ev_fork = a;
  h->ev_join = b;
  h->side_dev = dev;
  return s;
}

static int forward_impl(ttt_handle* h, const void* q, const void* k, const void* v, const ttt_weights* W0,
                        const ttt_eta* eta, int loss, int inner, int chunk, const ttt_options* opt, void* o,
                        const ttt_weights_out* W_out, void* workspace, size_t ws_bytes, void* stream,
                        bool may_create) {
  if (!h) return fail(nullptr, TTT_ERR_INVALID, "handle is NULL");
  h->err.clear();
  Opts op;
  int rc = check_request(h, loss, inner, chunk, opt, &op);
  if (rc) return rc;
  const ttt_config& c = h->cfg;
  if (!q || !k || !v || !o) return fail(h, TTT_ERR_INVALID, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(h, TTT_ERR_INVALID, "q, k, v and o must be 16-byte aligned");
  if (!W0) return fail(h, TTT_ERR_INVALID, "W0 is NULL");
  if (!eta) return fail(h, TTT_ERR_INVALID, "eta is NULL");
  if (!std::isfinite(eta->scale)) return fail(h, TTT_ERR_INVALID, "eta scale must be finite");
  const int nm = n_mats(inner);
  for (int i = 0; i < nm; ++i)
    if (!W0->w[i]) return fail(h, TTT_ERR_INVALID, "W0.w[%d] is NULL", i);
  const Layout L = make_layout(h, loss, inner, chunk, op);
  if (inner == TTT_INNER_VIT3 && W0->batch_stride != 0)
    return fail(h, TTT_ERR_UNSUPPORTED, "the ViT3 block takes W0 shared over the batch (batch_stride 0)");
  if (W0->batch_stride != 0 && W0->batch_stride < (long long)c.H * L.pb[0].msz)
    return fail(h, TTT_ERR_INVALID, "W0.batch_stride must be 0 or >= H*in*out (%lld)", (long long)c.H * L.pb[0].msz);
  if (!workspace) return fail(h, TTT_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
  if (ws_bytes < L.total) return fail(h, TTT_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(h, TTT_ERR_INVALID, "workspace must be 256-byte aligned");

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bool log = (c.flags & TTT_FLAG_LOG) || env_log();
  if (log)
    for (int i = 0; i < L.n; ++i) {
      const Plan& pl = L.pl[i];
      std::fprintf(stderr, "[ttt] B=%d H=%d(%d..%d) N=%d d=%d h=%d %s model=%d loss=%d chunk=%d nb=%d epochs=%d "
                   "mask=0x%x %s rule=%d grad=%s(S=%d) query=%s ws=%zu\n",
                   c.B, c.H, L.r[i].h0, L.r[i].h0 + L.r[i].hc - 1, c.N, c.d, pl.hid, c.dtype == TTT_BF16 ? "bf16" : "f32",
                   L.r[i].model, loss, chunk, pl.nb, op.epochs, range_mask(op.mask, L.r[i]),
                   op.causal ? "causal" : "write-then-query", op.rule,
                   pl.dwconv ? "dwconv" : pl.glu_grad ? "mfma_glu" : pl.mfma_fused_q ? "mfma_direct+readout"
                   : pl.mfma_direct ? "mfma_direct"
                   : pl.mfma_grad ? "mfma" : pl.lact_grad ? "mfma_swiglu"
                                                                       : pl.step_mfma ? "mfma_f32" : "generic",
                   pl.S_grad,
                   pl.dwconv ? "dwconv" : pl.glu_query ? "mfma_glu" : pl.mfma_query ? "mfma" : pl.lact_query ? "mfma_swiglu"
                                                                                                             : "generic",
                   L.total);
    }

  // the head ranges of a request are independent (disjoint heads of O, their
  // own workspace regions): the smaller ones run on the handle's second
  // stream, forked from and joined back to the caller's
  hipStream_t side = L.n > 1 ? side_stream(h, may_create) : nullptr;
  // hipGetLastError is per thread and sticky: drop an error some earlier,
  // unrelated runtime call left behind so that only our launches are checked.
  (void)hipGetLastError();
  const Call cl{q, k, v, o, W0, eta, W_out, chunk, st};
  Call cl_side = cl;
  cl_side.st = side;
  int timed = 0;                 // the timing hook brackets the range with the most heads
  for (int i = 1; i < L.n; ++i)
    if (L.r[i].hc > L.r[timed].hc) timed = i;
  if (side) {
    (void)hipEventRecord(h->ev_fork, st);
    (void)hipStreamWaitEvent(side, h->ev_fork, 0);
  }
  for (int i = 0; i < L.n; ++i)
    enqueue_range(h, L.r[i], L.pb[i], L.pl[i], op, ws + L.base[i], side && i != timed ? cl_side : cl, i == timed);
  if (side) {
    (void)hipEventRecord(h->ev_join, side);
    (void)hipStreamWaitEvent(st, h->ev_join, 0);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(h, e, "kernel launch");

  if (c.flags & TTT_FLAG_CHECK_FINITE) {
    int* flag = reinterpret_cast<int*>(ws + L.base[0] + L.pl[0].off_flag);
    launch_zero_flag(flag, st);   // a fill kernel, not a memset node (graph-capture safe)
    for (int i = 0; i < L.n; ++i) {
      // O once (every head), then each range's final state (contiguous: P * wsz floats)
      Problem pb = L.pb[i];
      pb.o = o;
      const Plan& pl = L.pl[i];
      float* wf[3] = {reinterpret_cast<float*>(ws + L.base[i] + pl.off_states) + (long long)(pl.nb - 1) * pl.state_stride,
                      nullptr, nullptr};
      const long long n_out = i == 0 ? (long long)c.B * c.H * c.N * c.d : 0;
      launch_check_finite(pb, n_out, wf, (long long)pl.P * pl.wsz, flag, st);
    }
    int hflag = 0;
    e = hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, st);
    if (e != hipSuccess) return hip_fail(h, e, "hipMemcpyAsync");
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamSynchronize");
    if (hflag) return fail(h, TTT_ERR_NONFINITE, "O or the final fast weights contain NaN/Inf");
  }
  return TTT_OK;
}

int ttt_forward_ex(ttt_handle* h, const void* q, const void* k, const void* v, const ttt_weights* W0,
                   const ttt_eta* eta, int loss, int inner, int chunk, const ttt_options* opt, void* o,
                   const ttt_weights_out* W_out, void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(h, q, k, v, W0, eta, loss, inner, chunk, opt, o, W_out, workspace, ws_bytes, stream, true);
}

}  // extern "C"

namespace ttt {
int forward_no_create(ttt_handle* h, const void* q, const void* k, const void* v, const ttt_weights* W0,
                      const ttt_eta* eta, int loss, int inner, int chunk, void* o, const ttt_weights_out* W_out,
                      void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(h, q, k, v, W0, eta, loss, inner, chunk, nullptr, o, W_out, workspace, ws_bytes, stream, false);
}
}  // namespace ttt

namespace {

// workspace of the backward: the forward's statistics, W*, the split-N
// partials and G, then the backward's own buffers
struct BwdPlan {
  int P, S, S_stats, S_kn;
  long long wsz;
  size_t off_stats_part, off_stats, off_knp;
  // generic-kernel path
  size_t off_states, off_part, off_gbuf, off_U, off_dpair, off_gG, off_gF;
  // fp32-MFMA path (GELU MLP, d and h multiples of 16): region offsets in the
  // order of BwdMfmaBufs
  bool mfma_shape;
  size_t off_m[18];
  size_t total;
};

int check_backward(ttt_handle* h, int loss, int inner) {
  const ttt_config& c = h->cfg;
  if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_DOT) return fail(h, TTT_ERR_INVALID, "unknown loss %d", loss);
  if (inner < TTT_INNER_LINEAR || inner > TTT_INNER_VIT3) return fail(h, TTT_ERR_INVALID, "unknown inner model %d", inner);
  if (inner != TTT_INNER_LINEAR && inner != TTT_INNER_MLP_GELU)
    return fail(h, TTT_ERR_UNSUPPORTED, "the outer-loop backward covers the linear and GELU-MLP inner models");
  if (inner == TTT_INNER_MLP_GELU && (c.hidden < 1 || c.hidden > 512))
    return fail(h, TTT_ERR_UNSUPPORTED, "hidden must be in 1..512 (got %d)", c.hidden);
  if (c.renorm) return fail(h, TTT_ERR_UNSUPPORTED, "the outer-loop backward has no re-norm");
  return TTT_OK;
}

BwdPlan make_bwd_plan(const ttt_handle* h, const Problem& pb) {
  const ttt_config& c = h->cfg;
  BwdPlan bp{};
  bp.P = pb.B * pb.H;
  bp.wsz = pb.msz * pb.nm;
  bp.S = choose_splits((long long)bp.P * ((pb.hid + 31) / 32), c.N, 16, 1024);
  bp.S_stats = c.key_norm ? stats_splits(bp.P, c.N) : 0;
  bp.S_kn = c.key_norm ? bwd_kn_splits(pb) : 0;
  const size_t f = sizeof(float), tok = (size_t)bp.P * c.N * c.d;
  size_t off = 0;
  bp.off_stats_part = off;
  if (c.key_norm) off = align256(off + f * (size_t)bp.P * bp.S_stats * 3 * c.d);
  bp.off_stats = off;
  if (c.key_norm) off = align256(off + f * (size_t)bp.P * c.d * 2);
  bp.off_knp = off;
  if (c.key_norm) off = align256(off + f * (size_t)bp.P * bp.S_kn * 2 * c.d);
  const size_t body = off;
  // the workspace holds either path (which one runs also depends on the
  // alignment of W0, known only at the call)
  bp.off_states = off;  off = align256(off + f * (size_t)bp.P * bp.wsz);
  bp.off_part = off;    off = align256(off + f * (size_t)bp.S * bp.P * bp.wsz);
  bp.off_gbuf = off;    off = align256(off + f * tok);
  bp.off_U = off;       off = align256(off + f * (size_t)bp.P * bp.wsz);
  bp.off_dpair = off;   off = align256(off + f * (size_t)bp.P * bp.wsz);
  bp.off_gG = off;      off = align256(off + f * tok);
  bp.off_gF = off;      off = align256(off + f * tok);
  size_t total = off;
  bp.mfma_shape = pb.inner == INNER_MLP && c.d % 16 == 0 && pb.hid % 16 == 0;
  if (bp.mfma_shape) {
    BwdMfmaSizes sz;
    bwd_mfma_sizes(pb, &sz);
    const long long n[18] = {sz.tok_d, sz.tok_d, sz.tok_d, sz.tok_d, sz.tok_d, sz.tok_d,          // X Q dO G F Fd
                             sz.tok_h, sz.tok_h, sz.tok_h, sz.tok_h, sz.tok_h, sz.tok_h, sz.tok_h,  // Z A dA dZ Zd Ad Ab
                             sz.KS * sz.wsz, sz.wsz, sz.wsz, sz.wsz, 0};                            // part dW Ws U
    off = body;
    for (int i = 0; i < 18; ++i) {
      bp.off_m[i] = off;
      off = align256(off + f * (size_t)n[i]);
    }
    if (off > total) total = off;
  }
  bp.total = total;
  return bp;
}

}  // namespace

extern "C" {

int ttt_backward_workspace_bytes(const ttt_handle* hc, int loss, int inner, size_t* bytes) {
  ttt_handle* h = const_cast<ttt_handle*>(hc);
  if (!h) return fail(nullptr, TTT_ERR_INVALID, "handle is NULL");
  if (!bytes) return fail(h, TTT_ERR_INVALID, "bytes is NULL");
  int rc = check_backward(h, loss, inner);
  if (rc) return rc;
  Range r[2];
  ranges_of(h->cfg, inner, r);
  *bytes = make_bwd_plan(h, make_problem(h, loss, r[0])).total;
  return TTT_OK;
}

int ttt_backward(ttt_handle* h, const void* q, const void* k, const void* v, const ttt_weights* W0,
                 const ttt_eta* eta, int loss, int inner, const void* dO, float* dq, float* dk, float* dv,
                 const ttt_weights_out* dW0, float* deta, void* workspace, size_t ws_bytes, void* stream) {
  if (!h) return fail(nullptr, TTT_ERR_INVALID, "handle is NULL");
  h->err.clear();
  int rc = check_backward(h, loss, inner);
  if (rc) return rc;
  const ttt_config& c = h->cfg;
  if (!q || !k || !v || !dO || !dq || !dk || !dv)
    return fail(h, TTT_ERR_INVALID, "q, k, v, dO, dq, dk and dv must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return fail(h, TTT_ERR_INVALID, "q, k, v, dO, dq, dk and dv must be 16-byte aligned");
  if (!W0) return fail(h, TTT_ERR_INVALID, "W0 is NULL");
  if (!eta) return fail(h, TTT_ERR_INVALID, "eta is NULL");
  if (!std::isfinite(eta->scale)) return fail(h, TTT_ERR_INVALID, "eta scale must be finite");
  const int nm = n_mats(inner);
  for (int i = 0; i < nm; ++i)
    if (!W0->w[i]) return fail(h, TTT_ERR_INVALID, "W0.w[%d] is NULL", i);
  Range r[2];
  ranges_of(c, inner, r);
  Problem pb = make_problem(h, loss, r[0]);
  if (W0->batch_stride != 0 && W0->batch_stride < (long long)c.H * pb.msz)
    return fail(h, TTT_ERR_INVALID, "W0.batch_stride must be 0 or >= H*in*out (%lld)", (long long)c.H * pb.msz);
  const BwdPlan bp = make_bwd_plan(h, pb);
  if (!workspace) return fail(h, TTT_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", bp.total);
  if (ws_bytes < bp.total) return fail(h, TTT_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, bp.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(h, TTT_ERR_INVALID, "workspace must be 256-byte aligned");

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  auto buf = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  pb.q = q; pb.k = k; pb.v = v; pb.o = nullptr;
  pb.eta_scale = eta->scale;
  pb.eta_tok = eta->per_token;
  pb.stats = c.key_norm ? buf(bp.off_stats) : nullptr;
  WRef w0{};
  for (int i = 0; i < 3; ++i) w0.m[i] = W0->w[i < nm ? i : 0];
  w0.sb = W0->batch_stride;
  w0.sh = pb.msz;
  (void)hipGetLastError();
  // the forward's step: key statistics, G and the split-N gradient at W0, W*
  if (c.key_norm) {
    launch_stats_partial(pb, bp.S_stats, buf(bp.off_stats_part), st);
    launch_stats_final(pb, bp.S_stats, buf(bp.off_stats_part), c.eps, buf(bp.off_stats), st);
  }
  // the fp32-MFMA path recomputes the step itself from whole-pair products
  const bool use_mfma = bp.mfma_shape && bwd_mfma_supported(pb, w0);
  if (!use_mfma) {
    launch_gen_grad_out(pb, w0, 0, c.N, buf(bp.off_gbuf), st);
    launch_gen_dW(pb, w0, 0, c.N, buf(bp.off_gbuf), bp.S, buf(bp.off_part), st);
    UpdateArgs ua{};
    ua.cur = w0;
    ua.w0 = w0;
    ua.part = buf(bp.off_part);
    ua.part_mode = PART_SPLITS;
    ua.S = bp.S;
    ua.part_pair_stride = (long long)bp.P * bp.wsz;
    ua.next = buf(bp.off_states);
    ua.mask = (1u << nm) - 1;
    ua.rule = RULE_GD;
    launch_update(pb, ua, st);
  }
  // the backward
  float* dw[3] = {nullptr, nullptr, nullptr};
  if (dW0)
    for (int i = 0; i < nm; ++i) dw[i] = dW0->w[i];
  if (use_mfma) {
    BwdMfmaBufs bb;
    float** slot[17] = {&bb.X, &bb.Q, &bb.dO, &bb.G, &bb.F, &bb.Fd, &bb.Z, &bb.A, &bb.dA, &bb.dZ,
                        &bb.Zd, &bb.Ad, &bb.Ab, &bb.part, &bb.dW, &bb.Ws, &bb.U};
    for (int i = 0; i < 17; ++i) *slot[i] = buf(bp.off_m[i]);
    bb.knp = buf(bp.off_knp);
    launch_backward_mfma(pb, w0, dO, bb, dq, dk, dv, deta, dw, W0->batch_stride == 0, bp.S_kn, st);
  } else {
    launch_backward(pb, w0, buf(bp.off_states), dO, bp.S, buf(bp.off_part), buf(bp.off_gbuf), buf(bp.off_U),
                    buf(bp.off_gG), buf(bp.off_gF), buf(bp.off_dpair), buf(bp.off_knp), bp.S_kn, dq, dk, dv, deta,
                    dw, W0->batch_stride == 0, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(h, e, "kernel launch");
  return TTT_OK;
}

int ttt_forward(ttt_handle* h, const void* q, const void* k, const void* v, const ttt_weights* W0,
                const ttt_eta* eta, int loss, int inner, int chunk, void* o, const ttt_weights_out* W_out,
                void* workspace, size_t ws_bytes, void* stream) {
  return ttt_forward_ex(h, q, k, v, W0, eta, loss, inner, chunk, nullptr, o, W_out, workspace, ws_bytes, stream);
}

}  // extern "C"
