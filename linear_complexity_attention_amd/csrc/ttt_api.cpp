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

int fail(ttt_handle* h, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (h) h->err = buf; else g_create_err = buf;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int n_mats(int inner) { return inner == TTT_INNER_LINEAR ? 1 : inner == TTT_INNER_SWIGLU ? 3 : 2; }

bool env_log() {
  const char* e = std::getenv("TTT_LOG");
  return e && e[0] == '1';
}

// Where every buffer of one request lives inside the caller's workspace.
struct Plan {
  // problem
  int P, nm, hid, nb, chunk, span;   // span: tokens of the longest update batch
  long long msz, wsz;                // elements per matrix / per pair
  // choices
  bool mfma_grad, mfma_query;        // GELU-MLP MFMA kernels
  bool lact_grad, lact_query;        // SwiGLU MFMA kernels
  int S_stats, S_grad;               // S_grad: partial slots of the gradient kernel
  int sk_G, sk_J;                    // stream-K geometry (MFMA gradient kernel)
  // byte offsets
  size_t off_stats_part, off_stats, off_states, off_part, off_gbuf, off_flag, total;
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

int check_request(ttt_handle* h, int loss, int inner, int chunk) {
  const ttt_config& c = h->cfg;
  if (loss != TTT_LOSS_MSE && loss != TTT_LOSS_DOT) return fail(h, TTT_ERR_INVALID, "unknown loss %d", loss);
  if (inner != TTT_INNER_LINEAR && inner != TTT_INNER_MLP_GELU && inner != TTT_INNER_SWIGLU)
    return fail(h, TTT_ERR_INVALID, "unknown inner model %d", inner);
  if (chunk < 0) return fail(h, TTT_ERR_INVALID, "chunk must be >= 0 (got %d)", chunk);
  if (chunk > 0 && c.key_norm)
    return fail(h, TTT_ERR_UNSUPPORTED,
                "key_norm with chunk > 0: whole-sequence key statistics would read future keys");
  if (inner != TTT_INNER_LINEAR && (c.hidden < 1 || c.hidden > 512))
    return fail(h, TTT_ERR_UNSUPPORTED, "hidden must be in 1..512 (got %d)", c.hidden);
  const long long nb = chunk ? (c.N + (long long)chunk - 1) / chunk : 1;
  if (nb > 65535) return fail(h, TTT_ERR_UNSUPPORTED, "too many chunks (%lld > 65535)", nb);
  return TTT_OK;
}

Problem make_problem(const ttt_handle* h, int loss, int inner) {
  const ttt_config& c = h->cfg;
  Problem pb{};
  pb.B = c.B; pb.H = c.H; pb.N = c.N; pb.d = c.d;
  pb.hid = inner == TTT_INNER_LINEAR ? c.d : c.hidden;
  pb.inner = inner == TTT_INNER_LINEAR ? INNER_LINEAR : inner == TTT_INNER_MLP_GELU ? INNER_MLP : INNER_SWIGLU;
  pb.loss = loss == TTT_LOSS_MSE ? LOSS_MSE : LOSS_DOT;
  pb.nm = n_mats(inner);
  pb.bf16 = c.dtype == TTT_BF16;
  pb.msz = (long long)c.d * pb.hid;
  return pb;
}

Plan make_plan(const ttt_handle* h, int loss, int inner, int chunk) {
  const ttt_config& c = h->cfg;
  Problem pb = make_problem(h, loss, inner);
  Plan pl{};
  pl.P = c.B * c.H;
  pl.nm = pb.nm;
  pl.hid = pb.hid;
  pl.chunk = chunk;
  pl.nb = chunk ? (c.N + chunk - 1) / chunk : 1;
  pl.span = chunk ? (chunk < c.N ? chunk : c.N) : c.N;
  pl.msz = pb.msz;
  pl.wsz = pb.msz * pb.nm;
  const bool generic_only = (c.flags & TTT_FLAG_FORCE_GENERIC) != 0;
  // A chain of several causal updates feeds each step's rounding into the next
  // (the recurrence amplifies weight perturbations), so bf16 weight operands are
  // used for a single update only; multi-chunk MLP gradients stay in fp32.
  pl.mfma_grad = !generic_only && mfma_full_supported(pb) && pl.nb == 1;
  pl.mfma_query = !generic_only && mfma_query_supported(pb);
  pl.lact_grad = !generic_only && !c.key_norm && lact_supported(pb);
  pl.lact_query = !generic_only && lact_readout_supported(pb);
  // key-stat slices: at most 4 workgroups per CU in total, so that all of them
  // run in one round (a partial second round would idle most of the chip)
  pl.S_stats = c.key_norm ? stats_splits(pl.P, c.N) : 0;
  if (pl.lact_grad) {
    pl.S_grad = lact_grad_splits(pb, pl.span);
  } else if (pl.mfma_grad) {
    int tpp_unused;
    mfma_grad_geometry(pb, pl.span, &pl.sk_G, &pl.sk_J, &tpp_unused);
    pl.S_grad = pl.sk_G * pl.sk_J;   // partial slots
  } else {
    const int outw = inner == TTT_INNER_LINEAR ? c.d : pb.hid;
    pl.S_grad = choose_splits((long long)pl.P * ((outw + 31) / 32), pl.span, 16, 1024);
  }
  size_t off = 0;
  pl.off_stats_part = off;
  if (c.key_norm) off = align256(off + sizeof(float) * (size_t)pl.P * pl.S_stats * 3 * c.d);
  pl.off_stats = off;
  if (c.key_norm) off = align256(off + sizeof(float) * (size_t)pl.P * c.d * 2);
  pl.off_states = off;
  pl.state_stride = (long long)pl.P * pl.wsz;
  off = align256(off + sizeof(float) * (size_t)pl.nb * pl.state_stride);
  pl.off_part = off;
  off = align256(off + sizeof(float) * (size_t)pl.S_grad * (pl.mfma_grad ? 1 : pl.P) * pl.wsz);
  pl.off_gbuf = off;
  if (!pl.mfma_grad && !pl.lact_grad) off = align256(off + sizeof(float) * (size_t)pl.P * pl.span * c.d);
  pl.off_flag = off;
  off = align256(off + 64);
  pl.total = off;
  return pl;
}

int hip_fail(ttt_handle* h, hipError_t e, const char* what) {
  return fail(h, TTT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

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
  delete h;
  return TTT_OK;
}

const char* ttt_last_error(const ttt_handle* h) { return h ? h->err.c_str() : g_create_err.c_str(); }

int ttt_workspace_bytes(const ttt_handle* hc, int loss, int inner, int chunk, size_t* bytes) {
  ttt_handle* h = const_cast<ttt_handle*>(hc);
  if (!h) return fail(nullptr, TTT_ERR_INVALID, "handle is NULL");
  if (!bytes) return fail(h, TTT_ERR_INVALID, "bytes is NULL");
  int rc = check_request(h, loss, inner, chunk);
  if (rc) return rc;
  *bytes = make_plan(h, loss, inner, chunk).total;
  return TTT_OK;
}

const char* ttt_path_name(const ttt_handle* hc, int loss, int inner, int chunk) {
  ttt_handle* h = const_cast<ttt_handle*>(hc);
  if (!h || check_request(h, loss, inner, chunk)) return nullptr;
  Plan pl = make_plan(h, loss, inner, chunk);
  if (pl.mfma_grad && pl.mfma_query) return "mfma";
  if (pl.mfma_query) return "generic_grad+mfma_query";
  if (pl.lact_grad && pl.lact_query) return "mfma_swiglu";
  if (pl.lact_query) return "generic_grad+mfma_swiglu_query";
  return "generic";
}

int ttt_forward(ttt_handle* h, const void* q, const void* k, const void* v, const ttt_weights* W0,
                const ttt_eta* eta, int loss, int inner, int chunk, void* o, const ttt_weights_out* W_out,
                void* workspace, size_t ws_bytes, void* stream) {
  if (!h) return fail(nullptr, TTT_ERR_INVALID, "handle is NULL");
  h->err.clear();
  int rc = check_request(h, loss, inner, chunk);
  if (rc) return rc;
  const ttt_config& c = h->cfg;
  if (!q || !k || !v || !o) return fail(h, TTT_ERR_INVALID, "q, k, v and o must be non-NULL");
  if (!W0) return fail(h, TTT_ERR_INVALID, "W0 is NULL");
  if (!eta) return fail(h, TTT_ERR_INVALID, "eta is NULL");
  if (!std::isfinite(eta->scale)) return fail(h, TTT_ERR_INVALID, "eta scale must be finite");
  const int nm = n_mats(inner);
  for (int i = 0; i < nm; ++i)
    if (!W0->w[i]) return fail(h, TTT_ERR_INVALID, "W0.w[%d] is NULL", i);
  Problem pb = make_problem(h, loss, inner);
  if (W0->batch_stride != 0 && W0->batch_stride < (long long)c.H * pb.msz)
    return fail(h, TTT_ERR_INVALID, "W0.batch_stride must be 0 or >= H*in*out (%lld)", (long long)c.H * pb.msz);
  Plan pl = make_plan(h, loss, inner, chunk);
  if (!workspace) return fail(h, TTT_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", pl.total);
  if (ws_bytes < pl.total) return fail(h, TTT_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, pl.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(h, TTT_ERR_INVALID, "workspace must be 256-byte aligned");

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* stats_part = reinterpret_cast<float*>(ws + pl.off_stats_part);
  float* stats = reinterpret_cast<float*>(ws + pl.off_stats);
  float* states = reinterpret_cast<float*>(ws + pl.off_states);
  float* part = reinterpret_cast<float*>(ws + pl.off_part);
  float* gbuf = reinterpret_cast<float*>(ws + pl.off_gbuf);
  int* flag = reinterpret_cast<int*>(ws + pl.off_flag);

  pb.q = q; pb.k = k; pb.v = v; pb.o = o;
  pb.eta_scale = eta->scale;
  pb.eta_tok = eta->per_token;
  pb.stats = c.key_norm ? stats : nullptr;

  const bool log = (c.flags & TTT_FLAG_LOG) || env_log();
  if (log)
    std::fprintf(stderr, "[ttt] B=%d H=%d N=%d d=%d h=%d %s inner=%d loss=%d chunk=%d nb=%d grad=%s(S=%d) query=%s ws=%zu\n",
                 c.B, c.H, c.N, c.d, pb.hid, pb.bf16 ? "bf16" : "f32", inner, loss, chunk, pl.nb,
                 pl.mfma_grad ? "mfma" : pl.lact_grad ? "mfma_swiglu" : "generic", pl.S_grad,
                 pl.mfma_query ? "mfma" : pl.lact_query ? "mfma_swiglu" : "generic", pl.total);

  WRef w0{};
  for (int i = 0; i < 3; ++i) w0.m[i] = i < nm ? W0->w[i] : W0->w[0];
  w0.sb = W0->batch_stride;
  w0.sh = pb.msz;

  auto state_ref = [&](int s) -> WRef {   // s >= 1
    WRef r{};
    float* base = states + (long long)(s - 1) * pl.state_stride;
    for (int i = 0; i < 3; ++i) r.m[i] = base + (long long)(i < nm ? i : 0) * pb.msz;
    r.sb = (long long)c.H * pl.wsz;
    r.sh = pl.wsz;
    return r;
  };

  // hipGetLastError is per thread and sticky: drop an error some earlier,
  // unrelated runtime call left behind so that only our launches are judged.
  (void)hipGetLastError();
  auto mark = [&](int i) {
    if (h->timing && h->events[i]) (void)hipEventRecord(h->events[i], st);
  };
  mark(0);
  if (c.key_norm) {
    launch_stats_partial(pb, pl.S_stats, stats_part, st);
    // the MFMA gradient kernel merges the slices itself; the generic kernels
    // read finished (mu, rstd) pairs
    if (!pl.mfma_grad) launch_stats_final(pb, pl.S_stats, stats_part, c.eps, stats, st);
  }
  mark(1);

  for (int b = 0; b < pl.nb; ++b) {
    const int t0 = chunk ? b * chunk : 0;
    const int nt = chunk ? std::min(chunk, c.N - t0) : c.N;
    const WRef cur = b == 0 ? w0 : state_ref(b);
    if (b == 0) mark(2);
    if (pl.lact_grad) {
      launch_lact_grad(pb, cur, t0, nt, pl.S_grad, eta->scale, part, st);
    } else if (pl.mfma_grad) {
      // the kernel accumulates eta_n-weighted (V_hat - V) or -eta_n V; the
      // scalar eta and the MSE constant 2/(n_b d) are applied to its partials
      const float scale = pb.loss == LOSS_MSE ? eta->scale * 2.0f / ((float)nt * (float)c.d) : eta->scale;
      launch_mfma_full_grad(pb, cur, t0, nt, scale, c.key_norm ? stats_part : nullptr, pl.S_stats, c.eps, part, st);
    } else {
      launch_gen_grad_out(pb, cur, t0, nt, gbuf, st);
      launch_gen_dW(pb, cur, t0, nt, gbuf, pl.S_grad, part, st);
    }
    if (b == 0) mark(3);
    UpdateArgs ua{};
    ua.cur = cur;
    ua.w0 = w0;
    ua.part = part;
    ua.part_mode = pl.mfma_grad ? PART_STREAMK : PART_SPLITS;
    ua.S = pl.S_grad;
    ua.part_pair_stride = (long long)pl.P * pl.wsz;
    if (pl.mfma_grad) mfma_grad_geometry(pb, nt, &ua.sk_G, &ua.sk_J, &ua.sk_tpp);
    ua.next = states + (long long)b * pl.state_stride;
    const bool last = b == pl.nb - 1;
    for (int i = 0; i < 3; ++i) ua.out[i] = (last && W_out && i < nm) ? W_out->w[i] : nullptr;
    ua.renorm = c.renorm;
    if (b == 0) mark(4);
    launch_update(pb, ua, st);
    if (b == 0) mark(5);
  }

  mark(6);
  if (pl.mfma_query) {
    launch_mfma_query(pb, w0, states, pl.state_stride, chunk ? pl.nb : 1, chunk, st);
  } else if (pl.lact_query) {
    launch_lact_readout(pb, w0, states, pl.state_stride, chunk ? pl.nb : 1, chunk, st);
  } else {
    launch_gen_query(pb, w0, states, pl.state_stride, chunk ? pl.nb : 1, chunk, st);
  }
  mark(7);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(h, e, "kernel launch");

  if (c.flags & TTT_FLAG_CHECK_FINITE) {
    launch_zero_flag(flag, st);   // a fill kernel, not a memset node (graph-capture safe)
    float* wf[3] = {nullptr, nullptr, nullptr};
    float* last = states + (long long)(pl.nb - 1) * pl.state_stride;
    wf[0] = last;   // the final state is contiguous: P * wsz floats
    launch_check_finite(pb, wf, (long long)pl.P * pl.wsz, flag, st);
    int hflag = 0;
    e = hipMemcpyAsync(&hflag, flag, sizeof(int), hipMemcpyDeviceToHost, st);
    if (e != hipSuccess) return hip_fail(h, e, "hipMemcpyAsync");
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamSynchronize");
    if (hflag) return fail(h, TTT_ERR_NONFINITE, "O or the final fast weights contain NaN/Inf");
  }
  return TTT_OK;
}

}  // extern "C"
