// C-ABI of the Kimi K3 LatentMoE layer forward (declarations and contract in include/k3moe.h).
//
// Stage order of one forward (Kimi K3 course, lesson 6 "LatentMoE", eq. 11 and eq. 13):
//   x_gemm   one pass over x for every x-consumer: router logits -> sigmoid scores,
//            W_down x -> z (bf16 or MXFP8), shared GLU hiddens -> bf16
//   topk     argtopk(s + b) and p renormalised from s
//   route    counts / offsets / expert-contiguous row order (replaces the expert-parallel
//            all-to-all dispatch with an on-device gather)
//   gateup   grouped GLU gate/up over the dispatched rows, SiLU(gate) * up -> h
//   down     grouped GLU down -> expert outputs O
//   combine  u = sum_j p_j O, RMSNorm -> n (latent) or u (full width)
//   y_gemm   y = [n | shared hiddens] [W_up | shared downs]^T   (or shared downs + u)
#include "../../include/k3moe.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "k3moe_internal.h"

using namespace k3;

namespace {

enum Stage { ST_X = 0, ST_TOPK, ST_ROUTE, ST_GATEUP, ST_DOWN, ST_COMBINE, ST_Y, ST_COUNT };
const char* kStageNames[ST_COUNT] = {"x_gemm", "topk", "route", "gateup", "down", "combine", "y_gemm"};

thread_local std::string g_create_error;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

struct k3moe_ctx {
  k3moe_config cfg;
  int le = 0;  // width the routed experts work in
  // packed layout
  int x_wwin = 0, x_P = 0, x_P_router = 0, x_P_down = 0, x_P_sh = 0;
  int y_K = 0, y_wwin = 0, y_P = 0;
  int gu_wwin = 0, gu_P = 0, dn_wwin = 0, dn_P = 0;
  size_t off_x = 0, off_y = 0, off_gu = 0, off_dn = 0, off_bias = 0, off_gamma = 0, total = 0;
  size_t gu_stride = 0, dn_stride = 0;
  // workspace layout (for max_tokens)
  size_t ws_scores = 0, ws_idx = 0, ws_p = 0, ws_counts = 0, ws_offsets = 0, ws_perm = 0, ws_inv = 0, ws_route = 0;
  size_t ws_z = 0, ws_zs = 0, ws_h = 0, ws_hs = 0, ws_o = 0, ws_abuf = 0, ws_u = 0, ws_partial = 0, ws_items = 0;
  size_t ws_total = 0;
  bool use_items = false;  // grouped row-tiled launches walk a work-item list (persistent grid)
  // state
  uint8_t* packed = nullptr;
  bool dense_packed = false;
  std::vector<uint8_t> routed_packed;
  int n_routed_packed = 0;
  std::string err;
  // profiling
  int prof_max = 0, prof_calls = 0;
  std::vector<hipEvent_t> events;  // [prof_max][ST_COUNT][2]
};

static int fail(k3moe_ctx* c, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c)
    c->err = buf;
  else
    g_create_error = buf;
  return code;
}

static int hip_fail(k3moe_ctx* c, hipError_t e, const char* what) {
  return fail(c, K3MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCHECK(c, expr, what)                 \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return hip_fail(c, e_, what); \
  } while (0)

extern "C" {

int32_t k3moe_stage_count(void) { return ST_COUNT; }

const char* k3moe_stage_name(int32_t stage) {
  return (stage >= 0 && stage < ST_COUNT) ? kStageNames[stage] : "";
}

const char* k3moe_last_error(const k3moe_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_create_error.c_str();
}

int k3moe_create(const k3moe_config* cfg, k3moe_ctx** out) {
  if (!out) return fail(nullptr, K3MOE_EINVAL, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(nullptr, K3MOE_EINVAL, "cfg is NULL");
  const k3moe_config& c = *cfg;
  if (c.latent_moe != 0 && c.latent_moe != 1) return fail(nullptr, K3MOE_EINVAL, "latent_moe must be 0 or 1");
  const int le = c.latent_moe ? c.latent : c.d_model;
  if (c.d_model <= 0 || c.d_model % 32 || le <= 0 || le % 32 || c.hidden <= 0 || c.hidden % 32)
    return fail(nullptr, K3MOE_EINVAL, "d_model, latent and hidden must be positive multiples of 32");
  if (c.n_shared < 0 || c.n_shared > 4) return fail(nullptr, K3MOE_EINVAL, "n_shared must be in [0, 4]");
  if (c.n_shared > 0 && (c.shared_hidden <= 0 || c.shared_hidden % 32))
    return fail(nullptr, K3MOE_EINVAL, "shared_hidden must be a positive multiple of 32");
  if (c.n_experts < 1 || c.n_experts > 2048) return fail(nullptr, K3MOE_EINVAL, "n_experts must be in [1, 2048]");
  if (c.top_k < 1 || c.top_k > c.n_experts || c.top_k > 64)
    return fail(nullptr, K3MOE_EINVAL, "top_k must be in [1, min(n_experts, 64)]");
  if (c.act != K3MOE_ACT_BF16 && c.act != K3MOE_ACT_MXFP8) return fail(nullptr, K3MOE_EINVAL, "unknown act");
  if (c.max_tokens < 1) return fail(nullptr, K3MOE_EINVAL, "max_tokens must be >= 1");
  if ((int64_t)c.max_tokens * c.top_k > (int64_t)1 << 30)
    return fail(nullptr, K3MOE_ETOOBIG, "max_tokens * top_k too large");
  if (le > 8192) return fail(nullptr, K3MOE_EUNSUPPORTED, "expert width above 8192");
  {
    // every GEMM operand must stay addressable by a 32-bit buffer offset
    const int64_t T = c.max_tokens, lim = ((int64_t)1 << 31) - ((int64_t)1 << 25);
    const int64_t yk = (c.latent_moe ? le : 0) + (int64_t)c.n_shared * c.shared_hidden;
    const int64_t worst = std::max({T * c.d_model * 2, T * c.top_k * c.hidden * 2, T * yk * 2, T * le * 2});
    if (worst > lim) return fail(nullptr, K3MOE_ETOOBIG, "max_tokens too large: an operand exceeds 2 GiB");
  }
  if (!(c.rms_eps >= 0.0f)) return fail(nullptr, K3MOE_EINVAL, "rms_eps must be >= 0");

  k3moe_ctx* x = new k3moe_ctx();
  x->cfg = c;
  x->le = le;
  const int d = c.d_model, l = c.latent, h = c.hidden, E = c.n_experts, Ns = c.n_shared, hs = c.shared_hidden;
  // x-consumer group: router panels, W_down panels (latent), shared GLU panels; K = d
  x->x_P_router = (int)ceil_div(E, kPanelRows);
  x->x_P_down = c.latent_moe ? (int)ceil_div(l, kPanelRows) : 0;
  x->x_P_sh = Ns > 0 ? (int)ceil_div(hs, 32) : 0;
  x->x_P = x->x_P_router + x->x_P_down + Ns * x->x_P_sh;
  x->x_wwin = (int)ceil_div(d, kWinK);
  // output group: [W_up | shared downs] (latent) or [shared downs] (full width); N = d
  x->y_K = (c.latent_moe ? l : 0) + Ns * hs;
  x->y_wwin = (int)ceil_div(x->y_K, kWinK);
  x->y_P = x->y_K > 0 ? (int)ceil_div(d, kPanelRows) : 0;
  // routed experts
  x->gu_P = h / 32;
  x->gu_wwin = (int)ceil_div(le, kWinK);
  x->dn_P = (int)ceil_div(le, kPanelRows);
  x->dn_wwin = (int)ceil_div(h, kWinK);
  x->gu_stride = (size_t)x->gu_P * x->gu_wwin * kPanelWinBytes;
  x->dn_stride = (size_t)x->dn_P * x->dn_wwin * kPanelWinBytes;
  size_t o = 0;
  x->off_gu = o;
  o += align256(x->gu_stride * E);
  x->off_dn = o;
  o += align256(x->dn_stride * E);
  x->off_x = o;
  o += align256((size_t)x->x_P * x->x_wwin * kPanelWinBytes);
  x->off_y = o;
  o += align256((size_t)x->y_P * x->y_wwin * kPanelWinBytes);
  x->off_bias = o;
  o += align256(sizeof(float) * E);
  x->off_gamma = o;
  o += align256(sizeof(float) * (c.latent_moe ? l : 1));
  x->total = o;
  // workspace
  const size_t T = c.max_tokens, k = c.top_k;
  size_t w = 0;
  auto take = [&](size_t bytes) {
    size_t at = w;
    w += align256(bytes);
    return at;
  };
  x->ws_scores = take(4 * T * E);
  x->ws_idx = take(4 * T * k);
  x->ws_p = take(4 * T * k);
  x->ws_counts = take(4 * (size_t)E);
  x->ws_offsets = take(4 * ((size_t)E + 1));
  x->ws_perm = take(4 * T * k);
  x->ws_inv = take(4 * T * k);
  x->ws_route = take((size_t)route_scratch_bytes(c.max_tokens, c.n_experts));
  const bool f8 = c.act == K3MOE_ACT_MXFP8;
  if (c.latent_moe) {
    x->ws_z = take((f8 ? 1 : 2) * T * l);
    x->ws_zs = take(f8 ? T * l / 32 : 0);
  }
  x->ws_h = take((f8 ? 1 : 2) * T * k * h);
  x->ws_hs = take(f8 ? T * k * h / 32 : 0);
  x->ws_o = take(4 * T * k * le);
  x->ws_abuf = take(2 * T * (size_t)x->y_K);
  x->ws_u = take(4 * T * le);
  x->ws_partial = take((size_t)gemm_partial_bytes());
  const int nblk_max = (int)std::max(ceil_div(x->gu_P, 4), ceil_div(x->dn_P, 4));
  x->use_items = tile_items_fit(c.max_tokens, E, nblk_max);
  x->ws_items = take(x->use_items ? (size_t)tile_items_bytes((int64_t)T * k, E, nblk_max) : 0);
  x->ws_total = w;
  x->routed_packed.assign(E, 0);
  *out = x;
  return K3MOE_OK;
}

void k3moe_destroy(k3moe_ctx* ctx) {
  if (!ctx) return;
  for (hipEvent_t e : ctx->events) (void)hipEventDestroy(e);
  delete ctx;
}

size_t k3moe_weight_bytes(const k3moe_ctx* ctx) { return ctx ? ctx->total : 0; }

size_t k3moe_workspace_bytes(const k3moe_ctx* ctx) { return ctx ? ctx->ws_total : 0; }

static bool mx_ok(const k3moe_mx& m) { return m.codes && m.scales; }

int k3moe_pack_weights(k3moe_ctx* ctx, const k3moe_weights* wts, void* packed_dev, void* stream) {
  if (!ctx) return K3MOE_EINVAL;
  if (!wts || !packed_dev) return fail(ctx, K3MOE_EINVAL, "weights or packed buffer is NULL");
  if ((uintptr_t)packed_dev % 256) return fail(ctx, K3MOE_EINVAL, "packed buffer must be 256-byte aligned");
  if (ctx->packed && ctx->packed != packed_dev)
    return fail(ctx, K3MOE_EINVAL, "packed buffer differs from the one bound by the first pack call");
  const k3moe_config& c = ctx->cfg;
  const int d = c.d_model, l = c.latent, h = c.hidden, E = c.n_experts, Ns = c.n_shared, hs = c.shared_hidden;
  const int le = ctx->le;
  hipStream_t s = (hipStream_t)stream;
  // validate everything before enqueuing anything
  if (wts->include_dense) {
    if (!mx_ok(wts->w_router) || !wts->router_bias) return fail(ctx, K3MOE_EINVAL, "router weights missing");
    if (c.latent_moe && (!mx_ok(wts->w_down) || !mx_ok(wts->w_up) || !wts->rms_gamma))
      return fail(ctx, K3MOE_EINVAL, "W_down, W_up or rms_gamma missing");
    if (Ns > 0) {
      if (!wts->sh_gate || !wts->sh_up || !wts->sh_down) return fail(ctx, K3MOE_EINVAL, "shared experts missing");
      for (int j = 0; j < Ns; ++j)
        if (!mx_ok(wts->sh_gate[j]) || !mx_ok(wts->sh_up[j]) || !mx_ok(wts->sh_down[j]))
          return fail(ctx, K3MOE_EINVAL, "shared expert %d has a NULL matrix", j);
    }
  }
  if (wts->routed_count < 0 || wts->routed_first < 0 || wts->routed_first + wts->routed_count > E)
    return fail(ctx, K3MOE_EINVAL, "routed expert range [%d, %d) outside [0, %d)", wts->routed_first,
                wts->routed_first + wts->routed_count, E);
  if (wts->routed_count > 0) {
    if (!wts->gate || !wts->up || !wts->down) return fail(ctx, K3MOE_EINVAL, "routed expert arrays missing");
    for (int i = 0; i < wts->routed_count; ++i)
      if (!mx_ok(wts->gate[i]) || !mx_ok(wts->up[i]) || !mx_ok(wts->down[i]))
        return fail(ctx, K3MOE_EINVAL, "routed expert %d has a NULL matrix", wts->routed_first + i);
  }
  ctx->packed = (uint8_t*)packed_dev;
  uint8_t* P = ctx->packed;
  auto src = [](const k3moe_mx& m, int N, int K) {
    PackSrc s;
    s.codes = (const uint8_t*)m.codes;
    s.scales = (const uint8_t*)m.scales;
    s.N = N;
    s.K = K;
    return s;
  };
  if (wts->include_dense) {
    PackJob j{};
    j.dst = P + ctx->off_x;
    j.wwin = ctx->x_wwin;
    j.p_off = 0;
    j.P = ctx->x_P_router;
    j.nseg = 1;
    j.src[0] = src(wts->w_router, E, d);
    HIPCHECK(ctx, launch_pack(j, s), "pack router");
    if (c.latent_moe) {
      j.p_off = ctx->x_P_router;
      j.P = ctx->x_P_down;
      j.src[0] = src(wts->w_down, l, d);
      HIPCHECK(ctx, launch_pack(j, s), "pack W_down");
    }
    for (int js = 0; js < Ns; ++js) {
      PackJob g{};
      g.dst = P + ctx->off_x;
      g.wwin = ctx->x_wwin;
      g.p_off = ctx->x_P_router + ctx->x_P_down + js * ctx->x_P_sh;
      g.P = ctx->x_P_sh;
      g.glu = 1;
      g.src[0] = src(wts->sh_gate[js], hs, d);
      g.src[1] = src(wts->sh_up[js], hs, d);
      HIPCHECK(ctx, launch_pack(g, s), "pack shared gate/up");
    }
    if (ctx->y_P > 0) {
      PackJob y{};
      y.dst = P + ctx->off_y;
      y.wwin = ctx->y_wwin;
      y.p_off = 0;
      y.P = ctx->y_P;
      int kb = 0, n = 0;
      if (c.latent_moe) {
        y.src[n] = src(wts->w_up, d, l);
        y.kb0[n++] = kb;
        kb += l / 32;
      }
      for (int js = 0; js < Ns; ++js) {
        y.src[n] = src(wts->sh_down[js], d, hs);
        y.kb0[n++] = kb;
        kb += hs / 32;
      }
      y.nseg = n;
      HIPCHECK(ctx, launch_pack(y, s), "pack output projection");
    }
    HIPCHECK(ctx, hipMemcpyAsync(P + ctx->off_bias, wts->router_bias, sizeof(float) * E, hipMemcpyDeviceToDevice, s),
             "copy router bias");
    if (c.latent_moe)
      HIPCHECK(ctx,
               hipMemcpyAsync(P + ctx->off_gamma, wts->rms_gamma, sizeof(float) * l, hipMemcpyDeviceToDevice, s),
               "copy rms gamma");
    ctx->dense_packed = true;
  }
  for (int i = 0; i < wts->routed_count; ++i) {
    const int e = wts->routed_first + i;
    PackJob g{};
    g.dst = P + ctx->off_gu + ctx->gu_stride * e;
    g.wwin = ctx->gu_wwin;
    g.P = ctx->gu_P;
    g.glu = 1;
    g.src[0] = src(wts->gate[i], h, le);
    g.src[1] = src(wts->up[i], h, le);
    HIPCHECK(ctx, launch_pack(g, s), "pack routed gate/up");
    PackJob dn{};
    dn.dst = P + ctx->off_dn + ctx->dn_stride * e;
    dn.wwin = ctx->dn_wwin;
    dn.P = ctx->dn_P;
    dn.nseg = 1;
    dn.src[0] = src(wts->down[i], le, h);
    HIPCHECK(ctx, launch_pack(dn, s), "pack routed down");
    if (!ctx->routed_packed[e]) {
      ctx->routed_packed[e] = 1;
      ctx->n_routed_packed++;
    }
  }
  return K3MOE_OK;
}

int k3moe_quantile_bias(k3moe_ctx* ctx, const float* scores_dev, int32_t T, float* bias_dev, void* stream) {
  if (!ctx) return K3MOE_EINVAL;
  if (!scores_dev || !bias_dev) return fail(ctx, K3MOE_EINVAL, "scores and bias must be non-null");
  if (T < 1 || T > 16384) return fail(ctx, K3MOE_ETOOBIG, "calibration batch T = %d outside [1, 16384]", T);
  const int64_t E = ctx->cfg.n_experts, k = ctx->cfg.top_k;
  const int m = (int)std::min<int64_t>(T, std::max<int64_t>(1, (2 * (int64_t)T * k + E) / (2 * E)));
  HIPCHECK(ctx, launch_quantile_bias(scores_dev, T, (int)E, m, bias_dev, (hipStream_t)stream), "quantile bias launch");
  return K3MOE_OK;
}

int k3moe_profile_begin(k3moe_ctx* ctx, int32_t max_calls) {
  if (!ctx) return K3MOE_EINVAL;
  if (max_calls < 1 || max_calls > 100000) return fail(ctx, K3MOE_EINVAL, "max_calls must be in [1, 100000]");
  const size_t need = (size_t)max_calls * ST_COUNT * 2;
  while (ctx->events.size() < need) {
    hipEvent_t e;
    HIPCHECK(ctx, hipEventCreate(&e), "hipEventCreate");
    ctx->events.push_back(e);
  }
  ctx->prof_max = max_calls;
  ctx->prof_calls = 0;
  return K3MOE_OK;
}

int k3moe_profile_end(k3moe_ctx* ctx, float* ms, int32_t n_stages, int32_t* calls) {
  if (!ctx) return K3MOE_EINVAL;
  if (!ms || n_stages < ST_COUNT) return fail(ctx, K3MOE_EINVAL, "ms must hold %d stages", (int)ST_COUNT);
  for (int st = 0; st < ST_COUNT; ++st) ms[st] = 0.0f;
  const int n = ctx->prof_calls;
  ctx->prof_max = 0;
  ctx->prof_calls = 0;
  for (int c = 0; c < n; ++c) {
    for (int st = 0; st < ST_COUNT; ++st) {
      hipEvent_t a = ctx->events[(c * ST_COUNT + st) * 2], b = ctx->events[(c * ST_COUNT + st) * 2 + 1];
      HIPCHECK(ctx, hipEventSynchronize(b), "hipEventSynchronize");
      float t = 0.0f;
      HIPCHECK(ctx, hipEventElapsedTime(&t, a, b), "hipEventElapsedTime");
      ms[st] += t;
    }
  }
  if (calls) *calls = n;
  return K3MOE_OK;
}

int k3moe_forward_ex(k3moe_ctx* ctx, const void* x_dev, int32_t T, void* y_dev, void* workspace_dev, void* stream,
                     const k3moe_taps* taps) {
  if (!ctx) return K3MOE_EINVAL;
  const k3moe_config& c = ctx->cfg;
  if (T < 0) return fail(ctx, K3MOE_EINVAL, "T must be >= 0");
  if (T > c.max_tokens) return fail(ctx, K3MOE_ETOOBIG, "T = %d above max_tokens = %d", T, c.max_tokens);
  if (!ctx->dense_packed || ctx->n_routed_packed != c.n_experts)
    return fail(ctx, K3MOE_ESTATE, "weights not packed (dense: %d, routed experts: %d of %d)", (int)ctx->dense_packed,
                ctx->n_routed_packed, c.n_experts);
  if (T == 0) return K3MOE_OK;
  if (!x_dev || !y_dev || !workspace_dev) return fail(ctx, K3MOE_EINVAL, "x, y or workspace is NULL");
  if ((uintptr_t)workspace_dev % 256) return fail(ctx, K3MOE_EINVAL, "workspace must be 256-byte aligned");
  if ((uintptr_t)x_dev % 16 || (uintptr_t)y_dev % 16) return fail(ctx, K3MOE_EINVAL, "x and y must be 16-byte aligned");
  if (x_dev == y_dev) return fail(ctx, K3MOE_EINVAL, "y may not alias x");

  hipStream_t s = (hipStream_t)stream;
  const int d = c.d_model, l = c.latent, h = c.hidden, E = c.n_experts, k = c.top_k, Ns = c.n_shared,
            hs = c.shared_hidden;
  const int le = ctx->le;
  const bool f8 = c.act == K3MOE_ACT_MXFP8;
  uint8_t* ws = (uint8_t*)workspace_dev;
  float* scores = (float*)(ws + ctx->ws_scores);
  int32_t* idx = (int32_t*)(ws + ctx->ws_idx);
  float* p = (float*)(ws + ctx->ws_p);
  int32_t* counts = (int32_t*)(ws + ctx->ws_counts);
  int32_t* offsets = (int32_t*)(ws + ctx->ws_offsets);
  int32_t* perm = (int32_t*)(ws + ctx->ws_perm);
  int32_t* inv = (int32_t*)(ws + ctx->ws_inv);
  uint8_t* z = ws + ctx->ws_z;
  uint8_t* zs = ws + ctx->ws_zs;
  uint8_t* H = ws + ctx->ws_h;
  uint8_t* Hs = ws + ctx->ws_hs;
  float* O = (float*)(ws + ctx->ws_o);
  uint16_t* abuf = (uint16_t*)(ws + ctx->ws_abuf);
  float* u = (float*)(ws + ctx->ws_u);
  const uint8_t* P = ctx->packed;
  const float* bias = (const float*)(P + ctx->off_bias);
  const float* gamma = (const float*)(P + ctx->off_gamma);

  const bool prof = ctx->prof_calls < ctx->prof_max;
  hipEvent_t* ev = prof ? &ctx->events[(size_t)ctx->prof_calls * ST_COUNT * 2] : nullptr;
  auto mark = [&](int st, int end) -> hipError_t {
    return prof ? hipEventRecord(ev[st * 2 + end], s) : hipSuccess;
  };

  // ---- x_gemm
  {
    GemmArgs a{};
    a.W = P + ctx->off_x;
    a.P = ctx->x_P;
    a.wwin = ctx->x_wwin;
    a.K = d;
    a.a_fmt = A_BF16;
    a.A = x_dev;
    a.lda = d;
    a.a_bytes = (int64_t)T * d * 2;
    a.M = T;
    int n = 0;
    EpiSeg& r = a.seg[n++];
    r.p0 = 0;
    r.p1 = ctx->x_P_router;
    r.mode = EPI_SIGMOID;
    r.ncols = E;
    r.out = scores;
    r.ldo = E;
    if (c.latent_moe) {
      EpiSeg& zg = a.seg[n++];
      zg.p0 = ctx->x_P_router;
      zg.p1 = ctx->x_P_router + ctx->x_P_down;
      zg.mode = f8 ? EPI_MXFP8 : EPI_BF16;
      zg.ncols = l;
      zg.out = z;
      zg.ldo = l;
      zg.out_scales = zs;
      zg.ldos = l / 32;
      if (taps && taps->z_f32) {
        zg.pre = taps->z_f32;
        zg.ldpre = l;
      }
    }
    for (int js = 0; js < Ns; ++js) {
      EpiSeg& sg = a.seg[n++];
      sg.p0 = ctx->x_P_router + ctx->x_P_down + js * ctx->x_P_sh;
      sg.p1 = sg.p0 + ctx->x_P_sh;
      sg.mode = EPI_SWIGLU_BF16;
      sg.ncols = hs;
      sg.out = abuf;
      sg.ldo = ctx->y_K;
      sg.col0 = (c.latent_moe ? l : 0) + js * hs;
    }
    a.nseg = n;
    HIPCHECK(ctx, mark(ST_X, 0), "event");
    a.partial = (float*)(ws + ctx->ws_partial);
    a.partial_bytes = gemm_partial_bytes();
    HIPCHECK(ctx, launch_panel_gemm(a, GEMM_X, s), "x_gemm launch");
    HIPCHECK(ctx, mark(ST_X, 1), "event");
  }
  // ---- topk
  HIPCHECK(ctx, mark(ST_TOPK, 0), "event");
  HIPCHECK(ctx, launch_topk(scores, bias, T, E, k, idx, p, s), "topk launch");
  HIPCHECK(ctx, mark(ST_TOPK, 1), "event");
  // ---- route
  HIPCHECK(ctx, mark(ST_ROUTE, 0), "event");
  HIPCHECK(ctx, launch_route(idx, T, E, k, counts, offsets, perm, inv, (int32_t*)(ws + ctx->ws_route), s),
           "route launch");
  HIPCHECK(ctx, mark(ST_ROUTE, 1), "event");
  // Which experts take the row-tiled GEMMs (whole 128-wide K windows, so both reduction widths must be
  // multiples of 128): with 32 or more rows per expert on average, all; with 8 or more, those with at
  // least 16 rows (the panel kernel, one pass per 16 rows, takes the rest: a skewed load puts hot
  // experts on the tiled kernel); with fewer (decode), none.
  int row_split = 0;
  if (le % 128 == 0 && h % 128 == 0) {
    if ((int64_t)T * k >= (int64_t)32 * E)
      row_split = 1;
    else if ((int64_t)T * k >= (int64_t)8 * E)
      row_split = 16;
  }
  // ---- gateup
  {
    GemmArgs a{};
    a.W = P + ctx->off_gu;
    a.w_group_stride = (int64_t)ctx->gu_stride;
    a.P = ctx->gu_P;
    a.wwin = ctx->gu_wwin;
    a.K = le;
    if (c.latent_moe) {
      a.a_fmt = f8 ? A_MXFP8 : A_BF16;
      a.A = z;
      a.lda = l;
      a.a_bytes = (int64_t)T * l * (f8 ? 1 : 2);
      a.A_scales = zs;
      a.ldas = l / 32;
      a.as_bytes = (int64_t)T * (l / 32);
    } else {
      a.a_fmt = A_BF16;
      a.A = x_dev;
      a.lda = d;
      a.a_bytes = (int64_t)T * d * 2;
    }
    a.rowmap = perm;
    a.offsets = offsets;
    a.n_groups = E;
    a.row_split = row_split;
    a.items = ctx->use_items ? (int32_t*)(ws + ctx->ws_items) : nullptr;
    EpiSeg& sg = a.seg[0];
    sg.p0 = 0;
    sg.p1 = ctx->gu_P;
    sg.mode = f8 ? EPI_SWIGLU_MXFP8 : EPI_SWIGLU_BF16;
    sg.ncols = h;
    sg.out = H;
    sg.ldo = h;
    sg.out_scales = Hs;
    sg.ldos = h / 32;
    if (taps && taps->h_f32) {
      sg.pre = taps->h_f32;
      sg.ldpre = h;
    }
    a.nseg = 1;
    HIPCHECK(ctx, mark(ST_GATEUP, 0), "event");
    HIPCHECK(ctx, launch_panel_gemm(a, GEMM_GATEUP, s), "gateup launch");
    HIPCHECK(ctx, mark(ST_GATEUP, 1), "event");
  }
  // ---- down
  {
    GemmArgs a{};
    a.W = P + ctx->off_dn;
    a.w_group_stride = (int64_t)ctx->dn_stride;
    a.P = ctx->dn_P;
    a.wwin = ctx->dn_wwin;
    a.K = h;
    a.a_fmt = f8 ? A_MXFP8 : A_BF16;
    a.A = H;
    a.lda = h;
    a.a_bytes = (int64_t)T * k * h * (f8 ? 1 : 2);
    a.A_scales = Hs;
    a.ldas = h / 32;
    a.as_bytes = (int64_t)T * k * (h / 32);
    a.offsets = offsets;
    a.n_groups = E;
    a.row_split = row_split;
    a.items = ctx->use_items ? (int32_t*)(ws + ctx->ws_items) : nullptr;
    EpiSeg& sg = a.seg[0];
    sg.p0 = 0;
    sg.p1 = ctx->dn_P;
    sg.mode = EPI_F32;
    sg.ncols = le;
    sg.out = O;
    sg.ldo = le;
    a.nseg = 1;
    HIPCHECK(ctx, mark(ST_DOWN, 0), "event");
    HIPCHECK(ctx, launch_panel_gemm(a, GEMM_DOWN, s), "down launch");
    HIPCHECK(ctx, mark(ST_DOWN, 1), "event");
  }
  // ---- combine (+ RMSNorm)
  HIPCHECK(ctx, mark(ST_COMBINE, 0), "event");
  if (c.latent_moe) {
    HIPCHECK(ctx,
             launch_combine(O, inv, p, T, k, le, gamma, c.rms_eps, 0, abuf, ctx->y_K, taps ? taps->u : nullptr, s),
             "combine launch");
  } else {
    HIPCHECK(ctx, launch_combine(O, inv, p, T, k, le, nullptr, 0.0f, 1, nullptr, 0, u, s), "combine launch");
  }
  HIPCHECK(ctx, mark(ST_COMBINE, 1), "event");
  // ---- y_gemm
  HIPCHECK(ctx, mark(ST_Y, 0), "event");
  if (ctx->y_P > 0) {
    GemmArgs a{};
    a.W = P + ctx->off_y;
    a.P = ctx->y_P;
    a.wwin = ctx->y_wwin;
    a.K = ctx->y_K;
    a.a_fmt = A_BF16;
    a.A = abuf;
    a.lda = ctx->y_K;
    a.a_bytes = (int64_t)T * ctx->y_K * 2;
    a.M = T;
    EpiSeg& sg = a.seg[0];
    sg.p0 = 0;
    sg.p1 = ctx->y_P;
    sg.mode = c.latent_moe ? EPI_BF16 : EPI_BF16_ADD;
    sg.ncols = d;
    sg.out = y_dev;
    sg.ldo = d;
    sg.addend = u;
    sg.ldadd = d;
    a.nseg = 1;
    a.partial = (float*)(ws + ctx->ws_partial);
    a.partial_bytes = gemm_partial_bytes();
    HIPCHECK(ctx, launch_panel_gemm(a, GEMM_Y, s), "y_gemm launch");
  } else {
    HIPCHECK(ctx, launch_f32_to_bf16(u, (uint16_t*)y_dev, (int64_t)T * d, s), "y convert launch");
  }
  HIPCHECK(ctx, mark(ST_Y, 1), "event");
  if (prof) ctx->prof_calls++;

  // ---- taps
  if (taps) {
    auto cp = [&](void* dst, const void* src_, size_t bytes) -> hipError_t {
      return dst ? hipMemcpyAsync(dst, src_, bytes, hipMemcpyDeviceToDevice, s) : hipSuccess;
    };
    const size_t Tk = (size_t)T * k;
    HIPCHECK(ctx, cp(taps->scores, scores, 4 * (size_t)T * E), "tap scores");
    HIPCHECK(ctx, cp(taps->topk_idx, idx, 4 * Tk), "tap idx");
    HIPCHECK(ctx, cp(taps->topk_p, p, 4 * Tk), "tap p");
    HIPCHECK(ctx, cp(taps->counts, counts, 4 * (size_t)E), "tap counts");
    HIPCHECK(ctx, cp(taps->offsets, offsets, 4 * ((size_t)E + 1)), "tap offsets");
    HIPCHECK(ctx, cp(taps->perm, perm, 4 * Tk), "tap perm");
    HIPCHECK(ctx, cp(taps->inv, inv, 4 * Tk), "tap inv");
    if (c.latent_moe) {
      HIPCHECK(ctx, cp(taps->z, z, (f8 ? 1 : 2) * (size_t)T * l), "tap z");
      if (f8) HIPCHECK(ctx, cp(taps->z_scales, zs, (size_t)T * l / 32), "tap z scales");
    }
    HIPCHECK(ctx, cp(taps->h, H, (f8 ? 1 : 2) * Tk * h), "tap h");
    if (f8) HIPCHECK(ctx, cp(taps->h_scales, Hs, Tk * h / 32), "tap h scales");
    HIPCHECK(ctx, cp(taps->expert_out, O, 4 * Tk * le), "tap expert_out");
    if (!c.latent_moe) HIPCHECK(ctx, cp(taps->u, u, 4 * (size_t)T * le), "tap u");
    if (c.latent_moe && taps->n)
      HIPCHECK(ctx,
               hipMemcpy2DAsync(taps->n, 2 * (size_t)l, abuf, 2 * (size_t)ctx->y_K, 2 * (size_t)l, T,
                                hipMemcpyDeviceToDevice, s),
               "tap n");
    if (Ns > 0 && taps->hs)
      HIPCHECK(ctx,
               hipMemcpy2DAsync(taps->hs, 2 * (size_t)Ns * hs, abuf + (c.latent_moe ? l : 0), 2 * (size_t)ctx->y_K,
                                2 * (size_t)Ns * hs, T, hipMemcpyDeviceToDevice, s),
               "tap hs");
  }
  return K3MOE_OK;
}

int k3moe_forward(k3moe_ctx* ctx, const void* x_dev, int32_t T, void* y_dev, void* workspace_dev, void* stream) {
  return k3moe_forward_ex(ctx, x_dev, T, y_dev, workspace_dev, stream, nullptr);
}

}  // extern "C"
