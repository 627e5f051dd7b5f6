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
// The first three are the "head", gateup and down the "experts", the last two the "tail": the
// expert-parallel entry points run them separately, k3moe_forward runs them in a row.
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

// Workspace of a forward over T tokens (T k dispatched rows): byte offsets of each buffer.
struct WsLayout {
  size_t scores = 0, idx = 0, p = 0, counts = 0, offsets = 0, perm = 0, inv = 0, route = 0;
  size_t z = 0, zs = 0, h = 0, hs = 0, o = 0, abuf = 0, u = 0, partial = 0, items = 0, t_gu = 0, t_d = 0;
  size_t total = 0;
  bool use_items = false;  // grouped row-tiled launches walk a work-item list (persistent grid)
};

}  // namespace

struct k3moe_ctx {
  k3moe_config cfg;
  int le = 0;  // width the routed experts work in
  // packed layout
  int x_wwin = 0, x_P = 0, x_P_router = 0, x_P_down = 0, x_P_sh = 0;
  int y_K = 0, y_wwin = 0, y_P = 0;
  int gu_wwin = 0, gu_P = 0, dn_wwin = 0, dn_P = 0;
  size_t off_x = 0, off_y = 0, off_gu = 0, off_dn = 0, off_bias = 0, off_gamma = 0, off_lora = 0, total = 0;
  size_t gu_stride = 0, dn_stride = 0;
  // per-expert BF16 LoRA block (lora_rank > 0): A_gu [2r][le], B_gu [h][2r] (gate | up per unit),
  // A_d [r][h], B_d [le][r]
  size_t lora_stride = 0, lo_agu = 0, lo_bgu = 0, lo_ad = 0, lo_bd = 0;
  WsLayout ws;  // at T = max_tokens
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

namespace {

WsLayout ws_layout(const k3moe_ctx& x, int64_t T_) {
  const k3moe_config& c = x.cfg;
  const size_t T = (size_t)T_, k = c.top_k, E = c.n_experts, l = c.latent, h = c.hidden, r = c.lora_rank;
  const bool f8 = c.act == K3MOE_ACT_MXFP8;
  WsLayout L;
  size_t w = 0;
  auto take = [&](size_t bytes) {
    size_t at = w;
    w += align256(bytes);
    return at;
  };
  L.scores = take(4 * T * E);
  L.idx = take(4 * T * k);
  L.p = take(4 * T * k);
  L.counts = take(4 * E);
  L.offsets = take(4 * (E + 1));
  L.perm = take(4 * T * k);
  L.inv = take(4 * T * k);
  L.route = take((size_t)route_scratch_bytes((int)T_, c.n_experts));
  if (c.latent_moe) {
    L.z = take((f8 ? 1 : 2) * T * l);
    L.zs = take(f8 ? T * l / 32 : 0);
  }
  L.h = take((f8 ? 1 : 2) * T * k * h);
  L.hs = take(f8 ? T * k * h / 32 : 0);
  L.o = take(4 * T * k * x.le);
  L.abuf = take(2 * T * (size_t)x.y_K);
  L.u = take(4 * T * x.le);
  L.partial = take((size_t)gemm_partial_bytes());
  const int nblk_max = (int)std::max(ceil_div(x.gu_P, 4), ceil_div(x.dn_P, 4));
  // a group's rows are bounded by the dispatched rows (an expert-parallel receiver's rows need not be
  // one per token)
  L.use_items = tile_items_fit((int64_t)T * k, c.n_experts, nblk_max);
  L.items = take(L.use_items ? (size_t)tile_items_bytes((int64_t)T * k, c.n_experts, nblk_max) : 0);
  L.t_gu = take(4 * T * k * 2 * r);
  L.t_d = take(4 * T * k * r);
  L.total = w;
  return L;
}

// Device pointers of one workspace.
struct Bufs {
  float* scores;
  int32_t *idx, *counts, *offsets, *perm, *inv, *route, *items;
  float* p;
  uint8_t *z, *zs, *H, *Hs;
  float *O, *u, *partial, *t_gu, *t_d;
  uint16_t* abuf;
  bool use_items;
};

Bufs bufs(const WsLayout& L, uint8_t* ws) {
  Bufs b;
  b.scores = (float*)(ws + L.scores);
  b.idx = (int32_t*)(ws + L.idx);
  b.p = (float*)(ws + L.p);
  b.counts = (int32_t*)(ws + L.counts);
  b.offsets = (int32_t*)(ws + L.offsets);
  b.perm = (int32_t*)(ws + L.perm);
  b.inv = (int32_t*)(ws + L.inv);
  b.route = (int32_t*)(ws + L.route);
  b.z = ws + L.z;
  b.zs = ws + L.zs;
  b.H = ws + L.h;
  b.Hs = ws + L.hs;
  b.O = (float*)(ws + L.o);
  b.abuf = (uint16_t*)(ws + L.abuf);
  b.u = (float*)(ws + L.u);
  b.partial = (float*)(ws + L.partial);
  b.items = L.use_items ? (int32_t*)(ws + L.items) : nullptr;
  b.t_gu = (float*)(ws + L.t_gu);
  b.t_d = (float*)(ws + L.t_d);
  b.use_items = L.use_items;
  return b;
}

}  // namespace

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

#define CHECK_OK(expr)            \
  do {                            \
    int rc_ = (expr);             \
    if (rc_ != K3MOE_OK) return rc_; \
  } while (0)

// Stage timing events of the current forward (null: not recorded).
struct Marks {
  hipEvent_t* ev = nullptr;
  hipStream_t s = nullptr;
  hipError_t operator()(int st, int end) const { return ev ? hipEventRecord(ev[st * 2 + end], s) : hipSuccess; }
};

// Which experts take the row-tiled GEMMs (whole 128-wide K windows, so both reduction widths must be
// multiples of 128): with 32 or more rows per expert on average, all; with 8 or more, those with at
// least 16 rows (the panel kernel, one pass per 16 rows, takes the rest: a skewed load puts hot
// experts on the tiled kernel); with fewer (decode), none.
static int row_split_for(const k3moe_ctx* ctx, int64_t rows, int n_groups) {
  if (ctx->le % 128 || ctx->cfg.hidden % 128) return 0;
  if (rows >= (int64_t)32 * n_groups) return 1;
  if (rows >= (int64_t)8 * n_groups) return 16;
  return 0;
}

// ---- head: x_gemm, topk, route
static int run_head(k3moe_ctx* ctx, const void* x_dev, int T, const Bufs& B, hipStream_t s, const k3moe_taps* taps,
                    const Marks& mark) {
  const k3moe_config& c = ctx->cfg;
  const int d = c.d_model, l = c.latent, E = c.n_experts, k = c.top_k, Ns = c.n_shared, hs = c.shared_hidden;
  const bool f8 = c.act == K3MOE_ACT_MXFP8;
  const uint8_t* P = ctx->packed;
  const float* bias = (const float*)(P + ctx->off_bias);
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
    r.out = B.scores;
    r.ldo = E;
    if (c.latent_moe) {
      EpiSeg& zg = a.seg[n++];
      zg.p0 = ctx->x_P_router;
      zg.p1 = ctx->x_P_router + ctx->x_P_down;
      zg.mode = f8 ? EPI_MXFP8 : EPI_BF16;
      zg.ncols = l;
      zg.out = B.z;
      zg.ldo = l;
      zg.out_scales = B.zs;
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
      sg.out = B.abuf;
      sg.ldo = ctx->y_K;
      sg.col0 = (c.latent_moe ? l : 0) + js * hs;
    }
    a.nseg = n;
    a.partial = B.partial;
    a.partial_bytes = gemm_partial_bytes();
    HIPCHECK(ctx, mark(ST_X, 0), "event");
    HIPCHECK(ctx, launch_panel_gemm(a, GEMM_X, s), "x_gemm launch");
    HIPCHECK(ctx, mark(ST_X, 1), "event");
  }
  HIPCHECK(ctx, mark(ST_TOPK, 0), "event");
  HIPCHECK(ctx, launch_topk(B.scores, bias, T, E, k, B.idx, B.p, s), "topk launch");
  HIPCHECK(ctx, mark(ST_TOPK, 1), "event");
  HIPCHECK(ctx, mark(ST_ROUTE, 0), "event");
  HIPCHECK(ctx, launch_route(B.idx, T, E, k, B.counts, B.offsets, B.perm, B.inv, B.route, s), "route launch");
  HIPCHECK(ctx, mark(ST_ROUTE, 1), "event");
  return K3MOE_OK;
}

// ---- experts: (LoRA first factor,) grouped gate/up + SwiGLU, (LoRA first factor,) grouped down.
// A: the routed input of `a_rows` rows (bf16 or E4M3 with scales), read through `rowmap` (null: row r
// of the dispatched order is row r of A); offsets: [n_groups + 1] device row ranges of the experts;
// R: dispatched rows (host). Writes h to B.H (+ B.Hs) and the expert outputs to O.
static int run_experts(k3moe_ctx* ctx, const void* A, const uint8_t* A_scales, int64_t a_rows, int64_t lda,
                       const int32_t* rowmap, const int32_t* offsets, int64_t R, const Bufs& B, float* O, hipStream_t s,
                       const k3moe_taps* taps, const Marks& mark) {
  const k3moe_config& c = ctx->cfg;
  const int h = c.hidden, E = c.n_experts, rank = c.lora_rank;
  const int le = ctx->le;
  const bool f8 = c.act == K3MOE_ACT_MXFP8;
  // the routed input: z (bf16 or MXFP8) in the latent layer, x (bf16) at full width
  const int afmt = c.latent_moe && f8 ? A_MXFP8 : A_BF16;
  const uint8_t* P = ctx->packed;
  const uint16_t* lora = (const uint16_t*)(P + ctx->off_lora);
  const int64_t lstride = (int64_t)(ctx->lora_stride / 2);
  const int row_split = row_split_for(ctx, R, E);
  // ---- gateup
  HIPCHECK(ctx, mark(ST_GATEUP, 0), "event");
  if (rank > 0) {
    LoraAArgs la{};
    la.A = A;
    la.lda = lda;
    la.a_bytes = a_rows * lda * (afmt == A_MXFP8 ? 1 : 2);
    la.A_scales = A_scales;
    la.ldas = lda / 32;
    la.as_bytes = a_rows * (lda / 32);
    la.a_fmt = afmt;
    la.n_groups = E;
    la.rowmap = rowmap;
    la.offsets = offsets;
    la.La = lora + ctx->lo_agu / 2;
    la.la_stride = lstride;
    la.N = 2 * rank;
    la.K = le;
    la.t = B.t_gu;
    la.ldt = 2 * rank;
    HIPCHECK(ctx, launch_lora_a(la, s), "LoRA gate/up first factor launch");
  }
  {
    GemmArgs a{};
    a.W = P + ctx->off_gu;
    a.w_group_stride = (int64_t)ctx->gu_stride;
    a.P = ctx->gu_P;
    a.wwin = ctx->gu_wwin;
    a.K = le;
    a.a_fmt = afmt;
    a.A = A;
    a.lda = lda;
    a.a_bytes = a_rows * lda * (afmt == A_MXFP8 ? 1 : 2);
    a.A_scales = A_scales;
    a.ldas = lda / 32;
    a.as_bytes = a_rows * (lda / 32);
    a.rowmap = rowmap;
    a.offsets = offsets;
    a.n_groups = E;
    a.row_split = row_split;
    a.M = (int32_t)R;  // rows over every group (the launcher picks kernels by rows per group)
    a.items = B.items;
    EpiSeg& sg = a.seg[0];
    sg.p0 = 0;
    sg.p1 = ctx->gu_P;
    sg.mode = f8 ? EPI_SWIGLU_MXFP8 : EPI_SWIGLU_BF16;
    sg.ncols = h;
    sg.out = B.H;
    sg.ldo = h;
    sg.out_scales = B.Hs;
    sg.ldos = h / 32;
    if (taps && taps->h_f32) {
      sg.pre = taps->h_f32;
      sg.ldpre = h;
    }
    a.nseg = 1;
    if (rank > 0) {
      a.lora_t = B.t_gu;
      a.lora_ldt = 2 * rank;
      a.lora_rank = rank;
      a.lora_b = lora + ctx->lo_bgu / 2;
      a.lora_b_stride = lstride;
      a.lora_ldb = 2 * rank;
    }
    HIPCHECK(ctx, launch_panel_gemm(a, GEMM_GATEUP, s), "gateup launch");
  }
  HIPCHECK(ctx, mark(ST_GATEUP, 1), "event");
  // ---- down
  HIPCHECK(ctx, mark(ST_DOWN, 0), "event");
  if (rank > 0) {
    LoraAArgs la{};
    la.A = B.H;
    la.lda = h;
    la.a_bytes = R * h * (f8 ? 1 : 2);
    la.A_scales = B.Hs;
    la.ldas = h / 32;
    la.as_bytes = R * (h / 32);
    la.a_fmt = f8 ? A_MXFP8 : A_BF16;
    la.n_groups = E;
    la.offsets = offsets;
    la.La = lora + ctx->lo_ad / 2;
    la.la_stride = lstride;
    la.N = rank;
    la.K = h;
    la.t = B.t_d;
    la.ldt = rank;
    HIPCHECK(ctx, launch_lora_a(la, s), "LoRA down first factor launch");
  }
  {
    GemmArgs a{};
    a.W = P + ctx->off_dn;
    a.w_group_stride = (int64_t)ctx->dn_stride;
    a.P = ctx->dn_P;
    a.wwin = ctx->dn_wwin;
    a.K = h;
    a.a_fmt = f8 ? A_MXFP8 : A_BF16;
    a.A = B.H;
    a.lda = h;
    a.a_bytes = R * h * (f8 ? 1 : 2);
    a.A_scales = B.Hs;
    a.ldas = h / 32;
    a.as_bytes = R * (h / 32);
    a.offsets = offsets;
    a.n_groups = E;
    a.row_split = row_split;
    a.M = (int32_t)R;  // rows over every group (the launcher picks kernels by rows per group)
    a.items = B.items;
    EpiSeg& sg = a.seg[0];
    sg.p0 = 0;
    sg.p1 = ctx->dn_P;
    sg.mode = EPI_F32;
    sg.ncols = le;
    sg.out = O;
    sg.ldo = le;
    a.nseg = 1;
    if (rank > 0) {
      a.lora_t = B.t_d;
      a.lora_ldt = rank;
      a.lora_rank = rank;
      a.lora_b = lora + ctx->lo_bd / 2;
      a.lora_b_stride = lstride;
      a.lora_ldb = rank;
    }
    HIPCHECK(ctx, launch_panel_gemm(a, GEMM_DOWN, s), "down launch");
  }
  HIPCHECK(ctx, mark(ST_DOWN, 1), "event");
  return K3MOE_OK;
}

// ---- tail: combine (+ RMSNorm), y_gemm
static int run_tail(k3moe_ctx* ctx, const float* O, int T, void* y_dev, const Bufs& B, hipStream_t s,
                    const k3moe_taps* taps, const Marks& mark) {
  const k3moe_config& c = ctx->cfg;
  const int d = c.d_model, k = c.top_k;
  const int le = ctx->le;
  const float* gamma = (const float*)(ctx->packed + ctx->off_gamma);
  HIPCHECK(ctx, mark(ST_COMBINE, 0), "event");
  if (c.latent_moe) {
    HIPCHECK(ctx,
             launch_combine(O, B.inv, B.p, T, k, le, gamma, c.rms_eps, 0, B.abuf, ctx->y_K, taps ? taps->u : nullptr,
                            s),
             "combine launch");
  } else {
    HIPCHECK(ctx, launch_combine(O, B.inv, B.p, T, k, le, nullptr, 0.0f, 1, nullptr, 0, B.u, s), "combine launch");
  }
  HIPCHECK(ctx, mark(ST_COMBINE, 1), "event");
  HIPCHECK(ctx, mark(ST_Y, 0), "event");
  if (ctx->y_P > 0) {
    GemmArgs a{};
    a.W = ctx->packed + ctx->off_y;
    a.P = ctx->y_P;
    a.wwin = ctx->y_wwin;
    a.K = ctx->y_K;
    a.a_fmt = A_BF16;
    a.A = B.abuf;
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
    sg.addend = B.u;
    sg.ldadd = d;
    a.nseg = 1;
    a.partial = B.partial;
    a.partial_bytes = gemm_partial_bytes();
    HIPCHECK(ctx, launch_panel_gemm(a, GEMM_Y, s), "y_gemm launch");
  } else {
    HIPCHECK(ctx, launch_f32_to_bf16(B.u, (uint16_t*)y_dev, (int64_t)T * d, s), "y convert launch");
  }
  HIPCHECK(ctx, mark(ST_Y, 1), "event");
  return K3MOE_OK;
}

static int check_forward_args(k3moe_ctx* ctx, const void* x_dev, int32_t T, const void* y_dev) {
  const k3moe_config& c = ctx->cfg;
  if (T < 0) return fail(ctx, K3MOE_EINVAL, "T must be >= 0");
  if (T > c.max_tokens) return fail(ctx, K3MOE_ETOOBIG, "T = %d above max_tokens = %d", T, c.max_tokens);
  if (!ctx->dense_packed || ctx->n_routed_packed != c.n_experts)
    return fail(ctx, K3MOE_ESTATE, "weights not packed (dense: %d, routed experts: %d of %d)", (int)ctx->dense_packed,
                ctx->n_routed_packed, c.n_experts);
  if (T == 0) return K3MOE_OK;
  if (!x_dev || !y_dev) return fail(ctx, K3MOE_EINVAL, "x or y is NULL");
  if ((uintptr_t)x_dev % 16 || (uintptr_t)y_dev % 16) return fail(ctx, K3MOE_EINVAL, "x and y must be 16-byte aligned");
  if (x_dev == y_dev) return fail(ctx, K3MOE_EINVAL, "y may not alias x");
  return K3MOE_OK;
}

static int forward_impl(k3moe_ctx* ctx, const void* x_dev, int32_t T, void* y_dev, uint8_t* ws, const WsLayout& L,
                        hipStream_t s, const k3moe_taps* taps) {
  const k3moe_config& c = ctx->cfg;
  const int l = c.latent, h = c.hidden, E = c.n_experts, k = c.top_k, Ns = c.n_shared, hs = c.shared_hidden;
  const int le = ctx->le;
  const bool f8 = c.act == K3MOE_ACT_MXFP8;
  const Bufs B = bufs(L, ws);
  const bool prof = ctx->prof_calls < ctx->prof_max;
  Marks mark;
  mark.s = s;
  mark.ev = prof ? &ctx->events[(size_t)ctx->prof_calls * ST_COUNT * 2] : nullptr;

  CHECK_OK(run_head(ctx, x_dev, T, B, s, taps, mark));
  if (c.latent_moe)
    CHECK_OK(run_experts(ctx, B.z, B.zs, T, l, B.perm, B.offsets, (int64_t)T * k, B, B.O, s, taps, mark));
  else
    CHECK_OK(run_experts(ctx, x_dev, nullptr, T, c.d_model, B.perm, B.offsets, (int64_t)T * k, B, B.O, s, taps, mark));
  CHECK_OK(run_tail(ctx, B.O, T, y_dev, B, s, taps, mark));
  if (prof) ctx->prof_calls++;

  if (taps) {
    auto cp = [&](void* dst, const void* src_, size_t bytes) -> hipError_t {
      return dst ? hipMemcpyAsync(dst, src_, bytes, hipMemcpyDeviceToDevice, s) : hipSuccess;
    };
    const size_t Tk = (size_t)T * k;
    HIPCHECK(ctx, cp(taps->scores, B.scores, 4 * (size_t)T * E), "tap scores");
    HIPCHECK(ctx, cp(taps->topk_idx, B.idx, 4 * Tk), "tap idx");
    HIPCHECK(ctx, cp(taps->topk_p, B.p, 4 * Tk), "tap p");
    HIPCHECK(ctx, cp(taps->counts, B.counts, 4 * (size_t)E), "tap counts");
    HIPCHECK(ctx, cp(taps->offsets, B.offsets, 4 * ((size_t)E + 1)), "tap offsets");
    HIPCHECK(ctx, cp(taps->perm, B.perm, 4 * Tk), "tap perm");
    HIPCHECK(ctx, cp(taps->inv, B.inv, 4 * Tk), "tap inv");
    if (c.latent_moe) {
      HIPCHECK(ctx, cp(taps->z, B.z, (f8 ? 1 : 2) * (size_t)T * l), "tap z");
      if (f8) HIPCHECK(ctx, cp(taps->z_scales, B.zs, (size_t)T * l / 32), "tap z scales");
    }
    HIPCHECK(ctx, cp(taps->h, B.H, (f8 ? 1 : 2) * Tk * h), "tap h");
    if (f8) HIPCHECK(ctx, cp(taps->h_scales, B.Hs, Tk * h / 32), "tap h scales");
    HIPCHECK(ctx, cp(taps->expert_out, B.O, 4 * Tk * le), "tap expert_out");
    if (!c.latent_moe) HIPCHECK(ctx, cp(taps->u, B.u, 4 * (size_t)T * le), "tap u");
    if (c.latent_moe && taps->n)
      HIPCHECK(ctx,
               hipMemcpy2DAsync(taps->n, 2 * (size_t)l, B.abuf, 2 * (size_t)ctx->y_K, 2 * (size_t)l, T,
                                hipMemcpyDeviceToDevice, s),
               "tap n");
    if (Ns > 0 && taps->hs)
      HIPCHECK(ctx,
               hipMemcpy2DAsync(taps->hs, 2 * (size_t)Ns * hs, B.abuf + (c.latent_moe ? l : 0), 2 * (size_t)ctx->y_K,
                                2 * (size_t)Ns * hs, T, hipMemcpyDeviceToDevice, s),
               "tap hs");
  }
  return K3MOE_OK;
}

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
  if (c.lora_rank < 0 || c.lora_rank > 32 || c.lora_rank % 8)
    return fail(nullptr, K3MOE_EINVAL, "lora_rank must be 0, 8, 16, 24 or 32");
  if ((int64_t)c.max_tokens * c.top_k > (int64_t)1 << 30)
    return fail(nullptr, K3MOE_ETOOBIG, "max_tokens * top_k too large");
  if (le > 8192) return fail(nullptr, K3MOE_EUNSUPPORTED, "expert width above 8192");
  {
    // every GEMM operand must stay addressable by a 32-bit buffer offset
    const int64_t T = c.max_tokens, lim = ((int64_t)1 << 31) - ((int64_t)1 << 25);
    const int64_t yk = (c.latent_moe ? le : 0) + (int64_t)c.n_shared * c.shared_hidden;
    const int64_t worst = std::max({T * c.d_model * 2, T * c.top_k * c.hidden * 2, T * yk * 2, T * le * 2,
                                    T * c.top_k * le * 2});
    if (worst > lim) return fail(nullptr, K3MOE_ETOOBIG, "max_tokens too large: an operand exceeds 2 GiB");
  }
  if (!(c.rms_eps >= 0.0f)) return fail(nullptr, K3MOE_EINVAL, "rms_eps must be >= 0");

  k3moe_ctx* x = new k3moe_ctx();
  x->cfg = c;
  x->le = le;
  const int d = c.d_model, l = c.latent, h = c.hidden, E = c.n_experts, Ns = c.n_shared, hs = c.shared_hidden;
  const int r = c.lora_rank;
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
  if (r > 0) {
    size_t o = 0;
    x->lo_agu = o;
    o += align256((size_t)2 * r * le * 2);
    x->lo_bgu = o;
    o += align256((size_t)h * 2 * r * 2);
    x->lo_ad = o;
    o += align256((size_t)r * h * 2);
    x->lo_bd = o;
    o += align256((size_t)le * r * 2);
    x->lora_stride = o;
  }
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
  x->off_lora = o;
  o += x->lora_stride * E;
  x->total = o;
  x->ws = ws_layout(*x, c.max_tokens);
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

size_t k3moe_workspace_bytes(const k3moe_ctx* ctx) { return ctx ? ctx->ws.total : 0; }

static bool mx_ok(const k3moe_mx& m) { return m.codes && m.scales; }

static bool lora_ok(const k3moe_lora& m) {
  return m.a_gate && m.b_gate && m.a_up && m.b_up && m.a_down && m.b_down;
}

int k3moe_pack_weights(k3moe_ctx* ctx, const k3moe_weights* wts, void* packed_dev, void* stream) {
  if (!ctx) return K3MOE_EINVAL;
  if (!wts || !packed_dev) return fail(ctx, K3MOE_EINVAL, "weights or packed buffer is NULL");
  if ((uintptr_t)packed_dev % 256) return fail(ctx, K3MOE_EINVAL, "packed buffer must be 256-byte aligned");
  if (ctx->packed && ctx->packed != packed_dev)
    return fail(ctx, K3MOE_EINVAL, "packed buffer differs from the one bound by the first pack call");
  const k3moe_config& c = ctx->cfg;
  const int d = c.d_model, l = c.latent, h = c.hidden, E = c.n_experts, Ns = c.n_shared, hs = c.shared_hidden;
  const int le = ctx->le, r = c.lora_rank;
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
    if (r > 0) {
      if (!wts->lora) return fail(ctx, K3MOE_EINVAL, "lora_rank > 0 but no LoRA deltas given");
      for (int i = 0; i < wts->routed_count; ++i)
        if (!lora_ok(wts->lora[i]))
          return fail(ctx, K3MOE_EINVAL, "routed expert %d has a NULL LoRA factor", wts->routed_first + i);
    }
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
    if (r > 0) {
      const k3moe_lora& lo = wts->lora[i];
      uint8_t* base = P + ctx->off_lora + ctx->lora_stride * e;
      const size_t arow = (size_t)r * le * 2;
      HIPCHECK(ctx, hipMemcpyAsync(base + ctx->lo_agu, lo.a_gate, arow, hipMemcpyDeviceToDevice, s), "pack LoRA");
      HIPCHECK(ctx, hipMemcpyAsync(base + ctx->lo_agu + arow, lo.a_up, arow, hipMemcpyDeviceToDevice, s), "pack LoRA");
      // B of gate and up side by side per hidden unit: row n = [b_gate[n, :] | b_up[n, :]]
      HIPCHECK(ctx,
               hipMemcpy2DAsync(base + ctx->lo_bgu, 4 * (size_t)r, lo.b_gate, 2 * (size_t)r, 2 * (size_t)r, h,
                                hipMemcpyDeviceToDevice, s),
               "pack LoRA");
      HIPCHECK(ctx,
               hipMemcpy2DAsync(base + ctx->lo_bgu + 2 * (size_t)r, 4 * (size_t)r, lo.b_up, 2 * (size_t)r,
                                2 * (size_t)r, h, hipMemcpyDeviceToDevice, s),
               "pack LoRA");
      HIPCHECK(ctx, hipMemcpyAsync(base + ctx->lo_ad, lo.a_down, (size_t)r * h * 2, hipMemcpyDeviceToDevice, s),
               "pack LoRA");
      HIPCHECK(ctx, hipMemcpyAsync(base + ctx->lo_bd, lo.b_down, (size_t)le * r * 2, hipMemcpyDeviceToDevice, s),
               "pack LoRA");
    }
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
  CHECK_OK(check_forward_args(ctx, x_dev, T, y_dev));
  if (T == 0) return K3MOE_OK;
  if (!workspace_dev) return fail(ctx, K3MOE_EINVAL, "workspace is NULL");
  if ((uintptr_t)workspace_dev % 256) return fail(ctx, K3MOE_EINVAL, "workspace must be 256-byte aligned");
  return forward_impl(ctx, x_dev, T, y_dev, (uint8_t*)workspace_dev, ctx->ws, (hipStream_t)stream, taps);
}

int k3moe_forward(k3moe_ctx* ctx, const void* x_dev, int32_t T, void* y_dev, void* workspace_dev, void* stream) {
  return k3moe_forward_ex(ctx, x_dev, T, y_dev, workspace_dev, stream, nullptr);
}

int k3moe_scratch_fits(const k3moe_ctx* ctx, int32_t T) {
  if (!ctx || T < 0 || T > ctx->cfg.max_tokens) return 0;
  return ws_layout(*ctx, T).total <= kScratchBytes ? 1 : 0;
}

int k3moe_forward_noalloc(k3moe_ctx* ctx, const void* x_dev, int32_t T, void* y_dev, void* stream) {
  if (!ctx) return K3MOE_EINVAL;
  CHECK_OK(check_forward_args(ctx, x_dev, T, y_dev));
  if (T == 0) return K3MOE_OK;
  const WsLayout L = ws_layout(*ctx, T);
  if (L.total > kScratchBytes)
    return fail(ctx, K3MOE_ETOOBIG, "T = %d needs %zu bytes of workspace, above the %zu-byte static scratch", T,
                L.total, kScratchBytes);
  void* scratch_ptr = nullptr;  // this device's copy of the static scratch array
  HIPCHECK(ctx, scratch_address(&scratch_ptr), "scratch address");
  return forward_impl(ctx, x_dev, T, y_dev, (uint8_t*)scratch_ptr, L, (hipStream_t)stream, nullptr);
}

int k3moe_forward_head(k3moe_ctx* ctx, const void* x_dev, int32_t T, void* workspace_dev, void* stream,
                       int32_t n_ranks, void* send_rows_dev, uint8_t* send_scales_dev, int32_t* send_counts_dev,
                       int32_t* expert_counts_dev) {
  if (!ctx) return K3MOE_EINVAL;
  const k3moe_config& c = ctx->cfg;
  const int E = c.n_experts, k = c.top_k;
  const bool f8 = c.act == K3MOE_ACT_MXFP8;
  if (T < 0) return fail(ctx, K3MOE_EINVAL, "T must be >= 0");
  if (T > c.max_tokens) return fail(ctx, K3MOE_ETOOBIG, "T = %d above max_tokens = %d", T, c.max_tokens);
  if (n_ranks < 1 || E % n_ranks) return fail(ctx, K3MOE_EINVAL, "n_ranks = %d must divide n_experts = %d", n_ranks, E);
  if (!ctx->dense_packed) return fail(ctx, K3MOE_ESTATE, "dense weights not packed");
  if (!workspace_dev || !send_counts_dev) return fail(ctx, K3MOE_EINVAL, "workspace or send counts is NULL");
  if (T > 0 && (!x_dev || !send_rows_dev || (f8 && c.latent_moe && !send_scales_dev)))
    return fail(ctx, K3MOE_EINVAL, "x, send rows or send scales (MXFP8) is NULL");
  if ((uintptr_t)workspace_dev % 256 || (uintptr_t)x_dev % 16 || (uintptr_t)send_rows_dev % 16)
    return fail(ctx, K3MOE_EINVAL, "workspace must be 256-byte and x and send rows 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const Bufs B = bufs(ctx->ws, (uint8_t*)workspace_dev);
  if (T > 0) {
    CHECK_OK(run_head(ctx, x_dev, T, B, s, nullptr, Marks{}));
    const int le = ctx->le;
    const bool a8 = f8 && c.latent_moe;  // the routed input: z (bf16 or MXFP8) or x (bf16)
    const uint8_t* src = c.latent_moe ? B.z : (const uint8_t*)x_dev;
    HIPCHECK(ctx,
             launch_gather_rows(src, (int64_t)le * (a8 ? 1 : 2), a8 ? B.zs : nullptr, a8 ? le / 32 : 0, B.perm,
                                (int64_t)T * k, (uint8_t*)send_rows_dev, a8 ? send_scales_dev : nullptr, s),
             "gather launch");
  } else {  // no tokens: every count is zero
    HIPCHECK(ctx, launch_fill_i32(B.offsets, E + 1, 0, s), "clear offsets");
    HIPCHECK(ctx, launch_fill_i32(B.counts, E, 0, s), "clear counts");
  }
  HIPCHECK(ctx, launch_send_counts(B.offsets, n_ranks, E / n_ranks, send_counts_dev, s), "send counts launch");
  if (expert_counts_dev)
    HIPCHECK(ctx, hipMemcpyAsync(expert_counts_dev, B.counts, 4 * (size_t)E, hipMemcpyDeviceToDevice, s),
             "copy counts");
  return K3MOE_OK;
}

int k3moe_experts_forward(k3moe_ctx* ctx, const void* rows_dev, const uint8_t* row_scales_dev, int32_t R,
                          const int32_t* expert_counts_dev, float* out_dev, void* workspace_dev, void* stream) {
  if (!ctx) return K3MOE_EINVAL;
  const k3moe_config& c = ctx->cfg;
  const bool a8 = c.act == K3MOE_ACT_MXFP8 && c.latent_moe;
  if (R < 0) return fail(ctx, K3MOE_EINVAL, "R must be >= 0");
  if ((int64_t)R > (int64_t)c.max_tokens * c.top_k)
    return fail(ctx, K3MOE_ETOOBIG, "R = %d above max_tokens * top_k = %lld", R, (long long)c.max_tokens * c.top_k);
  if (ctx->n_routed_packed != c.n_experts)
    return fail(ctx, K3MOE_ESTATE, "routed experts not packed (%d of %d)", ctx->n_routed_packed, c.n_experts);
  if (R == 0) return K3MOE_OK;
  if (!rows_dev || !expert_counts_dev || !out_dev || !workspace_dev || (a8 && !row_scales_dev))
    return fail(ctx, K3MOE_EINVAL, "rows, row scales (MXFP8), counts, out or workspace is NULL");
  if ((uintptr_t)workspace_dev % 256 || (uintptr_t)rows_dev % 16 || (uintptr_t)out_dev % 16)
    return fail(ctx, K3MOE_EINVAL, "workspace must be 256-byte and rows and out 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  const Bufs B = bufs(ctx->ws, (uint8_t*)workspace_dev);
  // the experts' row ranges from the received counts (clamped to the R rows given)
  HIPCHECK(ctx, launch_offsets(expert_counts_dev, c.n_experts, R, B.offsets, s), "offsets launch");
  return run_experts(ctx, rows_dev, row_scales_dev, R, ctx->le, nullptr, B.offsets, R, B, out_dev, s, nullptr,
                     Marks{});
}

int k3moe_forward_tail(k3moe_ctx* ctx, const float* expert_out_dev, int32_t T, void* y_dev, void* workspace_dev,
                       void* stream) {
  if (!ctx) return K3MOE_EINVAL;
  const k3moe_config& c = ctx->cfg;
  if (T < 0) return fail(ctx, K3MOE_EINVAL, "T must be >= 0");
  if (T > c.max_tokens) return fail(ctx, K3MOE_ETOOBIG, "T = %d above max_tokens = %d", T, c.max_tokens);
  if (!ctx->dense_packed) return fail(ctx, K3MOE_ESTATE, "dense weights not packed");
  if (T == 0) return K3MOE_OK;
  if (!expert_out_dev || !y_dev || !workspace_dev) return fail(ctx, K3MOE_EINVAL, "expert outputs, y or workspace is NULL");
  if ((uintptr_t)workspace_dev % 256 || (uintptr_t)expert_out_dev % 16 || (uintptr_t)y_dev % 16)
    return fail(ctx, K3MOE_EINVAL, "workspace must be 256-byte and expert outputs and y 16-byte aligned");
  const Bufs B = bufs(ctx->ws, (uint8_t*)workspace_dev);
  return run_tail(ctx, expert_out_dev, T, y_dev, B, (hipStream_t)stream, nullptr, Marks{});
}

int k3moe_stream_read(const void* buf_dev, size_t bytes, uint32_t* out_dev, void* stream) {
  if (!buf_dev || !out_dev || bytes == 0 || bytes % 16) return K3MOE_EINVAL;
  if (bytes > ((size_t)1 << 40)) return K3MOE_ETOOBIG;
  return launch_stream_read(buf_dev, (int64_t)bytes, out_dev, (hipStream_t)stream) == hipSuccess ? K3MOE_OK
                                                                                                 : K3MOE_EHIP;
}

}  // extern "C"
