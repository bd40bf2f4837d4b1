// C ABI of the MLA library: argument checks, workspace layout, launches.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/mla.h"
#include "mla_common.h"
#include "mla_internal.h"

using namespace mla;

namespace {

thread_local char g_err[512];

mla_status fail(mla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

mla_status hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

bool is_bf16(const mla_dims* d) { return d->dtype == MLA_BF16; }
int esize(const mla_dims* d) { return is_bf16(d) ? 2 : 4; }
int row_width(const mla_dims* d) { return d->d_latent + d->d_rope; }

mla_status check_dims(const mla_dims* d) {
  if (!d) return fail(MLA_ERR_INVALID_ARG, "dims is NULL");
  if (d->d_model <= 0 || d->n_heads <= 0 || d->d_latent <= 0 || d->d_q_latent <= 0 || d->d_nope <= 0 ||
      d->d_rope <= 0 || d->d_v <= 0)
    return fail(MLA_ERR_INVALID_ARG, "all dimensions must be positive");
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return fail(MLA_ERR_INVALID_ARG, "dtype %d", d->dtype);
  if ((d->d_rope & 1) || (d->d_latent & 1)) return fail(MLA_ERR_INVALID_ARG, "d_rope and d_latent must be even");
  if (!(d->rope_base > 0.f)) return fail(MLA_ERR_INVALID_ARG, "rope_base must be > 0");
  if (d->softmax_scale < 0.f || !isfinite(d->softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale");
  const int KB = is_bf16(d) ? 32 : 4;
  if (d->d_model % KB || d->d_q_latent % KB || (d->n_heads * d->d_latent) % KB)
    return fail(MLA_ERR_UNSUPPORTED, "d_model, d_q_latent and n_heads*d_latent must be multiples of %d", KB);
  if (d->weight_form != MLA_WEIGHTS_MERGED && d->weight_form != MLA_WEIGHTS_FACTORED)
    return fail(MLA_ERR_INVALID_ARG, "weight_form %d", d->weight_form);
  if (d->weight_form == MLA_WEIGHTS_FACTORED) {
    // reduction widths of the run-time factors, and whole 16-column tiles
    // per head for the per-head products
    if (d->d_nope % KB || d->d_latent % KB || (d->n_heads * d->d_v) % KB)
      return fail(MLA_ERR_UNSUPPORTED, "factored weights: d_nope, d_latent and n_heads*d_v must be multiples of %d", KB);
    if (d->d_latent % 16 || d->d_v % 16)
      return fail(MLA_ERR_UNSUPPORTED, "factored weights: d_latent and d_v must be multiples of 16");
  }
  return MLA_OK;
}

bool factored(const mla_dims* d) { return d->weight_form == MLA_WEIGHTS_FACTORED; }

mla_status check_attn_dims(const mla_dims* d) {
  if (!attn_supported(is_bf16(d), d->n_heads, d->d_latent, d->d_rope))
    return fail(MLA_ERR_UNSUPPORTED,
                "no attention kernel for dtype=%d H=%d d_latent=%d d_rope=%d (built: bf16 512+64, fp32 32+8)",
                d->dtype, d->n_heads, d->d_latent, d->d_rope);
  return MLA_OK;
}

float scale_of(const mla_dims* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)(d->d_nope + d->d_rope));
}

// ---------------------------------------------------------- absorbed ----
struct AbsLayout {
  size_t off[4], bytes[4], total;
  // factored form: byte offsets of W_UQ, W_QR, W_UKT, W_UK (region 2), W_UV, W_O (region 3)
  size_t uq, qr, ukt, uk, uv, wo;
};

size_t packed_bytes(const mla_dims* d, int K, int N) {
  const int KB = is_bf16(d) ? 32 : 4;
  return (size_t)ceil_div(K, KB) * KB * (size_t)ceil_div(N, 16) * 16 * esize(d);
}

AbsLayout abs_layout(const mla_dims* d) {
  const int R = row_width(d), H = d->n_heads;
  AbsLayout L{};
  size_t o = 0, end = 0;  // next free 256-byte boundary, end of the last matrix
  auto put = [&](int K, int N) {
    const size_t at = o;
    end = o + packed_bytes(d, K, N);
    o = align256(end);
    return at;
  };
  size_t ends[4];
  L.off[0] = put(d->d_model, R);
  ends[0] = end;
  L.off[1] = put(d->d_model, d->d_q_latent);
  ends[1] = end;
  L.off[2] = o;
  if (!factored(d)) {
    put(d->d_q_latent, H * R);
    ends[2] = end;
    L.off[3] = o;
    put(H * d->d_latent, d->d_model);
  } else {
    L.uq = put(d->d_q_latent, H * d->d_nope);
    L.qr = put(d->d_q_latent, H * d->d_rope);
    L.ukt = put(d->d_nope, H * d->d_latent);
    L.uk = put(d->d_latent, H * d->d_nope);
    ends[2] = end;
    L.off[3] = o;
    L.uv = put(d->d_latent, H * d->d_v);
    L.wo = put(H * d->d_v, d->d_model);
  }
  ends[3] = end;
  L.total = o;
  for (int i = 0; i < 4; ++i) L.bytes[i] = ends[i] - L.off[i];  // region i: its matrices and the gaps between them
  return L;
}

// ---------------------------------------------------------- workspace ----
struct WsLayout {
  size_t err, q, cq, qn, vo, ob, part, tile_off, attn_o, attn_lse, total;
  GemmPlan g_app, g_cq, g_q, g_out;
  // factored form: q_nope = c_Q W_UQ, q_pe, q_lat = q_nope[h] W_UK[h]^T,
  // v = o_lat[h] W_UV[h], y = v W_O
  GemmPlan g_qn, g_qr, g_qk, g_ov, g_oo;
  int G, V;
  bool plans_ok;
  // factored form, up to 16 rows: c_Q unsplit, then one fused launch for
  // q_nope, q_pe and q_lat (the per-head plans above are then unused)
  bool q_fused;
  // o_lat goes through a bf16 copy (ob) before the merged output
  // projection when that runs LDS-tiled: every column block re-reads the
  // whole A operand (at 64 rows as many bytes as the weights), which the
  // bf16 copy halves, and the 256 x 256 fp32-A tiling leaves LDS room for
  // three ring slots only.  (The factored form's per-head products read
  // each head's A columns in one block: nothing to save there.)
  bool stage_o;
};

// The fp32-A plan, or the bf16-A plan over a staged copy (stage_o) when the
// fp32 one is LDS-tiled and A has no column groups.
static GemmPlan plan_o(bool bf, int M, int K, int N, int ncu, int gt, int gs, bool* staged, size_t cap) {
  GemmPlan g = plan_gemm(M, K, N, bf, true, ncu, gt, gs, cap);
  if (bf && g.tiled == 1 && gt == 0) {
    const GemmPlan b = plan_gemm(M, K, N, bf, false, ncu, gt, gs, cap);
    if (b.tiled == 1) {
      *staged = true;
      return b;
    }
  }
  return g;
}

// cap: the most bytes the GEMMs' split-K partials may take (ws_fit).
WsLayout ws_layout(const mla_dims* d, int batch, int n_q, size_t cap = SIZE_MAX) {
  WsLayout W{};
  const bool bf = is_bf16(d);
  const int M = batch * n_q, R = row_width(d), H = d->n_heads;
  const int ncu = device_cus();
  W.g_app = plan_gemm(M, d->d_model, R, bf, false, ncu, 0, 0, cap);
  W.q_fused = factored(d) && q_fused_supported(bf, M, d->d_nope, d->d_rope, d->d_latent, d->d_q_latent);
  W.g_cq = plan_gemm(M, d->d_model, d->d_q_latent, bf, false, ncu, 0, 0, W.q_fused ? 0 : cap);
  size_t part = std::max(W.g_app.part_bytes, W.g_cq.part_bytes);
  if (!factored(d)) {
    W.g_q = plan_gemm(M, d->d_q_latent, H * R, bf, false, ncu, 0, 0, cap);
    W.g_out = plan_o(bf, M, H * d->d_latent, d->d_model, ncu, 0, 0, &W.stage_o, cap);
    part = std::max(part, std::max(W.g_q.part_bytes, W.g_out.part_bytes));
    W.plans_ok = true;
  } else {
    W.g_qn = plan_gemm(M, d->d_q_latent, H * d->d_nope, bf, false, ncu, 0, 0, cap);
    W.g_qr = plan_gemm(M, d->d_q_latent, H * d->d_rope, bf, false, ncu, 0, 0, cap);
    // per-head products: head h's output tiles read A columns h*K ..
    W.g_qk = plan_gemm(M, d->d_nope, H * d->d_latent, bf, false, ncu, d->d_latent / 16, d->d_nope, cap);
    W.g_ov = plan_o(bf, M, d->d_latent, H * d->d_v, ncu, d->d_v / 16, d->d_latent, &W.stage_o, cap);
    W.g_oo = plan_gemm(M, H * d->d_v, d->d_model, bf, false, ncu, 0, 0, cap);
    for (const GemmPlan* g : {&W.g_qn, &W.g_qr, &W.g_qk, &W.g_ov, &W.g_oo}) part = std::max(part, g->part_bytes);
    W.plans_ok = W.g_qk.tiled >= 0 && W.g_ov.tiled >= 0;
  }
  W.G = ncu;
  W.V = M;
  size_t o = 0;
  W.err = o; o = align256(o + 256);
  W.q = o; o = align256(o + (size_t)M * H * R * esize(d));
  W.cq = o; o = align256(o + (size_t)M * d->d_q_latent * esize(d));
  if (factored(d)) {
    W.qn = o; o = align256(o + (size_t)M * H * d->d_nope * esize(d));
    W.vo = o; o = align256(o + (size_t)M * H * d->d_v * esize(d));
  }
  if (W.stage_o) {
    W.ob = o; o = align256(o + (size_t)M * H * d->d_latent * 2);
  }
  W.part = o; o = align256(o + part);

  const int HG = attn_head_group(bf);
  const size_t U = (size_t)M * ((H + HG - 1) / HG);
  W.tile_off = o; o = align256(o + attn_sched_ints((int)U, W.G) * 4);
  const size_t slots = (size_t)W.G + U;
  W.attn_o = o; o = align256(o + slots * HG * d->d_latent * 4);
  W.attn_lse = o; o = align256(o + slots * HG * 4);
  W.total = o;
  return W;
}

// The layout of a call on a workspace of ws_bytes: that of ws_layout or,
// when its split-K partials do not fit, the plans whose partials fit the
// bytes the other regions leave (an unsplit plan needs none).  Every other
// region grows with the row count, so a workspace sized by
// mla_workspace_size for (batch, n_q) serves every call with fewer rows,
// although the K splits that fit best differ from one row count to another.
WsLayout ws_fit(const mla_dims* d, int batch, int n_q, size_t ws_bytes) {
  WsLayout W = ws_layout(d, batch, n_q);
  const size_t rest = W.total - (W.tile_off - W.part);  // all but the partial region
  if (W.total > ws_bytes && ws_bytes > rest) W = ws_layout(d, batch, n_q, (ws_bytes - rest) & ~(size_t)255);
  return W;
}

mla_status check_ws(const WsLayout& W, void* ws, size_t ws_bytes) {
  if (!W.plans_ok) return fail(MLA_ERR_UNSUPPORTED, "no GEMM configuration fits the per-head factored products");
  if (!ws) return fail(MLA_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < W.total) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, W.total);
  return MLA_OK;
}

mla_status check_cache(const mla_dims* d, const mla_cache* c, int batch) {
  if (!c || !c->pool) return fail(MLA_ERR_INVALID_ARG, "cache or cache->pool is NULL");
  if (!aligned(c->pool, 16)) return fail(MLA_ERR_INVALID_ARG, "cache pool must be 16-byte aligned");
  if (c->page_table) {
    if (c->page_size <= 0 || c->page_size % 32) return fail(MLA_ERR_INVALID_ARG, "page_size must be a positive multiple of 32");
    if (c->n_pages <= 0 || c->max_pages_per_seq <= 0) return fail(MLA_ERR_INVALID_ARG, "n_pages / max_pages_per_seq");
    if ((long)c->max_pages_per_seq * c->page_size > (long)INT32_MAX) return fail(MLA_ERR_INVALID_ARG, "capacity overflow");
  } else {
    if (c->s_max <= 0) return fail(MLA_ERR_INVALID_ARG, "contiguous cache needs s_max > 0");
  }
  if (c->row_format != MLA_ROWS_DTYPE && c->row_format != MLA_ROWS_E4M3)
    return fail(MLA_ERR_INVALID_ARG, "row_format %d", c->row_format);
  if (c->row_format == MLA_ROWS_E4M3) {
    if (!is_bf16(d)) return fail(MLA_ERR_UNSUPPORTED, "E4M3 cache rows need a bf16 layer");
    if (!c->scales || !aligned(c->scales, 4)) return fail(MLA_ERR_INVALID_ARG, "E4M3 cache needs 4-byte aligned scales");
    if (row_width(d) % 16) return fail(MLA_ERR_UNSUPPORTED, "E4M3 cache rows need R a multiple of 16");
  }
  (void)batch;
  return MLA_OK;
}

bool e4m3(const mla_cache* c) { return c->row_format == MLA_ROWS_E4M3; }

// The cache-store arguments for rows [M][R] fp32 at positions pos[b] + t.
StoreArgs store_args(const mla_dims* d, const mla_cache* c, const float* rows, const int32_t* pos, int M, int n_q,
                     bool rope, int32_t* err) {
  StoreArgs a{};
  a.rows = rows;
  a.pos = pos;
  a.M = M;
  a.n_q = n_q;
  a.R = row_width(d);
  a.d_latent = d->d_latent;
  a.d_rope = d->d_rope;
  a.rope = rope ? 1 : 0;
  a.rope_base = d->rope_base;
  a.format = e4m3(c) ? 1 : 0;
  a.bf16 = is_bf16(d) ? 1 : 0;
  a.pool = c->pool;
  a.scales = c->scales;
  a.page_table = c->page_table;
  a.paged = c->page_table != nullptr;
  a.page_size = c->page_size;
  a.n_pages = c->n_pages;
  a.max_pages = c->max_pages_per_seq;
  a.s_max = c->s_max;
  a.err = err;
  return a;
}

enum { G_APP = 0, G_CQ = 1, G_Q = 2, G_OUT = 3 };

mla_status run_gemm(const WsLayout& W, int which, const GemmPlan& g, bool bf16, bool a_f32, const void* A, int lda,
                    const void* Wp, unsigned char* ws, const EpiArgs& e, hipStream_t s) {
  (void)which;
  hipError_t err = launch_gemm(g, bf16, a_f32, A, lda, Wp, reinterpret_cast<float*>(ws + W.part), e, s);
  if (err != hipSuccess) return hip_fail(err, "gemm launch");
  return MLA_OK;
}

EpiArgs base_epi(int mode, void* out) {
  EpiArgs e{};
  e.mode = mode;
  e.out = out;
  return e;
}

mla_status q_proj_impl(const mla_dims* d, const WsLayout& W, const unsigned char* abs, const void* x,
                       const int32_t* kv_len, int batch, int n_q, void* q, unsigned char* ws, hipStream_t s) {
  const bool bf = is_bf16(d);
  const AbsLayout L = abs_layout(d);
  void* cq = ws + W.cq;
  mla_status st = run_gemm(W, G_CQ, W.g_cq, bf, false, x, d->d_model, abs + L.off[1], ws, base_epi(EPI_STORE_T, cq), s);
  if (st) return st;
  EpiArgs e = base_epi(EPI_Q, q);
  e.d_latent = d->d_latent; e.d_rope = d->d_rope; e.row = row_width(d); e.rope_base = d->rope_base;
  e.n_q = n_q; e.kv_len = kv_len;
  // column h*R + f of the merged product is element f of head h's row,
  // rotated from f = d_latent on
  e.qg_cols = row_width(d); e.qg_stride = row_width(d); e.q_off = 0; e.q_ld = d->n_heads * row_width(d);
  e.rope_from = d->d_latent;
  if (!factored(d)) {
    st = run_gemm(W, G_Q, W.g_q, bf, false, cq, d->d_q_latent, abs + L.off[2], ws, e, s);
    (void)batch;
    return st;
  }
  // factored: q_nope = c_Q W_UQ (all heads), rounded to dtype
  const int H = d->n_heads, R = row_width(d);
  if (W.q_fused) {
    QFusedArgs f{};
    f.cq = cq; f.w_uq = abs + L.uq; f.w_qr = abs + L.qr; f.w_ukt = abs + L.ukt;
    f.q = q; f.kv_len = kv_len;
    f.M = batch * n_q; f.n_q = n_q; f.H = H; f.d_q_latent = d->d_q_latent; f.rope_base = d->rope_base;
    hipError_t err = launch_q_fused(f, s);
    return err == hipSuccess ? MLA_OK : hip_fail(err, "fused query projection launch");
  }
  void* qn = ws + W.qn;
  st = run_gemm(W, G_Q, W.g_qn, bf, false, cq, d->d_q_latent, abs + L.uq, ws, base_epi(EPI_STORE_T, qn), s);
  if (st) return st;
  // q_pe[h] = RoPE(c_Q W_QR[h]) into columns d_L.. of head h's row
  e.qg_cols = d->d_rope; e.qg_stride = R; e.q_off = d->d_latent; e.q_ld = H * R; e.rope_from = 0;
  st = run_gemm(W, G_Q, W.g_qr, bf, false, cq, d->d_q_latent, abs + L.qr, ws, e, s);
  if (st) return st;
  // q_lat[h] = q_nope[h] W_UK[h]^T into columns 0..d_L of head h's row
  e.qg_cols = d->d_latent; e.qg_stride = R; e.q_off = 0; e.q_ld = H * R; e.rope_from = d->d_latent;
  st = run_gemm(W, G_Q, W.g_qk, bf, false, qn, H * d->d_nope, abs + L.ukt, ws, e, s);
  (void)batch;
  return st;
}

mla_status attention_impl(const mla_dims* d, const WsLayout& W, const void* q, const int32_t* kv_len, int batch,
                          int n_q, const mla_cache* c, float* o_lat, float* lse, unsigned char* ws, hipStream_t s,
                          int32_t* err = nullptr) {
  AttnArgs a{};
  a.q = q;
  a.pool = c->pool;
  a.page_table = c->page_table;
  a.paged = c->page_table != nullptr;
  a.page_size = a.paged ? c->page_size : 32;
  a.n_pages = c->n_pages;
  a.max_pages = c->max_pages_per_seq;
  a.s_max = c->s_max;
  a.kv_len = kv_len;
  a.B = batch;
  a.n_q = n_q;
  a.H = d->n_heads;
  a.V = batch * n_q;
  a.sched = reinterpret_cast<int32_t*>(ws + W.tile_off);  // plan storage, carved up by the launcher
  a.o_lat = o_lat;
  a.lse = lse;
  a.part_o = reinterpret_cast<float*>(ws + W.attn_o);
  a.part_lse = reinterpret_cast<float*>(ws + W.attn_lse);
  a.err = err ? err : reinterpret_cast<int32_t*>(ws + W.err);
  a.scale_log2 = scale_of(d) * 1.4426950408889634f;
  a.G = W.G;
  a.e4m3 = e4m3(c) ? 1 : 0;
  a.scales = c->scales;
  hipError_t e = launch_attention(a, is_bf16(d), s);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return MLA_OK;
}

mla_status check_common(const mla_dims* d, const void* absorbed, int batch, int n_q) {
  mla_status st = check_dims(d);
  if (st) return st;
  if (absorbed && !aligned(absorbed, 256)) return fail(MLA_ERR_INVALID_ARG, "absorbed buffer must be 256-byte aligned");
  if (batch <= 0 || n_q <= 0) return fail(MLA_ERR_INVALID_ARG, "batch (%d) and n_q (%d) must be positive", batch, n_q);
  if ((long)batch * n_q > (1L << 24)) return fail(MLA_ERR_INVALID_ARG, "batch*n_q too large");
  return MLA_OK;
}

// ----------------------------------------------------- expanded prefill ----
struct PfLayout {
  size_t err, cq, qe, ke, ve, vo, part, total;
  GemmPlan g_cq, g_qn, g_qr, g_k, g_v, g_oo;
  bool plans_ok;
};

PfLayout pf_layout(const mla_dims* d, int batch, int n_q, int s_max, size_t cap = SIZE_MAX) {
  PfLayout P{};
  const int M = batch * n_q, Mk = batch * s_max, H = d->n_heads, ncu = device_cus();
  const int QE = d->d_nope + d->d_rope;
  P.g_cq = plan_gemm(M, d->d_model, d->d_q_latent, true, false, ncu, 0, 0, cap);
  P.g_qn = plan_gemm(M, d->d_q_latent, H * d->d_nope, true, false, ncu, 0, 0, cap);
  P.g_qr = plan_gemm(M, d->d_q_latent, H * d->d_rope, true, false, ncu, 0, 0, cap);
  P.g_k = plan_gemm(Mk, d->d_latent, H * d->d_nope, true, false, ncu, 0, 0, cap);
  P.g_v = plan_gemm(Mk, d->d_latent, H * d->d_v, true, false, ncu, 0, 0, cap);
  P.g_oo = plan_gemm(M, H * d->d_v, d->d_model, true, false, ncu, 0, 0, cap);
  size_t part = 0;
  for (const GemmPlan* g : {&P.g_cq, &P.g_qn, &P.g_qr, &P.g_k, &P.g_v, &P.g_oo}) part = std::max(part, g->part_bytes);
  P.plans_ok = true;
  size_t o = 0;
  P.err = o; o = align256(o + 256);
  P.cq = o; o = align256(o + (size_t)M * d->d_q_latent * 2);
  P.qe = o; o = align256(o + (size_t)M * H * QE * 2);
  P.ke = o; o = align256(o + (size_t)Mk * H * d->d_nope * 2);
  P.ve = o; o = align256(o + (size_t)Mk * H * d->d_v * 2);
  P.vo = o; o = align256(o + (size_t)M * H * d->d_v * 2);
  P.part = o; o = align256(o + part);
  P.total = o;
  return P;
}

// As ws_fit, for the expanded prefill (the partial region comes last).
PfLayout pf_fit(const mla_dims* d, int batch, int n_q, int s_max, size_t ws_bytes) {
  PfLayout P = pf_layout(d, batch, n_q, s_max);
  if (P.total > ws_bytes && ws_bytes > P.part) P = pf_layout(d, batch, n_q, s_max, (ws_bytes - P.part) & ~(size_t)255);
  return P;
}

mla_status check_prefill(const mla_dims* d, int batch, int n_q, int s_max) {
  mla_status st = check_common(d, nullptr, batch, n_q);
  if (st) return st;
  if (!factored(d)) return fail(MLA_ERR_UNSUPPORTED, "expanded prefill needs the factored weight form");
  if (!prefill_supported(is_bf16(d), d->d_nope, d->d_rope, d->d_v))
    return fail(MLA_ERR_UNSUPPORTED, "expanded prefill is built for bf16, d_nope = d_v = 128, d_rope = 64");
  if (s_max <= 0 || (long)batch * s_max > (1L << 26)) return fail(MLA_ERR_INVALID_ARG, "s_max %d", s_max);
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_str(int32_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    default: return "MLA_ERR_UNKNOWN";
  }
}

const char* mla_last_error(void) { return g_err; }

const char* mla_version(void) { return "mla-gfx950 0.1"; }

mla_status mla_absorbed_layout(const mla_dims* d, size_t offsets[4], size_t bytes[4], size_t* total) {
  mla_status st = check_dims(d);
  if (st) return st;
  if (!total) return fail(MLA_ERR_INVALID_ARG, "total is NULL");
  const AbsLayout L = abs_layout(d);
  for (int i = 0; i < 4; ++i) {
    if (offsets) offsets[i] = L.off[i];
    if (bytes) bytes[i] = L.bytes[i];
  }
  *total = L.total;
  return MLA_OK;
}

mla_status mla_absorb_weights(const mla_dims* d, const mla_raw_weights* raw, void* absorbed, size_t absorbed_bytes,
                              void* stream) {
  mla_status st = check_dims(d);
  if (st) return st;
  if (!raw || !raw->W_DQ || !raw->W_UQ || !raw->W_QR || !raw->W_DKV || !raw->W_KR || !raw->W_UK || !raw->W_UV ||
      !raw->W_O)
    return fail(MLA_ERR_INVALID_ARG, "a raw weight pointer is NULL");
  if (!absorbed || !aligned(absorbed, 256)) return fail(MLA_ERR_INVALID_ARG, "absorbed must be non-NULL and 256-byte aligned");
  const AbsLayout L = abs_layout(d);
  if (absorbed_bytes < L.total) return fail(MLA_ERR_WORKSPACE, "absorbed %zu bytes < %zu needed", absorbed_bytes, L.total);
  unsigned char* ab = reinterpret_cast<unsigned char*>(absorbed);
  AbsorbArgs a{};
  a.d_model = d->d_model; a.H = d->n_heads; a.d_latent = d->d_latent; a.d_q_latent = d->d_q_latent;
  a.d_nope = d->d_nope; a.d_rope = d->d_rope; a.d_v = d->d_v;
  a.W_DQ = raw->W_DQ; a.W_UQ = raw->W_UQ; a.W_QR = raw->W_QR; a.W_DKV = raw->W_DKV; a.W_KR = raw->W_KR;
  a.W_UK = raw->W_UK; a.W_UV = raw->W_UV; a.W_O = raw->W_O;
  a.P_KV = ab + L.off[0]; a.P_DQ = ab + L.off[1]; a.P_QC = ab + L.off[2]; a.P_O = ab + L.off[3];
  a.factored = factored(d);
  a.P_UQ = ab + L.uq; a.P_QR = ab + L.qr; a.P_UKT = ab + L.ukt; a.P_UK = ab + L.uk; a.P_UV = ab + L.uv;
  a.P_WO = ab + L.wo;
  hipError_t e = launch_absorb(a, is_bf16(d), reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "absorb launch");
  return MLA_OK;
}

mla_status mla_workspace_size(const mla_dims* d, int32_t batch, int32_t n_q, size_t* bytes) {
  mla_status st = check_common(d, nullptr, batch, n_q);
  if (st) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  const WsLayout W = ws_layout(d, batch, n_q);
  if (!W.plans_ok) return fail(MLA_ERR_UNSUPPORTED, "no GEMM configuration fits the per-head factored products");
  *bytes = W.total;
  return MLA_OK;
}

mla_status mla_workspace_check(const mla_dims* d, int32_t batch, int32_t n_q, size_t ws_bytes) {
  mla_status st = check_common(d, nullptr, batch, n_q);
  if (st) return st;
  const WsLayout W = ws_fit(d, batch, n_q, ws_bytes);
  if (!W.plans_ok) return fail(MLA_ERR_UNSUPPORTED, "no GEMM configuration fits the per-head factored products");
  if (ws_bytes < W.total) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, W.total);
  return MLA_OK;
}

mla_status mla_read_device_error(void* workspace, int32_t* flags, void* stream) {
  if (!workspace || !flags) return fail(MLA_ERR_INVALID_ARG, "workspace and flags must be non-NULL");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t h = 0;
  hipError_t e = hipMemcpyAsync(&h, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the device error word");
  const int32_t zero = 0;
  e = hipMemcpyAsync(workspace, &zero, sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "clearing the device error word");
  *flags = h;
  return MLA_OK;
}

mla_status mla_compress_append(const mla_dims* d, const void* absorbed, const void* x, const int32_t* pos,
                               int32_t batch, int32_t n_q, const mla_cache* cache, void* workspace, size_t ws_bytes,
                               void* stream) {
  mla_status st = check_common(d, absorbed, batch, n_q);
  if (st) return st;
  if (!absorbed || !x || !pos) return fail(MLA_ERR_INVALID_ARG, "absorbed, x and pos must be non-NULL");
  if (!aligned(x, 16)) return fail(MLA_ERR_INVALID_ARG, "x must be 16-byte aligned");
  if ((st = check_cache(d, cache, batch))) return st;
  const WsLayout W = ws_fit(d, batch, n_q, ws_bytes);
  if ((st = check_ws(W, workspace, ws_bytes))) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf = is_bf16(d);
  const AbsLayout L = abs_layout(d);
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  if (e4m3(cache)) {
    // E4M3 rows: the GEMM leaves fp32 rows in the q region (unused by an
    // append), then one wave per row applies RoPE and quantises into the cache
    float* rows = reinterpret_cast<float*>(ws + W.q);
    st = run_gemm(W, G_APP, W.g_app, bf, false, x, d->d_model, reinterpret_cast<const unsigned char*>(absorbed) + L.off[0],
                  ws, base_epi(EPI_F32, rows), s);
    if (st) return st;
    hipError_t he = launch_cache_store(store_args(d, cache, rows, pos, batch * n_q, n_q, true,
                                                  reinterpret_cast<int32_t*>(ws + W.err)), s);
    if (he != hipSuccess) return hip_fail(he, "cache store launch");
    return MLA_OK;
  }
  EpiArgs e = base_epi(EPI_APPEND, nullptr);
  e.d_latent = d->d_latent; e.d_rope = d->d_rope; e.row = row_width(d); e.rope_base = d->rope_base;
  e.n_q = n_q; e.pos = pos;
  e.pool = cache->pool; e.page_table = cache->page_table; e.paged = cache->page_table != nullptr;
  e.page_size = cache->page_size; e.n_pages = cache->n_pages; e.max_pages = cache->max_pages_per_seq;
  e.s_max = cache->s_max;
  e.err = reinterpret_cast<int32_t*>(ws + W.err);
  return run_gemm(W, G_APP, W.g_app, bf, false, x, d->d_model, reinterpret_cast<const unsigned char*>(absorbed) + L.off[0],
                  ws, e, s);
}

mla_status mla_cache_store_rows(const mla_dims* d, const float* rows, const int32_t* pos, int32_t batch, int32_t n_q,
                                const mla_cache* cache, void* workspace, size_t ws_bytes, void* stream) {
  mla_status st = check_common(d, nullptr, batch, n_q);
  if (st) return st;
  if (!rows || !pos) return fail(MLA_ERR_INVALID_ARG, "rows and pos must be non-NULL");
  if (!aligned(rows, 16)) return fail(MLA_ERR_INVALID_ARG, "rows must be 16-byte aligned");
  if ((st = check_cache(d, cache, batch))) return st;
  // only the device error word (the first 256 bytes of any workspace) is used
  if (!workspace || !aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
  if (ws_bytes < 256) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < 256 needed", ws_bytes);
  hipError_t he = launch_cache_store(store_args(d, cache, rows, pos, batch * n_q, n_q, false,
                                                reinterpret_cast<int32_t*>(workspace)),
                                     reinterpret_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "cache store launch");
  return MLA_OK;
}

mla_status mla_q_proj(const mla_dims* d, const void* absorbed, const void* x, const int32_t* kv_len, int32_t batch,
                      int32_t n_q, void* q, void* workspace, size_t ws_bytes, void* stream) {
  mla_status st = check_common(d, absorbed, batch, n_q);
  if (st) return st;
  if (!absorbed || !x || !kv_len || !q) return fail(MLA_ERR_INVALID_ARG, "absorbed, x, kv_len and q must be non-NULL");
  if (!aligned(x, 16) || !aligned(q, 16)) return fail(MLA_ERR_INVALID_ARG, "x and q must be 16-byte aligned");
  const WsLayout W = ws_fit(d, batch, n_q, ws_bytes);
  if ((st = check_ws(W, workspace, ws_bytes))) return st;
  return q_proj_impl(d, W, reinterpret_cast<const unsigned char*>(absorbed), x, kv_len, batch, n_q, q,
                     reinterpret_cast<unsigned char*>(workspace), reinterpret_cast<hipStream_t>(stream));
}

mla_status mla_attention(const mla_dims* d, const void* q, const int32_t* kv_len, int32_t batch, int32_t n_q,
                         const mla_cache* cache, float* o_lat, float* lse, void* workspace, size_t ws_bytes,
                         void* stream) {
  mla_status st = check_common(d, nullptr, batch, n_q);
  if (st) return st;
  if ((st = check_attn_dims(d))) return st;
  if (!q || !kv_len || !o_lat) return fail(MLA_ERR_INVALID_ARG, "q, kv_len and o_lat must be non-NULL");
  if (!aligned(q, 16) || !aligned(o_lat, 16) || (lse && !aligned(lse, 4)))
    return fail(MLA_ERR_INVALID_ARG, "q and o_lat must be 16-byte aligned");
  if ((st = check_cache(d, cache, batch))) return st;
  const WsLayout W = ws_fit(d, batch, n_q, ws_bytes);
  if ((st = check_ws(W, workspace, ws_bytes))) return st;
  return attention_impl(d, W, q, kv_len, batch, n_q, cache, o_lat, lse, reinterpret_cast<unsigned char*>(workspace),
                        reinterpret_cast<hipStream_t>(stream));
}

// ------------------------------------------------ no-allocation variant ----
// The device scratch of mla_attention_noalloc: plan records, split partials
// and, when the caller passes no error word, a device error word.  One copy
// per GPU, held from the library's first use of it on that GPU until the
// process ends.  In host code `scratch` names a host-side stand-in: kernels
// and copies take the device address that hipGetSymbolAddress returns for
// the current device (g_scratch_dev), never the array's name.
constexpr size_t kScratchBytes = (size_t)96 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_dev[kMaxDevices] = {};

// Device address of this GPU's scratch, looked up once per device.
mla_status scratch_address(unsigned char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device %d: the scratch table covers %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, 256)) return fail(MLA_ERR_HIP, "scratch address %p is not 256-byte aligned", ptr);
    g_scratch_dev[dev] = reinterpret_cast<unsigned char*>(ptr);
  }
  *out = g_scratch_dev[dev];
  return MLA_OK;
}

// Attention regions inside the scratch for U (sequence, head group) units
// and G split work-groups: error word | plan records | partial O | partial lse.
size_t scratch_layout(const mla_dims* d, size_t U, int G, WsLayout* W) {
  const int HG = attn_head_group(is_bf16(d));
  const size_t slots = (size_t)G + U;
  size_t o = 0;
  W->err = o; o = align256(o + 256);
  W->tile_off = o; o = align256(o + attn_sched_ints((int)U, G) * 4);
  W->attn_o = o; o = align256(o + slots * HG * d->d_latent * 4);
  W->attn_lse = o; o = align256(o + slots * HG * 4);
  W->G = G;
  return o;
}
}  // namespace

mla_status mla_attention_noalloc(const mla_dims* d, const void* q, const int32_t* kv_len, int32_t batch, int32_t n_q,
                                 const mla_cache* cache, float* o_lat, float* lse, int32_t* dev_err, void* stream) {
  mla_status st = check_common(d, nullptr, batch, n_q);
  if (st) return st;
  if ((st = check_attn_dims(d))) return st;
  if (!q || !kv_len || !o_lat) return fail(MLA_ERR_INVALID_ARG, "q, kv_len and o_lat must be non-NULL");
  if (!aligned(q, 16) || !aligned(o_lat, 16) || (lse && !aligned(lse, 4)) || (dev_err && !aligned(dev_err, 4)))
    return fail(MLA_ERR_INVALID_ARG, "q and o_lat must be 16-byte aligned, lse and dev_err 4-byte aligned");
  if ((st = check_cache(d, cache, batch))) return st;
  const int HG = attn_head_group(is_bf16(d));
  const size_t U = (size_t)batch * n_q * ((d->n_heads + HG - 1) / HG);
  // as many split work-groups as there are CUs, fewer when the partials of
  // that many would not fit the scratch, never fewer than 8
  WsLayout W{};
  int G = std::min(device_cus(), 1024);
  while (G > 8 && (U > (size_t)(1 << 24) || scratch_layout(d, U, G, &W) > kScratchBytes)) --G;
  if (U > (size_t)(1 << 24) || scratch_layout(d, U, G, &W) > kScratchBytes)
    return fail(MLA_ERR_WORKSPACE, "%zu (sequence, head group) units need %zu scratch bytes, the maximum is %zu",
                U, scratch_layout(d, U, 8, &W), kScratchBytes);
  W.plans_ok = true;
  unsigned char* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return attention_impl(d, W, q, kv_len, batch, n_q, cache, o_lat, lse, ws, reinterpret_cast<hipStream_t>(stream),
                        dev_err);
}

mla_status mla_decode(const mla_dims* d, const void* absorbed, const void* x, const int32_t* kv_len, int32_t batch,
                      int32_t n_q, const mla_cache* cache, float* o_lat, float* lse, void* workspace, size_t ws_bytes,
                      void* stream) {
  mla_status st = check_common(d, absorbed, batch, n_q);
  if (st) return st;
  if ((st = check_attn_dims(d))) return st;
  if (!absorbed || !x || !kv_len || !o_lat) return fail(MLA_ERR_INVALID_ARG, "absorbed, x, kv_len and o_lat must be non-NULL");
  if (!aligned(x, 16) || !aligned(o_lat, 16)) return fail(MLA_ERR_INVALID_ARG, "x and o_lat must be 16-byte aligned");
  if ((st = check_cache(d, cache, batch))) return st;
  const WsLayout W = ws_fit(d, batch, n_q, ws_bytes);
  if ((st = check_ws(W, workspace, ws_bytes))) return st;
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = q_proj_impl(d, W, reinterpret_cast<const unsigned char*>(absorbed), x, kv_len, batch, n_q, ws + W.q, ws, s);
  if (st) return st;
  return attention_impl(d, W, ws + W.q, kv_len, batch, n_q, cache, o_lat, lse, ws, s);
}

mla_status mla_out_proj(const mla_dims* d, const void* absorbed, const float* o_lat, int32_t n_tok, float* y,
                        void* workspace, size_t ws_bytes, void* stream) {
  mla_status st = check_common(d, absorbed, n_tok, 1);
  if (st) return st;
  if (!absorbed || !o_lat || !y) return fail(MLA_ERR_INVALID_ARG, "absorbed, o_lat and y must be non-NULL");
  if (!aligned(o_lat, 16) || !aligned(y, 16)) return fail(MLA_ERR_INVALID_ARG, "o_lat and y must be 16-byte aligned");
  const WsLayout W = ws_fit(d, n_tok, 1, ws_bytes);
  if ((st = check_ws(W, workspace, ws_bytes))) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf = is_bf16(d);
  const AbsLayout L = abs_layout(d);
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  const unsigned char* ab = reinterpret_cast<const unsigned char*>(absorbed);
  const void* a_op = o_lat;
  if (W.stage_o) {
    const hipError_t e = launch_f32_to_bf16(o_lat, ws + W.ob, (size_t)n_tok * d->n_heads * d->d_latent, s);
    if (e != hipSuccess) return hip_fail(e, "o_lat conversion");
    a_op = ws + W.ob;
  }
  if (!factored(d))
    return run_gemm(W, G_OUT, W.g_out, bf, !W.stage_o, a_op, d->n_heads * d->d_latent, ab + L.off[3], ws,
                    base_epi(EPI_F32, y), s);
  // factored: v[h] = o_lat[h] W_UV[h] (rounded to dtype), then y = v W_O
  void* vo = ws + W.vo;
  st = run_gemm(W, G_OUT, W.g_ov, bf, !W.stage_o, a_op, d->n_heads * d->d_latent, ab + L.uv, ws,
                base_epi(EPI_STORE_T, vo), s);
  if (st) return st;
  return run_gemm(W, G_OUT, W.g_oo, bf, false, vo, d->n_heads * d->d_v, ab + L.wo, ws, base_epi(EPI_F32, y), s);
}

mla_status mla_prefill_workspace_size(const mla_dims* d, int32_t batch, int32_t n_q, int32_t s_max, size_t* bytes) {
  mla_status st = check_prefill(d, batch, n_q, s_max);
  if (st) return st;
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = pf_layout(d, batch, n_q, s_max).total;
  return MLA_OK;
}

mla_status mla_prefill_workspace_check(const mla_dims* d, int32_t batch, int32_t n_q, int32_t s_max, size_t ws_bytes) {
  mla_status st = check_prefill(d, batch, n_q, s_max);
  if (st) return st;
  const PfLayout P = pf_fit(d, batch, n_q, s_max, ws_bytes);
  if (ws_bytes < P.total) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, P.total);
  return MLA_OK;
}

mla_status mla_prefill_expanded(const mla_dims* d, const void* absorbed, const void* x, const int32_t* kv_len,
                                int32_t batch, int32_t n_q, const mla_cache* cache, float* y, float* lse,
                                void* workspace, size_t ws_bytes, void* stream) {
  if (!cache) return fail(MLA_ERR_INVALID_ARG, "cache is NULL");
  mla_status st = check_prefill(d, batch, n_q, cache->s_max);
  if (st) return st;
  if (absorbed && !aligned(absorbed, 256)) return fail(MLA_ERR_INVALID_ARG, "absorbed buffer must be 256-byte aligned");
  if (!absorbed || !x || !kv_len || !y) return fail(MLA_ERR_INVALID_ARG, "absorbed, x, kv_len and y must be non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(MLA_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  if ((st = check_cache(d, cache, batch))) return st;
  if (cache->page_table) return fail(MLA_ERR_UNSUPPORTED, "expanded prefill reads a contiguous cache");
  if (e4m3(cache)) return fail(MLA_ERR_UNSUPPORTED, "expanded prefill reads bf16 cache rows");
  const PfLayout P = pf_fit(d, batch, n_q, cache->s_max, ws_bytes);
  if (!workspace || !aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
  if (ws_bytes < P.total) return fail(MLA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, P.total);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  const unsigned char* ab = reinterpret_cast<const unsigned char*>(absorbed);
  const AbsLayout L = abs_layout(d);
  const int H = d->n_heads, R = row_width(d), QE = d->d_nope + d->d_rope;
  float* part = reinterpret_cast<float*>(ws + P.part);
  auto gemm = [&](const GemmPlan& g, bool a_f32, const void* A, int lda, const unsigned char* Wp, const EpiArgs& e,
                  const int32_t* row_len = nullptr) {
    hipError_t err = launch_gemm(g, true, a_f32, A, lda, Wp, part, e, s, row_len, cache->s_max);
    return err == hipSuccess ? MLA_OK : hip_fail(err, "gemm launch");
  };
  // queries: c_Q, then [q_nope | RoPE(q_pe)] per head (192 wide)
  void* cq = ws + P.cq;
  void* qe = ws + P.qe;
  if ((st = gemm(P.g_cq, false, x, d->d_model, ab + L.off[1], base_epi(EPI_STORE_T, cq)))) return st;
  EpiArgs e = base_epi(EPI_Q, qe);
  e.d_latent = d->d_latent; e.d_rope = d->d_rope; e.row = R; e.rope_base = d->rope_base;
  e.n_q = n_q; e.kv_len = kv_len;
  e.qg_cols = d->d_nope; e.qg_stride = QE; e.q_off = 0; e.q_ld = H * QE; e.rope_from = d->d_nope;
  if ((st = gemm(P.g_qn, false, cq, d->d_q_latent, ab + L.uq, e))) return st;
  e.qg_cols = d->d_rope; e.qg_stride = QE; e.q_off = d->d_nope; e.q_ld = H * QE; e.rope_from = 0;
  if ((st = gemm(P.g_qr, false, cq, d->d_q_latent, ab + L.qr, e))) return st;
  // per-head keys and values of the cache slots below kv_len (the only ones
  // the attention reads; blocks of slots past every sequence's length exit
  // at once): c W_UK[h], c W_UV[h]
  void* ke = ws + P.ke;
  void* ve = ws + P.ve;
  if ((st = gemm(P.g_k, false, cache->pool, R, ab + L.uk, base_epi(EPI_STORE_T, ke), kv_len))) return st;
  if ((st = gemm(P.g_v, false, cache->pool, R, ab + L.uv, base_epi(EPI_STORE_T, ve), kv_len))) return st;
  // causal attention per head, then y = sum_h v[h] W_O[h]
  PrefillArgs a{};
  a.qe = qe; a.ke = ke; a.ve = ve; a.pool = cache->pool; a.kv_len = kv_len;
  a.B = batch; a.n_q = n_q; a.H = H; a.s_max = cache->s_max;
  a.scale_log2 = scale_of(d) * 1.4426950408889634f;
  a.vo = ws + P.vo; a.lse = lse; a.err = reinterpret_cast<int32_t*>(ws + P.err);
  hipError_t err = launch_prefill_attention(a, s);
  if (err != hipSuccess) return hip_fail(err, "prefill attention launch");
  return gemm(P.g_oo, false, ws + P.vo, H * d->d_v, ab + L.wo, base_epi(EPI_F32, y));
}

}  // extern "C"
