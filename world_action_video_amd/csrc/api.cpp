// C-ABI layer: argument validation, workspace carving and the launch sequence of the DiT step.
// Every check happens before the first launch, so a non-OK status means nothing was enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/wam.h"
#include "kernels.h"

using namespace wam;

namespace {

thread_local std::string g_err;

// Event pairs around the QKV product of one layer, recorded on the pass's stream (process-wide, one
// user at a time).
struct QkvTimer {
  int layer = -1, n = 0;
  std::vector<hipEvent_t> ev;   // start, stop per sample
  void clear() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    ev.clear();
    layer = -1;
    n = 0;
  }
};
QkvTimer g_qkv_timer;

wam_status fail(wam_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_TRY(expr)                                                                        \
  do {                                                                                       \
    hipError_t e_ = (expr);                                                                  \
    if (e_ != hipSuccess) return fail(WAM_E_HIP, "%s: %s", #expr, hipGetErrorString(e_));     \
  } while (0)

constexpr int kMaxChunks = 8;   // 2 * n_chunks timesteps fit the time-MLP batch of 16

struct Geo {
  int D, H, d, F, L, P, A, La, Lv, Lq, Lc, Cin, br, freq;
  size_t esz;
  DType dt;
  bool mx;     // MXFP8 block projections (activations; weights too unless w4)
  bool w4;     // MXFP4 weights of the block projections
  int F1;      // rows of w_ff1 (2F for the SwiGLU variant)
  int Lt;      // text rows of the condition sequence (the image rows follow, then the state rows)
  int Li, Ls, Sd;   // image rows, state rows, state width
  bool img_x;  // image rows with their own projections and softmax (IMG_XATTN variant)
};

Geo geo_of(const wam_config& c) {
  Geo g;
  g.D = c.dim; g.H = c.heads; g.d = c.head_dim; g.F = c.ffn_dim; g.L = c.layers; g.P = c.patch_dim;
  g.A = c.action_dim; g.La = c.action_tokens; g.Lv = c.frames_per_chunk * c.grid_h * c.grid_w;
  g.Lq = g.Lv + g.La; g.Lc = c.ctx_text_len + c.ctx_img_len + c.ctx_state_len; g.Cin = c.ctx_in_dim;
  g.br = c.branches;
  g.Li = c.ctx_img_len; g.Ls = c.ctx_state_len; g.Sd = c.state_dim;
  g.freq = c.freq_dim;
  g.dt = c.dtype == WAM_BF16 ? DT_BF16 : DT_F32;
  g.esz = c.dtype == WAM_BF16 ? 2 : 4;
  g.mx = c.precision == WAM_PRECISION_MXFP8 || c.precision == WAM_PRECISION_MXFP4W;
  g.w4 = c.precision == WAM_PRECISION_MXFP4W;
  g.F1 = (c.variant & WAM_VARIANT_SWIGLU) ? 2 * c.ffn_dim : c.ffn_dim;
  g.Lt = c.ctx_text_len;
  g.img_x = (c.variant & WAM_VARIANT_IMG_XATTN) != 0;
  return g;
}

// Packed MXFP8 projections of one layer: codes [N][K] then scales [N][K/32] per matrix, 256-aligned.
enum { MX_QKV, MX_O, MX_CQ, MX_CO, MX_FF1, MX_FF2, MX_MATS };
struct MxMat { size_t codes, scales; int N, K; };
struct MxBlock { MxMat m[MX_MATS]; size_t total; };

MxBlock mx_block_of(const Geo& g) {
  MxBlock b{};
  const int NK[MX_MATS][2] = {{3 * g.D, g.D}, {g.D, g.D}, {g.D, g.D}, {g.D, g.D}, {g.F1, g.D}, {g.D, g.F}};
  size_t off = 0;
  for (int i = 0; i < MX_MATS; ++i) {
    b.m[i].N = NK[i][0];
    b.m[i].K = NK[i][1];
    b.m[i].codes = off;
    off += ((size_t)b.m[i].N * (g.w4 ? b.m[i].K / 2 : b.m[i].K) + 255) & ~size_t(255);
    b.m[i].scales = off;
    off += ((size_t)b.m[i].N * (b.m[i].K / 32) + 255) & ~size_t(255);
  }
  b.total = off;
  return b;
}

// Fragment-packed projections of one layer (launch_pack_weight's layout): the six matrices back to
// back in the order above, each N * K bf16 (a multiple of 4 KB, since N % 32 == 0 and K % 64 == 0).
// A band of 32 rows occupies the bytes its rows would unpacked, so row offsets that are multiples of
// 32 (the key / value rows of w_qkv) translate unchanged.
struct PkBlock { size_t off[MX_MATS]; int N[MX_MATS], K[MX_MATS]; size_t total; };

PkBlock pk_block_of(const Geo& g) {
  PkBlock b{};
  const int NK[MX_MATS][2] = {{3 * g.D, g.D}, {g.D, g.D}, {g.D, g.D}, {g.D, g.D}, {g.F1, g.D}, {g.D, g.F}};
  size_t off = 0;
  for (int i = 0; i < MX_MATS; ++i) {
    b.N[i] = NK[i][0];
    b.K[i] = NK[i][1];
    b.off[i] = off;
    off += (size_t)b.N[i] * b.K[i] * 2;
  }
  b.total = off;
  return b;
}

// every packed matrix must stay below 2 GiB (32-bit buffer offsets)
bool pk_fits(const Geo& g) {
  const PkBlock b = pk_block_of(g);
  for (int i = 0; i < MX_MATS; ++i)
    if ((long)b.N[i] * b.K[i] * 2 >= (1L << 31)) return false;
  return true;
}

wam_status check_cfg(const wam_config* c) {
  if (!c) return fail(WAM_E_ARG, "config is NULL");
  if (c->dtype != WAM_BF16 && c->dtype != WAM_F32) return fail(WAM_E_ARG, "unknown dtype %d", (int)c->dtype);
  if (c->dim <= 0 || c->heads <= 0 || c->layers <= 0 || c->ffn_dim <= 0 || c->freq_dim <= 0)
    return fail(WAM_E_SHAPE, "non-positive model size");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(WAM_E_SHAPE, "head_dim must be 64 or 128");
  if (c->dim != c->heads * c->head_dim) return fail(WAM_E_SHAPE, "dim != heads * head_dim");
  if (c->dim % 64 || c->ffn_dim % 64 || c->ctx_in_dim % 64 || c->ctx_in_dim <= 0)
    return fail(WAM_E_SHAPE, "dim, ffn_dim and ctx_in_dim must be multiples of 64");
  if (c->dim > 8192) return fail(WAM_E_SHAPE, "dim above 8192 is not supported");
  if (c->freq_dim % 8) return fail(WAM_E_SHAPE, "freq_dim must be a multiple of 8");
  if (c->patch_dim <= 0 || c->action_dim <= 0 || c->action_tokens < 0) return fail(WAM_E_SHAPE, "bad token sizes");
  if (c->patch_dim > 64 || c->action_dim > 64) return fail(WAM_E_SHAPE, "patch_dim and action_dim must be <= 64");
  if (c->frames_per_chunk <= 0 || c->grid_h <= 0 || c->grid_w <= 0) return fail(WAM_E_SHAPE, "bad chunk geometry");
  const int lq = c->frames_per_chunk * c->grid_h * c->grid_w + c->action_tokens;
  if (lq % 8 || lq < 32) return fail(WAM_E_SHAPE, "tokens per chunk (%d) must be a multiple of 8 and at least 32", lq);
  if (c->ctx_text_len <= 0 || c->ctx_img_len < 0) return fail(WAM_E_SHAPE, "bad condition lengths");
  if (c->branches != 1 && c->branches != 2) return fail(WAM_E_SHAPE, "branches must be 1 or 2");
  if (!(c->eps > 0.f) || !(c->rope_theta > 0.f)) return fail(WAM_E_ARG, "eps and rope_theta must be positive");
  if (c->variant & ~(WAM_VARIANT_FRAME_CAUSAL | WAM_VARIANT_RMS_NORM | WAM_VARIANT_SWIGLU | WAM_VARIANT_IMG_XATTN))
    return fail(WAM_E_UNSUPPORTED, "unknown variant bits 0x%x", c->variant);
  if ((c->variant & WAM_VARIANT_IMG_XATTN) && (c->ctx_img_len <= 0 || c->ctx_text_len % 8))
    return fail(WAM_E_SHAPE, "separate image cross-attention needs image tokens and ctx_text_len a multiple of 8");
  if (c->ctx_state_len < 0 || c->ctx_state_len > 64) return fail(WAM_E_SHAPE, "ctx_state_len must be in [0, 64]");
  if (c->ctx_state_len > 0 && (c->state_dim <= 0 || c->state_dim % 64 || c->state_dim > 4096))
    return fail(WAM_E_SHAPE, "state_dim must be a positive multiple of 64 (at most 4096)");
  if (c->ctx_state_len > 0 && (c->variant & WAM_VARIANT_IMG_XATTN))
    return fail(WAM_E_UNSUPPORTED, "state rows and the separate image cross-attention are not combined");
  if (c->precision != WAM_PRECISION_NATIVE && c->precision != WAM_PRECISION_MXFP8 &&
      c->precision != WAM_PRECISION_MXFP4W)
    return fail(WAM_E_UNSUPPORTED, "unknown precision %d", c->precision);
  if (c->precision != WAM_PRECISION_NATIVE && (c->dtype != WAM_BF16 || c->dim % 128 || c->ffn_dim % 128))
    return fail(WAM_E_UNSUPPORTED, "MXFP8 / MXFP4 projections need dtype bf16 and dim, ffn_dim multiples of 128");
  return WAM_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t h, y, qkv, qh, attn, ffn, rope, emb, h1, e, e6, partials, xq, xs, ctx_a, ctx_b, part, total;
  long part_elems;   // fp32 capacity of the split-K partial products
};

Layout layout_of(const Geo& g, int n) {
  Layout L{};
  const size_t R = (size_t)n * g.Lq, M = (size_t)g.br * R, G = 2 * (size_t)n;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
  L.h = take(M * g.D * 4);
  L.y = take(M * g.D * g.esz);
  L.qkv = take(M * 3 * g.D * g.esz);
  L.qh = take(M * g.D * g.esz);
  L.attn = take(M * g.D * g.esz);
  L.ffn = take(M * g.F * g.esz);
  L.rope = take(R * (g.d / 2) * sizeof(float2));
  L.emb = take(G * g.freq * 4);
  L.h1 = take(G * g.D * 4);
  L.e = take(G * g.D * 4);
  L.e6 = take(G * 6 * g.D * 4);
  L.partials = take(64 * 3 * 4);
  if (g.mx) {   // MXFP8 codes and scales of one projection input (up to ffn_dim columns)
    const size_t kmax = std::max(g.D, g.F);
    L.xq = take(M * kmax);
    L.xs = take(M * (kmax / 32));
  }
  size_t stack_total = off;
  // condition build (never concurrent with a pass on the same workspace): two [br*Lc][D] buffers
  const size_t cb = align256((size_t)g.br * g.Lc * g.D * g.esz);
  L.ctx_a = 0;
  L.ctx_b = cb;
  // split-K partial products (up to 4 splits of the widest D-column product), clear of both uses above;
  // the attention's key-split partials reuse the region (never live at the same time as a product's)
  const size_t Mmax = std::max(M, (size_t)g.br * g.Lc);
  L.part = align256(std::max(stack_total, 2 * cb));
  L.part_elems = (long)(4 * Mmax * g.D);
  if (g.dt == DT_BF16)   // the largest split any key count can take for this many query rows
    L.part_elems = std::max(L.part_elems, attn_split_floats((int)R, g.H, g.br, 1 << 28));
  L.total = L.part + align256((size_t)L.part_elems * 4);
  return L;
}

template <typename P> P* at(void* ws, size_t off) { return reinterpret_cast<P*>(reinterpret_cast<char*>(ws) + off); }

const char* const kBlockNames[] = {"mod", "w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "ln3_w", "ln3_b",
                                   "w_cq", "b_cq", "g_cq", "w_ck", "b_ck", "g_ck", "w_cv", "b_cv", "w_co",
                                   "b_co", "w_ff1", "b_ff1", "w_ff2", "b_ff2"};

bool unaligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; }

// pk_used: the configuration reads fragment-packed projections when a block supplies them (bf16,
// native precision); such a block's six unpacked projection matrices are then not read.
// pk_fit: the configuration's projections can be packed (each below 2 GiB).
wam_status check_block(const wam_block_weights* b, int l, bool mx, bool img_x, bool pk_used, bool pk_fit) {
  if (!b) return fail(WAM_E_ARG, "block weights of layer %d are NULL", l);
  const bool packed = pk_used && b->pk;
  if (packed && reinterpret_cast<uintptr_t>(b->pk) % 256)
    return fail(WAM_E_ARG, "layer %d: the packed projections (pk) must be 256-byte aligned", l);
  if (packed && !pk_fit) return fail(WAM_E_SHAPE, "layer %d: a projection is too large to pack (2 GiB)", l);
  if (img_x) {
    const void* q[5] = {b->w_cki, b->b_cki, b->g_cki, b->w_cvi, b->b_cvi};
    for (const void* x : q)
      if (!x || unaligned16(x))
        return fail(WAM_E_ARG, "layer %d: image key / value projections NULL or not 16-byte aligned", l);
  }
  if (mx && (!b->mx || reinterpret_cast<uintptr_t>(b->mx) % 256))
    return fail(WAM_E_ARG, "layer %d: MXFP8 precision needs the packed projections (mx, 256-byte aligned)", l);
  const void* const* p = reinterpret_cast<const void* const*>(b);
  auto replaced = [](const char* name) {   // a projection the packed copy stands in for
    for (const char* m : {"w_qkv", "w_o", "w_cq", "w_co", "w_ff1", "w_ff2"})
      if (!strcmp(name, m)) return true;
    return false;
  };
  for (int i = 0; i < (int)(sizeof(kBlockNames) / sizeof(kBlockNames[0])); ++i) {
    if (packed && replaced(kBlockNames[i])) continue;
    if (!p[i]) return fail(WAM_E_ARG, "layer %d: %s is NULL", l, kBlockNames[i]);
    if (unaligned16(p[i])) return fail(WAM_E_ARG, "layer %d: %s is not 16-byte aligned", l, kBlockNames[i]);
  }
  return WAM_OK;
}

wam_status check_weights(const wam_config* c, const wam_weights* w, bool need_blocks) {
  if (!w) return fail(WAM_E_ARG, "weights are NULL");
  if (!w->t_w1 || !w->t_b1 || !w->t_w2 || !w->t_b2 || !w->t_wp || !w->t_bp)
    return fail(WAM_E_ARG, "time-embedding weights are NULL");
  if (!w->pe_w || !w->pe_b || !w->ae_w || !w->ae_b) return fail(WAM_E_ARG, "token-embedding weights are NULL");
  if (!w->head_mod || !w->vo_w || !w->vo_b || !w->ao_w || !w->ao_b) return fail(WAM_E_ARG, "head weights are NULL");
  for (const void* q : {w->t_w1, w->t_b1, w->t_w2, w->t_b2, w->t_wp, w->t_bp, w->pe_w, w->pe_b, w->ae_w, w->ae_b,
                        w->head_mod, w->vo_w, w->vo_b, w->ao_w, w->ao_b})
    if (unaligned16(q)) return fail(WAM_E_ARG, "a global weight tensor is not 16-byte aligned");
  if (c->ctx_state_len > 0 && (!w->st_w || !w->st_b || unaligned16(w->st_w) || unaligned16(w->st_b)))
    return fail(WAM_E_ARG, "state encoder weights are NULL or not 16-byte aligned");
  if (need_blocks) {
    if (!w->blocks) return fail(WAM_E_ARG, "blocks array is NULL");
    for (int l = 0; l < c->layers; ++l) {
      wam_status st = check_block(&w->blocks[l], l, c->precision != WAM_PRECISION_NATIVE,
                                  (c->variant & WAM_VARIANT_IMG_XATTN) != 0,
                                  c->dtype == WAM_BF16 && c->precision == WAM_PRECISION_NATIVE, pk_fits(geo_of(*c)));
      if (st != WAM_OK) return st;
    }
  }
  return WAM_OK;
}

wam_status check_cache(const Geo& g, const wam_kv_cache* kv, int rows) {
  if (!kv || !kv->k || !kv->v) return fail(WAM_E_ARG, "KV cache pointers are NULL");
  if (unaligned16(kv->k) || unaligned16(kv->v)) return fail(WAM_E_ARG, "KV cache pointers are not 16-byte aligned");
  if (kv->branches != g.br) return fail(WAM_E_SHAPE, "cache branches %d != config branches %d", kv->branches, g.br);
  if (kv->capacity <= 0 || kv->capacity % 64) return fail(WAM_E_SHAPE, "cache capacity must be a positive multiple of 64");
  if (kv->length < 0 || kv->length % 8) return fail(WAM_E_SHAPE, "cache length must be a non-negative multiple of 8");
  if ((long)kv->length + rows > kv->capacity)
    return fail(WAM_E_CAPACITY, "cache capacity %d < length %d + %d new rows", kv->capacity, kv->length, rows);
  return WAM_OK;
}

wam_status check_ctx(const Geo& g, const wam_ctx_kv* cx) {
  if (!cx || !cx->k || !cx->v) return fail(WAM_E_ARG, "condition KV pointers are NULL");
  if (unaligned16(cx->k) || unaligned16(cx->v)) return fail(WAM_E_ARG, "condition KV pointers are not 16-byte aligned");
  if (cx->branches != g.br) return fail(WAM_E_SHAPE, "condition KV branches != config branches");
  if (cx->ctx_len != g.Lc) return fail(WAM_E_SHAPE, "condition length %d != %d", cx->ctx_len, g.Lc);
  if (cx->ctx_stride < g.Lc || cx->ctx_stride % 64) return fail(WAM_E_SHAPE, "ctx_stride must be a multiple of 64 >= ctx_len");
  // the image attention reads whole 32-key tiles of value rows that start at column Lt
  if (g.img_x && cx->ctx_stride < g.Lt + (g.Li + 31) / 32 * 32)
    return fail(WAM_E_SHAPE, "ctx_stride must hold ctx_text_len + ctx_img_len rounded up to 32");
  return WAM_OK;
}

// pointers of one layer inside the caches
template <typename X> X* layer_ptr(void* base, size_t elems_per_layer, int l, size_t esz) {
  return reinterpret_cast<X*>(reinterpret_cast<char*>(base) + (size_t)l * elems_per_layer * esz);
}

struct Pass {   // everything one pass needs
  const wam_config* cfg;
  Geo g;
  Layout L;
  void* ws;
  int n;        // chunks in this pass
  int R, M;     // rows per branch, total rows
  wam_kv_cache* kv;
  const wam_ctx_kv* cx;
  float* h;     // residual stream
  const float* e6;
  float2* rope;
  hipStream_t s;
};

RowMap rowmap(const Pass& p) { return RowMap{p.R, p.g.Lq, p.g.Lv}; }

GemmArgs gemm_args(const void* A, long lda, const void* W, long ldw, const void* bias, int M, int N, int K,
                   float* part = nullptr, long part_elems = 0) {
  GemmArgs a{};
  a.A = A; a.lda = lda; a.W = W; a.ldw = ldw; a.bias = reinterpret_cast<const float*>(bias);
  a.M = M; a.N = N; a.K = K;
  a.part = part; a.part_elems = part_elems;
  return a;
}

// AdaLN norm of a block input: y = LN(h) (1 + scale) + shift, rows modulated per chunk and token group
NormArgs adaln_args(const Pass& p, const float* mod, int shift_idx, int scale_idx) {
  NormArgs na{};
  na.X = p.h; na.Y = at<void>(p.ws, p.L.y); na.M = p.M; na.D = p.g.D; na.eps = p.cfg->eps; na.mode = NORM_ADALN;
  na.rm = rowmap(p); na.e6 = p.e6; na.mod = mod; na.shift_idx = shift_idx; na.scale_idx = scale_idx;
  na.rms = (p.cfg->variant & WAM_VARIANT_RMS_NORM) != 0;
  if (p.g.mx) {   // the block norms feed MXFP8 projections: they also write the quantised rows
    na.mxq = at<uint8_t>(p.ws, p.L.xq);
    na.mxs = at<uint8_t>(p.ws, p.L.xs);
  }
  return na;
}

// Output-head norm: y = LN(h) (1 + scale_h) + shift_h
NormArgs head_norm_args(const Pass& p, const wam_weights* w) {
  NormArgs na{};
  na.X = p.h; na.Y = at<void>(p.ws, p.L.y); na.M = p.M; na.D = p.g.D; na.eps = p.cfg->eps; na.mode = NORM_HEAD;
  na.rm = rowmap(p); na.e6 = at<float>(p.ws, p.L.e); na.mod = reinterpret_cast<const float*>(w->head_mod);
  na.rms = (p.cfg->variant & WAM_VARIANT_RMS_NORM) != 0;
  return na;
}

// MXFP8 projections: point the product at the quantised input rows in the workspace (quantising the
// bf16 rows src [M][K] first unless the block norm that wrote them already did) and at the layer's
// packed weights, matrix rows from row0 on.
hipError_t mx_operands(const Pass& p, const wam_block_weights& bw, GemmArgs& ga, const void* src, int mat, int row0) {
  const MxMat mm = mx_block_of(p.g).m[mat];
  uint8_t* xq = at<uint8_t>(p.ws, p.L.xq);
  uint8_t* xs = at<uint8_t>(p.ws, p.L.xs);
  const bool from_norm = mat == MX_QKV || mat == MX_CQ || mat == MX_FF1;
  const hipError_t e = from_norm ? hipSuccess : launch_mx_quantize(src, mm.K, DT_BF16, p.M, mm.K, xq, mm.K, xs, p.s);
  const char* base = reinterpret_cast<const char*>(bw.mx);
  ga.A = xq;
  ga.lda = mm.K;
  ga.As = xs;
  const int wrow = p.g.w4 ? mm.K / 2 : mm.K;   // bytes of one packed weight row
  ga.W = base + mm.codes + (size_t)row0 * wrow;
  ga.ldw = wrow;
  ga.w_fp4 = p.g.w4;
  ga.Ws = reinterpret_cast<const uint8_t*>(base + mm.scales + (size_t)row0 * (mm.K / 32));
  return e;
}

// One block. kv_only: stop after the keys/values of this layer are in the cache. pre_normed: y
// already holds this block's first AdaLN norm (written by the previous block's last product).
// after: the row stage that follows this block (the next block's first norm or the head norm), run
// together with the block's last product; nullptr for none.
wam_status run_block(const Pass& p, const wam_block_weights& bw, int l, bool kv_only, bool pre_normed,
                     const PostArgs* after) {
  const Geo& g = p.g;
  const DType dt = g.dt;
  const float eps = p.cfg->eps;
  const RowMap rm = rowmap(p);
  void* y = at<void>(p.ws, p.L.y);
  void* qkv = at<void>(p.ws, p.L.qkv);
  void* qh = at<void>(p.ws, p.L.qh);
  void* attn = at<void>(p.ws, p.L.attn);
  void* ffn = at<void>(p.ws, p.L.ffn);
  const size_t cache_layer = (size_t)g.br * g.H * p.kv->capacity * g.d;
  void* kc = layer_ptr<void>(p.kv->k, cache_layer, l, g.esz);
  void* vc = layer_ptr<void>(p.kv->v, cache_layer, l, g.esz);
  const int len = p.kv->length;
  const float* mod = reinterpret_cast<const float*>(bw.mod);
  float* part = at<float>(p.ws, p.L.part);
  const long part_n = p.L.part_elems;
  // fragment-packed projections (bf16, native precision): point the product at the packed copy
  const bool packed = dt == DT_BF16 && !g.mx && bw.pk != nullptr;
  const PkBlock pb = pk_block_of(g);
  auto use_packed = [&](GemmArgs& ga, int mat, int row0) {
    if (!packed) return;
    ga.W = reinterpret_cast<const char*>(bw.pk) + pb.off[mat] + (size_t)row0 * pb.K[mat] * 2;
    ga.w_packed = 1;
  };

  // (1) y = LN(h) (1 + scale1) + shift1
  if (!pre_normed) HIP_TRY(launch_norm(adaln_args(p, mod, 0, 1), dt, p.s));
  // (2) [q|k|v] = y Wqkv^T + b  (keys/values only for the last layer of an append)
  {
    const int col0 = kv_only ? g.D : 0;
    GemmArgs ga = gemm_args(y, g.D, reinterpret_cast<const char*>(bw.w_qkv) + (size_t)col0 * g.D * g.esz, g.D,
                            reinterpret_cast<const float*>(bw.b_qkv) + col0, p.M, 3 * g.D - col0, g.D, part, part_n);
    ga.C = reinterpret_cast<char*>(qkv) + (size_t)col0 * g.esz;
    ga.ldc = 3 * g.D;
    use_packed(ga, MX_QKV, col0);
    if (g.mx) HIP_TRY(mx_operands(p, bw, ga, y, MX_QKV, col0));
    QkvTimer& tm = g_qkv_timer;
    const bool timed = tm.layer == l && !kv_only && 2 * tm.n < (int)tm.ev.size();
    if (timed) HIP_TRY(hipEventRecord(tm.ev[2 * tm.n], p.s));
    HIP_TRY(launch_gemm(ga, dt, EPI_STORE, p.s));
    if (timed) {
      HIP_TRY(hipEventRecord(tm.ev[2 * tm.n + 1], p.s));
      ++tm.n;
    }
  }
  // (3) RMSNorm + RoPE of q (head-major) and k (into the cache), values into the cache
  QkNormArgs qa{};
  qa.src = qkv; qa.src_ld = 3 * g.D; qa.M = p.M; qa.D = g.D; qa.H = g.H; qa.d = g.d; qa.rows_per_branch = p.R;
  qa.eps = eps; qa.rope = p.rope; qa.rm = rm;
  qa.src_col = 0; qa.gain = reinterpret_cast<const float*>(bw.g_q);
  qa.dst = qh; qa.dst_bh_stride = (long)p.R * g.d; qa.dst_row0 = 0;
  QkNormArgs ka = qa;
  ka.src_col = g.D; ka.gain = reinterpret_cast<const float*>(bw.g_k);
  ka.dst = kc; ka.dst_bh_stride = (long)p.kv->capacity * g.d; ka.dst_row0 = len;
  VCacheArgs va{};
  va.src = qkv; va.src_ld = 3 * g.D; va.src_col = 2 * g.D; va.dst = vc; va.dst_bh_stride = (long)g.d * p.kv->capacity;
  va.dst_stride = p.kv->capacity; va.dst_col0 = len; va.rows_per_branch = p.R; va.br = g.br; va.H = g.H; va.d = g.d;
  HIP_TRY(launch_qkv_cache(kv_only ? nullptr : &qa, ka, va, dt, p.s));
  if (kv_only) return WAM_OK;

  // (4) chunk-causal self-attention over [cache ; this pass]
  AttnArgs aa{};
  aa.Q = qh; aa.K = kc; aa.Vt = vc; aa.O = attn;
  aa.q_bh_stride = (long)p.R * g.d; aa.k_bh_stride = (long)p.kv->capacity * g.d; aa.v_bh_stride = (long)g.d * p.kv->capacity;
  aa.v_stride = p.kv->capacity; aa.Lq_total = p.R; aa.H = g.H; aa.d = g.d; aa.br = g.br;
  const bool frame_causal = (p.cfg->variant & WAM_VARIANT_FRAME_CAUSAL) != 0;
  aa.kv_base = len; aa.chunk_q = p.n > 1 || frame_causal ? g.Lq : 0; aa.kv_total = len + p.R;
  aa.frame_tokens = frame_causal ? p.cfg->grid_h * p.cfg->grid_w : 0; aa.video_tokens = g.Lv;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)g.d));
  aa.part = part; aa.part_elems = part_n;
  HIP_TRY(launch_attention(aa, dt, p.s));
  // (5) h += gate1 * (o Wo^T + b), then (6) n3 = LN(h) w + b for the cross-attention queries
  {
    GemmArgs ga = gemm_args(attn, g.D, bw.w_o, g.D, bw.b_o, p.M, g.D, g.D, part, part_n);
    ga.H = p.h; ga.ldh = g.D; ga.rm = rm; ga.e6 = p.e6; ga.mod = mod; ga.gate_idx = 2; ga.D = g.D;
    PostArgs post{};
    post.mode = POST_NORM;
    post.na = adaln_args(p, mod, 0, 1);
    post.na.mode = NORM_AFFINE; post.na.w = reinterpret_cast<const float*>(bw.ln3_w);
    post.na.b = reinterpret_cast<const float*>(bw.ln3_b);
    use_packed(ga, MX_O, 0);
    if (g.mx) HIP_TRY(mx_operands(p, bw, ga, attn, MX_O, 0));
    HIP_TRY(launch_gemm_post(ga, dt, EPI_RESID_GATED, post, p.s));
  }
  // qc = RMS(n3 Wcq^T + b) g, head-major
  {
    GemmArgs ga = gemm_args(y, g.D, bw.w_cq, g.D, bw.b_cq, p.M, g.D, g.D, part, part_n);
    ga.C = qkv; ga.ldc = g.D;
    PostArgs post{};
    post.mode = POST_QK;
    post.qa = qa;
    post.qa.src_ld = g.D; post.qa.src_col = 0; post.qa.gain = reinterpret_cast<const float*>(bw.g_cq); post.qa.rope = nullptr;
    post.qa.dst = qh; post.qa.dst_bh_stride = (long)p.R * g.d; post.qa.dst_row0 = 0;
    use_packed(ga, MX_CQ, 0);
    if (g.mx) HIP_TRY(mx_operands(p, bw, ga, y, MX_CQ, 0));
    HIP_TRY(launch_gemm_post(ga, dt, EPI_STORE, post, p.s));
  }
  {
    const size_t ck_layer = (size_t)g.br * g.H * g.Lc * g.d, cv_layer = (size_t)g.br * g.H * g.d * p.cx->ctx_stride;
    AttnArgs ca{};
    ca.Q = qh; ca.K = layer_ptr<void>(p.cx->k, ck_layer, l, g.esz); ca.Vt = layer_ptr<void>(p.cx->v, cv_layer, l, g.esz);
    ca.O = attn; ca.q_bh_stride = (long)p.R * g.d; ca.k_bh_stride = (long)g.Lc * g.d;
    ca.v_bh_stride = (long)g.d * p.cx->ctx_stride; ca.v_stride = p.cx->ctx_stride;
    ca.Lq_total = p.R; ca.H = g.H; ca.d = g.d; ca.br = g.br; ca.kv_base = g.Lc; ca.chunk_q = 0; ca.kv_total = g.Lc;
    ca.scale_log2 = aa.scale_log2;
    ca.part = part; ca.part_elems = part_n;
    if (!g.img_x) {
      HIP_TRY(launch_attention(ca, dt, p.s));
    } else {   // text rows and image rows, each with its own softmax; the outputs are summed
      const int Li = g.Li;
      ca.kv_base = ca.kv_total = g.Lt;
      HIP_TRY(launch_attention(ca, dt, p.s));
      AttnArgs ci = ca;
      ci.K = reinterpret_cast<const char*>(ca.K) + (size_t)g.Lt * g.d * g.esz;
      ci.Vt = reinterpret_cast<const char*>(ca.Vt) + (size_t)g.Lt * g.esz;
      ci.kv_base = ci.kv_total = Li;
      ci.O = qkv;   // free here: the cross queries are already in qh
      HIP_TRY(launch_attention(ci, dt, p.s));
      HIP_TRY(launch_add(attn, qkv, (long)p.M * g.D, dt, p.s));
    }
  }
  // h += o Wco^T + b, then (7) y2 = LN(h) (1 + scale2) + shift2
  {
    GemmArgs ga = gemm_args(attn, g.D, bw.w_co, g.D, bw.b_co, p.M, g.D, g.D, part, part_n);
    ga.H = p.h; ga.ldh = g.D;
    PostArgs post{};
    post.mode = POST_NORM;
    post.na = adaln_args(p, mod, 3, 4);
    use_packed(ga, MX_CO, 0);
    if (g.mx) HIP_TRY(mx_operands(p, bw, ga, attn, MX_CO, 0));
    HIP_TRY(launch_gemm_post(ga, dt, EPI_RESID, post, p.s));
  }
  // FFN: h += gate2 * (GELU(y2 W1^T + b1) W2^T + b2); SwiGLU variant: W1 has 2F interleaved
  // [gate, up] rows and the product's epilogue writes SiLU(gate) * up
  {
    const bool swiglu = (p.cfg->variant & WAM_VARIANT_SWIGLU) != 0;
    GemmArgs ga = gemm_args(y, g.D, bw.w_ff1, g.D, bw.b_ff1, p.M, swiglu ? 2 * g.F : g.F, g.D, part, part_n);
    ga.C = ffn; ga.ldc = g.F;
    use_packed(ga, MX_FF1, 0);
    if (g.mx) HIP_TRY(mx_operands(p, bw, ga, y, MX_FF1, 0));
    HIP_TRY(launch_gemm(ga, dt, swiglu ? EPI_SWIGLU : EPI_GELU, p.s));
  }
  {
    GemmArgs ga = gemm_args(ffn, g.F, bw.w_ff2, g.F, bw.b_ff2, p.M, g.D, g.F, part, part_n);
    ga.H = p.h; ga.ldh = g.D; ga.rm = rm; ga.e6 = p.e6; ga.mod = mod; ga.gate_idx = 5; ga.D = g.D;
    PostArgs none{};
    none.mode = POST_NONE;
    use_packed(ga, MX_FF2, 0);
    if (g.mx) HIP_TRY(mx_operands(p, bw, ga, ffn, MX_FF2, 0));
    HIP_TRY(launch_gemm_post(ga, dt, EPI_RESID_GATED, after ? *after : none, p.s));
  }
  return WAM_OK;
}

wam_status time_embed(const Pass& p, const wam_weights* w, const float* t, int G, float* e, float* e6) {
  TimeArgs ta{};
  for (int i = 0; i < G; ++i) ta.t[i] = t[i];
  ta.G = G; ta.freq_dim = p.g.freq; ta.D = p.g.D;
  ta.w1 = w->t_w1; ta.w2 = w->t_w2; ta.wp = w->t_wp;
  ta.b1 = reinterpret_cast<const float*>(w->t_b1); ta.b2 = reinterpret_cast<const float*>(w->t_b2);
  ta.bp = reinterpret_cast<const float*>(w->t_bp);
  ta.emb = at<float>(p.ws, p.L.emb); ta.h1 = at<float>(p.ws, p.L.h1); ta.e = e; ta.e6 = e6;
  HIP_TRY(launch_time_mlp(ta, p.g.dt, p.s));
  return WAM_OK;
}

wam_status check_ws(const Layout& L, void* ws, size_t ws_bytes) {
  if (!ws) return fail(WAM_E_ARG, "workspace is NULL");
  if (ws_bytes < L.total) return fail(WAM_E_ARG, "workspace of %zu bytes < %zu needed", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(WAM_E_ARG, "workspace must be 256-byte aligned");
  return WAM_OK;
}

#define CHECK(expr)                      \
  do {                                   \
    wam_status st_ = (expr);             \
    if (st_ != WAM_OK) return st_;       \
  } while (0)

// the whole stack: time MLP, rotary table, embedding, blocks, heads (or only the K/V of an append)
wam_status stack_pass(const wam_config* cfg, const wam_weights* w, wam_kv_cache* kv, const wam_ctx_kv* cx, int n,
                      const float* xv, const float* xa, const float* tv, const float* ta, int start_frame,
                      float* vv, float* va, void* ws, size_t ws_bytes, hipStream_t s, bool append) {
  CHECK(check_cfg(cfg));
  const Geo g = geo_of(*cfg);
  if (n < 1 || n > kMaxChunks) return fail(WAM_E_SHAPE, "n_chunks must be in [1, %d]", kMaxChunks);
  CHECK(check_weights(cfg, w, true));
  CHECK(check_cache(g, kv, n * g.Lq));
  CHECK(check_ctx(g, cx));
  if (!xv || !xa) return fail(WAM_E_ARG, "latent pointers are NULL");
  if (!append && (!vv || !va || !tv || !ta)) return fail(WAM_E_ARG, "output or timestep pointers are NULL");
  if (start_frame < 0) return fail(WAM_E_ARG, "start_frame must be non-negative");
  const Layout L = layout_of(g, n);
  CHECK(check_ws(L, ws, ws_bytes));

  Pass p{};
  p.cfg = cfg; p.g = g; p.L = L; p.ws = ws; p.n = n; p.R = n * g.Lq; p.M = g.br * p.R; p.kv = kv; p.cx = cx;
  p.h = at<float>(ws, L.h); p.e6 = at<float>(ws, L.e6); p.rope = at<float2>(ws, L.rope); p.s = s;

  float tt[2 * kMaxChunks];
  for (int c = 0; c < n; ++c) {
    tt[2 * c] = append ? 1.f : tv[c];
    tt[2 * c + 1] = append ? 1.f : ta[c];
  }
  CHECK(time_embed(p, w, tt, 2 * n, at<float>(ws, L.e), at<float>(ws, L.e6)));
  HIP_TRY(launch_rope_table(p.rope, n, g.Lq, g.Lv, cfg->frames_per_chunk, cfg->grid_h, cfg->grid_w, start_frame, g.d,
                            cfg->rope_theta, s));
  EmbedArgs ea{};
  ea.xv = xv; ea.xa = xa; ea.pe_w = w->pe_w; ea.pe_b = reinterpret_cast<const float*>(w->pe_b);
  ea.ae_w = w->ae_w; ea.ae_b = reinterpret_cast<const float*>(w->ae_b); ea.H = p.h;
  ea.n_chunks = n; ea.Lv = g.Lv; ea.La = g.La; ea.P = g.P; ea.A = g.A; ea.D = g.D; ea.br = g.br;
  HIP_TRY(launch_embed(ea, g.dt, s));
  // Each block's first norm runs with the previous block's last product (the first one on its own);
  // the last block's product also runs the output-head norm.
  HIP_TRY(launch_norm(adaln_args(p, reinterpret_cast<const float*>(w->blocks[0].mod), 0, 1), g.dt, s));
  for (int l = 0; l < g.L; ++l) {
    PostArgs after{};
    const PostArgs* ap = nullptr;
    if (l + 1 < g.L) {
      after.mode = POST_NORM;
      after.na = adaln_args(p, reinterpret_cast<const float*>(w->blocks[l + 1].mod), 0, 1);
      ap = &after;
    } else if (!append) {
      after.mode = POST_NORM;
      after.na = head_norm_args(p, w);
      ap = &after;
    }
    CHECK(run_block(p, w->blocks[l], l, append && l == g.L - 1, true, ap));
  }
  if (append) return WAM_OK;

  // heads: v_video / v_action per token group from y = LN(h) (1 + scale_h) + shift_h
  HeadArgs hd{};
  hd.Y = at<void>(ws, L.y); hd.M = p.M; hd.D = g.D;
  hd.wv = w->vo_w; hd.bv = reinterpret_cast<const float*>(w->vo_b); hd.P = g.P;
  hd.wa = w->ao_w; hd.ba = reinterpret_cast<const float*>(w->ao_b); hd.A = g.A;
  hd.vv = vv; hd.va = va; hd.rm = rowmap(p);
  hd.part = at<float>(ws, L.part);
  hd.part_elems = L.part_elems;
  HIP_TRY(launch_head(hd, g.dt, s));
  return WAM_OK;
}

}  // namespace

extern "C" {

size_t wam_workspace_bytes(const wam_config* cfg, int n_chunks) {
  if (check_cfg(cfg) != WAM_OK || n_chunks < 1 || n_chunks > kMaxChunks) return 0;
  return layout_of(geo_of(*cfg), n_chunks).total;
}

wam_status wam_ctx_build(const wam_config* cfg, const wam_weights* w, const void* txt, const void* img,
                         const void* state, wam_ctx_kv* out, void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  const Geo g = geo_of(*cfg);
  CHECK(check_weights(cfg, w, true));
  CHECK(check_ctx(g, out));
  if (!txt || !w->txt_w || !w->txt_b) return fail(WAM_E_ARG, "text features or text projection are NULL");
  if (cfg->ctx_img_len > 0 && (!img || !w->img_w || !w->img_b)) return fail(WAM_E_ARG, "image features or projection are NULL");
  if (cfg->ctx_state_len > 0 && (!state || unaligned16(state))) return fail(WAM_E_ARG, "state is NULL or not 16-byte aligned");
  const Layout L = layout_of(g, 1);
  CHECK(check_ws(L, ws, ws_bytes));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ctx = at<void>(ws, L.ctx_a);
  void* tmp = at<void>(ws, L.ctx_b);
  float* part = at<float>(ws, L.part);
  const long part_n = L.part_elems;
  const int Lt = cfg->ctx_text_len, Li = cfg->ctx_img_len;
  for (int b = 0; b < g.br; ++b) {
    GemmArgs gt = gemm_args(reinterpret_cast<const char*>(txt) + (size_t)b * Lt * g.Cin * g.esz, g.Cin, w->txt_w, g.Cin,
                            w->txt_b, Lt, g.D, g.Cin, part, part_n);
    gt.C = reinterpret_cast<char*>(ctx) + (size_t)b * g.Lc * g.D * g.esz; gt.ldc = g.D;
    HIP_TRY(launch_gemm(gt, g.dt, EPI_STORE, s));
    if (Li > 0) {
      GemmArgs gi = gemm_args(img, g.Cin, w->img_w, g.Cin, w->img_b, Li, g.D, g.Cin, part, part_n);
      gi.C = reinterpret_cast<char*>(ctx) + ((size_t)b * g.Lc + Lt) * g.D * g.esz; gi.ldc = g.D;
      HIP_TRY(launch_gemm(gi, g.dt, EPI_STORE, s));
    }
    if (g.Ls > 0) {   // state rows after the image rows
      GemmArgs gs = gemm_args(state, g.Sd, w->st_w, g.Sd, w->st_b, g.Ls, g.D, g.Sd, part, part_n);
      gs.C = reinterpret_cast<char*>(ctx) + ((size_t)b * g.Lc + Lt + Li) * g.D * g.esz; gs.ldc = g.D;
      HIP_TRY(launch_gemm(gs, g.dt, EPI_STORE, s));
    }
  }
  const int M = g.br * g.Lc;
  const size_t ck_layer = (size_t)g.br * g.H * g.Lc * g.d, cv_layer = (size_t)g.br * g.H * g.d * out->ctx_stride;
  for (int l = 0; l < g.L; ++l) {
    const wam_block_weights& bw = w->blocks[l];
    GemmArgs gk = gemm_args(ctx, g.D, bw.w_ck, g.D, bw.b_ck, M, g.D, g.D, part, part_n);
    gk.C = tmp; gk.ldc = g.D;
    HIP_TRY(launch_gemm(gk, g.dt, EPI_STORE, s));
    QkNormArgs qa{};
    qa.src = tmp; qa.src_ld = g.D; qa.src_col = 0; qa.gain = reinterpret_cast<const float*>(bw.g_ck);
    qa.dst = layer_ptr<void>(out->k, ck_layer, l, g.esz); qa.dst_bh_stride = (long)g.Lc * g.d; qa.dst_row0 = 0;
    qa.M = M; qa.D = g.D; qa.H = g.H; qa.d = g.d; qa.rows_per_branch = g.Lc; qa.eps = cfg->eps; qa.rope = nullptr;
    qa.rm = RowMap{g.Lc, g.Lc, g.Lc};
    HIP_TRY(launch_qk_norm_rope(qa, g.dt, s));
    GemmArgs gv = gemm_args(ctx, g.D, bw.w_cv, g.D, bw.b_cv, M, g.D, g.D, part, part_n);
    gv.C = tmp; gv.ldc = g.D;
    HIP_TRY(launch_gemm(gv, g.dt, EPI_STORE, s));
    VCacheArgs va{};
    va.src = tmp; va.src_ld = g.D; va.src_col = 0; va.dst = layer_ptr<void>(out->v, cv_layer, l, g.esz);
    va.dst_bh_stride = (long)g.d * out->ctx_stride; va.dst_stride = out->ctx_stride; va.dst_col0 = 0;
    va.rows_per_branch = g.Lc; va.br = g.br; va.H = g.H; va.d = g.d;
    HIP_TRY(launch_v_to_cache(va, g.dt, s));
    if (g.img_x) {   // image rows of each branch again, with the image projections and gain
      const int Li = g.Li;
      for (int b = 0; b < g.br; ++b) {
        const char* src = reinterpret_cast<const char*>(ctx) + ((size_t)b * g.Lc + g.Lt) * g.D * g.esz;
        GemmArgs ik = gemm_args(src, g.D, bw.w_cki, g.D, bw.b_cki, Li, g.D, g.D, part, part_n);
        ik.C = tmp; ik.ldc = g.D;
        HIP_TRY(launch_gemm(ik, g.dt, EPI_STORE, s));
        QkNormArgs iq = qa;
        iq.src = tmp; iq.gain = reinterpret_cast<const float*>(bw.g_cki); iq.M = Li; iq.rows_per_branch = Li;
        iq.dst = layer_ptr<char>(out->k, ck_layer, l, g.esz) + (size_t)b * g.H * g.Lc * g.d * g.esz;
        iq.dst_row0 = g.Lt; iq.rm = RowMap{Li, Li, Li};
        HIP_TRY(launch_qk_norm_rope(iq, g.dt, s));
        GemmArgs iv = gemm_args(src, g.D, bw.w_cvi, g.D, bw.b_cvi, Li, g.D, g.D, part, part_n);
        iv.C = tmp; iv.ldc = g.D;
        HIP_TRY(launch_gemm(iv, g.dt, EPI_STORE, s));
        VCacheArgs ia = va;
        ia.src = tmp; ia.dst = layer_ptr<char>(out->v, cv_layer, l, g.esz) + (size_t)b * g.H * g.d * out->ctx_stride * g.esz;
        ia.dst_col0 = g.Lt; ia.rows_per_branch = Li; ia.br = 1;
        HIP_TRY(launch_v_to_cache(ia, g.dt, s));
      }
    }
  }
  return WAM_OK;
}

wam_status wam_ctx_set_state(const wam_config* cfg, const wam_weights* w, const void* state, wam_ctx_kv* ctx,
                             void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  const Geo g = geo_of(*cfg);
  if (g.Ls <= 0) return fail(WAM_E_SHAPE, "the configuration has no state rows (ctx_state_len = 0)");
  CHECK(check_weights(cfg, w, true));
  CHECK(check_ctx(g, ctx));
  if (!state || unaligned16(state)) return fail(WAM_E_ARG, "state is NULL or not 16-byte aligned");
  const Layout L = layout_of(g, 1);
  CHECK(check_ws(L, ws, ws_bytes));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* emb = at<void>(ws, L.ctx_a);   // [Ls][D]
  void* tmp = at<void>(ws, L.ctx_b);   // [Ls][D]
  float* part = at<float>(ws, L.part);
  const long part_n = L.part_elems;
  // a few rows: each projection as a row-parallel product over N / 32 workgroups
  const bool gemv = g.Ls <= 4;
  auto project = [&](const void* x, const void* W, const void* b, int K, void* y) -> hipError_t {
    if (gemv) return launch_gemv_store(W, reinterpret_cast<const float*>(b), x, K, y, g.D, g.Ls, g.D, K, g.dt, s);
    GemmArgs ga = gemm_args(x, K, W, K, b, g.Ls, g.D, K, part, part_n);
    ga.C = y; ga.ldc = g.D;
    return launch_gemm(ga, g.dt, EPI_STORE, s);
  };
  HIP_TRY(project(state, w->st_w, w->st_b, g.Sd, emb));
  const int row0 = g.Lt + g.Li;
  const size_t ck_layer = (size_t)g.br * g.H * g.Lc * g.d, cv_layer = (size_t)g.br * g.H * g.d * ctx->ctx_stride;
  for (int l = 0; l < g.L; ++l) {   // the rows are the same for both branches: project once, write per branch
    const wam_block_weights& bw = w->blocks[l];
    HIP_TRY(project(emb, bw.w_ck, bw.b_ck, g.D, tmp));
    for (int b = 0; b < g.br; ++b) {
      QkNormArgs qa{};
      qa.src = tmp; qa.src_ld = g.D; qa.src_col = 0; qa.gain = reinterpret_cast<const float*>(bw.g_ck);
      qa.dst = layer_ptr<char>(ctx->k, ck_layer, l, g.esz) + (size_t)b * g.H * g.Lc * g.d * g.esz;
      qa.dst_bh_stride = (long)g.Lc * g.d; qa.dst_row0 = row0;
      qa.M = g.Ls; qa.D = g.D; qa.H = g.H; qa.d = g.d; qa.rows_per_branch = g.Ls; qa.eps = cfg->eps; qa.rope = nullptr;
      qa.rm = RowMap{g.Ls, g.Ls, g.Ls};
      HIP_TRY(launch_qk_norm_rope(qa, g.dt, s));
    }
    HIP_TRY(project(emb, bw.w_cv, bw.b_cv, g.D, tmp));
    for (int b = 0; b < g.br; ++b) {
      VCacheArgs va{};
      va.src = tmp; va.src_ld = g.D; va.src_col = 0;
      va.dst = layer_ptr<char>(ctx->v, cv_layer, l, g.esz) + (size_t)b * g.H * g.d * ctx->ctx_stride * g.esz;
      va.dst_bh_stride = (long)g.d * ctx->ctx_stride; va.dst_stride = ctx->ctx_stride; va.dst_col0 = row0;
      va.rows_per_branch = g.Ls; va.br = 1; va.H = g.H; va.d = g.d;
      HIP_TRY(launch_v_to_cache(va, g.dt, s));
    }
  }
  return WAM_OK;
}

wam_status wam_time_embed(const wam_config* cfg, const wam_weights* w, const float* t, int n, float* e, float* e6,
                          void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  CHECK(check_weights(cfg, w, false));
  if (!t || !e || !e6) return fail(WAM_E_ARG, "timestep or output pointers are NULL");
  if (n < 1 || n > 2 * kMaxChunks) return fail(WAM_E_SHAPE, "n must be in [1, %d]", 2 * kMaxChunks);
  Pass p{};
  p.cfg = cfg; p.g = geo_of(*cfg); p.L = layout_of(p.g, kMaxChunks); p.ws = ws;
  p.s = reinterpret_cast<hipStream_t>(stream);
  const Layout need = layout_of(p.g, (n + 1) / 2);
  CHECK(check_ws(need, ws, ws_bytes));
  p.L = need;
  return time_embed(p, w, t, n, e, e6);
}

wam_status wam_dit_stack_fwd(const wam_config* cfg, const wam_weights* w, wam_kv_cache* cache, const wam_ctx_kv* ctx,
                             int n_chunks, const float* x_video, const float* x_action, const float* t_video,
                             const float* t_action, int start_frame, float* v_video, float* v_action, void* ws,
                             size_t ws_bytes, void* stream) {
  return stack_pass(cfg, w, cache, ctx, n_chunks, x_video, x_action, t_video, t_action, start_frame, v_video, v_action,
                    ws, ws_bytes, reinterpret_cast<hipStream_t>(stream), false);
}

wam_status wam_kv_append(const wam_config* cfg, const wam_weights* w, wam_kv_cache* cache, const wam_ctx_kv* ctx,
                         const float* x_video, const float* x_action, int start_frame, void* ws, size_t ws_bytes,
                         void* stream) {
  wam_status st = stack_pass(cfg, w, cache, ctx, 1, x_video, x_action, nullptr, nullptr, start_frame, nullptr, nullptr,
                             ws, ws_bytes, reinterpret_cast<hipStream_t>(stream), true);
  if (st == WAM_OK) cache->length += geo_of(*cfg).Lq;
  return st;
}

wam_status wam_dit_block_fwd(const wam_config* cfg, const wam_block_weights* bw, int layer, wam_kv_cache* cache,
                             const wam_ctx_kv* ctx, float* h, const float* e6, int n_chunks, int start_frame, int commit,
                             void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(cfg));
  const Geo g = geo_of(*cfg);
  if (layer < 0 || layer >= g.L) return fail(WAM_E_ARG, "layer %d out of range", layer);
  if (n_chunks < 1 || n_chunks > kMaxChunks) return fail(WAM_E_SHAPE, "n_chunks must be in [1, %d]", kMaxChunks);
  CHECK(check_block(bw, layer, g.mx, g.img_x, g.dt == DT_BF16 && !g.mx, pk_fits(g)));
  CHECK(check_cache(g, cache, n_chunks * g.Lq));
  CHECK(check_ctx(g, ctx));
  if (!h || !e6) return fail(WAM_E_ARG, "h or e6 is NULL");
  if (start_frame < 0) return fail(WAM_E_ARG, "start_frame must be non-negative");
  const Layout L = layout_of(g, n_chunks);
  CHECK(check_ws(L, ws, ws_bytes));
  Pass p{};
  p.cfg = cfg; p.g = g; p.L = L; p.ws = ws; p.n = n_chunks; p.R = n_chunks * g.Lq; p.M = g.br * p.R; p.kv = cache;
  p.cx = ctx; p.h = h; p.e6 = e6; p.rope = at<float2>(ws, L.rope); p.s = reinterpret_cast<hipStream_t>(stream);
  HIP_TRY(launch_rope_table(p.rope, n_chunks, g.Lq, g.Lv, cfg->frames_per_chunk, cfg->grid_h, cfg->grid_w, start_frame,
                            g.d, cfg->rope_theta, p.s));
  CHECK(run_block(p, *bw, layer, false, false, nullptr));
  if (commit) cache->length += n_chunks * g.Lq;
  return WAM_OK;
}

}  // extern "C"

namespace {

// Validation and launch shared by wam_flow_step and wam_flow_step_noalloc: the cosine partials go to
// the caller's workspace (ws, ws_bytes), or with library_scratch to the library's device scratch.
wam_status flow_step(float* x_video, float* x_action, const float* v_video, const float* v_action, int branches,
                     float guidance, int n_video, int n_action, float dt_video, float dt_action, float* g_video,
                     float* g_action, const float* prev_video, float* cos_parts, void* ws, size_t ws_bytes,
                     bool library_scratch, void* stream) {
  if (branches != 1 && branches != 2) return fail(WAM_E_SHAPE, "branches must be 1 or 2");
  if (n_video < 0 || n_action < 0) return fail(WAM_E_SHAPE, "negative sizes");
  if ((n_video && (!x_video || !v_video)) || (n_action && (!x_action || !v_action)))
    return fail(WAM_E_ARG, "latent or velocity pointers are NULL");
  if (prev_video && !cos_parts) return fail(WAM_E_ARG, "prev_video given without cos_parts");
  if (!std::isfinite(guidance) || !std::isfinite(dt_video) || !std::isfinite(dt_action))
    return fail(WAM_E_ARG, "non-finite scalar");
  const int nblocks = flow_partial_blocks(n_video, n_action);
  const size_t need = (size_t)nblocks * 3 * 4;
  float* partials = nullptr;
  if (prev_video && library_scratch) {
    size_t have = 0;
    HIP_TRY(flow_scratch(&partials, &have));
    if (need > have)
      return fail(WAM_E_ARG, "cosine partials need %zu bytes, above the %zu-byte library scratch", need, have);
  } else if (prev_video) {
    if (!ws || ws_bytes < need) return fail(WAM_E_ARG, "workspace too small for the cosine partials");
    partials = reinterpret_cast<float*>(ws);
  }
  FlowArgs fa{};
  fa.xv = x_video; fa.xa = x_action; fa.vv = v_video; fa.va = v_action; fa.br = branches; fa.w = guidance;
  fa.nv = n_video; fa.na = n_action; fa.dtv = dt_video; fa.dta = dt_action; fa.gv = g_video; fa.ga = g_action;
  fa.prev = prev_video; fa.partials = partials; fa.cos_parts = cos_parts;
  fa.nblocks = nblocks;
  HIP_TRY(launch_flow_step(fa, reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

}  // namespace

extern "C" {

wam_status wam_flow_step(float* x_video, float* x_action, const float* v_video, const float* v_action, int branches,
                         float guidance, int n_video, int n_action, float dt_video, float dt_action, float* g_video,
                         float* g_action, const float* prev_video, float* cos_parts, void* ws, size_t ws_bytes,
                         void* stream) {
  return flow_step(x_video, x_action, v_video, v_action, branches, guidance, n_video, n_action, dt_video, dt_action,
                   g_video, g_action, prev_video, cos_parts, ws, ws_bytes, false, stream);
}

wam_status wam_flow_step_noalloc(float* x_video, float* x_action, const float* v_video, const float* v_action,
                                 int branches, float guidance, int n_video, int n_action, float dt_video,
                                 float dt_action, float* g_video, float* g_action, const float* prev_video,
                                 float* cos_parts, void* stream) {
  return flow_step(x_video, x_action, v_video, v_action, branches, guidance, n_video, n_action, dt_video, dt_action,
                   g_video, g_action, prev_video, cos_parts, nullptr, 0, true, stream);
}

// ---- solvers of the denoising loop ------------------------------------------------------------------
// UniPC ([WS1] names it as the scheduler's solver; the published predictor UniP-p / corrector
// UniC-p in data-prediction form with B(h) = e^h - 1), for alpha_t = t, sigma_t = 1 - t,
// lambda_t = log(alpha_t / sigma_t): from s to t with h = lambda_t - lambda_s, earlier outputs at
// r_j = (lambda_j - lambda_s) / h (the corrector's new output at r = 1), D_j = (m_j - m_s) / r_j,
// h_phi_1 = e^{-h} - 1, h_phi_{k+1} = h_phi_k / (-h) - 1/k!, sum_j rho_j r_j^k = h_phi_{k+2} (k+1)! / B_h,
// x_t = (sigma_t / sigma_s) x_s - alpha_t h_phi_1 m_s - alpha_t B_h sum_j rho_j D_j.
// Weights are formed in double: x_new = a x_s + w[0] m_s + sum_j w[j] m_j (new output last).
struct UniUpdate {
  double a = 0.0;
  double w[5] = {0, 0, 0, 0, 0};
  int n = 0;   // entries of w used
};

static double half_log_snr(double t) { return std::log(t / (1.0 - t)); }

static UniUpdate unipc_update(double t_t, const double* hist, int order, bool corrector) {
  UniUpdate u;
  const double ts = hist[0];
  const double e = (ts * (1.0 - t_t)) / ((1.0 - ts) * t_t);   // e^{-h}: 0 from t = 0 or to t = 1
  const double z = e > 0.0 ? std::log(e) : -INFINITY;         // -h
  double hphi[6];                                             // hphi[k] = h_phi_{k+1}
  hphi[0] = e - 1.0;
  double fact = 1.0;
  for (int k = 1; k < 6; ++k) {
    fact *= k;
    hphi[k] = hphi[k - 1] / z - 1.0 / fact;
  }
  const double b_h = e - 1.0;
  double r[4];
  int nr = 0;
  for (int j = 1; j < order; ++j) r[nr++] = (half_log_snr(hist[j]) - half_log_snr(ts)) / -z;
  if (corrector) r[nr++] = 1.0;
  u.a = (1.0 - t_t) / (1.0 - ts);
  u.n = 1 + nr;
  u.w[0] = -t_t * hphi[0];
  if (nr == 0) return u;
  // Vandermonde system, Gaussian elimination with partial pivoting (nr <= 4)
  double A[4][5];
  fact = 1.0;
  for (int k = 0; k < nr; ++k) {
    fact *= (k + 1);
    for (int j = 0; j < nr; ++j) A[k][j] = std::pow(r[j], k);
    A[k][nr] = hphi[k + 1] * fact / b_h;
  }
  for (int c = 0; c < nr; ++c) {
    int piv = c;
    for (int i = c + 1; i < nr; ++i)
      if (std::fabs(A[i][c]) > std::fabs(A[piv][c])) piv = i;
    for (int j = 0; j <= nr; ++j) std::swap(A[c][j], A[piv][j]);
    for (int i = c + 1; i < nr; ++i) {
      const double f = A[i][c] / A[c][c];
      for (int j = c; j <= nr; ++j) A[i][j] -= f * A[c][j];
    }
  }
  double rho[4];
  for (int i = nr - 1; i >= 0; --i) {
    double acc = A[i][nr];
    for (int j = i + 1; j < nr; ++j) acc -= A[i][j] * rho[j];
    rho[i] = acc / A[i][i];
  }
  for (int j = 0; j < nr; ++j) {
    const double c = -t_t * b_h * rho[j] / r[j];
    u.w[j + 1] += c;
    u.w[0] -= c;
  }
  return u;
}

// predictor order of step k: 1 from t = 0, to t = 1 and after a step from t = 0 (lambda infinite)
static int unipc_order(const float* grid, int k, int order) {
  if (grid[k] <= 0.f || grid[k + 1] >= 1.f) return 1;
  int u = 1;
  while (u < order && k - u >= 0 && grid[k - u] > 0.f) ++u;
  return u;
}

// The chunk's denoising loop with CFG and velocity reuse; order 0 = Euler, 1..3 = UniPC.
static wam_status denoise_loop(const wam_config* cfg, const wam_weights* w, wam_kv_cache* cache, const wam_ctx_kv* ctx,
                               float* x_video, float* x_action, const float* grid, int n_steps, float guidance,
                               float tau, int max_consecutive_reuse, int start_frame, int order, bool corrector,
                               float* v_video, float* v_action, float* g_video, float* g_action, float* cos_parts,
                               float* state, void* ws, size_t ws_bytes, void* stream, int* dit_calls,
                               unsigned char* reused, const unsigned char* replay = nullptr,
                               float* cos_host = nullptr) {
  CHECK(check_cfg(cfg));
  if (!grid || n_steps < 1) return fail(WAM_E_ARG, "grid must hold n_steps + 1 >= 2 times");
  for (int k = 0; k <= n_steps; ++k)
    if (!std::isfinite(grid[k])) return fail(WAM_E_ARG, "non-finite time in the grid");
  if (!g_video || !g_action || !cos_parts) return fail(WAM_E_ARG, "guided-velocity or cosine buffers are NULL");
  if (!std::isfinite(tau) && !std::isinf(tau)) return fail(WAM_E_ARG, "tau is NaN");
  if (replay)
    for (int k = 0; k < std::min(n_steps, 2); ++k)
      if (replay[k]) return fail(WAM_E_ARG, "steps 0 and 1 always run the DiT: replay[%d] must be 0", k);
  if (order > 0) {
    if (order > 3) return fail(WAM_E_ARG, "UniPC order must be 1, 2 or 3");
    if (!state) return fail(WAM_E_ARG, "UniPC state buffer is NULL");
    if (grid[0] < 0.f || grid[n_steps] > 1.f) return fail(WAM_E_ARG, "UniPC times must lie in [0, 1]");
    for (int k = 0; k < n_steps; ++k)
      if (!(grid[k + 1] > grid[k])) return fail(WAM_E_ARG, "UniPC times must increase strictly");
    const size_t need = 256 + 64 * 3 * 4;
    if (!ws || ws_bytes < need) return fail(WAM_E_ARG, "workspace too small");
  }
  const Geo g = geo_of(*cfg);
  const int nv = g.Lv * g.P, na = g.La * g.A;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // reuse needs cos > tau with cos <= 1: a tau above 1 can never trigger it (no host read-back then);
  // a replayed mask decides by itself and reads the cosine back only to report it
  const bool may_reuse = !replay && tau <= 1.f;
  const bool read_cos = may_reuse || cos_host;
  int computed = 0, consecutive = 0, calls = 0, prev_order = 0;
  double cos_last = -2.0;   // cosine of the two most recent DiT-computed guided video velocities
  for (int k = 0; k < n_steps; ++k) {
    const float t = grid[k], dt = grid[k + 1] - grid[k];
    bool reuse = false;
    if (cos_host) cos_host[k] = k >= 2 && computed >= 2 ? (float)cos_last : NAN;
    if (replay)
      reuse = replay[k] != 0;
    else if (may_reuse && k >= 2 && computed >= 2 &&
             (max_consecutive_reuse < 0 || consecutive < max_consecutive_reuse))
      reuse = cos_last > (double)tau;
    if (!reuse)
      CHECK(wam_dit_stack_fwd(cfg, w, cache, ctx, 1, x_video, x_action, &t, &t, start_frame, v_video, v_action, ws,
                              ws_bytes, stream));
    // reused: the latest computed guided velocities; computed: guided velocities replace the previous
    // ones and the cosine compares new and previous
    const float* src_v = reuse ? g_video : v_video;
    const float* src_a = reuse ? g_action : v_action;
    const int br = reuse ? 1 : g.br;
    const float wgt = reuse ? 1.f : guidance;
    float* out_v = reuse ? nullptr : g_video;
    float* out_a = reuse ? nullptr : g_action;
    const float* prev = !reuse && computed >= 1 ? g_video : nullptr;
    if (order == 0) {
      CHECK(wam_flow_step(x_video, x_action, src_v, src_a, br, wgt, nv, na, dt, dt, out_v, out_a, prev,
                          prev ? cos_parts : nullptr, ws, ws_bytes, stream));
    } else {
      UnipcArgs ua{};
      ua.xv = x_video; ua.xa = x_action; ua.vv = src_v; ua.va = src_a; ua.br = br; ua.w = wgt;
      ua.nv = nv; ua.na = na; ua.sigma = 1.f - t; ua.gv = out_v; ua.ga = out_a; ua.prev = prev;
      ua.partials = reinterpret_cast<float*>(ws); ua.cos_parts = prev ? cos_parts : nullptr;
      ua.state = state;
      const int slots = order + 1;
      ua.slot_new = k % slots;
      if (corrector && k >= 1 && !reuse) {   // the previous step's corrector with this fresh output
        double hist[3];
        for (int j = 0; j < prev_order; ++j) hist[j] = grid[k - 1 - j];
        const UniUpdate c = unipc_update(t, hist, prev_order, true);
        ua.corr = 1; ua.cn = prev_order; ua.ca = (float)c.a; ua.ct = (float)c.w[c.n - 1];
        for (int j = 0; j < prev_order; ++j) {
          ua.cw[j] = (float)c.w[j];
          ua.cslot[j] = (k - 1 - j) % slots;
        }
      }
      const int p = unipc_order(grid, k, order);
      double hist[3];
      for (int j = 0; j < p; ++j) hist[j] = grid[k - j];
      const UniUpdate pu = unipc_update(grid[k + 1], hist, p, false);
      ua.pn = p; ua.pa = (float)pu.a;
      for (int j = 0; j < p; ++j) {
        ua.pw[j] = (float)pu.w[j];
        ua.pslot[j] = (k - j) % slots;
      }
      HIP_TRY(launch_unipc_step(ua, s));
      prev_order = p;
    }
    if (reuse) {
      ++consecutive;
    } else {
      ++computed;
      ++calls;
      consecutive = 0;
      if (read_cos && computed >= 2 && k + 1 < n_steps) {
        float parts[3];
        HIP_TRY(hipMemcpyAsync(parts, cos_parts, sizeof(parts), hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
        const double den = std::sqrt((double)parts[1] * (double)parts[2]);
        cos_last = den > 0.0 ? (double)parts[0] / den : 0.0;
      }
    }
    if (reused) reused[k] = reuse ? 1 : 0;
  }
  if (dit_calls) *dit_calls = calls;
  return WAM_OK;
}

wam_status wam_denoise_chunk(const wam_config* cfg, const wam_weights* w, wam_kv_cache* cache, const wam_ctx_kv* ctx,
                             float* x_video, float* x_action, const float* grid, int n_steps, float guidance, float tau,
                             int max_consecutive_reuse, int start_frame, float* v_video, float* v_action, float* g_video,
                             float* g_action, float* cos_parts, void* ws, size_t ws_bytes, void* stream, int* dit_calls,
                             unsigned char* reused) {
  return denoise_loop(cfg, w, cache, ctx, x_video, x_action, grid, n_steps, guidance, tau, max_consecutive_reuse,
                      start_frame, 0, false, v_video, v_action, g_video, g_action, cos_parts, nullptr, ws, ws_bytes,
                      stream, dit_calls, reused);
}

wam_status wam_denoise_chunk_replay(const wam_config* cfg, const wam_weights* w, wam_kv_cache* cache,
                                    const wam_ctx_kv* ctx, float* x_video, float* x_action, const float* grid,
                                    int n_steps, float guidance, const unsigned char* replay, int start_frame,
                                    float* v_video, float* v_action, float* g_video, float* g_action, float* cos_parts,
                                    void* ws, size_t ws_bytes, void* stream, int* dit_calls, float* cosines) {
  if (!replay) return fail(WAM_E_ARG, "replay mask is NULL");
  return denoise_loop(cfg, w, cache, ctx, x_video, x_action, grid, n_steps, guidance, 2.f, -1, start_frame, 0, false,
                      v_video, v_action, g_video, g_action, cos_parts, nullptr, ws, ws_bytes, stream, dit_calls,
                      nullptr, replay, cosines);
}

wam_status wam_denoise_chunk_unipc(const wam_config* cfg, const wam_weights* w, wam_kv_cache* cache,
                                   const wam_ctx_kv* ctx, float* x_video, float* x_action, const float* grid,
                                   int n_steps, float guidance, float tau, int max_consecutive_reuse, int start_frame,
                                   int order, int corrector, float* v_video, float* v_action, float* g_video,
                                   float* g_action, float* cos_parts, float* state, void* ws, size_t ws_bytes,
                                   void* stream, int* dit_calls, unsigned char* reused) {
  if (order < 1) return fail(WAM_E_ARG, "UniPC order must be 1, 2 or 3");
  return denoise_loop(cfg, w, cache, ctx, x_video, x_action, grid, n_steps, guidance, tau, max_consecutive_reuse,
                      start_frame, order, corrector != 0, v_video, v_action, g_video, g_action, cos_parts, state, ws,
                      ws_bytes, stream, dit_calls, reused);
}

wam_status wam_op_linear(wam_dtype dtype, const void* A, int lda, const void* W, int ldw, const float* bias, void* C,
                         int ldc, int M, int N, int K, int act, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != WAM_BF16 && dtype != WAM_F32) return fail(WAM_E_ARG, "unknown dtype");
  if (!A || !W || !C) return fail(WAM_E_ARG, "NULL operand");
  if (M < 0 || N < 0 || K <= 0 || K % 64) return fail(WAM_E_SHAPE, "K must be a positive multiple of 64");
  if (lda < K || ldw < K || ldc < (act == 2 ? N / 2 : N)) return fail(WAM_E_SHAPE, "leading dimensions too small");
  const int epu = dtype == WAM_BF16 ? 8 : 4;
  if (lda % epu || ldw % epu) return fail(WAM_E_SHAPE, "lda/ldw must keep rows 16-byte aligned");
  if (act < 0 || act > 2) return fail(WAM_E_ARG, "act must be 0, 1 or 2");
  if (act == 2 && N % 2) return fail(WAM_E_SHAPE, "SwiGLU needs an even N");
  const long esz = dtype == WAM_BF16 ? 2 : 4;
  if ((long)M * lda * esz >= (1L << 31) || (long)N * ldw * esz >= (1L << 31))
    return fail(WAM_E_SHAPE, "A and W must each stay below 2 GiB (32-bit buffer offsets): split the product");
  if (ws && reinterpret_cast<uintptr_t>(ws) % 256) return fail(WAM_E_ARG, "workspace must be 256-byte aligned");
  GemmArgs ga = gemm_args(A, lda, W, ldw, bias, M, N, K, ws ? reinterpret_cast<float*>(ws) : nullptr,
                          ws ? (long)(ws_bytes / 4) : 0);
  ga.C = C;
  ga.ldc = ldc;
  HIP_TRY(launch_gemm(ga, dtype == WAM_BF16 ? DT_BF16 : DT_F32, act == 2 ? EPI_SWIGLU : act ? EPI_GELU : EPI_STORE,
                      reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_op_split_finish(const float* part, int splits, int M, int N, const float* bias, float* h,
                               const float* e6, const float* mod_gate, int gate_idx, const float* mod_norm,
                               int shift_idx, int scale_idx, int rms, float eps, void* y, void* stream) {
  if (!part || !h || !e6 || !mod_norm || !y || (gate_idx >= 0 && !mod_gate)) return fail(WAM_E_ARG, "NULL buffer");
  if (splits < 2 || splits > 4) return fail(WAM_E_SHAPE, "splits must be 2, 3 or 4");
  if (M < 0 || N <= 0 || N % 4 || N > 8192) return fail(WAM_E_SHAPE, "N must be a positive multiple of 4 up to 8192");
  if (gate_idx > 5 || shift_idx < 0 || shift_idx > 5 || scale_idx < 0 || scale_idx > 5)
    return fail(WAM_E_ARG, "modulation slots must be in 0..5");
  if (!(eps > 0.f)) return fail(WAM_E_ARG, "eps must be positive");
  if (unaligned16(part) || unaligned16(h) || unaligned16(e6) || unaligned16(mod_norm) || unaligned16(y) ||
      (bias && unaligned16(bias)) || (gate_idx >= 0 && unaligned16(mod_gate)))
    return fail(WAM_E_ARG, "buffers must be 16-byte aligned");
  if (M == 0) return WAM_OK;
  const RowMap rm{M, M, M};   // one row type: every row takes slot block 0 of e6
  GemmArgs ga{};
  ga.bias = bias; ga.H = h; ga.ldh = N; ga.M = M; ga.N = N; ga.K = 0; ga.rm = rm;
  ga.e6 = e6; ga.mod = mod_gate; ga.gate_idx = gate_idx < 0 ? 0 : gate_idx; ga.D = N;
  ga.part = const_cast<float*>(part); ga.part_elems = (long)splits * M * N;
  PostArgs post{};
  post.mode = POST_NORM;
  NormArgs& na = post.na;
  na.X = h; na.Y = y; na.M = M; na.D = N; na.eps = eps; na.mode = NORM_ADALN; na.rm = rm;
  na.e6 = e6; na.mod = mod_norm; na.shift_idx = shift_idx; na.scale_idx = scale_idx; na.rms = rms != 0;
  HIP_TRY(launch_split_finish(ga, gate_idx >= 0 ? EPI_RESID_GATED : EPI_RESID, post, splits,
                              reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_op_modulated_norm(const float* x, int M, int D, const float* e6, const float* mod, int shift_idx,
                                 int scale_idx, int rms, float eps, void* y, void* stream) {
  if (!x || !e6 || !mod || !y) return fail(WAM_E_ARG, "NULL buffer");
  if (M < 0 || D <= 0 || D % 4 || D > 8192) return fail(WAM_E_SHAPE, "D must be a positive multiple of 4 up to 8192");
  if (shift_idx < 0 || shift_idx > 5 || scale_idx < 0 || scale_idx > 5)
    return fail(WAM_E_ARG, "modulation slots must be in 0..5");
  if (!(eps > 0.f)) return fail(WAM_E_ARG, "eps must be positive");
  if (unaligned16(x) || unaligned16(e6) || unaligned16(mod) || unaligned16(y))
    return fail(WAM_E_ARG, "buffers must be 16-byte aligned");
  if (M == 0) return WAM_OK;
  NormArgs na{};
  na.X = x; na.Y = y; na.M = M; na.D = D; na.eps = eps; na.mode = NORM_ADALN; na.rm = RowMap{M, M, M};
  na.e6 = e6; na.mod = mod; na.shift_idx = shift_idx; na.scale_idx = scale_idx; na.rms = rms != 0;
  HIP_TRY(launch_norm(na, DT_BF16, reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_op_qkv_cache(const void* qkv, int br, int rows, int Lq, int Lv, int H, int d, const float* g_q,
                            const float* g_k, float eps, const float* rope, void* q_out, void* k_cache, void* v_cache,
                            int cap, int row0, void* stream) {
  if (!qkv || !g_q || !g_k || !rope || !q_out || !k_cache || !v_cache) return fail(WAM_E_ARG, "NULL buffer");
  if (d != 64 && d != 128) return fail(WAM_E_SHAPE, "head dim must be 64 or 128");
  if (br < 1 || H < 1 || (long)H * d > 8192) return fail(WAM_E_SHAPE, "need br >= 1 and 1 <= H d <= 8192");
  if (rows < 0 || rows % 8 || row0 < 0 || row0 % 8 || cap % 8 || row0 + rows > cap)
    return fail(WAM_E_SHAPE, "rows, row0 and cap must be multiples of 8 with row0 + rows <= cap");
  if (Lq < 1 || Lv < 0 || Lv > Lq) return fail(WAM_E_SHAPE, "need 0 <= Lv <= Lq");
  if (!(eps > 0.f)) return fail(WAM_E_ARG, "eps must be positive");
  if (unaligned16(qkv) || unaligned16(g_q) || unaligned16(g_k) || unaligned16(rope) || unaligned16(q_out) ||
      unaligned16(k_cache) || unaligned16(v_cache))
    return fail(WAM_E_ARG, "buffers must be 16-byte aligned");
  if (rows == 0) return WAM_OK;
  const int D = H * d;
  QkNormArgs qa{};
  qa.src = qkv; qa.src_ld = 3L * D; qa.src_col = 0; qa.gain = g_q;
  qa.dst = q_out; qa.dst_bh_stride = (long)rows * d; qa.dst_row0 = 0;
  qa.M = br * rows; qa.D = D; qa.H = H; qa.d = d; qa.rows_per_branch = rows; qa.eps = eps;
  qa.rope = reinterpret_cast<const float2*>(rope); qa.rm = RowMap{rows, Lq, Lv};
  QkNormArgs ka = qa;
  ka.src_col = D; ka.gain = g_k; ka.dst = k_cache; ka.dst_bh_stride = (long)cap * d; ka.dst_row0 = row0;
  VCacheArgs va{};
  va.src = qkv; va.src_ld = 3L * D; va.src_col = 2 * D; va.dst = v_cache; va.dst_bh_stride = (long)d * cap;
  va.dst_stride = cap; va.dst_col0 = row0; va.rows_per_branch = rows; va.br = br; va.H = H; va.d = d;
  HIP_TRY(launch_qkv_cache(&qa, ka, va, DT_BF16, reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_mx_quantize(wam_dtype dtype, const void* src, int ld, int rows, int cols, void* codes, int ldq,
                           void* scales, void* stream) {
  if (dtype != WAM_BF16 && dtype != WAM_F32) return fail(WAM_E_ARG, "unknown dtype");
  if (!src || !codes || !scales) return fail(WAM_E_ARG, "NULL buffer");
  if (rows < 0 || cols <= 0 || cols % 32) return fail(WAM_E_SHAPE, "cols must be a positive multiple of 32");
  if (ld < cols || ldq < cols || ldq % 16 || ld % (dtype == WAM_BF16 ? 8 : 4))
    return fail(WAM_E_SHAPE, "ld must keep rows 16-byte aligned and ldq be a multiple of 16, both >= cols");
  if (unaligned16(src) || unaligned16(codes)) return fail(WAM_E_ARG, "src and codes must be 16-byte aligned");
  HIP_TRY(launch_mx_quantize(src, ld, dtype == WAM_BF16 ? DT_BF16 : DT_F32, rows, cols, reinterpret_cast<uint8_t*>(codes),
                             ldq, reinterpret_cast<uint8_t*>(scales), reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_mx4_quantize(wam_dtype dtype, const void* src, int ld, int rows, int cols, void* codes, int ldq,
                            void* scales, void* stream) {
  if (dtype != WAM_BF16 && dtype != WAM_F32) return fail(WAM_E_ARG, "unknown dtype");
  if (!src || !codes || !scales) return fail(WAM_E_ARG, "NULL buffer");
  if (rows < 0 || cols <= 0 || cols % 32) return fail(WAM_E_SHAPE, "cols must be a positive multiple of 32");
  if (ld < cols || ldq < cols / 2 || ldq % 16 || ld % (dtype == WAM_BF16 ? 8 : 4))
    return fail(WAM_E_SHAPE, "ld must keep rows 16-byte aligned and be >= cols; ldq a multiple of 16, >= cols / 2");
  if (unaligned16(src) || unaligned16(codes)) return fail(WAM_E_ARG, "src and codes must be 16-byte aligned");
  HIP_TRY(launch_mx4_quantize(src, ld, dtype == WAM_BF16 ? DT_BF16 : DT_F32, rows, cols,
                              reinterpret_cast<uint8_t*>(codes), ldq, reinterpret_cast<uint8_t*>(scales),
                              reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_op_linear_mx(const void* A, const void* A_scales, int lda, const void* W, const void* W_scales, int ldw,
                            int w_format, const float* bias, void* C, int ldc, int M, int N, int K, int act, void* ws,
                            size_t ws_bytes, void* stream) {
  if (!A || !A_scales || !W || !W_scales || !C) return fail(WAM_E_ARG, "NULL operand");
  if (M < 0 || N <= 0 || K <= 0 || K % 128) return fail(WAM_E_SHAPE, "K must be a positive multiple of 128");
  if (N % 4) return fail(WAM_E_SHAPE, "N must be a multiple of 4");
  if (act < 0 || act > 2) return fail(WAM_E_ARG, "act must be 0, 1 or 2");
  if (w_format != WAM_MX_E4M3 && w_format != WAM_MX_E2M1) return fail(WAM_E_ARG, "unknown weight format");
  const int wbytes = w_format == WAM_MX_E2M1 ? K / 2 : K;
  if (lda < K || ldw < wbytes || lda % 16 || ldw % 16)
    return fail(WAM_E_SHAPE, "lda / ldw must be multiples of 16 holding a row (K codes, K / 2 bytes for e2m1)");
  if (ldc < (act == 2 ? N / 2 : N) || ldc % 4) return fail(WAM_E_SHAPE, "ldc too small or not a multiple of 4");
  if ((long)M * lda >= (1L << 31) || (long)N * ldw >= (1L << 31))
    return fail(WAM_E_SHAPE, "A and W codes must each stay below 2 GiB (32-bit buffer offsets): split the product");
  if (unaligned16(A) || unaligned16(W) || reinterpret_cast<uintptr_t>(C) % 8 || (bias && unaligned16(bias)))
    return fail(WAM_E_ARG, "A, W (16 bytes), C (8 bytes) and bias (16 bytes) alignment");
  if (reinterpret_cast<uintptr_t>(A_scales) % 4 || reinterpret_cast<uintptr_t>(W_scales) % 4)
    return fail(WAM_E_ARG, "scale arrays must be 4-byte aligned");
  if (ws && reinterpret_cast<uintptr_t>(ws) % 256) return fail(WAM_E_ARG, "workspace must be 256-byte aligned");
  GemmArgs ga = gemm_args(A, lda, W, ldw, bias, M, N, K, ws ? reinterpret_cast<float*>(ws) : nullptr,
                          ws ? (long)(ws_bytes / 4) : 0);
  ga.C = C;
  ga.ldc = ldc;
  ga.As = reinterpret_cast<const uint8_t*>(A_scales);
  ga.Ws = reinterpret_cast<const uint8_t*>(W_scales);
  ga.w_fp4 = w_format == WAM_MX_E2M1;
  HIP_TRY(launch_gemm_mx(ga, act == 2 ? EPI_SWIGLU : act ? EPI_GELU : EPI_STORE, reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_weights_for_embodiment(const wam_weights* w, int id, wam_weights* out) {
  if (!w || !out) return fail(WAM_E_ARG, "weights or out is NULL");
  if (!w->embodiments || id < 0 || id >= w->n_embodiments)
    return fail(WAM_E_ARG, "embodiment %d outside the table of %d", id, w->embodiments ? w->n_embodiments : 0);
  const wam_action_io& e = w->embodiments[id];
  if (!e.ae_w || !e.ae_b || !e.ao_w || !e.ao_b) return fail(WAM_E_ARG, "embodiment %d: action matrices are NULL", id);
  wam_weights r = *w;
  r.ae_w = e.ae_w;
  r.ae_b = e.ae_b;
  r.ao_w = e.ao_w;
  r.ao_b = e.ao_b;
  *out = r;
  return WAM_OK;
}

size_t wam_mx_block_bytes(const wam_config* cfg) {
  if (check_cfg(cfg) != WAM_OK) return 0;
  const Geo g = geo_of(*cfg);
  if (g.dt != DT_BF16 || g.D % 128 || g.F % 128) return 0;
  return mx_block_of(g).total;
}

wam_status wam_mx_pack_block(const wam_config* cfg, const wam_block_weights* bw, void* dst, size_t dst_bytes,
                             void* stream) {
  CHECK(check_cfg(cfg));
  const Geo g = geo_of(*cfg);
  if (g.dt != DT_BF16 || g.D % 128 || g.F % 128)
    return fail(WAM_E_UNSUPPORTED, "MXFP8 packing needs dtype bf16 and dim, ffn_dim multiples of 128");
  if (!bw) return fail(WAM_E_ARG, "block weights are NULL");
  const MxBlock b = mx_block_of(g);
  if (!dst || reinterpret_cast<uintptr_t>(dst) % 256) return fail(WAM_E_ARG, "dst must be a 256-byte aligned buffer");
  if (dst_bytes < b.total) return fail(WAM_E_ARG, "dst holds %zu bytes, the packed layer needs %zu", dst_bytes, b.total);
  const void* W[MX_MATS] = {bw->w_qkv, bw->w_o, bw->w_cq, bw->w_co, bw->w_ff1, bw->w_ff2};
  const char* names[MX_MATS] = {"w_qkv", "w_o", "w_cq", "w_co", "w_ff1", "w_ff2"};
  for (int i = 0; i < MX_MATS; ++i)
    if (!W[i] || unaligned16(W[i])) return fail(WAM_E_ARG, "%s is NULL or not 16-byte aligned", names[i]);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* base = reinterpret_cast<char*>(dst);
  for (int i = 0; i < MX_MATS; ++i) {
    const MxMat& m = b.m[i];
    uint8_t* codes = reinterpret_cast<uint8_t*>(base + m.codes);
    uint8_t* scales = reinterpret_cast<uint8_t*>(base + m.scales);
    if (g.w4)
      HIP_TRY(launch_mx4_quantize(W[i], m.K, DT_BF16, m.N, m.K, codes, m.K / 2, scales, s));
    else
      HIP_TRY(launch_mx_quantize(W[i], m.K, DT_BF16, m.N, m.K, codes, m.K, scales, s));
  }
  return WAM_OK;
}

size_t wam_pack_block_bytes(const wam_config* cfg) {
  if (check_cfg(cfg) != WAM_OK) return 0;
  const Geo g = geo_of(*cfg);
  if (g.dt != DT_BF16 || !pk_fits(g)) return 0;
  return pk_block_of(g).total;
}

wam_status wam_pack_block(const wam_config* cfg, const wam_block_weights* bw, void* dst, size_t dst_bytes,
                          void* stream) {
  CHECK(check_cfg(cfg));
  const Geo g = geo_of(*cfg);
  if (g.dt != DT_BF16) return fail(WAM_E_UNSUPPORTED, "packed projections need dtype bf16");
  if (!pk_fits(g)) return fail(WAM_E_SHAPE, "a projection is too large to pack (2 GiB)");
  if (!bw) return fail(WAM_E_ARG, "block weights are NULL");
  const PkBlock b = pk_block_of(g);
  if (!dst || reinterpret_cast<uintptr_t>(dst) % 256) return fail(WAM_E_ARG, "dst must be a 256-byte aligned buffer");
  if (dst_bytes < b.total) return fail(WAM_E_ARG, "dst holds %zu bytes, the packed layer needs %zu", dst_bytes, b.total);
  const void* W[MX_MATS] = {bw->w_qkv, bw->w_o, bw->w_cq, bw->w_co, bw->w_ff1, bw->w_ff2};
  const char* names[MX_MATS] = {"w_qkv", "w_o", "w_cq", "w_co", "w_ff1", "w_ff2"};
  for (int i = 0; i < MX_MATS; ++i)
    if (!W[i] || unaligned16(W[i])) return fail(WAM_E_ARG, "%s is NULL or not 16-byte aligned", names[i]);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int i = 0; i < MX_MATS; ++i)
    HIP_TRY(launch_pack_weight(W[i], b.K[i], b.N[i], b.K[i], reinterpret_cast<char*>(dst) + b.off[i], s));
  return WAM_OK;
}

wam_status wam_pack_weight(const void* W, int ldw, int N, int K, void* dst, void* stream) {
  if (!W || !dst) return fail(WAM_E_ARG, "NULL operand");
  if (unaligned16(W) || unaligned16(dst)) return fail(WAM_E_ARG, "W and dst must be 16-byte aligned");
  if (N <= 0 || K <= 0 || N % 32 || K % 64) return fail(WAM_E_SHAPE, "N must be a multiple of 32 and K of 64");
  if (ldw < K || ldw % 8) return fail(WAM_E_SHAPE, "ldw must be >= K and a multiple of 8");
  if ((long)N * K * 2 >= (1L << 31)) return fail(WAM_E_SHAPE, "the packed matrix must stay below 2 GiB");
  HIP_TRY(launch_pack_weight(W, ldw, N, K, dst, reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_op_linear_packed(const void* A, int lda, const void* Wp, const float* bias, void* C, int ldc, int M,
                                int N, int K, int act, void* ws, size_t ws_bytes, void* stream) {
  if (!A || !Wp || !C) return fail(WAM_E_ARG, "NULL operand");
  if (M < 0 || N <= 0 || N % 32 || K <= 0 || K % 64) return fail(WAM_E_SHAPE, "N must be a multiple of 32 and K of 64");
  if (lda < K || lda % 8 || ldc < (act == 2 ? N / 2 : N) || ldc % 4)
    return fail(WAM_E_SHAPE, "lda must be >= K and a multiple of 8, ldc wide enough and a multiple of 4");
  if (act < 0 || act > 2) return fail(WAM_E_ARG, "act must be 0, 1 or 2");
  if (unaligned16(A) || unaligned16(Wp) || reinterpret_cast<uintptr_t>(C) % 8 || (bias && unaligned16(bias)))
    return fail(WAM_E_ARG, "A, Wp and bias must be 16-byte aligned, C 8-byte aligned");
  if ((long)M * lda * 2 >= (1L << 31) || (long)N * K * 2 >= (1L << 31))
    return fail(WAM_E_SHAPE, "A and W must each stay below 2 GiB (32-bit buffer offsets): split the product");
  if (ws && reinterpret_cast<uintptr_t>(ws) % 256) return fail(WAM_E_ARG, "workspace must be 256-byte aligned");
  if (M == 0) return WAM_OK;
  GemmArgs ga = gemm_args(A, lda, Wp, K, bias, M, N, K, ws ? reinterpret_cast<float*>(ws) : nullptr,
                          ws ? (long)(ws_bytes / 4) : 0);
  ga.C = C;
  ga.ldc = ldc;
  ga.w_packed = 1;
  HIP_TRY(launch_gemm(ga, DT_BF16, act == 2 ? EPI_SWIGLU : act ? EPI_GELU : EPI_STORE,
                      reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_op_attention(wam_dtype dtype, const void* Q, const void* K, const void* Vt, void* O, int br, int heads,
                            int head_dim, int Lq, int k_rows, int v_stride, int kv_base, int chunk_q, int kv_total,
                            void* ws, size_t ws_bytes, void* stream) {
  if (dtype != WAM_BF16 && dtype != WAM_F32) return fail(WAM_E_ARG, "unknown dtype");
  if (!Q || !K || !Vt || !O) return fail(WAM_E_ARG, "NULL operand");
  if (head_dim != 64 && head_dim != 128) return fail(WAM_E_SHAPE, "head_dim must be 64 or 128");
  if (br <= 0 || heads <= 0 || Lq < 0 || kv_total <= 0 || kv_base < 0) return fail(WAM_E_SHAPE, "bad sizes");
  if (k_rows < kv_total || v_stride < kv_total || v_stride % 8) return fail(WAM_E_SHAPE, "k_rows/v_stride too small");
  if (ws && reinterpret_cast<uintptr_t>(ws) % 256) return fail(WAM_E_ARG, "workspace must be 256-byte aligned");
  AttnArgs a{};
  a.Q = Q; a.K = K; a.Vt = Vt; a.O = O;
  a.q_bh_stride = (long)Lq * head_dim; a.k_bh_stride = (long)k_rows * head_dim; a.v_bh_stride = (long)head_dim * v_stride;
  a.v_stride = v_stride; a.Lq_total = Lq; a.H = heads; a.d = head_dim; a.br = br;
  a.kv_base = kv_base; a.chunk_q = chunk_q; a.kv_total = kv_total;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  a.part = reinterpret_cast<float*>(ws); a.part_elems = ws ? (long)(ws_bytes / 4) : 0;
  HIP_TRY(launch_attention(a, dtype == WAM_BF16 ? DT_BF16 : DT_F32, reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_op_attention_mx(const void* Q, const void* Q_scales, const void* K, const void* K_scales, const void* Vt,
                               const void* Vt_scales, void* O, int br, int heads, int Lq, int k_rows, int v_stride,
                               int kv_base, int chunk_q, int kv_total, void* stream) {
  if (!Q || !Q_scales || !K || !K_scales || !Vt || !Vt_scales || !O) return fail(WAM_E_ARG, "NULL operand");
  if (unaligned16(Q) || unaligned16(K) || unaligned16(Vt) || unaligned16(Vt_scales) || unaligned16(O) ||
      reinterpret_cast<uintptr_t>(Q_scales) % 4 || reinterpret_cast<uintptr_t>(K_scales) % 4)
    return fail(WAM_E_ARG, "codes, V^T scales and O must be 16-byte aligned, Q/K scales 4-byte aligned");
  if (br <= 0 || heads <= 0 || Lq <= 0 || kv_total <= 0 || kv_base < 0 || chunk_q < 0)
    return fail(WAM_E_SHAPE, "bad sizes");
  if (k_rows < kv_total || v_stride % 64 || v_stride < (kv_total + 63) / 64 * 64)
    return fail(WAM_E_SHAPE, "k_rows must be >= kv_total and v_stride a multiple of 64 covering kv_total");
  if ((long)k_rows * 128 > INT32_MAX || (long)v_stride * 128 > INT32_MAX)
    return fail(WAM_E_SHAPE, "one head's keys exceed 2 GiB");
  AttnMxArgs a{};
  a.Q = static_cast<const uint8_t*>(Q); a.Qs = static_cast<const uint8_t*>(Q_scales);
  a.K = static_cast<const uint8_t*>(K); a.Ks = static_cast<const uint8_t*>(K_scales);
  a.Vt = static_cast<const uint8_t*>(Vt); a.Vs = static_cast<const uint8_t*>(Vt_scales); a.O = O;
  a.q_bh = (long)Lq * 128; a.qs_bh = (long)Lq * 4; a.k_bh = (long)k_rows * 128; a.ks_bh = (long)k_rows * 4;
  a.v_bh = 128L * v_stride; a.vs_bh = (long)(v_stride / 32) * 128;
  a.v_stride = v_stride; a.Lq = Lq; a.H = heads; a.br = br; a.kv_base = kv_base; a.chunk_q = chunk_q;
  a.kv_total = kv_total;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt(128.0));
  HIP_TRY(launch_attention_mx(a, reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_kv_evict(const wam_config* cfg, wam_kv_cache* cache, int drop_rows, int frame_shift, void* stream) {
  CHECK(check_cfg(cfg));
  const Geo g = geo_of(*cfg);
  if (!cache || !cache->k || !cache->v) return fail(WAM_E_ARG, "KV cache pointers are NULL");
  if (unaligned16(cache->k) || unaligned16(cache->v)) return fail(WAM_E_ARG, "KV cache pointers are not 16-byte aligned");
  if (cache->branches != g.br) return fail(WAM_E_SHAPE, "cache branches %d != config branches %d", cache->branches, g.br);
  if (cache->capacity <= 0 || cache->capacity % 64) return fail(WAM_E_SHAPE, "cache capacity must be a positive multiple of 64");
  if (drop_rows < 0 || drop_rows % g.Lq || drop_rows > cache->length)
    return fail(WAM_E_SHAPE, "drop_rows (%d) must be whole chunks of %d rows, at most the length %d", drop_rows, g.Lq,
                cache->length);
  if (drop_rows == 0) return WAM_OK;
  KvEvictArgs a{};
  a.k = cache->k; a.v = cache->v;
  a.blocks = g.L * g.br * g.H; a.cap = cache->capacity; a.d = g.d; a.len = cache->length; a.drop = drop_rows;
  a.Lq = g.Lq; a.Lv = g.Lv;
  // frame axis: the first d_t / 2 pairs of a head, d_t = d - 2 * 2 floor(d / 6), freq theta^(-2j / d_t)
  const int dh = 2 * (g.d / 6), dt = g.d - 2 * dh;
  a.frame_pairs = dt / 2;
  for (int j = 0; j < a.frame_pairs; ++j) {
    const double ang = -(double)frame_shift * std::pow((double)cfg->rope_theta, -2.0 * j / (double)dt);
    a.cs[j] = make_float2((float)std::cos(ang), (float)std::sin(ang));
  }
  HIP_TRY(launch_kv_evict(a, g.dt, reinterpret_cast<hipStream_t>(stream)));
  cache->length -= drop_rows;
  return WAM_OK;
}

void wam_kv_reset(wam_kv_cache* cache) {
  if (cache) cache->length = 0;
}

const char* wam_last_error(void) { return g_err.c_str(); }

wam_status wam_qkv_timer_config(int layer, int max_samples) {
  g_qkv_timer.clear();
  if (layer < 0) return WAM_OK;
  if (max_samples < 1 || max_samples > 4096) return fail(WAM_E_ARG, "max_samples must be in [1, 4096]");
  for (int i = 0; i < 2 * max_samples; ++i) {
    hipEvent_t e;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      g_qkv_timer.clear();
      return fail(WAM_E_HIP, "hipEventCreate: %s", hipGetErrorString(err));
    }
    g_qkv_timer.ev.push_back(e);
  }
  g_qkv_timer.layer = layer;
  return WAM_OK;
}

wam_status wam_mfma_peak_probe(float* out, int workgroups, int iters, void* stream) {
  if (!out) return fail(WAM_E_ARG, "out is NULL");
  if (workgroups < 1 || workgroups > 65536 || iters < 1) return fail(WAM_E_ARG, "workgroups in [1, 65536], iters >= 1");
  HIP_TRY(launch_mfma_peak(out, workgroups, iters, reinterpret_cast<hipStream_t>(stream)));
  return WAM_OK;
}

wam_status wam_qkv_timer_read(float* ms, int cap, int* n) {
  if (!n || (cap > 0 && !ms) || cap < 0) return fail(WAM_E_ARG, "n is NULL, or ms is NULL with cap > 0");
  QkvTimer& tm = g_qkv_timer;
  *n = tm.n;
  for (int i = 0; i < tm.n && i < cap; ++i) {
    hipError_t err = hipEventSynchronize(tm.ev[2 * i + 1]);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms[i], tm.ev[2 * i], tm.ev[2 * i + 1]);
    if (err != hipSuccess) return fail(WAM_E_HIP, "timer event: %s", hipGetErrorString(err));
  }
  tm.n = 0;
  return WAM_OK;
}

}  // extern "C"
