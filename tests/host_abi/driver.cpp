// Drives every C-ABI entry point of the DiT library through its host logic (validation, workspace
// carving, launch sequence) with fake device addresses, against the host stand-ins of stubs.cpp.
// Built with -fsanitize=address,undefined by tests/test_host_sanitized.py; exit status 0 and the
// line "host_abi: OK" when every call returned the expected status and every launch stayed inside
// its buffers.
#include <cmath>
#include <cstdio>
#include <vector>

#include "../../include/wam.h"
#include "stubs.h"

namespace {
int g_fail = 0;
uintptr_t g_next = (uintptr_t)1 << 40;   // fake device address space

void* dev(size_t bytes, const std::string& name) {
  g_next = (g_next + 255) & ~(uintptr_t)255;
  void* p = reinterpret_cast<void*>(g_next);
  host_abi::register_region(p, bytes ? bytes : 1, name);
  g_next += bytes + 256;
  return p;
}
void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "host_abi: %s returned %d, expected %d (%s)\n", what, got, want, wam_last_error());
    ++g_fail;
  }
}

struct Model {
  wam_config c{};
  std::vector<wam_block_weights> blocks;
  wam_weights w{};
  wam_kv_cache kv{};
  wam_ctx_kv cx{};
  void* ws = nullptr;
  size_t ws_bytes = 0;
  int Lv = 0, Lq = 0, Lc = 0;
};

wam_config config(bool full, wam_dtype dt) {
  wam_config c{};
  if (full) {
    c.dim = 5120; c.heads = 40; c.head_dim = 128; c.ffn_dim = 13824; c.layers = 40;
    c.grid_h = 11; c.grid_w = 20; c.ctx_in_dim = 1536; c.ctx_text_len = 512; c.ctx_img_len = 257;
  } else {
    c.dim = 256; c.heads = 4; c.head_dim = 64; c.ffn_dim = 1024; c.layers = 2;
    c.grid_h = 8; c.grid_w = 8; c.ctx_in_dim = 256; c.ctx_text_len = 32; c.ctx_img_len = 0;
  }
  c.freq_dim = 256; c.patch_dim = 64; c.action_dim = 8; c.action_tokens = 24; c.frames_per_chunk = 2;
  c.branches = 2; c.rope_theta = 10000.f; c.eps = 1e-6f; c.dtype = dt; c.state_dim = 64;
  return c;
}

// packed: each block gets its fragment-packed projections (wam_pack_block) and loses the six unpacked
// matrices, so a read of those would fall outside every registered region
Model build(const wam_config& c, int cache_chunks, bool packed = false) {
  Model m;
  m.c = c;
  const size_t e = c.dtype == WAM_BF16 ? 2 : 4, D = c.dim, F = c.ffn_dim;
  const size_t F1 = (c.variant & WAM_VARIANT_SWIGLU) ? 2 * F : F;
  m.Lv = c.frames_per_chunk * c.grid_h * c.grid_w;
  m.Lq = m.Lv + c.action_tokens;
  m.Lc = c.ctx_text_len + c.ctx_img_len + c.ctx_state_len;
  m.blocks.resize(c.layers);
  for (int l = 0; l < c.layers; ++l) {
    wam_block_weights& b = m.blocks[l];
    b.mod = dev(6 * D * 4, "mod");
    b.w_qkv = dev(3 * D * D * e, "w_qkv"); b.b_qkv = dev(3 * D * 4, "b_qkv");
    b.g_q = dev(D * 4, "g_q"); b.g_k = dev(D * 4, "g_k");
    b.w_o = dev(D * D * e, "w_o"); b.b_o = dev(D * 4, "b_o");
    b.ln3_w = dev(D * 4, "ln3_w"); b.ln3_b = dev(D * 4, "ln3_b");
    b.w_cq = dev(D * D * e, "w_cq"); b.b_cq = dev(D * 4, "b_cq"); b.g_cq = dev(D * 4, "g_cq");
    b.w_ck = dev(D * D * e, "w_ck"); b.b_ck = dev(D * 4, "b_ck"); b.g_ck = dev(D * 4, "g_ck");
    b.w_cv = dev(D * D * e, "w_cv"); b.b_cv = dev(D * 4, "b_cv");
    b.w_co = dev(D * D * e, "w_co"); b.b_co = dev(D * 4, "b_co");
    b.w_ff1 = dev(F1 * D * e, "w_ff1"); b.b_ff1 = dev(F1 * 4, "b_ff1");
    b.w_ff2 = dev(D * F * e, "w_ff2"); b.b_ff2 = dev(D * 4, "b_ff2");
    if (c.variant & WAM_VARIANT_IMG_XATTN) {
      b.w_cki = dev(D * D * e, "w_cki"); b.b_cki = dev(D * 4, "b_cki"); b.g_cki = dev(D * 4, "g_cki");
      b.w_cvi = dev(D * D * e, "w_cvi"); b.b_cvi = dev(D * 4, "b_cvi");
    }
    if (c.precision != WAM_PRECISION_NATIVE) b.mx = dev(wam_mx_block_bytes(&c), "mx arena");
    if (packed) {
      const size_t pk_bytes = wam_pack_block_bytes(&c);
      if (!pk_bytes) { std::fprintf(stderr, "host_abi: packed size 0\n"); ++g_fail; }
      void* pk = dev(pk_bytes, "packed projections");
      expect(wam_pack_block(&c, &b, pk, pk_bytes, nullptr), WAM_OK, "pack_block");
      expect(wam_pack_block(&c, &b, pk, pk_bytes - 256, nullptr), WAM_E_ARG, "pack_block into a short arena");
      b.pk = pk;
      b.w_qkv = b.w_o = b.w_cq = b.w_co = b.w_ff1 = b.w_ff2 = nullptr;
    }
  }
  wam_weights& w = m.w;
  w.blocks = m.blocks.data();
  w.t_w1 = dev(D * c.freq_dim * e, "t_w1"); w.t_b1 = dev(D * 4, "t_b1");
  w.t_w2 = dev(D * D * e, "t_w2"); w.t_b2 = dev(D * 4, "t_b2");
  w.t_wp = dev(6 * D * D * e, "t_wp"); w.t_bp = dev(6 * D * 4, "t_bp");
  w.pe_w = dev(D * c.patch_dim * e, "pe_w"); w.pe_b = dev(D * 4, "pe_b");
  w.ae_w = dev(D * c.action_dim * e, "ae_w"); w.ae_b = dev(D * 4, "ae_b");
  w.head_mod = dev(2 * D * 4, "head_mod");
  w.vo_w = dev((size_t)c.patch_dim * D * e, "vo_w"); w.vo_b = dev(c.patch_dim * 4, "vo_b");
  w.ao_w = dev((size_t)c.action_dim * D * e, "ao_w"); w.ao_b = dev(c.action_dim * 4, "ao_b");
  w.txt_w = dev(D * c.ctx_in_dim * e, "txt_w"); w.txt_b = dev(D * 4, "txt_b");
  if (c.ctx_img_len) { w.img_w = dev(D * c.ctx_in_dim * e, "img_w"); w.img_b = dev(D * 4, "img_b"); }
  if (c.ctx_state_len) { w.st_w = dev(D * c.state_dim * e, "st_w"); w.st_b = dev(D * 4, "st_b"); }
  const int cap = ((cache_chunks * m.Lq + 63) / 64) * 64;
  const size_t blk = (size_t)c.branches * c.heads * cap * c.head_dim * e;
  m.kv = wam_kv_cache{dev(c.layers * blk, "cache k"), dev(c.layers * blk, "cache v"), c.branches, cap, 0};
  const int stride = ((m.Lc + 31) / 32 * 32 + 63) / 64 * 64 + 64;
  m.cx = wam_ctx_kv{dev((size_t)c.layers * c.branches * c.heads * m.Lc * c.head_dim * e, "ctx k"),
                    dev((size_t)c.layers * c.branches * c.heads * c.head_dim * stride * e, "ctx v"), c.branches, m.Lc,
                    stride};
  m.ws_bytes = wam_workspace_bytes(&c, 2);
  if (!m.ws_bytes) { std::fprintf(stderr, "host_abi: workspace size 0\n"); ++g_fail; }
  m.ws = dev(m.ws_bytes, "workspace");
  return m;
}

void scenario(const char* name, const wam_config& c, bool packed = false) {
  std::fprintf(stderr, "host_abi: scenario %s\n", name);
  Model m = build(c, 5, packed);
  const size_t e = c.dtype == WAM_BF16 ? 2 : 4;
  const int Lv = m.Lv, La = c.action_tokens, P = c.patch_dim, A = c.action_dim, br = c.branches;
  void* txt = dev((size_t)br * c.ctx_text_len * c.ctx_in_dim * e, "txt");
  void* img = c.ctx_img_len ? dev((size_t)c.ctx_img_len * c.ctx_in_dim * e, "img") : nullptr;
  void* st = c.ctx_state_len ? dev((size_t)c.ctx_state_len * c.state_dim * e, "state") : nullptr;
  expect(wam_ctx_build(&m.c, &m.w, txt, img, st, &m.cx, m.ws, m.ws_bytes, nullptr), WAM_OK, "ctx_build");
  if (st) expect(wam_ctx_set_state(&m.c, &m.w, st, &m.cx, m.ws, m.ws_bytes, nullptr), WAM_OK, "ctx_set_state");
  float* xv = static_cast<float*>(dev((size_t)2 * Lv * P * 4, "x video"));
  float* xa = static_cast<float*>(dev((size_t)2 * La * A * 4, "x action"));
  float* vv = static_cast<float*>(dev((size_t)br * 2 * Lv * P * 4, "v video"));
  float* va = static_cast<float*>(dev((size_t)br * 2 * La * A * 4, "v action"));
  const float t1[2] = {0.3f, 0.6f}, t2[2] = {0.5f, 0.9f};
  float* e1 = static_cast<float*>(dev(4 * c.dim * 4, "e"));
  float* e6 = static_cast<float*>(dev(4 * 6 * c.dim * 4, "e6"));
  expect(wam_time_embed(&m.c, &m.w, t1, 2, e1, e6, m.ws, m.ws_bytes, nullptr), WAM_OK, "time_embed");
  expect(wam_kv_append(&m.c, &m.w, &m.kv, &m.cx, xv, xa, 0, m.ws, m.ws_bytes, nullptr), WAM_OK, "kv_append 1");
  expect(wam_kv_append(&m.c, &m.w, &m.kv, &m.cx, xv, xa, 2, m.ws, m.ws_bytes, nullptr), WAM_OK, "kv_append 2");
  expect(m.kv.length, 2 * m.Lq, "cache length after two appends");
  expect(wam_dit_stack_fwd(&m.c, &m.w, &m.kv, &m.cx, 1, xv, xa, t1, t2, 4, vv, va, m.ws, m.ws_bytes, nullptr), WAM_OK,
         "stack_fwd 1 chunk");
  expect(wam_dit_stack_fwd(&m.c, &m.w, &m.kv, &m.cx, 2, xv, xa, t1, t2, 4, vv, va, m.ws, m.ws_bytes, nullptr), WAM_OK,
         "stack_fwd 2 chunks");
  float* h = static_cast<float*>(dev((size_t)br * 2 * m.Lq * c.dim * 4, "h"));
  expect(wam_dit_block_fwd(&m.c, &m.blocks[0], 0, &m.kv, &m.cx, h, e6, 2, 4, 0, m.ws, m.ws_bytes, nullptr), WAM_OK,
         "block_fwd 2 chunks");
  expect(wam_dit_block_fwd(&m.c, &m.blocks[c.layers - 1], c.layers - 1, &m.kv, &m.cx, h, e6, 1, 4, 1, m.ws, m.ws_bytes,
                           nullptr), WAM_OK, "block_fwd commit");
  expect(m.kv.length, 3 * m.Lq, "cache length after a committing block");
  expect(wam_kv_evict(&m.c, &m.kv, m.Lq, c.frames_per_chunk, nullptr), WAM_OK, "kv_evict");
  expect(m.kv.length, 2 * m.Lq, "cache length after eviction");
  // the denoising loops: no reuse (tau > 1), reuse decided by the read-back similarity, replay, UniPC
  const int nv = Lv * P, na = La * A;
  float* gv = static_cast<float*>(dev(nv * 4, "g video"));
  float* ga = static_cast<float*>(dev(na * 4, "g action"));
  float* cp = static_cast<float*>(dev(12, "cos parts"));
  float grid[17];
  for (int k = 0; k <= 16; ++k) grid[k] = k / 16.f;
  int calls = 0;
  unsigned char flags[16];
  expect(wam_denoise_chunk(&m.c, &m.w, &m.kv, &m.cx, xv, xa, grid, 16, 5.f, 2.f, -1, 4, vv, va, gv, ga, cp, m.ws,
                           m.ws_bytes, nullptr, &calls, flags), WAM_OK, "denoise tau 2");
  expect(calls, 16, "denoise tau 2 calls");
  host_abi::g_cos_parts[0] = 0.999f;   // cosine 0.999 > 0.99: every step after the second reuses
  expect(wam_denoise_chunk(&m.c, &m.w, &m.kv, &m.cx, xv, xa, grid, 16, 5.f, 0.99f, -1, 4, vv, va, gv, ga, cp, m.ws,
                           m.ws_bytes, nullptr, &calls, flags), WAM_OK, "denoise tau 0.99");
  expect(calls, 2, "denoise tau 0.99 calls");
  host_abi::g_cos_parts[0] = 0.5f;
  unsigned char replay[16] = {0, 0, 1, 0, 1, 1, 0, 0, 0, 1, 0, 0, 0, 0, 1, 0};
  float cos[16];
  expect(wam_denoise_chunk_replay(&m.c, &m.w, &m.kv, &m.cx, xv, xa, grid, 16, 5.f, replay, 4, vv, va, gv, ga, cp, m.ws,
                                  m.ws_bytes, nullptr, &calls, cos), WAM_OK, "denoise replay");
  expect(calls, 11, "denoise replay calls");
  expect(std::isnan(cos[1]) && std::fabs(cos[2] - 0.5f) < 1e-6f ? 1 : 0, 1, "replay cosines");
  float* state = static_cast<float*>(dev((size_t)5 * (nv + na) * 4, "unipc state"));
  expect(wam_denoise_chunk_unipc(&m.c, &m.w, &m.kv, &m.cx, xv, xa, grid, 16, 5.f, 2.f, -1, 4, 2, 1, vv, va, gv, ga, cp,
                                 state, m.ws, m.ws_bytes, nullptr, &calls, flags), WAM_OK, "denoise unipc");
  expect(wam_flow_step(xv, xa, vv, va, br, 5.f, nv, na, 0.1f, 0.1f, gv, ga, gv, cp, m.ws, m.ws_bytes, nullptr), WAM_OK,
         "flow_step");
  expect(wam_flow_step_noalloc(xv, xa, vv, va, br, 5.f, nv, na, 0.1f, 0.1f, gv, ga, gv, cp, nullptr), WAM_OK,
         "flow_step_noalloc");
  // errors: every one before any launch
  const long before = host_abi::g_launches;
  long launched = 0;
  wam_kv_cache small = m.kv;
  small.capacity = 64;
  expect(wam_dit_stack_fwd(&m.c, &m.w, &small, &m.cx, 1, xv, xa, t1, t2, 4, vv, va, m.ws, m.ws_bytes, nullptr),
         WAM_E_CAPACITY, "stack_fwd over capacity");
  expect(wam_dit_stack_fwd(nullptr, &m.w, &m.kv, &m.cx, 1, xv, xa, t1, t2, 4, vv, va, m.ws, m.ws_bytes, nullptr),
         WAM_E_ARG, "stack_fwd NULL config");
  expect(wam_dit_stack_fwd(&m.c, &m.w, &m.kv, &m.cx, 9, xv, xa, t1, t2, 4, vv, va, m.ws, m.ws_bytes, nullptr),
         WAM_E_SHAPE, "stack_fwd 9 chunks");
  expect(wam_dit_stack_fwd(&m.c, &m.w, &m.kv, &m.cx, 1, xv, xa, t1, t2, 4, vv, va, m.ws, 16, nullptr), WAM_E_ARG,
         "stack_fwd small workspace");
  expect(wam_dit_block_fwd(&m.c, &m.blocks[0], c.layers, &m.kv, &m.cx, h, e6, 1, 4, 0, m.ws, m.ws_bytes, nullptr),
         WAM_E_ARG, "block_fwd bad layer");
  const int len = m.kv.length;
  expect(wam_dit_block_fwd(&m.c, &m.blocks[0], 0, &small, &m.cx, h, e6, 1, 4, 1, m.ws, m.ws_bytes, nullptr),
         WAM_E_CAPACITY, "block_fwd commit over capacity");
  expect(m.kv.length, len, "length unchanged by a failed call");
  expect(wam_kv_evict(&m.c, &m.kv, m.Lq + 8, 0, nullptr), WAM_E_SHAPE, "evict partial chunk");
  if (packed) {   // a misaligned packed arena is rejected before anything runs
    const void* pk = m.blocks[0].pk;
    m.blocks[0].pk = static_cast<const char*>(pk) + 16;
    expect(wam_dit_stack_fwd(&m.c, &m.w, &m.kv, &m.cx, 1, xv, xa, t1, t2, 4, vv, va, m.ws, m.ws_bytes, nullptr),
           WAM_E_ARG, "stack_fwd with a misaligned packed arena");
    m.blocks[0].pk = pk;
  }
  unsigned char bad[16] = {0, 1};   // step 1 always runs the DiT
  expect(wam_denoise_chunk_replay(&m.c, &m.w, &m.kv, &m.cx, xv, xa, grid, 16, 5.f, bad, 4, vv, va, gv, ga, cp, m.ws,
                                  m.ws_bytes, nullptr, &calls, cos), WAM_E_ARG, "replay skipping step 1");
  launched = host_abi::g_launches - before;
  if (launched) { std::fprintf(stderr, "host_abi: %ld launches by calls that had to fail\n", launched); ++g_fail; }
  wam_kv_reset(&m.kv);
  expect(m.kv.length, 0, "kv_reset");
  host_abi::clear_regions();
}
}  // namespace

int main() {
  // kernel-level calls
  {
    void* a = dev(1 << 20, "A");
    void* wt = dev(1 << 20, "W");
    void* cc = dev(1 << 20, "C");
    expect(wam_op_linear(WAM_BF16, a, 64, wt, 64, nullptr, cc, 64, 64, 64, 64, 0, nullptr, 0, nullptr), WAM_OK, "op_linear");
    expect(wam_op_linear(WAM_BF16, a, 64, wt, 64, nullptr, cc, 64, 64, 64, 60, 0, nullptr, 0, nullptr), WAM_E_SHAPE,
           "op_linear K not a multiple of 64");
    expect(wam_op_attention(WAM_BF16, a, wt, cc, a, 1, 2, 64, 32, 64, 64, 0, 0, 64, nullptr, 0, nullptr), WAM_OK,
           "op_attention");
    void* wp = dev(64 * 64 * 2, "packed W");
    expect(wam_pack_weight(wt, 64, 64, 64, wp, nullptr), WAM_OK, "pack_weight");
    expect(wam_op_linear_packed(a, 64, wp, nullptr, cc, 64, 64, 64, 64, 0, nullptr, 0, nullptr), WAM_OK,
           "op_linear_packed");
    expect(wam_op_linear_packed(a, 64, wp, nullptr, cc, 64, 40, 64, 64, 2, nullptr, 0, nullptr), WAM_OK,
           "op_linear_packed swiglu");
    {
      const long before_pk = host_abi::g_launches;
      expect(wam_pack_weight(wt, 64, 48, 64, wp, nullptr), WAM_E_SHAPE, "pack_weight N not a multiple of 32");
      expect(wam_pack_weight(wt, 60, 64, 64, wp, nullptr), WAM_E_SHAPE, "pack_weight ldw below K");
      expect(wam_op_linear_packed(a, 64, wp, nullptr, cc, 64, 64, 48, 64, 0, nullptr, 0, nullptr), WAM_E_SHAPE,
             "op_linear_packed N not a multiple of 32");
      expect(wam_op_linear_packed(a, 64, wp, nullptr, cc, 64, 64, 64, 64, 3, nullptr, 0, nullptr), WAM_E_ARG,
             "op_linear_packed act 3");
      expect(wam_op_linear_packed(a, 64, static_cast<char*>(wp) + 8, nullptr, cc, 64, 64, 64, 64, 0, nullptr, 0,
                                  nullptr), WAM_E_ARG, "op_linear_packed misaligned W");
      wam_config cf = config(false, WAM_F32);
      expect((int)wam_pack_block_bytes(&cf), 0, "pack_block_bytes f32");
      wam_block_weights nb{};
      expect(wam_pack_block(&cf, &nb, wp, 1 << 20, nullptr), WAM_E_UNSUPPORTED, "pack_block f32");
      expect((int)(host_abi::g_launches - before_pk), 0, "no launch by a rejected packing call");
    }
    float* o = static_cast<float*>(dev(256 * 256 * 4, "probe"));
    expect(wam_mfma_peak_probe(o, 256, 8, nullptr), WAM_OK, "mfma peak probe");
    expect(wam_mfma_peak_probe(o, 0, 8, nullptr), WAM_E_ARG, "mfma peak probe, no workgroups");
    expect(wam_qkv_timer_config(0, 2), WAM_OK, "qkv timer");
    int n = -1;
    float ms[2];
    expect(wam_qkv_timer_read(ms, 2, &n), WAM_OK, "qkv timer read");
    expect(wam_qkv_timer_config(-1, 1), WAM_OK, "qkv timer off");
    const int M = 40, N = 1024;
    float* part = static_cast<float*>(dev((size_t)3 * M * N * 4, "finish partials"));
    float* hh = static_cast<float*>(dev((size_t)M * N * 4, "finish h"));
    float* e6v = static_cast<float*>(dev((size_t)6 * N * 4, "finish e6"));
    float* mg = static_cast<float*>(dev((size_t)6 * N * 4, "finish gate offsets"));
    float* mn = static_cast<float*>(dev((size_t)6 * N * 4, "finish norm offsets"));
    void* yy = dev((size_t)M * N * 2, "finish y");
    expect(wam_op_split_finish(part, 3, M, N, e6v, hh, e6v, mg, 5, mn, 0, 1, 0, 1e-6f, yy, nullptr), WAM_OK,
           "op_split_finish gated");
    expect(wam_op_split_finish(part, 3, M, N, nullptr, hh, e6v, nullptr, -1, mn, 3, 4, 1, 1e-6f, yy, nullptr), WAM_OK,
           "op_split_finish plain");
    expect(wam_op_modulated_norm(hh, M, N, e6v, mn, 0, 1, 0, 1e-6f, yy, nullptr), WAM_OK, "op_modulated_norm");
    const long before_bad = host_abi::g_launches;
    expect(wam_op_split_finish(part, 5, M, N, nullptr, hh, e6v, mg, 5, mn, 0, 1, 0, 1e-6f, yy, nullptr), WAM_E_SHAPE,
           "op_split_finish 5 splits");
    expect(wam_op_split_finish(part, 3, M, N, nullptr, hh, e6v, nullptr, 2, mn, 0, 1, 0, 1e-6f, yy, nullptr), WAM_E_ARG,
           "op_split_finish gate without offsets");
    expect(wam_op_modulated_norm(hh, M, N + 2, e6v, mn, 0, 1, 0, 1e-6f, yy, nullptr), WAM_E_SHAPE,
           "op_modulated_norm D not a multiple of 4");
    expect(wam_op_modulated_norm(hh, M, N, e6v, mn, 0, 6, 0, 1e-6f, yy, nullptr), WAM_E_ARG,
           "op_modulated_norm slot 6");
    expect((int)(host_abi::g_launches - before_bad), 0, "no launch by a rejected op");
    {
      const int br = 2, rows = 48, H = 4, d = 64, D = H * d, cap = 64;
      void* qkv = dev((size_t)br * rows * 3 * D * 2, "qkv rows");
      float* gq = static_cast<float*>(dev((size_t)D * 4, "g_q"));
      float* gk = static_cast<float*>(dev((size_t)D * 4, "g_k"));
      float* rope = static_cast<float*>(dev((size_t)rows * d * 4, "rope table"));
      void* qo = dev((size_t)br * H * rows * d * 2, "q out");
      void* kc = dev((size_t)br * H * cap * d * 2, "k cache");
      void* vc = dev((size_t)br * H * d * cap * 2, "v cache");
      expect(wam_op_qkv_cache(qkv, br, rows, 24, 20, H, d, gq, gk, 1e-6f, rope, qo, kc, vc, cap, 16, nullptr), WAM_OK,
             "op_qkv_cache");
      const long before_q = host_abi::g_launches;
      expect(wam_op_qkv_cache(qkv, br, rows, 24, 20, H, d, gq, gk, 1e-6f, rope, qo, kc, vc, cap, 24, nullptr),
             WAM_E_SHAPE, "op_qkv_cache past the cache");
      expect(wam_op_qkv_cache(qkv, br, rows, 24, 20, H, 96, gq, gk, 1e-6f, rope, qo, kc, vc, cap, 0, nullptr),
             WAM_E_SHAPE, "op_qkv_cache head dim 96");
      expect((int)(host_abi::g_launches - before_q), 0, "no launch by a rejected q/k/v op");
    }
    host_abi::clear_regions();
  }
  scenario("tiny bf16", config(false, WAM_BF16));
  scenario("tiny f32", config(false, WAM_F32));
  {
    wam_config c = config(false, WAM_BF16);
    c.variant = WAM_VARIANT_FRAME_CAUSAL | WAM_VARIANT_RMS_NORM | WAM_VARIANT_SWIGLU | WAM_VARIANT_IMG_XATTN;
    c.ctx_img_len = 16;
    scenario("tiny variants", c);
  }
  {
    wam_config c = config(false, WAM_BF16);
    c.ctx_state_len = 3;
    scenario("tiny state rows", c);
  }
  {
    wam_config c = config(false, WAM_BF16);
    c.precision = WAM_PRECISION_MXFP8;
    scenario("tiny mxfp8", c);
    c.precision = WAM_PRECISION_MXFP4W;
    scenario("tiny mxfp4 weights", c);
  }
  scenario("tiny bf16, packed projections", config(false, WAM_BF16), true);
  {
    wam_config c = config(false, WAM_BF16);
    c.variant = WAM_VARIANT_SWIGLU;
    scenario("tiny swiglu, packed projections", c, true);
  }
  scenario("full width bf16, 40 layers", config(true, WAM_BF16));
  scenario("full width bf16, 40 layers, packed projections", config(true, WAM_BF16), true);
  if (g_fail || host_abi::g_errors) {
    std::fprintf(stderr, "host_abi: %d failed expectations, %d launch-bound errors\n", g_fail, host_abi::g_errors);
    return 1;
  }
  std::printf("host_abi: OK (%ld launches checked)\n", host_abi::g_launches);
  return 0;
}
