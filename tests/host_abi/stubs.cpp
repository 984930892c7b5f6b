// Host-only stand-ins for the kernel launchers and the few HIP runtime calls of the C-ABI layer, so
// that layer can be built with the host compiler under AddressSanitizer / UndefinedBehaviorSanitizer
// and driven without a GPU. No stand-in dereferences a device pointer: each checks that every
// buffer a launch would touch lies inside a region the driver registered (fake device addresses),
// and counts the launch.
#include "stubs.h"

#include <cstdio>
#include <vector>

#include "../../world_action_video_amd/csrc/kernels.h"

namespace host_abi {
struct Region { uintptr_t base; size_t bytes; std::string name; };
static std::vector<Region> g_regions;
int g_errors = 0;
long g_launches = 0;
float g_cos_parts[3] = {0.5f, 1.f, 1.f};

void register_region(const void* base, size_t bytes, const std::string& name) {
  g_regions.push_back({reinterpret_cast<uintptr_t>(base), bytes, name});
}
void clear_regions() { g_regions.clear(); }

void check(const void* p, size_t bytes, const char* what) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (!p) {
    std::fprintf(stderr, "host_abi: %s is NULL\n", what);
    ++g_errors;
    return;
  }
  for (const Region& r : g_regions)
    if (a >= r.base && a + bytes <= r.base + r.bytes) return;
  std::fprintf(stderr, "host_abi: %s [%#lx, +%zu) outside every registered buffer\n", what, (unsigned long)a, bytes);
  ++g_errors;
}
}  // namespace host_abi

using host_abi::check;

namespace wam {
static size_t esz(DType dt) { return dt == DT_BF16 ? 2 : 4; }

static void check_gemm(const GemmArgs& a, size_t ea, size_t ew, size_t ec, Epi epi) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) { std::fprintf(stderr, "host_abi: gemm sizes\n"); ++host_abi::g_errors; return; }
  check(a.A, ((size_t)(a.M - 1) * a.lda + a.K) * ea, "gemm A");
  if (a.w_packed) check(a.W, (size_t)a.N * a.K * 2, "gemm packed W");
  else check(a.W, ((size_t)(a.N - 1) * a.ldw + a.K) * ew, "gemm W");
  if (a.bias) check(a.bias, (size_t)a.N * 4, "gemm bias");
  if (epi == EPI_RESID || epi == EPI_RESID_GATED) check(a.H, ((size_t)(a.M - 1) * a.ldh + a.N) * 4, "gemm H");
  else if (epi == EPI_SWIGLU) check(a.C, ((size_t)(a.M - 1) * a.ldc + a.N / 2) * ec, "gemm C");
  else if (epi != EPI_ROWSEL_F32) check(a.C, ((size_t)(a.M - 1) * a.ldc + a.N) * ec, "gemm C");
  if (a.part) check(a.part, (size_t)a.part_elems * 4, "gemm split-K partials");
}
hipError_t launch_gemm(const GemmArgs& a, DType dt, Epi epi, hipStream_t) {
  ++host_abi::g_launches;
  check_gemm(a, esz(dt), esz(dt), esz(dt), epi);
  return hipSuccess;
}
hipError_t launch_pack_weight(const void* W, long ldw, int N, int K, void* Wp, hipStream_t) {
  ++host_abi::g_launches;
  check(W, ((size_t)(N - 1) * ldw + K) * 2, "pack source");
  check(Wp, (size_t)N * K * 2, "pack destination");
  return hipSuccess;
}
hipError_t launch_gemm_mx(const GemmArgs& a, Epi epi, hipStream_t) {
  ++host_abi::g_launches;
  check_gemm(a, 1, 1, 2, epi);
  check(a.As, (size_t)a.M * (a.K / 32), "gemm A scales");
  check(a.Ws, (size_t)a.N * (a.K / 32), "gemm W scales");
  return hipSuccess;
}
static void check_norm(const NormArgs& n, DType dt) {
  check(n.X, (size_t)n.M * n.D * 4, "norm X");
  check(n.Y, (size_t)n.M * n.D * esz(dt), "norm Y");
  if (n.mxq) check(n.mxq, (size_t)n.M * n.D, "norm MXFP8 codes");
}
hipError_t launch_gemm_post(const GemmArgs& a, DType dt, Epi epi, const PostArgs& p, hipStream_t s) {
  if (dt == DT_BF16 && a.As) launch_gemm_mx(a, epi, s); else launch_gemm(a, dt, epi, s);
  if (p.mode == POST_NORM) check_norm(p.na, dt);
  return hipSuccess;
}
hipError_t launch_split_finish(const GemmArgs& a, Epi epi, const PostArgs& p, int splits, hipStream_t) {
  ++host_abi::g_launches;
  check(a.part, (size_t)splits * a.M * a.N * 4, "finish partials");
  if (a.bias) check(a.bias, (size_t)a.N * 4, "finish bias");
  if (epi == EPI_RESID || epi == EPI_RESID_GATED) check(a.H, ((size_t)(a.M - 1) * a.ldh + a.N) * 4, "finish H");
  if (epi == EPI_RESID_GATED) check(a.mod, (size_t)6 * a.D * 4, "finish gate offsets");
  if (p.mode == POST_NORM) {
    check_norm(p.na, DT_BF16);
    check(p.na.mod, (size_t)6 * p.na.D * 4, "finish norm offsets");
  }
  return hipSuccess;
}
hipError_t launch_mx_quantize(const void* src, long ld, DType dt, int rows, int cols, uint8_t* codes, long ldq,
                              uint8_t* scales, hipStream_t) {
  ++host_abi::g_launches;
  check(src, ((size_t)(rows - 1) * ld + cols) * esz(dt), "mx source");
  check(codes, (size_t)(rows - 1) * ldq + cols, "mx codes");
  check(scales, (size_t)rows * (cols / 32), "mx scales");
  return hipSuccess;
}
hipError_t launch_mx4_quantize(const void* src, long ld, DType dt, int rows, int cols, uint8_t* codes, long ldq,
                               uint8_t* scales, hipStream_t) {
  ++host_abi::g_launches;
  check(src, ((size_t)(rows - 1) * ld + cols) * esz(dt), "mx4 source");
  check(codes, (size_t)(rows - 1) * ldq + cols / 2, "mx4 codes");
  check(scales, (size_t)rows * (cols / 32), "mx4 scales");
  return hipSuccess;
}
hipError_t launch_attention_mx(const AttnMxArgs&, hipStream_t) { ++host_abi::g_launches; return hipSuccess; }
hipError_t launch_attention(const AttnArgs& a, DType dt, hipStream_t) {
  ++host_abi::g_launches;
  const size_t e = esz(dt), bh = (size_t)a.br * a.H;
  check(a.Q, ((bh - 1) * a.q_bh_stride + (size_t)a.Lq_total * a.d) * e, "attention Q");
  check(a.K, ((bh - 1) * a.k_bh_stride + (size_t)a.kv_total * a.d) * e, "attention K");
  check(a.Vt, ((bh - 1) * a.v_bh_stride + (size_t)(a.d - 1) * a.v_stride + a.kv_total) * e, "attention Vt");
  check(a.O, (size_t)a.br * a.Lq_total * a.H * a.d * e, "attention O");
  return hipSuccess;
}
int attn_kv_splits(int, int, int, int) { return 1; }
long attn_split_floats(int, int, int, int) { return 0; }
hipError_t launch_norm(const NormArgs& a, DType dt, hipStream_t) {
  ++host_abi::g_launches;
  check_norm(a, dt);
  return hipSuccess;
}
hipError_t launch_gemv_store(const void* W, const float*, const void* x, long ldx, void* y, long ldy, int G, int N,
                             int K, DType dt, hipStream_t) {
  ++host_abi::g_launches;
  check(W, (size_t)N * K * esz(dt), "gemv W");
  check(x, ((size_t)(G - 1) * ldx + K) * esz(dt), "gemv x");
  check(y, ((size_t)(G - 1) * ldy + N) * esz(dt), "gemv y");
  return hipSuccess;
}
hipError_t launch_add(void* dst, const void* src, long n, DType dt, hipStream_t) {
  ++host_abi::g_launches;
  check(dst, (size_t)n * esz(dt), "add dst");
  check(src, (size_t)n * esz(dt), "add src");
  return hipSuccess;
}
static void check_qk(const QkNormArgs& a, DType dt, const char* what) {
  const size_t e = esz(dt);
  const int br = a.M / a.rows_per_branch;
  check(a.src, ((size_t)(a.M - 1) * a.src_ld + a.src_col + a.D) * e, what);
  check(a.dst, ((size_t)(br * a.H - 1) * a.dst_bh_stride + (size_t)(a.dst_row0 + a.rows_per_branch) * a.d) * e, what);
}
hipError_t launch_qk_norm_rope(const QkNormArgs& a, DType dt, hipStream_t) {
  ++host_abi::g_launches;
  check_qk(a, dt, "q/k norm");
  return hipSuccess;
}
static void check_v(const VCacheArgs& v, DType dt) {
  const size_t e = esz(dt);
  check(v.src, ((size_t)(v.br * v.rows_per_branch - 1) * v.src_ld + v.src_col + (size_t)v.H * v.d) * e, "value source");
  check(v.dst, ((size_t)(v.br * v.H - 1) * v.dst_bh_stride + (size_t)(v.d - 1) * v.dst_stride + v.dst_col0 +
                v.rows_per_branch) * e, "value cache");
}
hipError_t launch_v_to_cache(const VCacheArgs& a, DType dt, hipStream_t) {
  ++host_abi::g_launches;
  check_v(a, dt);
  return hipSuccess;
}
hipError_t launch_qkv_cache(const QkNormArgs* q, const QkNormArgs& k, const VCacheArgs& v, DType dt, hipStream_t) {
  ++host_abi::g_launches;
  if (q) check_qk(*q, dt, "q norm");
  check_qk(k, dt, "k norm");
  check_v(v, dt);
  return hipSuccess;
}
hipError_t launch_kv_evict(const KvEvictArgs& a, DType dt, hipStream_t) {
  ++host_abi::g_launches;
  check(a.k, (size_t)a.blocks * a.cap * a.d * esz(dt), "evict keys");
  check(a.v, (size_t)a.blocks * a.d * a.cap * esz(dt), "evict values");
  return hipSuccess;
}
hipError_t launch_rope_table(float2* t, int n, int Lq, int, int, int, int, int, int d, float, hipStream_t) {
  ++host_abi::g_launches;
  check(t, (size_t)n * Lq * (d / 2) * sizeof(float2), "rope table");
  return hipSuccess;
}
hipError_t launch_embed(const EmbedArgs& a, DType, hipStream_t) {
  ++host_abi::g_launches;
  check(a.xv, (size_t)a.n_chunks * a.Lv * a.P * 4, "embed video latents");
  check(a.xa, (size_t)a.n_chunks * a.La * a.A * 4, "embed action latents");
  check(a.H, (size_t)a.br * a.n_chunks * (a.Lv + a.La) * a.D * 4, "embed H");
  return hipSuccess;
}
hipError_t launch_time_mlp(const TimeArgs& a, DType, hipStream_t) {
  ++host_abi::g_launches;
  check(a.e, (size_t)a.G * a.D * 4, "time e");
  check(a.e6, (size_t)a.G * 6 * a.D * 4, "time e6");
  check(a.emb, (size_t)a.G * a.freq_dim * 4, "time sinusoid");
  check(a.h1, (size_t)a.G * a.D * 4, "time hidden");
  return hipSuccess;
}
hipError_t launch_flow_step(const FlowArgs& a, hipStream_t) {
  ++host_abi::g_launches;
  if (a.nv) { check(a.xv, (size_t)a.nv * 4, "flow x video"); check(a.vv, (size_t)a.br * a.nv * 4, "flow v video"); }
  if (a.na) { check(a.xa, (size_t)a.na * 4, "flow x action"); check(a.va, (size_t)a.br * a.na * 4, "flow v action"); }
  if (a.prev) check(a.partials, (size_t)a.nblocks * 12, "flow partials");
  return hipSuccess;
}
hipError_t launch_unipc_step(const UnipcArgs& a, hipStream_t) {
  ++host_abi::g_launches;
  check(a.state, (size_t)5 * (a.nv + a.na) * 4, "unipc state");
  return hipSuccess;
}
hipError_t launch_head(const HeadArgs& a, DType dt, hipStream_t) {
  ++host_abi::g_launches;
  check(a.Y, (size_t)a.M * a.D * esz(dt), "head input");
  return hipSuccess;
}
int flow_partial_blocks(int nv, int na) {
  const long units = ((long)nv + na + 3) / 4;
  const long b = (units + 1023) / 1024;
  return (int)(b < 1 ? 1 : b > 512 ? 512 : b);
}
hipError_t launch_mfma_peak(float* out, int wg, int, hipStream_t) {
  ++host_abi::g_launches;
  check(out, (size_t)wg * 256 * 4, "peak probe output");
  return hipSuccess;
}
static float g_scratch_stub[512 * 3];
hipError_t flow_scratch(float** p, size_t* bytes) {
  host_abi::register_region(g_scratch_stub, sizeof g_scratch_stub, "library scratch");
  *p = g_scratch_stub;
  *bytes = sizeof g_scratch_stub;
  return hipSuccess;
}
}  // namespace wam

// ---- the HIP runtime calls of the C-ABI layer (events of the measurement hook, the 12-byte
// similarity read-back of the denoising loop)
hipError_t hipEventCreate(hipEvent_t* e) { static int dummy; *e = reinterpret_cast<hipEvent_t>(&dummy); return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) { *ms = 1.f; return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t) {
  if (kind != hipMemcpyDeviceToHost || bytes != sizeof host_abi::g_cos_parts) { ++host_abi::g_errors; return hipErrorInvalidValue; }
  check(src, bytes, "similarity read-back");
  std::memcpy(dst, host_abi::g_cos_parts, bytes);
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub"; }
