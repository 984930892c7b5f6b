// Launchers of the gfx950 kernels (host-callable, no torch types). Each returns the HIP status of
// its launch; shapes are validated by the C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wam {

enum DType { DT_BF16 = 0, DT_F32 = 1 };

// ---- GEMM: C[m][n] = sum_k A[m][k] W[n][k] (+ bias[n]) followed by an epilogue ----------------
enum Epi {
  EPI_STORE = 0,        // C (element type T) = acc + bias
  EPI_GELU = 1,         // C (T) = gelu_tanh(acc + bias)
  EPI_RESID = 2,        // H (fp32) += acc + bias
  EPI_RESID_GATED = 3,  // H (fp32) += gate[row group][n] * (acc + bias), gate = e6[chunk][group][gi] + mod[gi]
  EPI_ROWSEL_F32 = 4,   // fp32 output of the rows of one token group, gathered per branch (output heads)
  EPI_SWIGLU = 5,       // C[m][j] (T) = silu(acc[m][2j] + bias[2j]) * (acc[m][2j+1] + bias[2j+1]), N even
};

struct RowMap {       // how a GEMM row maps to (branch, chunk, token group)
  int rows_per_branch;  // n_chunks * Lq
  int Lq, Lv;           // tokens per chunk, video tokens per chunk
};

struct GemmArgs {
  const void* A; long lda;   // [M][K], element type T
  const void* W; long ldw;   // [N][K], element type T (nn.Linear layout)
  const float* bias;         // [N] or nullptr
  void* C; long ldc;         // EPI_STORE / EPI_GELU / EPI_ROWSEL_F32 output
  float* H; long ldh;        // EPI_RESID* fp32 residual stream
  int M, N, K;
  RowMap rm;
  const float* e6;           // EPI_RESID_GATED: [n_chunks][2][6][D]
  const float* mod;          // EPI_RESID_GATED: [6][D]
  int gate_idx, D;
  int sel_group;             // EPI_ROWSEL_F32: 0 = video rows, 1 = action rows
  float* part;               // split-K scratch: [splits][M][N] partial products (nullptr: no split), fp32,
                             //   or bf16 when part_bf16 is set (the block's fused split path)
  long part_elems;           // capacity of `part` in floats
  const uint8_t* As;         // MXFP8 operands only: e8m0 scales of A [M][K/32] and of W [N][K/32]
  const uint8_t* Ws;         //   (A and W then hold fp8 e4m3 codes, lda / ldw in bytes)
  int w_fp4;                 // MXFP8 operands only: W holds e2m1 nibbles (two k per byte, low first)
  int part_bf16;             // split-K partials stored as bf16 (each rounded once), read back by the finish
  int w_packed;              // bf16 only: W holds the fragment-packed layout of launch_pack_weight (ldw
                             //   unused; N % 32 == 0, K % 64 == 0, N * K * 2 < 2^31)
};

hipError_t launch_gemm(const GemmArgs& a, DType dt, Epi epi, hipStream_t s);
// Fragment-packed copy of a bf16 matrix W [N][K] (row stride ldw elements) for the products with
// w_packed set: Wp holds N * K bf16 in blocks of 32 rows x 16 k, 64 lanes x 16 bytes each, lane l
// holding row 32 b + l % 32 at k 16 c + 8 (l / 32) .. + 7, blocks of a row band consecutive along k.
// N % 32 == 0, K % 64 == 0, ldw % 8 == 0, 16-byte aligned pointers.
hipError_t launch_pack_weight(const void* W, long ldw, int N, int K, void* Wp, hipStream_t s);
// MXFP8 product ([N569] real-time optimisations: quantised projections; the OCP microscaling format
// that gfx950's scaled MFMA reads): A, W fp8 e4m3 with one power-of-two scale per 32 consecutive k,
// fp32 accumulation, the same epilogues as the bf16 product (bf16 outputs). K % 128 == 0, N % 4 == 0.
hipError_t launch_gemm_mx(const GemmArgs& a, Epi epi, hipStream_t s);
// Quantise rows of a bf16 / fp32 matrix to MXFP8: codes [rows][cols] (row stride ldq bytes) and scales
// [rows][cols/32]; cols % 32 == 0.
hipError_t launch_mx_quantize(const void* src, long ld_src, DType dt, int rows, int cols, uint8_t* codes, long ldq,
                              uint8_t* scales, hipStream_t s);
// The same for MXFP4 (e2m1 elements, block exponent floor(log2 amax) - 2): codes two per byte, low
// nibble first, [rows][ldq] bytes with ldq >= cols / 2.
hipError_t launch_mx4_quantize(const void* src, long ld_src, DType dt, int rows, int cols, uint8_t* codes, long ldq,
                               uint8_t* scales, hipStream_t s);

// ---- attention ----------------------------------------------------------------------------------
struct AttnArgs {
  const void* Q;      // [br][H][Lq_total][d]
  const void* K;      // [br][H][k_rows][d]     (k_rows = row capacity of one head's key block)
  const void* Vt;     // [br][H][d][v_stride]   (values stored key-contiguous)
  void* O;            // [br * Lq_total][H * d] row-major
  long q_bh_stride, k_bh_stride, v_bh_stride;   // elements between consecutive (branch, head) blocks
  int v_stride;       // keys per row of Vt
  int Lq_total, H, d, br;
  int kv_base;        // keys visible to every query (cached clean chunks)
  int chunk_q;        // queries per chunk (for the chunk-causal limit); <= 0: no chunk limit
  int kv_total;       // total keys present (kv_base + current keys)
  float scale_log2;   // log2(e) / sqrt(d)
  float* part;        // scratch for key-split partial outputs (nullptr: never split)
  long part_elems;    // capacity of `part` in floats
  int kv_splits;      // set by launch_attention: key ranges per query block (1 = no split)
  int frame_tokens;   // > 0 (with chunk_q > 0): frame-causal inside a chunk, frames of this many tokens
  int video_tokens;   // video tokens at the start of each chunk (frame-causal only)
};
// MXFP8 attention (head dim 128): e4m3 codes with e8m0 scales per 32 values; byte strides between
// consecutive (branch, head) blocks.
struct AttnMxArgs {
  const uint8_t* Q;    // [br][H][Lq][128] codes
  const uint8_t* Qs;   // [br][H][Lq][4] scales (blocks of 32 head-dim values)
  const uint8_t* K;    // [br][H][k_rows][128]
  const uint8_t* Ks;   // [br][H][k_rows][4]
  const uint8_t* Vt;   // [br][H][128][v_stride] (key-contiguous)
  const uint8_t* Vs;   // [br][H][v_stride / 32][128] (block-major: the 128 rows' scales of key block kb)
  void* O;             // bf16 [br * Lq][H * 128]
  long q_bh, qs_bh, k_bh, ks_bh, v_bh, vs_bh;
  int v_stride, Lq, H, br, kv_base, chunk_q, kv_total;
  float scale_log2;    // log2(e) / sqrt(128)
};
hipError_t launch_attention_mx(const AttnMxArgs& a, hipStream_t s);

// Keys visible to query q: a prefix [0, limit) of the key rows. Cached keys (below kv_base) are
// always visible; inside the pass, keys up to the end of the query's chunk (chunk_q > 0), or with
// frame_tokens > 0 up to the end of the query's frame for video queries.
__host__ __device__ inline int attn_limit(const AttnArgs& a, int q) {
  int lim = a.kv_total;
  if (a.chunk_q > 0) {
    const int loc = q % a.chunk_q;
    int inside = a.chunk_q;
    if (a.frame_tokens > 0 && loc < a.video_tokens) inside = (loc / a.frame_tokens + 1) * a.frame_tokens;
    const int c = a.kv_base + (q - loc) + inside;
    lim = c < lim ? c : lim;
  }
  return lim;
}
hipError_t launch_attention(const AttnArgs& a, DType dt, hipStream_t s);
// Key ranges per query block the bf16 kernel takes for these sizes (flash-decoding-style split when
// the query blocks alone would leave most CUs idle), and the scratch floats that split needs.
int attn_kv_splits(int Lq_total, int H, int br, int kv_total);
long attn_split_floats(int Lq_total, int H, int br, int kv_total);

// ---- row-wise kernels -----------------------------------------------------------------------------
enum NormMode {
  NORM_ADALN = 0,       // LN(x) (1 + scale) + shift, scale/shift from e6 (+ layer offset)
  NORM_AFFINE = 1,      // LN(x) w + b
  NORM_HEAD = 2,        // LN(x) (1 + head_mod[1] + e) + head_mod[0] + e
};
struct NormArgs {
  const float* X;       // [M][D] fp32 residual stream
  void* Y;              // [M][D] T
  int M, D;
  float eps;
  NormMode mode;
  RowMap rm;
  const float* e6;      // ADALN: [n_chunks][2][6][D]; HEAD: e [n_chunks][2][D]
  const float* mod;     // ADALN: [6][D] layer offset; HEAD: head_mod [2][D]
  int shift_idx, scale_idx;
  const float* w;       // AFFINE
  const float* b;
  int rms;              // RMSNorm (no mean subtraction) in place of LayerNorm
  uint8_t* mxq;         // bf16 only, optional: MXFP8 copy of Y, codes [M][D] and scales [M][D/32]
  uint8_t* mxs;         //   (D % 32 == 0), quantised from the stored bf16 values
};
hipError_t launch_norm(const NormArgs& a, DType dt, hipStream_t s);
// y[g][n] = x[g] . W[n] + bias[n] for g < G <= 4 rows (storage type in and out, fp32 sums; bias may be
// NULL); K and ldx multiples of 16 bytes' worth of elements, 16-byte aligned W and x.
hipError_t launch_gemv_store(const void* W, const float* bias, const void* x, long ldx, void* y, long ldy, int G, int N,
                             int K, DType dt, hipStream_t s);
// dst[i] += src[i] for i < n (elements of the storage type; n % 8 == 0, 16-byte aligned pointers)
hipError_t launch_add(void* dst, const void* src, long n, DType dt, hipStream_t s);

struct QkNormArgs {
  const void* src; long src_ld;     // rows of the projection output ([M][src_ld], T)
  int src_col;                      // first column of this tensor in a row
  const float* gain;                // [D]
  void* dst;                        // head-major destination [br][H][dst_rows][d]
  long dst_bh_stride;               // elements between consecutive (branch, head) blocks
  int dst_row0;                     // first destination row (cache length for keys)
  int M, D, H, d;
  int rows_per_branch;
  float eps;
  const float2* rope;               // [rows_per_branch][d/2] (cos, sin) or nullptr; rows of action tokens unused
  RowMap rm;
};
hipError_t launch_qk_norm_rope(const QkNormArgs& a, DType dt, hipStream_t s);

// Row stage that follows a product. POST_NORM: the LayerNorm `na` of the product's updated residual
// rows (na.X is the product's H); POST_QK: the q/k RMSNorm `qa` of the product's output rows (qa.src
// is the product's C; no rotary embedding). When the product is split over K, the stage runs in the
// kernel that sums the partials (one workgroup per row), otherwise as its own launch afterwards.
enum PostMode { POST_NONE = 0, POST_NORM = 1, POST_QK = 2 };
struct PostArgs {
  PostMode mode;
  NormArgs na;
  QkNormArgs qa;
};
hipError_t launch_gemm_post(const GemmArgs& a, DType dt, Epi epi, const PostArgs& post, hipStream_t s);
// The finishing row kernel of a split product on its own: sums a.part[0 .. splits-1] in split order,
// adds a.bias, applies the epilogue (EPI_RESID / EPI_RESID_GATED into a.H, or EPI_STORE feeding
// POST_QK) and runs the row stage `post` (bf16 only, 2 <= splits <= 4, N % 4 == 0, N <= 8192).
hipError_t launch_split_finish(const GemmArgs& a, Epi epi, const PostArgs& post, int splits, hipStream_t s);

struct VCacheArgs {
  const void* src; long src_ld; int src_col;   // v = src[row][src_col + h*d + j]
  void* dst; long dst_bh_stride; int dst_stride; int dst_col0;   // Vt[b][h][j][dst_col0 + r]
  int rows_per_branch, br, H, d;
};
hipError_t launch_v_to_cache(const VCacheArgs& a, DType dt, hipStream_t s);
// q (optional) and k norms plus the value transpose in one launch (bf16; other cases run the three
// launches above)
hipError_t launch_qkv_cache(const QkNormArgs* q, const QkNormArgs& k, const VCacheArgs& v, DType dt, hipStream_t s);

// Sliding-window eviction: keep rows [drop, len) of every (layer, branch, head) block, moved to the
// front, with the frame-axis pairs of video keys rotated by (cos, sin) = cs[j] (j < frame_pairs).
struct KvEvictArgs {
  void* k;            // [blocks][cap][d]
  void* v;            // [blocks][d][cap]
  int blocks, cap, d, len, drop;
  int Lq, Lv;         // rows per cached chunk, video rows first (drop is a multiple of Lq)
  int frame_pairs;    // channel pairs (2j, 2j+1) of a head on the frame axis
  float2 cs[64];
};
hipError_t launch_kv_evict(const KvEvictArgs& a, DType dt, hipStream_t s);

// rotary (cos, sin) table for the video tokens of n_chunks chunks, written for every row of a branch
hipError_t launch_rope_table(float2* table, int n_chunks, int Lq, int Lv, int frames_per_chunk, int grid_h,
                             int grid_w, int start_frame, int head_dim, float theta, hipStream_t s);

// token embedding: h[b][row] = x_video/x_action row times the patch/action linear, for every branch
struct EmbedArgs {
  const float* xv; const float* xa;
  const void* pe_w; const float* pe_b; const void* ae_w; const float* ae_b;
  float* H;
  int n_chunks, Lv, La, P, A, D, br;
};
hipError_t launch_embed(const EmbedArgs& a, DType dt, hipStream_t s);

// small-batch matrix-vector products for the time embedding path
struct TimeArgs {
  float t[16];             // [G] timesteps, passed by value (host scalars)
  int G, freq_dim, D;
  const void *w1, *w2, *wp; const float *b1, *b2, *bp;
  float* emb;              // [G][freq_dim] scratch
  float* h1;               // [G][D] scratch
  float* e;                // [G][D] out
  float* e6;               // [G][6D] out
};
hipError_t launch_time_mlp(const TimeArgs& a, DType dt, hipStream_t s);

struct FlowArgs {
  float* xv; float* xa;
  const float* vv; const float* va;   // [br][n]
  int br; float w;
  int nv, na;
  float dtv, dta;
  float* gv; float* ga;               // guided velocities out (optional)
  const float* prev;                  // previous guided video velocity (optional)
  float* partials;                    // [nblocks][3] scratch
  float* cos_parts;                   // [3] out
  int nblocks;
};
hipError_t launch_flow_step(const FlowArgs& a, hipStream_t s);

// One UniPC step on the concatenated [video | action] latent (n = nv + na): the guided velocity g
// (as in the flow step), the data prediction m = x + sigma g, optionally the previous step's
// corrector xs = ca x_prev + sum_j cw[j] m_{cslot[j]} + ct m, then the predictor
// x_next = pa xs + pw[0] m + sum_{j>=1} pw[j] m_{pslot[j]}. `state` holds `slots` data predictions
// of n floats each followed by x_prev; m goes to slot `slot_new`, xs to x_prev.
struct UnipcArgs {
  float* xv; float* xa;
  const float* vv; const float* va;   // [br][n] model outputs, or a reused guided velocity (br = 1, w = 1)
  int br; float w;
  int nv, na;
  float sigma;
  float* gv; float* ga;               // guided velocities out (optional)
  const float* prev;                  // previous guided video velocity (optional, cosine partials)
  float* partials; float* cos_parts;
  float* state;
  int slot_new;
  int corr, cn; float ca, ct; float cw[4]; int cslot[4];
  int pn; float pa; float pw[4]; int pslot[4];
};
hipError_t launch_unipc_step(const UnipcArgs& a, hipStream_t s);

// Output heads: video rows (first Lv of each chunk) -> Wv [P][D], action rows -> Wa [A][D], written
// token-major per branch to vv [br][n*Lv][P] and va [br][n*La][A]. K is split `splits` ways into
// fp32 partials part[splits][M][64] (summed in order by the second kernel). P, A <= 64.
struct HeadArgs {
  const void* Y; int M, D;
  const void* wv; const float* bv; int P;
  const void* wa; const float* ba; int A;
  float* vv; float* va;
  RowMap rm;
  float* part; long part_elems;   // scratch for the K slices' partial outputs (fp32 capacity)
  int splits;                      // set by launch_head
};
hipError_t launch_head(const HeadArgs& a, DType dt, hipStream_t s);
// workgroups (and [3] partial-sum slots) of the flow step for these sizes: 1 .. 512
int flow_partial_blocks(int nv, int na);
// Matrix-core peak probe: `workgroups` x 256 threads, each wave `iters` x 8 independent bf16
// 32x32x16 MFMAs (32768 flops each); one float per thread to `out`.
hipError_t launch_mfma_peak(float* out, int workgroups, int iters, hipStream_t s);
// Device address (for the current device) and size of the library-owned flow-step scratch.
hipError_t flow_scratch(float** ptr, size_t* bytes);

}  // namespace wam
