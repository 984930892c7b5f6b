// Row-wise and small kernels of the DiT step: LayerNorm + adaLN modulation, q/k RMSNorm + 3-D
// rotary embedding with the head-major / KV-cache scatter, the value transpose into the cache,
// the rotary table, token embedding, the time-embedding MLP and the fused CFG + Euler + cosine
// update. All statistics are accumulated in fp32 with a fixed reduction order (deterministic).
#include "common.h"
#include "kernels.h"

namespace wam {

// ------------------------------------------------------------------------------------------------
// LayerNorm (+ modulation): one workgroup per row, D/4 float4 per row spread over 256 threads.
// ------------------------------------------------------------------------------------------------
static constexpr int NORM_MAXV = 8;   // up to D = 8192

template <typename T>
__global__ void __launch_bounds__(256) norm_kernel(NormArgs a) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const float4* x4 = reinterpret_cast<const float4*>(a.X + (long)row * a.D);
  const int nv = a.D / 4;
  float4 xv[NORM_MAXV];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NORM_MAXV; ++k) {
    const int i = tid + 256 * k;
    if (i < nv) {
      xv[k] = x4[i];
      s += (xv[k].x + xv[k].y) + (xv[k].z + xv[k].w);
    }
  }
  const float mean = block_sum<256>(s, red) / (float)a.D;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NORM_MAXV; ++k) {
    const int i = tid + 256 * k;
    if (i < nv) {
      const float d0 = xv[k].x - mean, d1 = xv[k].y - mean, d2 = xv[k].z - mean, d3 = xv[k].w - mean;
      ss += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
    }
  }
  const float var = block_sum<256>(ss, red) / (float)a.D;
  const float rstd = 1.f / sqrtf(var + a.eps);

  const float* shift = nullptr;
  const float* scale = nullptr;
  const float* shift2 = nullptr;
  const float* scale2 = nullptr;
  if (a.mode != NORM_AFFINE) {
    const int rb = row % a.rm.rows_per_branch;
    const int ch = rb / a.rm.Lq, grp = (rb % a.rm.Lq) < a.rm.Lv ? 0 : 1;
    if (a.mode == NORM_ADALN) {
      const float* e6 = a.e6 + (long)(ch * 2 + grp) * 6 * a.D;
      shift = e6 + (long)a.shift_idx * a.D;
      scale = e6 + (long)a.scale_idx * a.D;
      shift2 = a.mod + (long)a.shift_idx * a.D;
      scale2 = a.mod + (long)a.scale_idx * a.D;
    } else {  // NORM_HEAD: e [n][2][D] + head_mod [2][D]
      const float* e = a.e6 + (long)(ch * 2 + grp) * a.D;
      shift = e;
      scale = e;
      shift2 = a.mod;
      scale2 = a.mod + a.D;
    }
  }
  T* y = reinterpret_cast<T*>(a.Y) + (long)row * a.D;
#pragma unroll
  for (int k = 0; k < NORM_MAXV; ++k) {
    const int i = tid + 256 * k;
    if (i >= nv) continue;
    float v[4] = {(xv[k].x - mean) * rstd, (xv[k].y - mean) * rstd, (xv[k].z - mean) * rstd, (xv[k].w - mean) * rstd};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = 4 * i + c;
      if (a.mode == NORM_AFFINE) {
        v[c] = v[c] * a.w[col] + a.b[col];
      } else {
        const float sh = shift[col] + shift2[col];
        const float sc = scale[col] + scale2[col];
        v[c] = v[c] * (1.f + sc) + sh;
      }
    }
    if constexpr (sizeof(T) == 2) {
      const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
      reinterpret_cast<uint2*>(y)[i] = make_uint2(lo, hi);
    } else {
      reinterpret_cast<float4*>(y)[i] = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

hipError_t launch_norm(const NormArgs& a, DType dt, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.D % 4 || a.D > 4 * 256 * NORM_MAXV) return hipErrorInvalidValue;
  if (dt == DT_BF16) hipLaunchKernelGGL(norm_kernel<bf16_t>, dim3(a.M), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(norm_kernel<float>, dim3(a.M), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// q/k RMSNorm over the full width + rotary embedding of video rows + scatter to head-major rows.
// One workgroup per row; thread t handles channel pairs (2p, 2p+1), p = t + 256 k.
// ------------------------------------------------------------------------------------------------
static constexpr int QK_MAXP = 16;   // up to D = 8192

template <typename T>
__global__ void __launch_bounds__(256) qk_norm_rope_kernel(QkNormArgs a) {
  __shared__ float red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const T* src = reinterpret_cast<const T*>(a.src) + (long)row * a.src_ld + a.src_col;
  const int np = a.D / 2;
  float x0[QK_MAXP], x1[QK_MAXP];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < QK_MAXP; ++k) {
    const int p = tid + 256 * k;
    if (p < np) {
      x0[k] = Elem<T>::load(src + 2 * p);
      x1[k] = Elem<T>::load(src + 2 * p + 1);
      ss += x0[k] * x0[k] + x1[k] * x1[k];
    }
  }
  const float ms = block_sum<256>(ss, red) / (float)a.D;
  const float rstd = 1.f / sqrtf(ms + a.eps);
  const int b = row / a.rows_per_branch, rb = row % a.rows_per_branch;
  const bool video = (rb % a.rm.Lq) < a.rm.Lv;
  const int half_d = a.d / 2;
  T* dst = reinterpret_cast<T*>(a.dst);
#pragma unroll
  for (int k = 0; k < QK_MAXP; ++k) {
    const int p = tid + 256 * k;
    if (p >= np) continue;
    float y0 = x0[k] * rstd * a.gain[2 * p];
    float y1 = x1[k] * rstd * a.gain[2 * p + 1];
    const int hh = (2 * p) / a.d, j = p % half_d;
    if (a.rope && video) {
      const float2 cs = a.rope[(long)rb * half_d + j];
      const float r0 = y0 * cs.x - y1 * cs.y;
      const float r1 = y0 * cs.y + y1 * cs.x;
      y0 = r0;
      y1 = r1;
    }
    T* o = dst + ((long)b * a.H + hh) * a.dst_bh_stride + (long)(a.dst_row0 + rb) * a.d + 2 * j;
    o[0] = Elem<T>::from_f(y0);
    o[1] = Elem<T>::from_f(y1);
  }
}

hipError_t launch_qk_norm_rope(const QkNormArgs& a, DType dt, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.D % 2 || a.D > 2 * 256 * QK_MAXP) return hipErrorInvalidValue;
  if (dt == DT_BF16) hipLaunchKernelGGL(qk_norm_rope_kernel<bf16_t>, dim3(a.M), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(qk_norm_rope_kernel<float>, dim3(a.M), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Values into the cache, key-contiguous: Vt[b][h][j][col0 + r] = src[b*R + r][src_col + h*d + j].
// Tiles of 64 rows x one head go through LDS so both the reads and the writes are contiguous.
// ------------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) v_to_cache_kernel(VCacheArgs a) {
  constexpr int PITCH = D + 2;          // odd word pitch for bf16 / even+2 for f32 against conflicts
  __shared__ T tile[64 * PITCH];
  const int r0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const T* src = reinterpret_cast<const T*>(a.src);
  for (int e = tid; e < 64 * D; e += 256) {
    const int r = e / D, j = e % D;
    const int rr = r0 + r;
    tile[r * PITCH + j] = rr < a.rows_per_branch ? src[((long)b * a.rows_per_branch + rr) * a.src_ld + a.src_col + h * D + j] : T(0);
  }
  __syncthreads();
  T* dst = reinterpret_cast<T*>(a.dst) + ((long)b * a.H + h) * a.dst_bh_stride;
  for (int e = tid; e < 64 * D; e += 256) {
    const int j = e / 64, r = e % 64;
    const int rr = r0 + r;
    if (rr < a.rows_per_branch) dst[(long)j * a.dst_stride + a.dst_col0 + rr] = tile[r * PITCH + j];
  }
}

hipError_t launch_v_to_cache(const VCacheArgs& a, DType dt, hipStream_t s) {
  if (a.rows_per_branch <= 0) return hipSuccess;
  const dim3 grid((a.rows_per_branch + 63) / 64, a.H, a.br);
  if (dt == DT_BF16) {
    if (a.d == 128) hipLaunchKernelGGL((v_to_cache_kernel<bf16_t, 128>), grid, dim3(256), 0, s, a);
    else if (a.d == 64) hipLaunchKernelGGL((v_to_cache_kernel<bf16_t, 64>), grid, dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
  } else {
    if (a.d == 128) hipLaunchKernelGGL((v_to_cache_kernel<float, 128>), grid, dim3(256), 0, s, a);
    else if (a.d == 64) hipLaunchKernelGGL((v_to_cache_kernel<float, 64>), grid, dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Rotary table: for every row of a branch, (cos, sin) of each channel pair. Video rows use
// (frame, patch row, patch column) on the (d_t, d_h, d_w) = (d - 2*2floor(d/6), 2floor(d/6),
// 2floor(d/6)) split with frequencies theta^(-2j'/d_axis); angles are formed in double precision.
// ------------------------------------------------------------------------------------------------
__global__ void rope_table_kernel(float2* table, int rows, int Lq, int Lv, int Fc, int Hp, int Wp, int start_frame,
                                  int d, float theta) {
  const int half_d = d / 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)rows * half_d) return;
  const int rb = (int)(idx / half_d), j = (int)(idx % half_d);
  const int ch = rb / Lq, loc = rb % Lq;
  if (loc >= Lv) {
    table[idx] = make_float2(1.f, 0.f);
    return;
  }
  const int dh = 2 * (d / 6), dt = d - 2 * dh;
  const int f = start_frame + ch * Fc + loc / (Hp * Wp);
  const int pr = (loc / Wp) % Hp, pc = loc % Wp;
  int pos, jj, da;
  if (j < dt / 2) { pos = f; jj = j; da = dt; }
  else if (j < dt / 2 + dh / 2) { pos = pr; jj = j - dt / 2; da = dh; }
  else { pos = pc; jj = j - dt / 2 - dh / 2; da = dh; }
  const double freq = pow((double)theta, -2.0 * jj / (double)da);
  const double ang = (double)pos * freq;
  table[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

hipError_t launch_rope_table(float2* table, int n_chunks, int Lq, int Lv, int Fc, int Hp, int Wp, int start_frame,
                             int d, float theta, hipStream_t s) {
  const int rows = n_chunks * Lq;
  const long n = (long)rows * (d / 2);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, table, rows, Lq, Lv, Fc, Hp,
                     Wp, start_frame, d, theta);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Token embedding: per branch b and row r of chunk c, h = x W^T + bias with the patch linear for
// video rows and the action linear for action rows. One thread per output column.
// ------------------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) embed_kernel(EmbedArgs a) {
  extern __shared__ float xrow[];
  const int rb = blockIdx.x, Lq = a.Lv + a.La;
  const int ch = rb / Lq, loc = rb % Lq;
  const bool video = loc < a.Lv;
  const int K = video ? a.P : a.A;
  const float* x = video ? a.xv + ((long)ch * a.Lv + loc) * a.P : a.xa + ((long)ch * a.La + (loc - a.Lv)) * a.A;
  for (int k = threadIdx.x; k < K; k += blockDim.x) xrow[k] = x[k];
  __syncthreads();
  const T* Wm = reinterpret_cast<const T*>(video ? a.pe_w : a.ae_w);
  const float* bias = video ? a.pe_b : a.ae_b;
  const int R = a.n_chunks * Lq;
  for (int n = blockIdx.y * blockDim.x + threadIdx.x; n < a.D; n += gridDim.y * blockDim.x) {
    float acc = 0.f;
    const T* wr = Wm + (long)n * K;
    for (int k = 0; k < K; ++k) acc += xrow[k] * Elem<T>::load(wr + k);
    acc += bias[n];
    for (int b = 0; b < a.br; ++b) a.H[((long)b * R + rb) * a.D + n] = acc;
  }
}

hipError_t launch_embed(const EmbedArgs& a, DType dt, hipStream_t s) {
  const int R = a.n_chunks * (a.Lv + a.La);
  if (R <= 0) return hipSuccess;
  const dim3 grid(R, (a.D + 255) / 256);
  const size_t sh = sizeof(float) * (size_t)(a.P > a.A ? a.P : a.A);
  if (dt == DT_BF16) hipLaunchKernelGGL(embed_kernel<bf16_t>, grid, dim3(256), sh, s, a);
  else hipLaunchKernelGGL(embed_kernel<float>, grid, dim3(256), sh, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Time embedding MLP (G = 2 * n_chunks timesteps):
//   emb = [cos(s w_i) ; sin(s w_i)], s = 1000 (1 - t), w_i = 10000^(-i/half)   (double precision)
//   h1 = SiLU(W1 emb + b1);  e = W2 h1 + b2;  e6 = Wp SiLU(e) + bp
// The products are batched matrix-vector products: one wave per output row streams that row of
// W once with 16-byte loads and serves all G vectors (HBM-bound on W).
// ------------------------------------------------------------------------------------------------
static constexpr int TIME_GMAX = 16;

struct TimeSteps { float t[TIME_GMAX]; };

__global__ void sinusoid_kernel(TimeSteps ts, int freq_dim, float* emb) {
  const int g = blockIdx.x, half = freq_dim / 2;
  const double s = 1000.0 * (1.0 - (double)ts.t[g]);
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double w = pow(10000.0, -(double)i / (double)half);
    emb[(long)g * freq_dim + i] = (float)cos(s * w);
    emb[(long)g * freq_dim + half + i] = (float)sin(s * w);
  }
}

template <typename T>
__global__ void __launch_bounds__(256) gemv_kernel(const T* W, const float* bias, const float* x, float* y, int N, int K,
                                                   int G, int silu_in, int silu_out) {
  constexpr int EPU = 16 / sizeof(T);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + wave;
  if (n >= N) return;
  float acc[TIME_GMAX];
#pragma unroll
  for (int g = 0; g < TIME_GMAX; ++g) acc[g] = 0.f;
  const T* wr = W + (long)n * K;
  for (int k0 = lane * EPU; k0 < K; k0 += 64 * EPU) {
    const uint4 raw = *reinterpret_cast<const uint4*>(wr + k0);
    const T* we = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < EPU; ++e) {
      const float wv = Elem<T>::to_f(we[e]);
#pragma unroll
      for (int g = 0; g < TIME_GMAX; ++g) {
        if (g < G) {
          float xv = x[(long)g * K + k0 + e];
          if (silu_in) xv = silu_f(xv);
          acc[g] += wv * xv;
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < TIME_GMAX; ++g) {
    if (g < G) {
      float v = wave_sum(acc[g]);
      if (lane == 0) {
        v += bias[n];
        if (silu_out) v = silu_f(v);
        y[(long)g * N + n] = v;
      }
    }
  }
}

template <typename T>
static void launch_gemv(const void* W, const float* b, const float* x, float* y, int N, int K, int G, int si, int so,
                        hipStream_t s) {
  hipLaunchKernelGGL(gemv_kernel<T>, dim3((N + 3) / 4), dim3(256), 0, s, reinterpret_cast<const T*>(W), b, x, y, N, K, G,
                     si, so);
}

hipError_t launch_time_mlp(const TimeArgs& a, DType dt, hipStream_t s) {
  if (a.G <= 0) return hipSuccess;
  if (a.G > TIME_GMAX) return hipErrorInvalidValue;
  const int EPU = dt == DT_BF16 ? 8 : 4;
  if (a.freq_dim % EPU || a.D % EPU) return hipErrorInvalidValue;
  TimeSteps ts;
  for (int g = 0; g < TIME_GMAX; ++g) ts.t[g] = g < a.G ? a.t[g] : 0.f;
  hipLaunchKernelGGL(sinusoid_kernel, dim3(a.G), dim3(128), 0, s, ts, a.freq_dim, a.emb);
  if (dt == DT_BF16) {
    launch_gemv<bf16_t>(a.w1, a.b1, a.emb, a.h1, a.D, a.freq_dim, a.G, 0, 1, s);
    launch_gemv<bf16_t>(a.w2, a.b2, a.h1, a.e, a.D, a.D, a.G, 0, 0, s);
    launch_gemv<bf16_t>(a.wp, a.bp, a.e, a.e6, 6 * a.D, a.D, a.G, 1, 0, s);
  } else {
    launch_gemv<float>(a.w1, a.b1, a.emb, a.h1, a.D, a.freq_dim, a.G, 0, 1, s);
    launch_gemv<float>(a.w2, a.b2, a.h1, a.e, a.D, a.D, a.G, 0, 0, s);
    launch_gemv<float>(a.wp, a.bp, a.e, a.e6, 6 * a.D, a.D, a.G, 1, 0, s);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Flow-matching update: guided velocity g = w v_cond + (1 - w) v_uncond (or v when one branch),
// x += dt g per modality, optional store of g, and partial sums of <g, prev>, |g|^2, |prev|^2 over
// the video part for the cosine used by velocity reuse. Fixed grid => fixed reduction order.
// ------------------------------------------------------------------------------------------------
static constexpr int FLOW_BLOCKS = 64;
int flow_partial_blocks(int) { return FLOW_BLOCKS; }

__global__ void __launch_bounds__(256) flow_kernel(FlowArgs a) {
  __shared__ float red[4];
  const float wc = a.w, wu = 1.f - a.w;
  float dot = 0.f, gg = 0.f, pp = 0.f;
  const int n = a.nv + a.na;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += FLOW_BLOCKS * 256) {
    const bool video = i < a.nv;
    const int k = video ? i : i - a.nv;
    const float* v = video ? a.vv : a.va;
    const int nn = video ? a.nv : a.na;
    float g = v[k];
    if (a.br == 2) g = wc * v[k] + wu * v[nn + k];
    if (video) {
      a.xv[k] += a.dtv * g;
      if (a.prev) {
        const float p = a.prev[k];
        dot += g * p;
        gg += g * g;
        pp += p * p;
      }
      if (a.gv) a.gv[k] = g;
    } else {
      a.xa[k] += a.dta * g;
      if (a.ga) a.ga[k] = g;
    }
  }
  if (a.prev) {
    dot = block_sum<256>(dot, red);
    gg = block_sum<256>(gg, red);
    pp = block_sum<256>(pp, red);
    if (threadIdx.x == 0) {
      a.partials[blockIdx.x * 3 + 0] = dot;
      a.partials[blockIdx.x * 3 + 1] = gg;
      a.partials[blockIdx.x * 3 + 2] = pp;
    }
  }
}

__global__ void flow_reduce_kernel(const float* partials, float* out) {
  if (threadIdx.x < 3) {
    float s = 0.f;
    for (int b = 0; b < FLOW_BLOCKS; ++b) s += partials[b * 3 + threadIdx.x];
    out[threadIdx.x] = s;
  }
}

hipError_t launch_flow_step(const FlowArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(flow_kernel, dim3(FLOW_BLOCKS), dim3(256), 0, s, a);
  if (a.prev && a.cos_parts) hipLaunchKernelGGL(flow_reduce_kernel, dim3(1), dim3(64), 0, s, a.partials, a.cos_parts);
  return hipGetLastError();
}

}  // namespace wam
