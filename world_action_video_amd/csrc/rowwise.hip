// Row-wise and small kernels of the DiT step: LayerNorm + adaLN modulation, q/k RMSNorm + 3-D
// rotary embedding with the head-major / KV-cache scatter, the value transpose into the cache,
// the rotary table, token embedding, the time-embedding MLP and the fused CFG + Euler + cosine
// update. All statistics are accumulated in fp32 with a fixed reduction order (deterministic).
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace wam {

// ------------------------------------------------------------------------------------------------
// LayerNorm (+ modulation): a 256-thread workgroup per row, over R consecutive rows per workgroup
// (more rows per workgroup only for tall inputs, where workgroup dispatch would otherwise pace the
// kernel); thread t holds columns 4 (t + 256 k), k < G. The row's fp32 input and its per-column
// vectors, combined into one multiplier and one addend (1 + scale, shift for the adaLN and head modes;
// w, b for the affine mode), are all loaded before the reductions; the vectors are kept while the
// next row has the same token group. Mean and variance are two workgroup reductions in a fixed order.
// With a.rms the mean is taken as zero: RMSNorm.
// ------------------------------------------------------------------------------------------------
template <typename T, int G>
__global__ void __launch_bounds__(256) norm_kernel(NormArgs a, int R) {
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int nv = a.D / 4;
  const int r0 = blockIdx.x * R, r1 = min(a.M, r0 + R);
  float4 mv[G], av[G];
  int have = -2;   // token group whose vectors mv / av hold (-1: the affine weights)
  for (int row = r0; row < r1; ++row) {
    const float4* x4 = reinterpret_cast<const float4*>(a.X + (long)row * a.D);
    float4 xv[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int q = t + 256 * k;
      xv[k] = q < nv ? x4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    int grp_id = -1;
    if (a.mode != NORM_AFFINE) {
      const int rb = row % a.rm.rows_per_branch;
      grp_id = (rb / a.rm.Lq) * 2 + ((rb % a.rm.Lq) < a.rm.Lv ? 0 : 1);
    }
    if (grp_id != have) {   // uniform across the workgroup
      have = grp_id;
      const float4 *sh = nullptr, *sc = nullptr, *sh2 = nullptr, *sc2 = nullptr;
      if (a.mode == NORM_ADALN) {
        const float* e6 = a.e6 + (long)grp_id * 6 * a.D;
        sh = reinterpret_cast<const float4*>(e6 + (long)a.shift_idx * a.D);
        sc = reinterpret_cast<const float4*>(e6 + (long)a.scale_idx * a.D);
        sh2 = reinterpret_cast<const float4*>(a.mod + (long)a.shift_idx * a.D);
        sc2 = reinterpret_cast<const float4*>(a.mod + (long)a.scale_idx * a.D);
      } else if (a.mode == NORM_HEAD) {   // e [n][2][D] + head_mod [2][D]
        const float* e = a.e6 + (long)grp_id * a.D;
        sh = sc = reinterpret_cast<const float4*>(e);
        sh2 = reinterpret_cast<const float4*>(a.mod);
        sc2 = reinterpret_cast<const float4*>(a.mod + a.D);
      }
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const int q = t + 256 * k;
        mv[k] = av[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q >= nv) continue;
        if (a.mode == NORM_AFFINE) {
          mv[k] = reinterpret_cast<const float4*>(a.w)[q];
          av[k] = reinterpret_cast<const float4*>(a.b)[q];
        } else {
          const float4 p = sh[q], p2 = sh2[q], r = sc[q], r2 = sc2[q];
          mv[k] = make_float4(1.f + (r.x + r2.x), 1.f + (r.y + r2.y), 1.f + (r.z + r2.z), 1.f + (r.w + r2.w));
          av[k] = make_float4(p.x + p2.x, p.y + p2.y, p.z + p2.z, p.w + p2.w);
        }
      }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < G; ++k) s += (xv[k].x + xv[k].y) + (xv[k].z + xv[k].w);
    const float mean = a.rms ? 0.f : block_sum<256>(s, red) / (float)a.D;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      if (t + 256 * k >= nv) continue;
      const float d0 = xv[k].x - mean, d1 = xv[k].y - mean, d2 = xv[k].z - mean, d3 = xv[k].w - mean;
      ss += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
    }
    const float rstd = 1.f / sqrtf(block_sum<256>(ss, red) / (float)a.D + a.eps);

    T* y = reinterpret_cast<T*>(a.Y) + (long)row * a.D;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int q = t + 256 * k;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (q < nv)
        v = make_float4((xv[k].x - mean) * rstd * mv[k].x + av[k].x, (xv[k].y - mean) * rstd * mv[k].y + av[k].y,
                        (xv[k].z - mean) * rstd * mv[k].z + av[k].z, (xv[k].w - mean) * rstd * mv[k].w + av[k].w);
      if constexpr (sizeof(T) == 2) {
        if (q < nv) reinterpret_cast<uint2*>(y)[q] = make_uint2(pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w));
        if (a.mxq && 256 * k < nv) {   // MXFP8 copy of the stored (bf16-rounded) row; whole waves call it
          v = make_float4(bf16_round(v.x), bf16_round(v.y), bf16_round(v.z), bf16_round(v.w));
          mx_store_quad(v, q < nv, a.mxq + (long)row * a.D, a.mxs + (long)row * (a.D / 32), q);
        }
      } else {
        if (q < nv) reinterpret_cast<float4*>(y)[q] = v;
      }
    }
  }
}

// dst += src elementwise, eight elements (bf16) or four (fp32) per 16-byte access; sums in fp32
template <typename T>
__global__ void __launch_bounds__(256) add_kernel(T* dst, const T* src, long n16) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  uint4 a = reinterpret_cast<const uint4*>(dst)[i];
  const uint4 b = reinterpret_cast<const uint4*>(src)[i];
  uint32_t* pa = reinterpret_cast<uint32_t*>(&a);
  const uint32_t* pb = reinterpret_cast<const uint32_t*>(&b);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if constexpr (sizeof(T) == 2) {
      const float lo = __uint_as_float(pa[k] << 16) + __uint_as_float(pb[k] << 16);
      const float hi = __uint_as_float(pa[k] & 0xffff0000u) + __uint_as_float(pb[k] & 0xffff0000u);
      pa[k] = pack2_bf16(lo, hi);
    } else {
      pa[k] = __float_as_uint(__uint_as_float(pa[k]) + __uint_as_float(pb[k]));
    }
  }
  reinterpret_cast<uint4*>(dst)[i] = a;
}

hipError_t launch_add(void* dst, const void* src, long n, DType dt, hipStream_t s) {
  const long per = dt == DT_BF16 ? 8 : 4;
  if (n <= 0) return hipSuccess;
  if (n % per || reinterpret_cast<uintptr_t>(dst) % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return hipErrorInvalidValue;
  const long n16 = n / per;
  const dim3 grid((unsigned)((n16 + 255) / 256)), block(256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL((add_kernel<bf16_t>), grid, block, 0, s, reinterpret_cast<bf16_t*>(dst),
                       reinterpret_cast<const bf16_t*>(src), n16);
  else
    hipLaunchKernelGGL((add_kernel<float>), grid, block, 0, s, reinterpret_cast<float*>(dst),
                       reinterpret_cast<const float*>(src), n16);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_norm_t(const NormArgs& a, hipStream_t s) {
  // rows per workgroup: one up to 8192 rows, then enough for about 8192 workgroups, at most 8
  const int R = a.M <= 8192 ? 1 : min(8, (a.M + 8191) / 8192);
  const dim3 grid((a.M + R - 1) / R), block(256);
  const int g = (a.D / 4 + 255) / 256;   // float4 groups per thread
  if (g <= 1) hipLaunchKernelGGL((norm_kernel<T, 1>), grid, block, 0, s, a, R);
  else if (g <= 2) hipLaunchKernelGGL((norm_kernel<T, 2>), grid, block, 0, s, a, R);
  else if (g <= 5) hipLaunchKernelGGL((norm_kernel<T, 5>), grid, block, 0, s, a, R);
  else if (g <= 8) hipLaunchKernelGGL((norm_kernel<T, 8>), grid, block, 0, s, a, R);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_norm(const NormArgs& a, DType dt, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.D % 4 || a.D > 8192) return hipErrorInvalidValue;
  return dt == DT_BF16 ? launch_norm_t<bf16_t>(a, s) : launch_norm_t<float>(a, s);
}

// ------------------------------------------------------------------------------------------------
// q/k RMSNorm over the full width + rotary embedding of video rows + scatter to head-major rows.
// One wave per row; each lane owns groups of 8 consecutive channels (16-byte loads and stores; a
// group never straddles a head since the head dim is a multiple of 8). The row's values are loaded in
// one batch with no control flow between the loads (lanes past the row's end read its last group and
// drop it); the workgroup meanwhile copies the gain into LDS (`stage`), so one memory round trip
// precedes the sum of squares. The output is rstd * R(x * g): gain, rotation, then the row scale.
// ------------------------------------------------------------------------------------------------
template <int GPL>
struct GainLds {   // the gain of a width of up to 512 GPL channels, copied once per workgroup
  float4 v[GPL * 128];
  static_assert(GPL * 128 % 256 == 0, "whole rounds of the 256 threads");
  static constexpr int GS = GPL * 128 / 256;   // quads per thread
};

// `valid` false: the wave only takes part in the workgroup's staging (its loads read the last row).
template <typename T, int GPL>
__device__ __forceinline__ void qk_row(const QkNormArgs& a, int row, bool valid, int lane, GainLds<GPL>& gl) {
  constexpr int EPU = 16 / sizeof(T);            // elements per 16-byte unit
  constexpr int UPG = 8 / EPU;                   // units per group of 8 channels
  if (!valid) row = a.M - 1;
  // The gain's loads go out first (clamped to its end: the copies past the width are never read, and
  // no branch separates the loads), the row's right behind them.
  constexpr int GS = GainLds<GPL>::GS;
  float4 gt[GS];
#pragma unroll
  for (int j = 0; j < GS; ++j)
    gt[j] = reinterpret_cast<const float4*>(a.gain)[min((int)threadIdx.x + 256 * j, a.D / 4 - 1)];
  const T* src = reinterpret_cast<const T*>(a.src) + (long)row * a.src_ld + a.src_col;
  const int ng = a.D / 8;
  const int b = row / a.rows_per_branch, rb = row % a.rows_per_branch;
  const bool rotate = a.rope && (rb % a.rm.Lq) < a.rm.Lv;   // video rows only
  const int half_d = a.d / 2;
  uint4 u[GPL][UPG];
#pragma unroll
  for (int k = 0; k < GPL; ++k) {
    const int ch0 = min(lane + 64 * k, ng - 1) * 8;
#pragma unroll
    for (int q = 0; q < UPG; ++q) u[k][q] = reinterpret_cast<const uint4*>(src + ch0)[q];
  }
  // A lane's groups are 512 channels apart: when d divides 512 they sit at the same offset inside
  // their heads and share one set of rotary entries, loaded once.
  const bool one_cs = rotate && 512 % a.d == 0;
  float2 cs_lane[4];
  if (one_cs) {
    const float2* cs = a.rope + (long)rb * half_d + ((8 * lane) % a.d) / 2;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) cs_lane[pp] = cs[pp];
  }
#pragma unroll
  for (int j = 0; j < GS; ++j) gl.v[threadIdx.x + 256 * j] = gt[j];
  __syncthreads();
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < GPL; ++k) {
    const bool in = lane + 64 * k < ng;
    const T* e = reinterpret_cast<const T*>(u[k]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float x = Elem<T>::to_f(e[c]);
      ss += in ? x * x : 0.f;
    }
  }
  const float rstd = 1.f / sqrtf(wave_sum(ss) / (float)a.D + a.eps);
  if (!valid) return;
  T* dst = reinterpret_cast<T*>(a.dst);
  // cs(k, ch0, pp): rotary entry pp of group k (the lane's shared set, or loaded per group), so the
  // two cases run as separate loops and the shared case waits on no load.
  auto emit = [&](auto cs) {
#pragma unroll
    for (int k = 0; k < GPL; ++k) {
      const int gi = lane + 64 * k;
      if (gi >= ng) continue;
      const int ch0 = gi * 8, hh = ch0 / a.d;
      const float4 g0 = gl.v[ch0 / 4], g1 = gl.v[ch0 / 4 + 1];
      const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const T* e = reinterpret_cast<const T*>(u[k]);
      float y[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = Elem<T>::to_f(e[c]) * g[c];
      if (rotate) {
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const float2 t = cs(ch0, pp);
          const float r0 = y[2 * pp] * t.x - y[2 * pp + 1] * t.y;
          const float r1 = y[2 * pp] * t.y + y[2 * pp + 1] * t.x;
          y[2 * pp] = r0;
          y[2 * pp + 1] = r1;
        }
      }
      T* o = dst + ((long)b * a.H + hh) * a.dst_bh_stride + (long)(a.dst_row0 + rb) * a.d + ch0 % a.d;
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c] = y[c] * rstd;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint4*>(o) = make_uint4(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]),
                                                  pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7]));
      } else {
        reinterpret_cast<float4*>(o)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(o)[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  };
  if (one_cs || !rotate)
    emit([&](int, int pp) { return cs_lane[pp]; });
  else
    emit([&](int ch0, int pp) { return a.rope[(long)rb * half_d + (ch0 % a.d) / 2 + pp]; });
}

template <typename T, int GPL>
__global__ void __launch_bounds__(256) qk_norm_rope_kernel(QkNormArgs a) {
  __shared__ GainLds<GPL> gl;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  qk_row<T, GPL>(a, row, row < a.M, threadIdx.x & 63, gl);
}

template <typename T>
static hipError_t launch_qk_t(const QkNormArgs& a, hipStream_t s) {
  const dim3 grid((a.M + 3) / 4), block(256);
  const int gpl = (a.D / 8 + 63) / 64;
  if (gpl <= 2) hipLaunchKernelGGL((qk_norm_rope_kernel<T, 2>), grid, block, 0, s, a);
  else if (gpl <= 4) hipLaunchKernelGGL((qk_norm_rope_kernel<T, 4>), grid, block, 0, s, a);
  else if (gpl <= 10) hipLaunchKernelGGL((qk_norm_rope_kernel<T, 10>), grid, block, 0, s, a);
  else if (gpl <= 16) hipLaunchKernelGGL((qk_norm_rope_kernel<T, 16>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const QkNormArgs& a, DType dt, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.D % 8 || a.D > 8192 || a.d % 8) return hipErrorInvalidValue;
  return dt == DT_BF16 ? launch_qk_t<bf16_t>(a, s) : launch_qk_t<float>(a, s);
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

// ------------------------------------------------------------------------------------------------
// One launch for everything that follows the QKV projection (bf16): q RMSNorm + RoPE to head-major
// rows, k RMSNorm + RoPE into the key cache, v transposed into the value cache. Block ranges of the
// 1-D grid select the part, so the three run side by side. The value part moves 8x8 element blocks
// through registers: each thread reads 8 rows x 16 bytes (one head's 8 channels) and writes 8 cache
// rows x 16 bytes (8 consecutive keys), so both sides are 16-byte accesses.
// ------------------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void v_block_bf16(const VCacheArgs& a, int blk) {
  constexpr int CB = D / 8;                      // 8-channel column blocks per head
  constexpr int RB = 256 / CB;                   // 8-row blocks per workgroup
  const int R = a.rows_per_branch;
  const int nrb = (R + RB * 8 - 1) / (RB * 8);
  const int rblk = blk % nrb, h = (blk / nrb) % a.H, b = blk / (nrb * a.H);
  const int cb = threadIdx.x % CB, rbk = threadIdx.x / CB;
  const int r0 = rblk * RB * 8 + rbk * 8;        // rows per branch are a multiple of 8
  if (r0 >= R) return;
  const bf16_t* src = reinterpret_cast<const bf16_t*>(a.src) + ((long)b * R + r0) * a.src_ld + a.src_col + h * D + cb * 8;
  uint4 x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = *reinterpret_cast<const uint4*>(src + (long)i * a.src_ld);
  bf16_t* dst = reinterpret_cast<bf16_t*>(a.dst) + ((long)b * a.H + h) * a.dst_bh_stride + (long)(cb * 8) * a.dst_stride +
                a.dst_col0 + r0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // channel c of the 8 rows: element c of each row's unit
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (reinterpret_cast<const uint32_t*>(&x[2 * i])[c >> 1] >> ((c & 1) * 16)) & 0xFFFFu;
      const uint32_t hi = (reinterpret_cast<const uint32_t*>(&x[2 * i + 1])[c >> 1] >> ((c & 1) * 16)) & 0xFFFFu;
      w[i] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(dst + (long)c * a.dst_stride) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int GPL, int D>
__global__ void __launch_bounds__(256) qkv_cache_kernel(QkNormArgs q, QkNormArgs k, VCacheArgs v, int nq_blk, int nk_blk) {
  __shared__ GainLds<GPL> gl;
  int blk = blockIdx.x;
  const int row4 = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (blk < nk_blk) {
    const int row = blk * 4 + row4;
    qk_row<bf16_t, GPL>(k, row, row < k.M, lane, gl);
    return;
  }
  blk -= nk_blk;
  if (blk < nq_blk) {
    const int row = blk * 4 + row4;
    qk_row<bf16_t, GPL>(q, row, row < q.M, lane, gl);
    return;
  }
  v_block_bf16<D>(v, blk - nq_blk);
}

hipError_t launch_qkv_cache(const QkNormArgs* q, const QkNormArgs& k, const VCacheArgs& v, DType dt, hipStream_t s) {
  if (k.M <= 0) return hipSuccess;
  const bool fused = dt == DT_BF16 && (v.d == 128 || v.d == 64) && v.rows_per_branch % 8 == 0 && v.dst_col0 % 8 == 0 &&
                     v.dst_stride % 8 == 0 && v.src_ld % 8 == 0 && v.src_col % 8 == 0 && k.D % 8 == 0 &&
                     k.D <= 8192 && k.d % 8 == 0 && (!q || (q->D == k.D && q->M == k.M));
  if (!fused) {
    hipError_t e = hipSuccess;
    if (q) e = launch_qk_norm_rope(*q, dt, s);
    if (e == hipSuccess) e = launch_qk_norm_rope(k, dt, s);
    if (e == hipSuccess) e = launch_v_to_cache(v, dt, s);
    return e;
  }
  const int nk_blk = (k.M + 3) / 4, nq_blk = q ? (q->M + 3) / 4 : 0;
  const int rows_per_wg = 8 * (256 / (v.d / 8));
  const int nv_blk = (v.rows_per_branch + rows_per_wg - 1) / rows_per_wg * v.H * v.br;
  const dim3 grid(nk_blk + nq_blk + nv_blk), block(256);
  const QkNormArgs qq = q ? *q : k;
  const int gpl = (k.D / 8 + 63) / 64;
#define WAM_QKV(G)                                                                                              \
  if (v.d == 128) hipLaunchKernelGGL((qkv_cache_kernel<G, 128>), grid, block, 0, s, qq, k, v, nq_blk, nk_blk); \
  else hipLaunchKernelGGL((qkv_cache_kernel<G, 64>), grid, block, 0, s, qq, k, v, nq_blk, nk_blk);
  if (gpl <= 2) { WAM_QKV(2) }
  else if (gpl <= 4) { WAM_QKV(4) }
  else if (gpl <= 10) { WAM_QKV(10) }
  else { WAM_QKV(16) }
#undef WAM_QKV
  return hipGetLastError();
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
// Sliding attention window ([WS1] continuous requests: the attention window releases old KV and
// the frame position restarts). Every (layer, branch, head) block keeps rows [drop, len), moved to
// [0, len - drop); keys of video rows get their frame-axis pairs rotated by -shift * freq(j) on the
// way: rotations compose, so a key rotated for frame f becomes the key of frame f - shift. Values
// move along their key-contiguous rows. One workgroup per block moves it front to back in rounds:
// a round's data are in registers before any of it is stored (the barrier sits between), and later
// rounds read only rows past every row written so far, so the overlapping in-place move is safe.
// ------------------------------------------------------------------------------------------------
static constexpr int EVICT_PER = 4;   // 16-byte units per thread per round

template <typename T, int D>
__global__ void __launch_bounds__(256) kv_evict_k_kernel(KvEvictArgs a) {
  constexpr int EPU = 16 / sizeof(T), U = D / EPU, ROWS = 256 * EVICT_PER / U;
  T* base = reinterpret_cast<T*>(a.k) + (long)blockIdx.x * a.cap * D;
  const int keep = a.len - a.drop;
  for (int r0 = 0; r0 < keep; r0 += ROWS) {
    uint4 v[EVICT_PER];
#pragma unroll
    for (int i = 0; i < EVICT_PER; ++i) {
      const int x = threadIdx.x + 256 * i, row = r0 + x / U, u = x % U;
      v[i] = make_uint4(0, 0, 0, 0);
      if (row >= keep) continue;
      v[i] = reinterpret_cast<const uint4*>(base + (long)(row + a.drop) * D)[u];
      const int j0 = u * EPU / 2;   // first channel pair of the unit
      if ((row % a.Lq) >= a.Lv || j0 >= a.frame_pairs) continue;
      T* e = reinterpret_cast<T*>(&v[i]);
#pragma unroll
      for (int pp = 0; pp < EPU / 2; ++pp) {
        if (j0 + pp >= a.frame_pairs) break;
        const float2 t = a.cs[j0 + pp];
        const float x0 = Elem<T>::to_f(e[2 * pp]), x1 = Elem<T>::to_f(e[2 * pp + 1]);
        e[2 * pp] = Elem<T>::from_f(x0 * t.x - x1 * t.y);
        e[2 * pp + 1] = Elem<T>::from_f(x0 * t.y + x1 * t.x);
      }
    }
    // every thread's loads have returned before any store of the round
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < EVICT_PER; ++i) {
      const int x = threadIdx.x + 256 * i, row = r0 + x / U, u = x % U;
      if (row < keep) reinterpret_cast<uint4*>(base + (long)row * D)[u] = v[i];
    }
    __syncthreads();
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(256) kv_evict_v_kernel(KvEvictArgs a) {
  constexpr int EPU = 16 / sizeof(T), KU = 256 * EVICT_PER / D;   // key units per row per round
  T* base = reinterpret_cast<T*>(a.v) + (long)blockIdx.x * D * a.cap;
  const int keep = a.len - a.drop;   // a multiple of 8 keys, so of EPU
  for (int k0 = 0; k0 < keep; k0 += KU * EPU) {
    uint4 v[EVICT_PER];
#pragma unroll
    for (int i = 0; i < EVICT_PER; ++i) {
      const int x = threadIdx.x + 256 * i, j = x / KU, key = k0 + (x % KU) * EPU;
      v[i] = key < keep ? *reinterpret_cast<const uint4*>(base + (long)j * a.cap + a.drop + key) : make_uint4(0, 0, 0, 0);
    }
    // every thread's loads have returned before any store of the round
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < EVICT_PER; ++i) {
      const int x = threadIdx.x + 256 * i, j = x / KU, key = k0 + (x % KU) * EPU;
      if (key < keep) *reinterpret_cast<uint4*>(base + (long)j * a.cap + key) = v[i];
    }
    __syncthreads();
  }
}

hipError_t launch_kv_evict(const KvEvictArgs& a, DType dt, hipStream_t s) {
  if (a.len - a.drop <= 0 || a.drop <= 0 || a.blocks <= 0) return hipSuccess;
  if (a.d != 64 && a.d != 128) return hipErrorInvalidValue;
  const dim3 grid(a.blocks), block(256);
#define WAM_EVICT(T, D)                                                  \
  hipLaunchKernelGGL((kv_evict_k_kernel<T, D>), grid, block, 0, s, a); \
  hipLaunchKernelGGL((kv_evict_v_kernel<T, D>), grid, block, 0, s, a);
  if (dt == DT_BF16) {
    if (a.d == 128) { WAM_EVICT(bf16_t, 128) } else { WAM_EVICT(bf16_t, 64) }
  } else {
    if (a.d == 128) { WAM_EVICT(float, 128) } else { WAM_EVICT(float, 64) }
  }
#undef WAM_EVICT
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Token embedding: per branch b and row r of chunk c, h = x W^T + bias with the patch linear for
// video rows and the action linear for action rows. A workgroup computes 16 rows x 256 columns:
// the 16 input rows sit in LDS, each thread streams one weight row once and serves all 16 rows.
// ------------------------------------------------------------------------------------------------
static constexpr int EMB_ROWS = 16;

// PC / AC > 0: compile-time patch / action widths (weights held in registers); 0: any width.
template <typename T, int PC, int AC>
__global__ void __launch_bounds__(256) embed_kernel(EmbedArgs a) {
  extern __shared__ float xs[];                      // [EMB_ROWS][Kmax]
  const int Lq = a.Lv + a.La, R = a.n_chunks * Lq;
  const int P = PC > 0 ? PC : a.P, A = AC > 0 ? AC : a.A;
  const int Kmax = P > A ? P : A;
  const int r0 = blockIdx.x * EMB_ROWS;
  for (int e = threadIdx.x; e < EMB_ROWS * Kmax; e += 256) {
    const int rr = e / Kmax, k = e % Kmax, rb = r0 + rr;
    float v = 0.f;
    if (rb < R) {
      const int ch = rb / Lq, loc = rb % Lq;
      if (loc < a.Lv) { if (k < P) v = a.xv[((long)ch * a.Lv + loc) * P + k]; }
      else if (k < A) v = a.xa[((long)ch * a.La + (loc - a.Lv)) * A + k];
    }
    xs[e] = v;
  }
  __syncthreads();
  const int n = blockIdx.y * 256 + threadIdx.x;
  if (n >= a.D) return;
  const T* wpr = reinterpret_cast<const T*>(a.pe_w) + (long)n * P;
  const T* war = reinterpret_cast<const T*>(a.ae_w) + (long)n * A;
  const float bv = a.pe_b[n], ba = a.ae_b[n];
  if constexpr (PC > 0 && AC > 0) {
    float wv[PC], wa[AC];
#pragma unroll
    for (int k = 0; k < PC; ++k) wv[k] = Elem<T>::load(wpr + k);
#pragma unroll
    for (int k = 0; k < AC; ++k) wa[k] = Elem<T>::load(war + k);
    for (int rr = 0; rr < EMB_ROWS; ++rr) {
      const int rb = r0 + rr;
      if (rb >= R) break;
      const float* x = xs + rr * Kmax;
      float acc = 0.f;
      if ((rb % Lq) < a.Lv) {
#pragma unroll
        for (int k = 0; k < PC; ++k) acc += x[k] * wv[k];
        acc += bv;
      } else {
#pragma unroll
        for (int k = 0; k < AC; ++k) acc += x[k] * wa[k];
        acc += ba;
      }
      for (int b = 0; b < a.br; ++b) a.H[((long)b * R + rb) * a.D + n] = acc;
    }
  } else {
    for (int rr = 0; rr < EMB_ROWS; ++rr) {
      const int rb = r0 + rr;
      if (rb >= R) break;
      const float* x = xs + rr * Kmax;
      float acc = 0.f;
      if ((rb % Lq) < a.Lv) {
        for (int k = 0; k < P; ++k) acc += x[k] * Elem<T>::load(wpr + k);
        acc += bv;
      } else {
        for (int k = 0; k < A; ++k) acc += x[k] * Elem<T>::load(war + k);
        acc += ba;
      }
      for (int b = 0; b < a.br; ++b) a.H[((long)b * R + rb) * a.D + n] = acc;
    }
  }
}

template <typename T>
static void launch_embed_t(const EmbedArgs& a, dim3 grid, size_t sh, hipStream_t s) {
  if (a.P == 64 && a.A == 8) hipLaunchKernelGGL((embed_kernel<T, 64, 8>), grid, dim3(256), sh, s, a);
  else hipLaunchKernelGGL((embed_kernel<T, 0, 0>), grid, dim3(256), sh, s, a);
}

hipError_t launch_embed(const EmbedArgs& a, DType dt, hipStream_t s) {
  const int R = a.n_chunks * (a.Lv + a.La);
  if (R <= 0) return hipSuccess;
  const dim3 grid((R + EMB_ROWS - 1) / EMB_ROWS, (a.D + 255) / 256);
  const size_t sh = sizeof(float) * EMB_ROWS * (size_t)(a.P > a.A ? a.P : a.A);
  if (sh > 48 * 1024) return hipErrorInvalidValue;
  if (dt == DT_BF16) launch_embed_t<bf16_t>(a, grid, sh, s);
  else launch_embed_t<float>(a, grid, sh, s);
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

// NR output rows per wave share each load of x; used for the common small batches (G <= 4).
template <typename T, int G, int NR>
__global__ void __launch_bounds__(256) gemv_rows_kernel(const T* W, const float* bias, const float* x, float* y, int N,
                                                        int K, int silu_in, int silu_out) {
  constexpr int EPU = 16 / sizeof(T);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * NR;
  if (n0 >= N) return;
  float acc[NR][G];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[r][g] = 0.f;
  for (int k0 = lane * EPU; k0 < K; k0 += 64 * EPU) {
    float xv[G][EPU];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float4* xp = reinterpret_cast<const float4*>(x + (long)g * K + k0);
#pragma unroll
      for (int q = 0; q < EPU / 4; ++q) {
        const float4 t = xp[q];
        xv[g][4 * q] = t.x; xv[g][4 * q + 1] = t.y; xv[g][4 * q + 2] = t.z; xv[g][4 * q + 3] = t.w;
      }
      if (silu_in) {
#pragma unroll
        for (int e = 0; e < EPU; ++e) xv[g][e] = silu_f(xv[g][e]);
      }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (n0 + r >= N) break;
      const uint4 raw = *reinterpret_cast<const uint4*>(W + (long)(n0 + r) * K + k0);
      const T* we = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const float wv = Elem<T>::to_f(we[e]);
#pragma unroll
        for (int g = 0; g < G; ++g) acc[r][g] += wv * xv[g][e];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float v = wave_sum(acc[r][g]);
      if (lane == 0 && n0 + r < N) {
        v += bias[n0 + r];
        if (silu_out) v = silu_f(v);
        y[(long)g * N + n0 + r] = v;
      }
    }
  }
}

// y[g][n] = sum_k x[g][k] W[n][k] + bias[n] for a few rows g < G of x, in the storage type: the one-row
// products of a state update spread over N / 32 workgroups instead of a handful of GEMM tiles.
template <typename T, int G, int NR>
__global__ void __launch_bounds__(256) gemv_store_kernel(const T* W, const float* bias, const T* x, long ldx, T* y,
                                                         long ldy, int N, int K) {
  constexpr int EPU = 16 / sizeof(T);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * NR;
  if (n0 >= N) return;
  float acc[NR][G];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[r][g] = 0.f;
  for (int k0 = lane * EPU; k0 < K; k0 += 64 * EPU) {
    float xv[G][EPU];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 raw = *reinterpret_cast<const uint4*>(x + (long)g * ldx + k0);
      const T* xe = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int e = 0; e < EPU; ++e) xv[g][e] = Elem<T>::to_f(xe[e]);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (n0 + r >= N) break;
      const uint4 raw = *reinterpret_cast<const uint4*>(W + (long)(n0 + r) * K + k0);
      const T* we = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int e = 0; e < EPU; ++e) {
        const float wv = Elem<T>::to_f(we[e]);
#pragma unroll
        for (int g = 0; g < G; ++g) acc[r][g] += wv * xv[g][e];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float v = wave_sum(acc[r][g]);
      if (lane == 0 && n0 + r < N) Elem<T>::store(y + (long)g * ldy + n0 + r, v + (bias ? bias[n0 + r] : 0.f));
    }
  }
}

hipError_t launch_gemv_store(const void* W, const float* bias, const void* x, long ldx, void* y, long ldy, int G, int N,
                             int K, DType dt, hipStream_t s) {
  if (G <= 0 || N <= 0) return hipSuccess;
  const int epu = dt == DT_BF16 ? 8 : 4;
  if (G > 4 || K % epu || ldx % epu || reinterpret_cast<uintptr_t>(W) % 16 || reinterpret_cast<uintptr_t>(x) % 16)
    return hipErrorInvalidValue;
  constexpr int NR = 2;
  const dim3 grid((N + 4 * NR - 1) / (4 * NR)), block(256);
#define WAM_GEMV(T, GG)                                                                                         \
  hipLaunchKernelGGL((gemv_store_kernel<T, GG, NR>), grid, block, 0, s, reinterpret_cast<const T*>(W), bias,  \
                     reinterpret_cast<const T*>(x), ldx, reinterpret_cast<T*>(y), ldy, N, K)
  if (dt == DT_BF16) {
    if (G == 1) WAM_GEMV(bf16_t, 1); else if (G == 2) WAM_GEMV(bf16_t, 2); else if (G == 3) WAM_GEMV(bf16_t, 3); else WAM_GEMV(bf16_t, 4);
  } else {
    if (G == 1) WAM_GEMV(float, 1); else if (G == 2) WAM_GEMV(float, 2); else if (G == 3) WAM_GEMV(float, 3); else WAM_GEMV(float, 4);
  }
#undef WAM_GEMV
  return hipGetLastError();
}

template <typename T>
static void launch_gemv(const void* W, const float* b, const float* x, float* y, int N, int K, int G, int si, int so,
                        hipStream_t s) {
  const T* w = reinterpret_cast<const T*>(W);
  constexpr int NR = 8;
  const dim3 grid((N + 4 * NR - 1) / (4 * NR));
  if (G == 2) hipLaunchKernelGGL((gemv_rows_kernel<T, 2, NR>), grid, dim3(256), 0, s, w, b, x, y, N, K, si, so);
  else if (G == 4) hipLaunchKernelGGL((gemv_rows_kernel<T, 4, NR>), grid, dim3(256), 0, s, w, b, x, y, N, K, si, so);
  else hipLaunchKernelGGL(gemv_kernel<T>, dim3((N + 3) / 4), dim3(256), 0, s, w, b, x, y, N, K, G, si, so);
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
// the video part for the cosine used by velocity reuse. The grid is a fixed function of the sizes
// (about four vectors per thread, at most FLOW_MAX_BLOCKS workgroups), so for given sizes the
// reduction order is fixed. VEC = 4 moves float4s when every size and pointer allows it. The
// velocities are read, and x and g written, with the nontemporal hint: each is touched once here,
// and on a latent past the Infinity Cache the streaming accesses with a grid of two workgroups per
// CU move the 24 bytes per element faster than cached ones with more workgroups.
// ------------------------------------------------------------------------------------------------
static constexpr int FLOW_BLOCKS = 64;        // the UniPC step's grid
static constexpr int FLOW_MAX_BLOCKS = 512;

__device__ __forceinline__ float nt_load(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float4 nt_load(const float4* p) {
  return make_float4(__builtin_nontemporal_load(&p->x), __builtin_nontemporal_load(&p->y),
                     __builtin_nontemporal_load(&p->z), __builtin_nontemporal_load(&p->w));
}
__device__ __forceinline__ void nt_store(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void nt_store(float4* p, float4 v) {
  __builtin_nontemporal_store(v.x, &p->x); __builtin_nontemporal_store(v.y, &p->y);
  __builtin_nontemporal_store(v.z, &p->z); __builtin_nontemporal_store(v.w, &p->w);
}

static bool flow_vec4(const FlowArgs& a) {
  auto al = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  return a.nv % 4 == 0 && a.na % 4 == 0 && al(a.xv) && al(a.xa) && al(a.vv) && al(a.va) && al(a.gv) && al(a.ga) &&
         al(a.prev);
}
int flow_partial_blocks(int nv, int na) {
  const long units = ((long)nv + na + 3) / 4;
  return (int)std::max(1L, std::min((long)FLOW_MAX_BLOCKS, (units + 1023) / 1024));
}

template <int VEC>
__global__ void __launch_bounds__(256) flow_kernel(FlowArgs a) {
  using V = typename std::conditional<VEC == 4, float4, float>::type;
  __shared__ float red[4];
  const float wc = a.w, wu = 1.f - a.w;
  float dot = 0.f, gg = 0.f, pp = 0.f;
  const long uv = a.nv / VEC, n = uv + a.na / VEC;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const bool video = i < uv;
    const long k = video ? i : i - uv;
    const V* v = reinterpret_cast<const V*>(video ? a.vv : a.va);
    const long nn = (video ? a.nv : a.na) / VEC;
    V g = nt_load(v + k);
    if (a.br == 2) {
      const V u = nt_load(v + nn + k);
      if constexpr (VEC == 4) {
        g.x = wc * g.x + wu * u.x; g.y = wc * g.y + wu * u.y; g.z = wc * g.z + wu * u.z; g.w = wc * g.w + wu * u.w;
      } else {
        g = wc * g + wu * u;
      }
    }
    V* xp = reinterpret_cast<V*>(video ? a.xv : a.xa) + k;
    const float dt = video ? a.dtv : a.dta;
    V x = *xp;
    if constexpr (VEC == 4) {
      x.x += dt * g.x; x.y += dt * g.y; x.z += dt * g.z; x.w += dt * g.w;
    } else {
      x += dt * g;
    }
    nt_store(xp, x);
    if (video) {
      if (a.prev) {
        V p = reinterpret_cast<const V*>(a.prev)[k];
        if constexpr (VEC == 4) {
          dot += g.x * p.x; dot += g.y * p.y; dot += g.z * p.z; dot += g.w * p.w;
          gg += g.x * g.x; gg += g.y * g.y; gg += g.z * g.z; gg += g.w * g.w;
          pp += p.x * p.x; pp += p.y * p.y; pp += p.z * p.z; pp += p.w * p.w;
        } else {
          dot += g * p; gg += g * g; pp += p * p;
        }
      }
      if (a.gv) nt_store(reinterpret_cast<V*>(a.gv) + k, g);
    } else if (a.ga) {
      nt_store(reinterpret_cast<V*>(a.ga) + k, g);
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

// float4 form: the video and the action part each run their own grid-stride loop, four of a
// thread's float4s per pass with every load of the pass issued before any arithmetic (positions past
// the end re-read the last float4; their results are dropped), and the branch count, the cosine
// and the velocity store are compile-time cases, so no control flow sits between the loads. A
// thread visits the video float4s in the same order as the single-loop form, so the cosine partials
// are summed in that order.
template <bool TWO, bool PREV, bool GOUT>
__device__ __forceinline__ void flow_range4(const float4* v, long nn, float4* x,
                                            const float4* prev, float4* gout, float wc,
                                            float wu, float dt, float& dot, float& gg, float& pp) {
  constexpr int U = 4;
  const long S = (long)gridDim.x * 256;
  for (long i0 = (long)blockIdx.x * 256 + threadIdx.x; i0 < nn; i0 += U * S) {
    float4 cv[U], uv[U], xv[U], pv[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const long i = min(i0 + j * S, nn - 1);
      cv[j] = nt_load(v + i);
      if constexpr (TWO) uv[j] = nt_load(v + nn + i);
      xv[j] = x[i];
      if constexpr (PREV) pv[j] = prev[i];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const long i = i0 + j * S;
      if (i < nn) {
        float4 g = cv[j];
        if constexpr (TWO) {
          const float4 u = uv[j];
          g.x = wc * g.x + wu * u.x; g.y = wc * g.y + wu * u.y; g.z = wc * g.z + wu * u.z; g.w = wc * g.w + wu * u.w;
        }
        float4 xn = xv[j];
        xn.x += dt * g.x; xn.y += dt * g.y; xn.z += dt * g.z; xn.w += dt * g.w;
        nt_store(x + i, xn);
        if constexpr (PREV) {
          const float4 q = pv[j];
          dot += g.x * q.x; dot += g.y * q.y; dot += g.z * q.z; dot += g.w * q.w;
          gg += g.x * g.x; gg += g.y * g.y; gg += g.z * g.z; gg += g.w * g.w;
          pp += q.x * q.x; pp += q.y * q.y; pp += q.z * q.z; pp += q.w * q.w;
        }
        if constexpr (GOUT) nt_store(gout + i, g);
      }
    }
  }
}

template <bool TWO>
__device__ __forceinline__ void flow_parts4(const FlowArgs& a, float& dot, float& gg, float& pp) {
  const float wc = TWO ? a.w : 1.f, wu = TWO ? 1.f - a.w : 0.f;
  const float4* vv = reinterpret_cast<const float4*>(a.vv);
  const float4* va = reinterpret_cast<const float4*>(a.va);
  float4* xv = reinterpret_cast<float4*>(a.xv);
  float4* xa = reinterpret_cast<float4*>(a.xa);
  const float4* pr = reinterpret_cast<const float4*>(a.prev);
  float4* gv = reinterpret_cast<float4*>(a.gv);
  float4* ga = reinterpret_cast<float4*>(a.ga);
  const long nv = a.nv / 4, na = a.na / 4;
  if (a.prev) {
    if (a.gv) flow_range4<TWO, true, true>(vv, nv, xv, pr, gv, wc, wu, a.dtv, dot, gg, pp);
    else flow_range4<TWO, true, false>(vv, nv, xv, pr, gv, wc, wu, a.dtv, dot, gg, pp);
  } else {
    if (a.gv) flow_range4<TWO, false, true>(vv, nv, xv, pr, gv, wc, wu, a.dtv, dot, gg, pp);
    else flow_range4<TWO, false, false>(vv, nv, xv, pr, gv, wc, wu, a.dtv, dot, gg, pp);
  }
  if (a.ga) flow_range4<TWO, false, true>(va, na, xa, nullptr, ga, wc, wu, a.dta, dot, gg, pp);
  else flow_range4<TWO, false, false>(va, na, xa, nullptr, ga, wc, wu, a.dta, dot, gg, pp);
}

__global__ void __launch_bounds__(256) flow4_kernel(FlowArgs a) {
  __shared__ float red[4];
  float dot = 0.f, gg = 0.f, pp = 0.f;
  if (a.br == 2) flow_parts4<true>(a, dot, gg, pp);
  else flow_parts4<false>(a, dot, gg, pp);
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

// One wave: lane l sums blocks l, l + 64, ... in order, then a fixed butterfly across the lanes.
__global__ void __launch_bounds__(64) flow_reduce_kernel(const float* partials, int nblocks, float* out) {
  float s[3] = {0.f, 0.f, 0.f};
  for (int b = threadIdx.x; b < nblocks; b += 64)
#pragma unroll
    for (int c = 0; c < 3; ++c) s[c] += partials[b * 3 + c];
#pragma unroll
  for (int c = 0; c < 3; ++c) s[c] = wave_sum(s[c]);
  if (threadIdx.x == 0) {
    out[0] = s[0]; out[1] = s[1]; out[2] = s[2];
  }
}

hipError_t launch_flow_step(const FlowArgs& a, hipStream_t s) {
  const bool v4 = flow_vec4(a);
  const int nb = a.nblocks;
  if (nb < 1 || nb > FLOW_MAX_BLOCKS) return hipErrorInvalidValue;
  if (v4) hipLaunchKernelGGL(flow4_kernel, dim3(nb), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(flow_kernel<1>, dim3(nb), dim3(256), 0, s, a);
  if (a.prev && a.cos_parts) hipLaunchKernelGGL(flow_reduce_kernel, dim3(1), dim3(64), 0, s, a.partials, nb, a.cos_parts);
  return hipGetLastError();
}

// Library-owned scratch of the allocation-free flow step (wam_flow_step_noalloc): the per-workgroup
// cosine partials of one call, FLOW_MAX_BLOCKS x 3 floats (6 KB). Each GPU holds its own copy; host
// code reaches it only through the address that hipGetSymbolAddress returns for the current device,
// looked up once per device and kept (the array's name is not a device address on the host).
constexpr size_t kFlowScratchFloats = (size_t)FLOW_MAX_BLOCKS * 3;
static __device__ __align__(256) float scratch[kFlowScratchFloats];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static float* g_scratch_ptr[kMaxDevices];   // per device, nullptr until looked up

hipError_t flow_scratch(float** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kFlowScratchFloats * sizeof(float);
  return hipSuccess;
}

// ------------------------------------------------------------------------------------------------
// UniPC step ([WS1] names UniPC as the scheduler's solver; the published predictor-corrector in
// data-prediction form). Elementwise over the concatenated latent with weights from the host; the
// cosine partials of the guided video velocity are reduced exactly as in the flow step.
// ------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) unipc_kernel(UnipcArgs a) {
  __shared__ float red[4];
  const float wc = a.w, wu = 1.f - a.w;
  float dot = 0.f, gg = 0.f, pp = 0.f;
  const int n = a.nv + a.na;
  float* xprev = a.state + (long)4 * n;   // after the four data-prediction slots
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += FLOW_BLOCKS * 256) {
    const bool video = i < a.nv;
    const int k = video ? i : i - a.nv;
    const float* v = video ? a.vv : a.va;
    const int nn = video ? a.nv : a.na;
    float g = v[k];
    if (a.br == 2) g = wc * v[k] + wu * v[nn + k];
    float* xp = video ? a.xv + k : a.xa + k;
    const float x = *xp;
    const float m = x + a.sigma * g;
    float xs = x;
    if (a.corr) {
      xs = a.ca * xprev[i];
      for (int j = 0; j < a.cn; ++j) xs += a.cw[j] * a.state[(long)a.cslot[j] * n + i];
      xs += a.ct * m;
    }
    float xn = a.pa * xs + a.pw[0] * m;
    for (int j = 1; j < a.pn; ++j) xn += a.pw[j] * a.state[(long)a.pslot[j] * n + i];
    a.state[(long)a.slot_new * n + i] = m;
    xprev[i] = xs;
    *xp = xn;
    if (video) {
      if (a.prev) {
        const float p = a.prev[k];
        dot += g * p;
        gg += g * g;
        pp += p * p;
      }
      if (a.gv) a.gv[k] = g;
    } else if (a.ga) {
      a.ga[k] = g;
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

hipError_t launch_unipc_step(const UnipcArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(unipc_kernel, dim3(FLOW_BLOCKS), dim3(256), 0, s, a);
  if (a.prev && a.cos_parts)
    hipLaunchKernelGGL(flow_reduce_kernel, dim3(1), dim3(64), 0, s, a.partials, FLOW_BLOCKS, a.cos_parts);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// Output heads (fp32, or bf16 with unaligned operands). A workgroup takes 16 rows and one K slice (at most 320 columns): the slice of both
// head matrices and of the 16 rows goes to LDS once with coalesced 16-byte loads (video head rows
// 0 .. P-1, action head rows 64 .. 64+A-1, the activation rows after them; rows padded by 8
// elements so a wave's 64 weight-row reads hit distinct banks), then each wave computes 4 rows, lane
// n accumulating output n of each from LDS weight row n (fp32, k in order). The second kernel sums the slices in order, adds the bias and writes the row to its
// token-group output.
// ------------------------------------------------------------------------------------------------
constexpr int HEAD_ROWS = 16, HEAD_KMAX = 320;

template <typename T>
__global__ void __launch_bounds__(256) head_partial_kernel(HeadArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char head_lds[];
  T* wl = reinterpret_cast<T*>(head_lds);
  constexpr int EPU = 16 / sizeof(T);
  const int m0 = blockIdx.x * HEAD_ROWS, sp = blockIdx.y;
  const int kspan = a.D / a.splits, k0 = sp * kspan, pitch = kspan + 8;
  const int groups = kspan / 8;                              // 8-element groups per weight row
  T* yl = wl + (64 + a.A) * pitch;                          // the workgroup's activation rows
  for (int x = threadIdx.x; x < (a.P + a.A + HEAD_ROWS) * groups; x += 256) {
    const int r = x / groups, gidx = x % groups;
    const T* src;
    T* dst;
    if (r < a.P + a.A) {
      const bool vrow = r < a.P;
      src = reinterpret_cast<const T*>(vrow ? a.wv : a.wa) + (long)(vrow ? r : r - a.P) * a.D + k0 + gidx * 8;
      dst = wl + (vrow ? r : 64 + r - a.P) * pitch + gidx * 8;
    } else {
      const int yr = r - a.P - a.A;
      src = reinterpret_cast<const T*>(a.Y) + (long)min(m0 + yr, a.M - 1) * a.D + k0 + gidx * 8;
      dst = yl + yr * pitch + gidx * 8;
    }
#pragma unroll
    for (int u = 0; u < 8 / EPU; ++u) reinterpret_cast<uint4*>(dst)[u] = reinterpret_cast<const uint4*>(src)[u];
  }
  __syncthreads();
  const int n = threadIdx.x & 63, mb = m0 + (threadIdx.x >> 6) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const T* wrow[4];
  const T* yrow[4];
  bool act[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = min(mb + r, a.M - 1);
    const bool video = (m % a.rm.rows_per_branch) % a.rm.Lq < a.rm.Lv;
    act[r] = mb + r < a.M && n < (video ? a.P : a.A);
    wrow[r] = wl + (video ? n : 64 + min(n, a.A - 1)) * pitch;
    yrow[r] = yl + (mb + r - m0 < HEAD_ROWS ? mb + r - m0 : 0) * pitch;
  }
  for (int k = 0; k < kspan; k += 8) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float yv[8], wv[8];
#pragma unroll
      for (int u = 0; u < 8 / EPU; ++u) {
        const uint4 yy = *reinterpret_cast<const uint4*>(yrow[r] + k + u * EPU);
        const uint4 ww = *reinterpret_cast<const uint4*>(wrow[r] + k + u * EPU);
        const T* ye = reinterpret_cast<const T*>(&yy);
        const T* we = reinterpret_cast<const T*>(&ww);
#pragma unroll
        for (int e = 0; e < EPU; ++e) {
          yv[u * EPU + e] = Elem<T>::to_f(ye[e]);
          wv[u * EPU + e] = Elem<T>::to_f(we[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r] = fmaf(yv[e], wv[e], acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (act[r]) a.part[((long)sp * a.M + mb + r) * 64 + n] = acc[r];
}

// bf16 heads on the matrix cores: a wave takes 32 rows and one K slice and forms, with 32x32x16
// MFMAs (weight block first, so a lane holds one row's outputs in four runs of four), VB 32-column
// blocks of the video head and AB of the action head for those rows; each row keeps the outputs of
// the head its token belongs to. Operands come straight from memory (16 bytes per lane and step; the
// two head matrices, under 1 MB, stay in L2). Weight rows past P (A) and activation rows past M
// re-read the last one; their results are dropped. The slice's partial sums go to
// part[slice][row][64] like the LDS kernel's, and head_reduce_kernel sums them in slice order.
template <int VB, int AB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) head_mfma_kernel(HeadArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sp = blockIdx.y * 4 + wave;   // K slice (wave-uniform)
  if (sp >= a.splits) return;
  const int kspan = a.D / a.splits, k0 = sp * kspan;
  const int l32 = lane & 31, hk = (lane >> 5) * 8;
  const int row = blockIdx.x * 32 + l32;
  const bf16_t* y = reinterpret_cast<const bf16_t*>(a.Y) + (long)min(row, a.M - 1) * a.D + k0 + hk;
  const bf16_t* wv[VB];
  const bf16_t* wa[AB];
#pragma unroll
  for (int b = 0; b < VB; ++b)
    wv[b] = reinterpret_cast<const bf16_t*>(a.wv) + (long)min(b * 32 + l32, a.P - 1) * a.D + k0 + hk;
#pragma unroll
  for (int b = 0; b < AB; ++b)
    wa[b] = reinterpret_cast<const bf16_t*>(a.wa) + (long)min(b * 32 + l32, a.A - 1) * a.D + k0 + hk;
  floatx16 accv[VB], acca[AB];
#pragma unroll
  for (int b = 0; b < VB; ++b) accv[b] = floatx16{};
#pragma unroll
  for (int b = 0; b < AB; ++b) acca[b] = floatx16{};
  // five 16-column steps per pass, every load of the pass issued before its products, with no branch
  // between them: a step past the slice re-reads the last one and its activation fragment becomes
  // zero (a select), so its products add exact zeros
  constexpr int C = 5;
  for (int k = 0; k < kspan; k += 16 * C) {
    uint4 yf[C];
    bf16x8_t vf[C][VB], af[C][AB];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int kk = min(k + 16 * c, kspan - 16);
      yf[c] = *reinterpret_cast<const uint4*>(y + kk);
#pragma unroll
      for (int b = 0; b < VB; ++b) vf[c][b] = *reinterpret_cast<const bf16x8_t*>(wv[b] + kk);
#pragma unroll
      for (int b = 0; b < AB; ++b) af[c][b] = *reinterpret_cast<const bf16x8_t*>(wa[b] + kk);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool in = k + 16 * c < kspan;
      const uint4 yv = make_uint4(in ? yf[c].x : 0u, in ? yf[c].y : 0u, in ? yf[c].z : 0u, in ? yf[c].w : 0u);
      const bf16x8_t yb = __builtin_bit_cast(bf16x8_t, yv);
#pragma unroll
      for (int b = 0; b < VB; ++b) accv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[c][b], yb, accv[b], 0, 0, 0);
#pragma unroll
      for (int b = 0; b < AB; ++b) acca[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[c][b], yb, acca[b], 0, 0, 0);
    }
  }
  if (row >= a.M) return;
  const bool video = (row % a.rm.rows_per_branch) % a.rm.Lq < a.rm.Lv;
  float* dst = a.part + ((long)sp * a.M + row) * 64;
  // register e of block b holds output b * 32 + 8 (e / 4) + 4 (lane / 32) + e % 4 of this row
  auto put = [&](const floatx16& acc, int b, int nout) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n0 = b * 32 + 8 * q + 4 * (lane >> 5);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n0 + e < nout) dst[n0 + e] = acc[4 * q + e];
    }
  };
  if (video) {
#pragma unroll
    for (int b = 0; b < VB; ++b) put(accv[b], b, a.P);
  } else {
#pragma unroll
    for (int b = 0; b < AB; ++b) put(acca[b], b, a.A);
  }
}

__global__ void __launch_bounds__(256) head_reduce_kernel(HeadArgs a) {
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6), n = threadIdx.x & 63;
  if (m >= a.M) return;
  const int b = m / a.rm.rows_per_branch, rb = m % a.rm.rows_per_branch;
  const int ch = rb / a.rm.Lq, loc = rb % a.rm.Lq;
  const int nch = a.rm.rows_per_branch / a.rm.Lq, La = a.rm.Lq - a.rm.Lv;
  const bool video = loc < a.rm.Lv;
  const int nout = video ? a.P : a.A;
  if (n >= nout) return;
  // the slices in order; their loads issued eight at a time
  const float* pp = a.part + (long)m * 64 + n;
  const long st = (long)a.M * 64;
  float v = 0.f;
  int sp = 0;
  for (; sp + 8 <= a.splits; sp += 8) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = pp[(sp + j) * st];
#pragma unroll
    for (int j = 0; j < 8; ++j) v += x[j];
  }
  for (; sp < a.splits; ++sp) v += pp[sp * st];
  v += video ? a.bv[n] : a.ba[n];
  if (video) a.vv[((long)(b * nch + ch) * a.rm.Lv + loc) * a.P + n] = v;
  else a.va[((long)(b * nch + ch) * La + (loc - a.rm.Lv)) * a.A + n] = v;
}

hipError_t launch_head(const HeadArgs& a0, DType dt, hipStream_t s) {
  if (a0.M <= 0) return hipSuccess;
  if (a0.P > 64 || a0.A > 64 || a0.P < 1 || a0.A < 1 || a0.D % 8) return hipErrorInvalidValue;
  HeadArgs a = a0;
  // bf16 with 16-byte aligned operands: the matrix-core kernel, with K slices of a whole number of
  // 16-column steps (up to 32 slices of at least 160 columns), four slices per workgroup
  const bool al16 = reinterpret_cast<uintptr_t>(a.Y) % 16 == 0 && reinterpret_cast<uintptr_t>(a.wv) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(a.wa) % 16 == 0;
  if (dt == DT_BF16 && al16 && a.D % 16 == 0) {
    int sp = std::min(32, std::max(1, a.D / 160));
    while (sp > 1 && (a.D % (16 * sp) || (long)sp * a.M * 64 > a.part_elems)) --sp;
    if ((long)sp * a.M * 64 <= a.part_elems) {
      a.splits = sp;
      const dim3 grid((a.M + 31) / 32, (sp + 3) / 4), block(256);
      const int vb = (a.P + 31) / 32, ab = (a.A + 31) / 32;
      if (vb == 1 && ab == 1) hipLaunchKernelGGL((head_mfma_kernel<1, 1>), grid, block, 0, s, a);
      else if (vb == 1) hipLaunchKernelGGL((head_mfma_kernel<1, 2>), grid, block, 0, s, a);
      else if (ab == 1) hipLaunchKernelGGL((head_mfma_kernel<2, 1>), grid, block, 0, s, a);
      else hipLaunchKernelGGL((head_mfma_kernel<2, 2>), grid, block, 0, s, a);
      hipLaunchKernelGGL(head_reduce_kernel, dim3((a.M + 3) / 4), block, 0, s, a);
      return hipGetLastError();
    }
  }
  // the fewest K slices of at most HEAD_KMAX columns, each a whole number of 8-column groups
  // (and whose weight slices fit the 64 KB of dynamic LDS)
  const size_t esz = dt == DT_BF16 ? 2 : 4;
  auto lds_of = [&](int sp) { return (size_t)(64 + a.A + HEAD_ROWS) * (a.D / sp + 8) * esz; };
  a.splits = 1;
  while (a.splits <= a.D / 8 && (a.D / a.splits > HEAD_KMAX || a.D % (8 * a.splits) || lds_of(a.splits) > 65536))
    ++a.splits;
  if (a.splits > a.D / 8 || (long)a.splits * a.M * 64 > a.part_elems) return hipErrorInvalidValue;
  const size_t lds = lds_of(a.splits);
  const dim3 grid((a.M + HEAD_ROWS - 1) / HEAD_ROWS, a.splits), block(256);
  if (dt == DT_BF16) hipLaunchKernelGGL(head_partial_kernel<bf16_t>, grid, block, lds, s, a);
  else hipLaunchKernelGGL(head_partial_kernel<float>, grid, block, lds, s, a);
  hipLaunchKernelGGL(head_reduce_kernel, dim3((a.M + 3) / 4), block, 0, s, a);
  return hipGetLastError();
}

}  // namespace wam
