// Flash-style attention for the chunk-causal self-attention over the KV cache and for the
// cross-attention over the condition tokens.
//
// One workgroup = 4 waves = 128 queries of one (branch, head); each wave owns 32 queries. Keys
// stream through LDS in tiles of 64 (double-buffered, register-staged loads). Per tile a wave
// computes S^T = K Q^T with 32x32 MFMAs, so every lane holds the scores of ONE query (lane mod 32)
// for 32 of the 64 keys; the other 32 sit in the partner lane (lane xor 32). The row max therefore
// needs a single cross-lane exchange, and the rescale factor of the running output is a per-lane
// scalar. The key rows fed to the MFMA are permuted (bits 2 and 3 of the row index swapped) so that
// the score registers come out exactly in the operand layout of the next product, O^T += V^T P^T:
// the probabilities never leave registers. Values are stored key-contiguous (V^T) so their operand
// fragments are plain 16-byte LDS reads.
//
// Masking is by select: a score whose key is at or beyond the query's limit becomes -inf before the
// max, so its probability is exactly 0 and hidden keys cannot influence the result. The limit of
// query q is min(kv_total, kv_base + (q / chunk_q + 1) * chunk_q): cached clean chunks are always
// visible, current-chunk keys up to the end of the query's own chunk (bidirectional inside a chunk),
// never later chunks. Value rows past kv_total are zero-filled in LDS.
#include "common.h"
#include "kernels.h"

namespace wam {

static constexpr int ATT_BQ = 128, ATT_BKV = 64;

__device__ __forceinline__ int swap_bits_2_3(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <typename T, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_kernel(AttnArgs a) {
  constexpr int EPU = 16 / sizeof(T);
  constexpr int KU = D * (int)sizeof(T) / 16;          // 16-byte units per K row (D elements)
  constexpr int VU = ATT_BKV * (int)sizeof(T) / 16;    // 16-byte units per V^T row (64 keys)
  constexpr int K_UNITS = ATT_BKV * KU, V_UNITS = D * VU;
  constexpr int K_PER_T = K_UNITS / 256, V_PER_T = V_UNITS / 256;
  constexpr int UPF = 8 / EPU;
  constexpr int DC = D / 16;                            // k16 chunks over the head dim
  constexpr int DB = D / 32;                            // 32-row blocks of the output O^T
  __shared__ uint4 smem[2][K_UNITS + V_UNITS];
  // LDS swizzles (16-byte units XOR a row-dependent phase) chosen so that each 16-lane pass of a
  // fragment read (16 rows, one logical unit) covers distinct banks: rows of 256 bytes or more
  // take phase row mod 16; 128-byte rows take (row / 2) mod 8 (row pairs share a bank line).
  auto kswz = [](int row) { return KU >= 16 ? (row & 15) : ((row >> 1) & 7); };
  auto vswz = [](int row) { return VU >= 16 ? (row & 15) : ((row >> 1) & 7); };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  // XCD-aware order: workgroup w runs on XCD w mod 8; give each XCD a contiguous range of
  // (branch, head, query tile) items, query tiles fastest, so the tiles that stream the same keys and
  // values share one L2.
  const int nq = (a.Lq_total + ATT_BQ - 1) / ATT_BQ;
  const int items = nq * a.H * a.br;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int per = items >> 3, rem = items & 7;
  if (kx >= per + (xcd < rem ? 1 : 0)) return;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + kx;
  const int qt = item % nq, bh_i = item / nq;
  const int h = bh_i % a.H, b = bh_i / a.H;
  const int qblk = qt * ATT_BQ;
  const long bh = (long)b * a.H + h;
  const T* Q = reinterpret_cast<const T*>(a.Q) + bh * a.q_bh_stride;
  const T* K = reinterpret_cast<const T*>(a.K) + bh * a.k_bh_stride;
  const T* Vt = reinterpret_cast<const T*>(a.Vt) + bh * a.v_bh_stride;

  auto limit_of = [&](int q) {
    int lim = a.kv_total;
    if (a.chunk_q > 0) {
      const int c = a.kv_base + (q / a.chunk_q + 1) * a.chunk_q;
      lim = c < lim ? c : lim;
    }
    return lim;
  };
  const int q_last = min(qblk + ATT_BQ, a.Lq_total) - 1;
  const int kv_wg = limit_of(q_last);                   // limits grow with q: the last query sees most
  const int n_tiles = (kv_wg + ATT_BKV - 1) / ATT_BKV;

  // this lane's query and its key limit
  const int q = qblk + wave * 32 + l32;
  const bool q_ok = q < a.Lq_total;
  const int my_lim = q_ok ? limit_of(q) : 0;
  // smallest limit among this wave's valid queries (the first one); 0 if the wave has none
  const int q_first = qblk + wave * 32;
  const int wave_lim = q_first < a.Lq_total ? limit_of(q_first) : 0;

  // Q^T fragments (B operand of S^T = K Q^T): lane (query l32, half) holds Q[q][16c + 8 half .. +8]
  Frag<T> qf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    uint4* dst = reinterpret_cast<uint4*>(&qf[c]);
#pragma unroll
    for (int u = 0; u < UPF; ++u)
      dst[u] = q_ok ? *reinterpret_cast<const uint4*>(Q + (long)q * D + c * 16 + half * 8 + u * EPU)
                    : make_uint4(0, 0, 0, 0);
  }

  uint4 rk[K_PER_T], rv[V_PER_T];
  auto gload = [&](int kt) {
    const int key0 = kt * ATT_BKV;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int u = tid + 256 * i, row = u / KU, unit = u % KU;
      const int key = key0 + row;
      rk[i] = key < a.kv_total ? *reinterpret_cast<const uint4*>(K + (long)key * D + unit * EPU) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + 256 * i, row = u / VU, unit = u % VU;
      const int kfirst = key0 + unit * EPU;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kfirst < a.kv_total) {
        v = *reinterpret_cast<const uint4*>(Vt + (long)row * a.v_stride + kfirst);
        const int valid = a.kv_total - kfirst;
        if (valid < EPU) {
          T* e = reinterpret_cast<T*>(&v);
#pragma unroll
          for (int x = 0; x < EPU; ++x)
            if (x >= valid) e[x] = T(0);
        }
      }
      rv[i] = v;
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int u = tid + 256 * i, row = u / KU, unit = u % KU;
      smem[st][row * KU + (unit ^ kswz(row))] = rk[i];
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + 256 * i, row = u / VU, unit = u % VU;
      smem[st][K_UNITS + row * VU + (unit ^ vswz(row))] = rv[i];
    }
  };

  floatx16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;

  if (n_tiles > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < n_tiles; ++kt) {
    if (kt + 1 < n_tiles) gload(kt + 1);
    const uint4* sk = smem[kt & 1];
    const uint4* sv = sk + K_UNITS;
    const int key0 = kt * ATT_BKV;

    // S^T blocks: rows = keys (permuted), columns = this wave's 32 queries
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = floatx16{};
      const int row = kb * 32 + swap_bits_2_3(l32);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        Frag<T> kf;
        uint4* dst = reinterpret_cast<uint4*>(&kf);
        const int u0 = (c * 16 + half * 8) / EPU;
#pragma unroll
        for (int u = 0; u < UPF; ++u) dst[u] = sk[row * KU + ((u0 + u) ^ kswz(row))];
        mfma_k16(s[kb], kf, qf[c]);
      }
    }
    // register e of block kb holds key key0 + 32 kb + 16 (e / 8) + 8 half + (e % 8). Limits rise with
    // the query index, so a tile entirely below the wave's first limit needs no mask.
    float tmax = -INFINITY;
    if (key0 + ATT_BKV <= wave_lim) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[kb][e] *= a.scale_log2;
          tmax = fmaxf(tmax, s[kb][e]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + kb * 32 + 16 * (e >> 3) + 8 * half + (e & 7);
          const float v = key < my_lim ? s[kb][e] * a.scale_log2 : -INFINITY;
          s[kb][e] = v;
          tmax = fmaxf(tmax, v);
        }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    // a query with no visible key yet keeps m = -inf: its probabilities and alpha are 0 and o, l stay 0
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
    Frag<T> pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(s[kb][8 * j + e] - m_use);
          psum += p[e];
        }
        pack_frag(pf[kb][j], p);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      const int row = db * 32 + l32;     // head-dim index of this lane's V^T row
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          Frag<T> vf;
          uint4* dst = reinterpret_cast<uint4*>(&vf);
          const int u0 = (kb * 32 + 16 * j + 8 * half) / EPU;
#pragma unroll
          for (int u = 0; u < UPF; ++u) dst[u] = sv[row * VU + ((u0 + u) ^ vswz(row))];
          mfma_k16(o[db], vf, pf[kb][j]);
        }
    }
    if (kt + 1 < n_tiles) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- normalise and write O[b * Lq_total + q][h * D + dd] through LDS (rows become contiguous)
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  constexpr int SROW = D + EPU;   // staging row pitch: one 16-byte pad unit against bank conflicts
  static_assert(4 * 32 * SROW * (int)sizeof(T) <= 2 * (K_UNITS + V_UNITS) * 16, "staging fits in LDS");
  T* stage = reinterpret_cast<T*>(&smem[0][0]) + wave * 32 * SROW;   // [32 queries][SROW]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) stage[l32 * SROW + db * 32 + acc_row(e, lane)] = Elem<T>::from_f(o[db][e] * inv);
  __syncthreads();
  constexpr int ROW_UNITS = D * (int)sizeof(T) / 16;
  T* O = reinterpret_cast<T*>(a.O);
  for (int u = lane; u < 32 * ROW_UNITS; u += 64) {
    const int r = u / ROW_UNITS, c = u % ROW_UNITS;
    const int qq = qblk + wave * 32 + r;
    if (qq < a.Lq_total)
      *reinterpret_cast<uint4*>(O + ((long)b * a.Lq_total + qq) * ((long)a.H * D) + (long)h * D + c * EPU) =
          reinterpret_cast<const uint4*>(stage + r * SROW)[c];
  }
}

template <typename T, int D>
static hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  const int items = ((a.Lq_total + ATT_BQ - 1) / ATT_BQ) * a.H * a.br;
  const dim3 grid(8 * ((items + 7) / 8)), block(256);
  hipLaunchKernelGGL((attn_kernel<T, D>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, DType dt, hipStream_t s) {
  if (a.Lq_total <= 0) return hipSuccess;
  if (dt == DT_BF16) {
    if (a.d == 128) return launch_t<bf16_t, 128>(a, s);
    if (a.d == 64) return launch_t<bf16_t, 64>(a, s);
  } else {
    if (a.d == 128) return launch_t<float, 128>(a, s);
    if (a.d == 64) return launch_t<float, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace wam
