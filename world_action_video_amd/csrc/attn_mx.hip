// Attention on MXFP8 operands with MXFP8 probabilities (the softmax kept in fp8 e4m3 beside the fp8
// projections, as the mixed-precision passage of the DreamZero walk-through on real-time
// optimisations describes), head dimension 128.
//
// Same plan as the bf16 kernel: one workgroup = 4 waves = 128 queries of one (branch, head), keys
// streamed through an LDS ring filled by direct-to-LDS copies, S^T = K Q^T with the key rows
// permuted so that each lane holds one query's scores in the operand layout of O^T += V^T P^T. Here a
// tile is 64 keys and both products are v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, one e8m0
// scale per 32 values of an operand row):
//   - Q, K are MXFP8 along the head dimension, V^T along keys; their scale bytes come with the tile.
//   - The softmax reference m is kept an integer (log2 units), so p = 2^(s - m) differs from the
//     p of any other integer reference by a power of two, which the MX rule maps to the same codes.
//   - Each query's p over a 32-key block is quantised to e4m3 with the block's shared exponent
//     (floor(log2 max) - 8), saturated at 448, nearest even; the block's two halves sit in the lane
//     pair (l, l xor 32), one exchange gives the block maximum.
//   - The normaliser is the sum of the unquantised p.
// Keys past kv_total read as zero codes (buffer range) or are zeroed in LDS (values), and their
// probabilities are exactly 0, so nothing past kv_total reaches the output.
#include "common.h"
#include "kernels.h"

#pragma clang diagnostic ignored "-Winline-asm"   // M0 is written by the LDS-copy assembly

namespace wam {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int MXA_D = 128, MXA_BKV = 64, MXA_NW = 4, MXA_NS = 4, MXA_BQ = 32 * MXA_NW;
constexpr int MXA_KB = MXA_BKV * MXA_D;            // K codes of a tile (64 rows x 128 bytes)
constexpr int MXA_VB = MXA_D * MXA_BKV;            // V^T codes of a tile (128 rows x 64 bytes)
constexpr int MXA_KS = MXA_KB + MXA_VB;            // K scales (64 keys x 4 bytes; 1 KB region)
constexpr int MXA_VS = MXA_KS + 1024;              // V^T scales (2 key blocks x 128 rows; 1 KB region)
constexpr int MXA_SB = MXA_VS + 1024;              // stage bytes
constexpr int MXA_PER = 5;                         // copies per wave and tile: 4 of codes, 1 of scales

__device__ __forceinline__ void mxa_copy16(int lds_addr, int voffset, __amdgpu_buffer_rsrc_t rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voffset), "s"(rsrc) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void mxa_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }
__device__ __forceinline__ void mxa_hand_over() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void mxa_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void mxa_settle(uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }
__device__ __forceinline__ void mxa_settle(uint32_t& v) { asm volatile("" : "+v"(v)); }

// 16-byte units of a 128-byte K row / 64-byte V^T row are XOR-swizzled by row
__device__ __forceinline__ int mxa_kswz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int mxa_vswz(int row) { return (row >> 2) & 3; }
// key (within a 32-key subtile) fed to MFMA row rho = 8a + 4h + b: 16h + 4a + b, so register e of
// lane (q, h) holds key 16h + e
__device__ __forceinline__ int mxa_key_of_row(int rho) { return ((rho & 4) << 2) | ((rho >> 3) << 2) | (rho & 3); }

__device__ __forceinline__ int mxa_limit(const AttnMxArgs& a, int q) {
  int lim = a.kv_total;
  if (a.chunk_q > 0) lim = min(lim, a.kv_base + (q / a.chunk_q + 1) * a.chunk_q);
  return lim;
}

__device__ __forceinline__ i32x8 mxa_frag(uint4 lo, uint4 hi) {
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__global__ void __launch_bounds__(MXA_NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_mx_kernel(AttnMxArgs a) {
  constexpr int D = MXA_D, NS = MXA_NS, SB = MXA_SB, DB = D / 32;
  __shared__ __attribute__((aligned(1024))) uint4 smem[NS * SB / 16];
  char* lds = reinterpret_cast<char*>(smem);
  static_assert(MXA_NW * 32 * (D + 8) * 2 <= NS * SB, "output staging fits in LDS");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;

  // work unit in XCD-aware order: consecutive query blocks of one (branch, head) share an XCD
  const int nq = (a.Lq + MXA_BQ - 1) / MXA_BQ, units = nq * a.H * a.br;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int per = units >> 3, rem = units & 7;
  if (kx >= per + (xcd < rem ? 1 : 0)) return;
  const int unit = xcd * per + (xcd < rem ? xcd : rem) + kx;
  const int qt = unit % nq, bh = unit / nq, b = bh / a.H, h = bh % a.H;
  const int qblk = qt * MXA_BQ;
  const int q = qblk + wave * 32 + l32;
  const bool q_ok = q < a.Lq;
  const int qrow = q_ok ? q : a.Lq - 1;
  const int my_lim = q_ok ? mxa_limit(a, q) : 0;
  const int q_first = qblk + wave * 32;
  const int wave_lim = q_first < a.Lq ? mxa_limit(a, q_first) : 0;
  const int n_tiles = (mxa_limit(a, min(qblk + MXA_BQ, a.Lq) - 1) + MXA_BKV - 1) / MXA_BKV;
  const int last = n_tiles - 1;
  const int tail_tile = (a.kv_total % MXA_BKV) ? a.kv_total / MXA_BKV : -1;

  // ---- copies: waves 0, 1 take the K codes (rows 32 w .. 32 w + 31), waves 2, 3 the V^T codes (rows
  // 64 (w - 2) ..); every wave adds one 1 KB copy of a scale block (waves 0, 1: K scales; 2, 3: V^T
  // scales; the two copies of a pair write the same bytes). Lanes 16..63 of a scale copy refetch
  // the block's last 16 bytes into the unused rest of the 1 KB region.
  const bool kwave = wave < 2;
  const uint8_t* kb = a.K + (long)bh * a.k_bh;
  const uint8_t* vb = a.Vt + (long)bh * a.v_bh;
  const uint8_t* ksb = a.Ks + (long)bh * a.ks_bh;
  const uint8_t* vsb = a.Vs + (long)bh * a.vs_bh;
  const int nvb = (a.kv_total + 31) / 32;   // key blocks holding at least one key
  const __amdgpu_buffer_rsrc_t rcode = kwave
      ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kb), (short)0, a.kv_total * D, 0x00020000)
      : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vb), (short)0, D * a.v_stride, 0x00020000);
  const __amdgpu_buffer_rsrc_t rscale = kwave
      ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ksb), (short)0, a.kv_total * 4, 0x00020000)
      : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vsb), (short)0, nvb * D, 0x00020000);
  const int code_stride = kwave ? MXA_BKV * D : MXA_BKV;   // bytes from one tile to the next
  const int scale_stride = kwave ? MXA_BKV * 4 : 2 * D;
  int voff[4], ldst[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = (wave & 1) * 4 + j;   // 1 KB piece of the K (or V^T) block
    if (kwave) {
      const int row = i * 8 + (lane >> 3);
      voff[j] = row * D + (((lane & 7) ^ mxa_kswz(row)) * 16);
      ldst[j] = i * 1024;
    } else {
      const int row = i * 16 + (lane >> 2);
      voff[j] = row * a.v_stride + (((lane & 3) ^ mxa_vswz(row)) * 16);
      ldst[j] = MXA_KB + i * 1024;
    }
  }
  const int soff = min(lane, 15) * 16;
  const int sdst = kwave ? MXA_KS : MXA_VS;
  const int lds_base = (int)(uintptr_t)lds;
  auto copy = [&](int t, int stage) {
    const int tt = min(t, last);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      mxa_copy16(__builtin_amdgcn_readfirstlane(lds_base + stage * SB + ldst[j]), voff[j] + tt * code_stride, rcode);
    mxa_copy16(__builtin_amdgcn_readfirstlane(lds_base + stage * SB + sdst), soff + tt * scale_stride, rscale);
  };
  // value codes of keys at or past kv_total in the tile that holds kv_total become zero
  auto zero_tail = [&](int stage) {
    char* vbase = lds + stage * SB + MXA_KB;
    const int k0 = tail_tile * MXA_BKV;
    for (int x = tid; x < D * 4; x += MXA_NW * 64) {
      const int row = x >> 2, slot = x & 3;
      const int kfirst = k0 + 16 * (slot ^ mxa_vswz(row));
      if (kfirst + 16 <= a.kv_total) continue;
      uint4* p = reinterpret_cast<uint4*>(vbase + row * 64 + slot * 16);
      uint4 v = *p;
      uint8_t* e = reinterpret_cast<uint8_t*>(&v);
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (kfirst + k >= a.kv_total) e[k] = 0;
      *p = v;
    }
  };

  // ---- query fragments and scales (lane (q, h): head-dim bytes 64 c + 16 h and 64 c + 32 + 16 h)
  const uint8_t* qp = a.Q + (long)bh * a.q_bh + (long)qrow * D;
  uint4 qraw[4];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    qraw[2 * c] = *reinterpret_cast<const uint4*>(qp + 64 * c + 16 * half);
    qraw[2 * c + 1] = *reinterpret_cast<const uint4*>(qp + 64 * c + 32 + 16 * half);
  }
  uint32_t qsc = *reinterpret_cast<const uint32_t*>(a.Qs + (long)bh * a.qs_bh + (long)qrow * 4);

  floatx16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = floatx16{};
  float m_ref = -INFINITY, l_run = 0.f;   // integer reference in log2 units
  const float cs = a.scale_log2;

  // key fragments of subtile j, chunk c, and the key rows' scale words
  const int krow0 = mxa_key_of_row(l32);
  i32x8 kf[2][2];
  uint32_t ksc[2];
  auto load_k = [&](int stage) {
    const char* sk = lds + stage * SB;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 32 * j + krow0;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint4 lo = *reinterpret_cast<const uint4*>(sk + r * D + (((4 * c + half) ^ mxa_kswz(r)) * 16));
        const uint4 hi = *reinterpret_cast<const uint4*>(sk + r * D + (((4 * c + 2 + half) ^ mxa_kswz(r)) * 16));
        kf[j][c] = mxa_frag(lo, hi);
      }
      ksc[j] = *reinterpret_cast<const uint32_t*>(sk + MXA_KS + r * 4);
    }
  };

  if (n_tiles > 0) {
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) copy(t, t);
    mxa_vmcnt<MXA_PER * (NS - 2)>();
    mxa_hand_over();
    if (tail_tile == 0) {
      zero_tail(0);
      mxa_barrier();
    }
    load_k(0);
  }
  // consume the query loads here, so no wait of the compiler's inside the loop covers the copies
#pragma unroll
  for (int i = 0; i < 4; ++i) mxa_settle(qraw[i]);
  mxa_settle(qsc);
  const i32x8 qf[2] = {mxa_frag(qraw[0], qraw[1]), mxa_frag(qraw[2], qraw[3])};

  for (int kt = 0; kt < n_tiles; ++kt) {
    const char* sb = lds + (kt % NS) * SB;
    // (1) S^T = K Q^T for the two 32-key subtiles
    floatx16 s[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      s[j] = floatx16{};
#pragma unroll
      for (int c = 0; c < 2; ++c)
        s[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[j][c], qf[c], s[j], 0, 0, 0,
                                                               (int)(ksc[j] >> (8 * (2 * c + half))), 0,
                                                               (int)(qsc >> (8 * (2 * c + half))));
    }
    // (2) value fragments (lane (row, h): keys 16 h .. and 32 + 16 h ..) and their scale bytes
    i32x8 vf[DB];
    int vsc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = db * 32 + l32;
      const uint4 lo = *reinterpret_cast<const uint4*>(sb + MXA_KB + row * 64 + ((half ^ mxa_vswz(row)) * 16));
      const uint4 hi = *reinterpret_cast<const uint4*>(sb + MXA_KB + row * 64 + (((2 + half) ^ mxa_vswz(row)) * 16));
      vf[db] = mxa_frag(lo, hi);
      vsc[db] = (int)*reinterpret_cast<const uint8_t*>(sb + MXA_VS + half * D + row);
    }
    // (3) hand-over: tile kt+1 visible everywhere, the stage of tile kt-1 free
    mxa_vmcnt<MXA_PER * (NS - 3)>();
    mxa_hand_over();
    if (kt + 1 == tail_tile) {
      zero_tail((kt + 1) % NS);
      mxa_barrier();
    }
    // (4) request tile kt+NS-1 into the stage of tile kt-1; (5) next tile's key fragments
    copy(kt + NS - 1, (kt + NS - 1) % NS);
    load_k((kt + 1) % NS);
    // (6) softmax with an integer reference; register e of s[j] holds key kt*64 + 32 j + 16 h + e
    const int key0 = kt * MXA_BKV;
    float tmax = -INFINITY;
    if (key0 + MXA_BKV <= wave_lim) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[j][e]);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + 32 * j + 16 * half + e;
          s[j][e] = key < my_lim ? s[j][e] : -INFINITY;
          tmax = fmaxf(tmax, s[j][e]);
        }
    }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
      tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * cs;
    }
    if (__any(tmax > m_ref + 8.f)) {
      const float m_new = ceilf(fmaxf(m_ref, tmax));
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);   // a power of two
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
    }
    const float moff = m_ref == -INFINITY ? 0.f : m_ref;
    float p[2][16];
    float pmax[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      pmax[j] = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[j][e] = __builtin_amdgcn_exp2f(fmaf(s[j][e], cs, -moff));
        l_run += p[j][e];
        pmax[j] = fmaxf(pmax[j], p[j][e]);
      }
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(pmax[j]), __float_as_uint(pmax[j]), false, false);
      pmax[j] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // (7) P in MXFP8 (block j = subtile j), then O^T += V^T P^T
    int pe[2];
    uint32_t pw[8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      pe[j] = mx_block_exponent(pmax[j]);
      const float inv = mx_inv_scale(pe[j]);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        pw[4 * j + g] = mx_pack4(p[j][4 * g] * inv, p[j][4 * g + 1] * inv, p[j][4 * g + 2] * inv, p[j][4 * g + 3] * inv);
    }
    const i32x8 pf = i32x8{(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3], (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
    const int psc = (half ? pe[1] : pe[0]) + 127;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[db], pf, o[db], 0, 0, 0, vsc[db], 0, psc);
  }
  mxa_vmcnt<0>();
  mxa_barrier();

  // ---- normalise, stage each wave's 32 x 128 block through LDS, write whole 16-byte row pieces
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  constexpr int SROW = D + 8;
  bf16_t* stage = reinterpret_cast<bf16_t*>(smem) + wave * 32 * SROW;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) stage[l32 * SROW + db * 32 + acc_row(e, lane)] = f32_to_bf16(o[db][e] * inv);
  __syncthreads();
  bf16_t* O = reinterpret_cast<bf16_t*>(a.O);
  for (int u = lane; u < 32 * (D / 8); u += 64) {
    const int r = u / (D / 8), cu = u % (D / 8);
    const int qq = qblk + wave * 32 + r;
    if (qq < a.Lq)
      *reinterpret_cast<uint4*>(O + ((long)b * a.Lq + qq) * ((long)a.H * D) + (long)h * D + cu * 8) =
          reinterpret_cast<const uint4*>(stage + r * SROW)[cu];
  }
}

}  // namespace

hipError_t launch_attention_mx(const AttnMxArgs& a, hipStream_t s) {
  const int units = (a.Lq + MXA_BQ - 1) / MXA_BQ * a.H * a.br;
  if (units <= 0) return hipSuccess;
  const dim3 grid((unsigned)((units + 7) / 8 * 8)), block(MXA_NW * 64);
  hipLaunchKernelGGL(attn_mx_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace wam
