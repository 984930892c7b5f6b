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
// query q (attn_limit) is min(kv_total, kv_base + (q / chunk_q + 1) * chunk_q): cached clean chunks
// are always visible, current-chunk keys up to the end of the query's own chunk (bidirectional
// inside a chunk), never later chunks; with the frame-causal variant a video query's limit ends at
// its own frame instead. Limits never decrease with q. Value rows past kv_total are zero-filled in LDS.
#include "common.h"
#include "kernels.h"

#include <algorithm>

#pragma clang diagnostic ignored "-Winline-asm"   // M0 is written by the LDS-copy assembly

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

  auto limit_of = [&](int q) { return attn_limit(a, q); };
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

// ------------------------------------------------------------------------------------------------
// bf16 kernel with 32-key tiles copied global -> LDS by the buffer unit (buffer_load ... lds), in a
// ring of NS stages: tile t+NS-1 is requested while tile t computes, so about NS-1 tiles of compute
// cover the memory latency and no registers stage the copies. Each 1 KB copy instruction writes
// 64 lanes x 16 bytes contiguously; which 16-byte unit a lane fetches implements the XOR swizzle. The copies are issued from inline assembly (M0 holds the LDS destination) and
// waited for with explicit vmcnt counts before the barrier that hands a stage over, so the compiler
// neither drains them at barriers nor waits for them before unrelated LDS reads.
//
// Softmax bookkeeping follows the online (running max) formulation with a lazy reference: the
// running max used as the exponent offset is raised (and the output rescaled) only when a tile's max
// exceeds it by more than 2^8 for some query of the wave; otherwise probabilities up to 2^8 are
// accumulated against the old reference. The final normalisation divides by the sum accumulated
// against the same reference, so the result is the exact softmax (rescaling is exact up to
// rounding). p = exp2(s c - m), c = log2(e)/sqrt(d), comes out of the score product itself: the
// query fragments are pre-scaled by c (rounded to bf16 once more) and the first MFMA of a tile
// accumulates onto a block holding -m, so the exponent needs no vector arithmetic.
// The row sum is taken over the bf16-rounded probabilities (dot products of the packed pairs with
// ones), i.e. over exactly the weights the value product uses, and the tile maximum is a tree of
// three-input maxima (no NaN-quieting steps: scores are finite or -inf by construction).
//
// Keys at or past kv_total read as zero (the copy's buffer range ends there) and are masked; values
// past kv_total are zeroed in LDS once their tile has landed, so stale rows never meet a zero
// probability as 0 * inf or 0 * NaN.
// ------------------------------------------------------------------------------------------------
static constexpr int AT3_BKV = 32;   // keys per tile
static constexpr int AT3_NW = 4;     // waves (x 32 queries) per workgroup
static constexpr int AT3_PART = 66 * 64;   // floats of one wave's key-split partial: up to 64 accumulators, max, sum

template <int N>
__device__ __forceinline__ void vmcnt_wait() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

__device__ __forceinline__ void lds_copy16(int lds_addr, int voffset, __amdgpu_buffer_rsrc_t rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voffset), "s"(rsrc) : "memory", "m0");
}

// The compiler cannot see the lds_copy16 loads, so a wait it places for its own loads in a loop
// header would also drain every copy in flight. Consuming the query fragments once before the loop
// moves that wait out of the loop.
__device__ __forceinline__ void settle(uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }

// copies land in LDS without LDS-counter traffic: handing a stage over needs only vmcnt and a barrier
__device__ __forceinline__ void lds_hand_over() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One workgroup's share: NW waves x 32 queries of one (branch, head), taken in XCD-aware order
// (consecutive query blocks of a head share one XCD's L2), with each query's chunk-causal key limit.
// With `splits` > 1 each query block is a unit of `splits` workgroups, one per contiguous range of
// its key tiles; the units of one block are consecutive, so they also share an XCD.
template <int NW>
struct AttnItem {
  static constexpr int BQ = 32 * NW;
  bool valid = false, q_ok = false;
  int item = 0, split = 0, b = 0, h = 0, qblk = 0, n_tiles = 0, q = 0, my_lim = 0, wave_lim = 0;
  long bh = 0;
  __device__ __forceinline__ static int limit_of(const AttnArgs& a, int q) { return attn_limit(a, q); }
  __device__ __forceinline__ static int blocks(const AttnArgs& a) { return (a.Lq_total + BQ - 1) / BQ * a.H * a.br; }
  // the workgroup's unit from its index in XCD order
  __device__ __forceinline__ AttnItem(const AttnArgs& a, int wave, int l32, int splits) {
    const int units = blocks(a) * splits;
    const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
    const int per = units >> 3, rem = units & 7;
    if (kx >= per + (xcd < rem ? 1 : 0)) return;
    const int unit = xcd * per + (xcd < rem ? xcd : rem) + kx;
    init(a, unit / splits, wave, l32);
    split = unit % splits;
  }
  // query block `it` directly (the merge of key-split partials)
  __device__ __forceinline__ static AttnItem block(const AttnArgs& a, int it, int wave, int l32) {
    AttnItem r;
    r.init(a, it, wave, l32);
    return r;
  }
  AttnItem() = default;
  __device__ __forceinline__ void init(const AttnArgs& a, int it, int wave, int l32) {
    valid = true;
    item = it;
    const int nq = (a.Lq_total + BQ - 1) / BQ;
    const int qt = it % nq, bh_i = it / nq;
    h = bh_i % a.H;
    b = bh_i / a.H;
    qblk = qt * BQ;
    bh = (long)b * a.H + h;
    const int q_last = min(qblk + BQ, a.Lq_total) - 1;
    n_tiles = (limit_of(a, q_last) + AT3_BKV - 1) / AT3_BKV;
    q = qblk + wave * 32 + l32;
    q_ok = q < a.Lq_total;
    my_lim = q_ok ? limit_of(a, q) : 0;
    const int q_first = qblk + wave * 32;   // the limit grows with the query: the wave's first is its least
    wave_lim = q_first < a.Lq_total ? limit_of(a, q_first) : 0;
  }
};

// The LDS ring. Stage s holds the K block of a 32-key tile (32 rows of D bf16, 16-byte units XOR
// swizzled by row) followed by its V^T block (D rows of 32 keys, 64 bytes each). Waves
// 0 .. K_INSTR/PER_WAVE - 1 copy the K block and the others the V^T block, so each wave has a single
// source and no branches. Lane offsets are for tile 0; tile t adds t * tile_stride. Requests past
// the last tile refetch the last tile into a free stage.
template <int D, int NS, int NW>
struct KvRing {
  static constexpr int KU = D / 8;                      // 16-byte units per K row
  static constexpr int K_ROWS_I = 64 / KU;              // K rows per 1 KB copy
  static constexpr int K_INSTR = AT3_BKV / K_ROWS_I;    // copies per K tile
  static constexpr int V_INSTR = D / 16;                // copies per V^T tile (16 rows each)
  // waves that copy: all when the copies split evenly over them, else the first four (the others
  // only compute; their vmcnt waits are then trivially met)
  static constexpr int COPY_WAVES = (K_INSTR + V_INSTR) % NW == 0 ? NW : 4;
  static constexpr int PER_WAVE = (K_INSTR + V_INSTR) / COPY_WAVES;
  static constexpr int KB = AT3_BKV * D * 2, SB = KB + D * AT3_BKV * 2;   // K block, stage bytes
  static_assert((K_INSTR + V_INSTR) % COPY_WAVES == 0 && COPY_WAVES <= NW, "copies split evenly over the copy waves");
  static_assert(K_INSTR % PER_WAVE == 0, "a wave copies either keys or values");
  __device__ __forceinline__ static int kswz(int row) { return KU >= 16 ? (row & 15) : ((row >> 1) & 7); }
  __device__ __forceinline__ static int vswz(int row) { return (row >> 2) & 3; }   // four 64-B rows share a bank line

  int lds_base, tile_stride, last;
  bool copier;
  int voff[PER_WAVE], ldst[PER_WAVE];
  __amdgpu_buffer_rsrc_t rsrc;

  __device__ __forceinline__ KvRing(const AttnArgs& a, long bh, const char* lds, int wave, int lane, int n_tiles) {
    using T = bf16_t;
    lds_base = (int)(uintptr_t)lds;   // low 32 bits of a generic LDS pointer: its LDS address
    last = n_tiles - 1;
    // buffer ranges: keys of this (branch, head) up to kv_total; all value rows of its block
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(reinterpret_cast<const T*>(a.K) + bh * a.k_bh_stride), (short)0, a.kv_total * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(reinterpret_cast<const T*>(a.Vt) + bh * a.v_bh_stride), (short)0, D * a.v_stride * 2, 0x00020000);
    copier = wave < COPY_WAVES;
    const bool kwave = wave * PER_WAVE < K_INSTR;
    rsrc = kwave ? rk : rv;
    tile_stride = kwave ? AT3_BKV * D * 2 : AT3_BKV * 2;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int i = min(wave * PER_WAVE + j, K_INSTR + V_INSTR - 1);   // copy index within the tile
      const int ki = i, vi = i - K_INSTR;
      const int krow = ki * K_ROWS_I + lane / KU, vrow = vi * 16 + (lane >> 2);
      voff[j] = kwave ? krow * D * 2 + ((lane % KU) ^ kswz(krow)) * 16
                      : vrow * a.v_stride * 2 + ((lane & 3) ^ vswz(vrow)) * 16;
      ldst[j] = kwave ? ki * 1024 : KB + vi * 1024;
    }
  }
  __device__ __forceinline__ void copy(int t, int stage) const {
    if constexpr (COPY_WAVES < NW)
      if (!copier) return;   // wave-uniform
    const int toff = min(t, last) * tile_stride;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j)   // the LDS address is wave-uniform (M0 takes a scalar)
      lds_copy16(__builtin_amdgcn_readfirstlane(lds_base + stage * SB + ldst[j]), voff[j] + toff, rsrc);
  }
  // values past kv_total in the tile that holds kv_total (once it has landed) become zero
  __device__ __forceinline__ static void zero_tail(char* lds, int stage, int tail_tile, int kv_total, int tid) {
    using T = bf16_t;
    char* vb = lds + stage * SB + KB;
    const int k0 = tail_tile * AT3_BKV;
    for (int x = tid; x < D * 4; x += NW * 64) {
      const int row = x >> 2, u = x & 3;
      const int kfirst = k0 + u * 8;
      if (kfirst + 8 <= kv_total) continue;
      uint4* p = reinterpret_cast<uint4*>(vb + row * 64 + ((u ^ vswz(row)) * 16));
      uint4 v = *p;
      T* e = reinterpret_cast<T*>(&v);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (kfirst + k >= kv_total) e[k] = T(0);
      *p = v;
    }
  }
};

// Query fragments of the 32x32x16 products: lane l holds query l % 32, head-dim elements
// 16 c + 8 (l / 32) .. + 8. Lanes past the last query read the last query's row (no branch around
// the loads); their results are never stored.
template <int D, int NW>
__device__ __forceinline__ void load_q_frags(const AttnArgs& a, const AttnItem<NW>& it, int half, uint4 (&qf)[D / 16]) {
  const bf16_t* Q = reinterpret_cast<const bf16_t*>(a.Q) + it.bh * a.q_bh_stride;
  const int q_row = it.q_ok ? it.q : a.Lq_total - 1;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) qf[c] = *reinterpret_cast<const uint4*>(Q + (long)q_row * D + c * 16 + half * 8);
}

// Normalise, stage each wave's 32 x D block through LDS and write whole 16-byte row pieces.
// The caller has drained every copy and synchronised the workgroup (the ring is reused).
template <int D, int NW>
__device__ __forceinline__ void store_output(uint4* smem, const floatx16 (&o)[D / 32], float l_run, const AttnArgs& a,
                                             const AttnItem<NW>& it, int wave, int lane) {
  using T = bf16_t;
  const int l32 = lane & 31;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  constexpr int SROW = D + 8;
  T* stage = reinterpret_cast<T*>(smem) + wave * 32 * SROW;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) stage[l32 * SROW + db * 32 + acc_row(e, lane)] = f32_to_bf16(o[db][e] * inv);
  __syncthreads();
  constexpr int ROW_UNITS = D / 8;
  T* O = reinterpret_cast<T*>(a.O);
  for (int u = lane; u < 32 * ROW_UNITS; u += 64) {
    const int r = u / ROW_UNITS, cu = u % ROW_UNITS;
    const int qq = it.qblk + wave * 32 + r;
    if (qq < a.Lq_total)
      *reinterpret_cast<uint4*>(O + ((long)it.b * a.Lq_total + qq) * ((long)a.H * D) + (long)it.h * D + cu * 8) =
          reinterpret_cast<const uint4*>(stage + r * SROW)[cu];
  }
}

__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Row maximum of the 16 relative scores a lane holds (-inf start), then with the partner lane's 16.
__device__ __forceinline__ float tile_max_rel(const floatx16& s) {
  const float a0 = vmax3(s[0], s[1], s[2]), a1 = vmax3(s[3], s[4], s[5]), a2 = vmax3(s[6], s[7], s[8]);
  const float a3 = vmax3(s[9], s[10], s[11]), a4 = vmax3(s[12], s[13], s[14]);
  const float m = vmax3(vmax3(a0, a1, a2), vmax3(a3, a4, s[15]), -INFINITY);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return vmax3(__uint_as_float(sw[0]), __uint_as_float(sw[1]), -INFINITY);
}

// Eight bf16 values times c, rounded back to bf16 (to nearest even).
__device__ __forceinline__ uint4 scale_bf16x8(uint4 v, float c) {
  auto sc = [c](uint32_t w) { return pack2_bf16(__uint_as_float(w << 16) * c, __uint_as_float(w & 0xffff0000u) * c); };
  return make_uint4(sc(v.x), sc(v.y), sc(v.z), sc(v.w));
}

// Scores of keys at or past the lane's limit become -inf (select). Register e holds key
// key0 + 8 half + 16 (e / 8) + e % 8, so each test compares a constant with lim - key0 - 8 half.
__device__ __forceinline__ void mask_tile(floatx16& s, int key0, int half, int lim) {
  const int rel = lim - key0 - 8 * half;
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = 16 * (e >> 3) + (e & 7) < rel ? s[e] : -INFINITY;
}

// Per tile kt: scores from K fragments already in registers, value fragments requested, stage
// hand-over (tile kt+1 visible, stage of tile kt-1 free), copy of tile kt+NS-1 requested, K
// fragments of tile kt+1 requested, then the softmax and the value product, so LDS latency hides
// behind matrix and vector work. Tile kt+1's copies were requested NS-3 tiles earlier.
template <int D, int NS, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn3_kernel(AttnArgs a) {
  using Ring = KvRing<D, NS, NW>;
  constexpr int KB = Ring::KB, SB = Ring::SB, DC = D / 16, DB = D / 32;
  static_assert(NS >= 4, "the hand-over waits for copies issued NS-3 tiles ahead");
  static_assert(NW * 32 * (D + 8) * 2 <= NS * SB, "output staging fits in LDS");
  __shared__ __attribute__((aligned(1024))) uint4 smem[NS * SB / 16];
  char* lds = reinterpret_cast<char*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const AttnItem<NW> it(a, wave, l32, a.kv_splits);
  if (!it.valid) return;
  // this workgroup's key tiles [t0, t1): all of them, or one contiguous range of a key split
  const int t0 = it.split * it.n_tiles / a.kv_splits, t1 = (it.split + 1) * it.n_tiles / a.kv_splits;
  const int nt = t1 - t0;
  const Ring ring(a, it.bh, lds, wave, lane, t1);
  const int tail_tile = (a.kv_total % AT3_BKV) ? a.kv_total / AT3_BKV : -1;

  uint4 qf[DC];
  load_q_frags<D, NW>(a, it, half, qf);
  floatx16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = floatx16{};
  // The query fragments are multiplied by log2(e)/sqrt(d) once (one more bf16 rounding of each
  // query element), so scores leave the product in log2 units; the product starts from -m_ref
  // (negm, the lane's reference broadcast over its 16 scores), so they also leave it relative to the
  // reference and go straight into exp2. m_ref = -inf: no visible key yet (negm holds 0). thr is
  // the relative score that raises the reference: any visible score while there is none, else 2^8.
#pragma unroll
  for (int cc = 0; cc < DC; ++cc) qf[cc] = scale_bf16x8(qf[cc], a.scale_log2);
  float m_ref = -INFINITY, l_run = 0.f, thr = -INFINITY;
  floatx16 negm = floatx16{};

  const int srow = swap_bits_2_3(l32);
  uint4 kf[DC];
  auto load_kf = [&](int stage) {
    const char* sk = lds + stage * SB + srow * (D * 2);
#pragma unroll
    for (int cc = 0; cc < DC; ++cc) kf[cc] = *reinterpret_cast<const uint4*>(sk + (((2 * cc + half) ^ Ring::kswz(srow)) * 16));
  };
  // stage of the range's tile t0 + i is i % NS
  if (nt > 0) {
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) ring.copy(t0 + t, t);
    vmcnt_wait<Ring::PER_WAVE * (NS - 2)>();
    lds_hand_over();
    if (tail_tile == t0) {
      Ring::zero_tail(lds, 0, tail_tile, a.kv_total, tid);
      lds_barrier();
    }
    load_kf(0);
  }
#pragma unroll
  for (int cc = 0; cc < DC; ++cc) settle(qf[cc]);
  for (int i = 0; i < nt; ++i) {
    const int kt = t0 + i;
    const char* sb = lds + (i % NS) * SB;
    // (1) S^T = K Q^T for 32 keys (rows permuted) x this wave's 32 queries
    floatx16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[0]),
                                                         __builtin_bit_cast(bf16x8_t, qf[0]), negm, 0, 0, 0);
#pragma unroll
    for (int cc = 1; cc < DC; ++cc)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[cc]), __builtin_bit_cast(bf16x8_t, qf[cc]), s,
                                                  0, 0, 0);
    // (2) value fragments of this tile
    uint4 vf[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int row = db * 32 + l32;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        vf[db][j] = *reinterpret_cast<const uint4*>(sb + KB + row * 64 + (((2 * j + half) ^ Ring::vswz(row)) * 16));
    }
    // (3) hand-over: this wave's copies of tile kt+1 have landed, then everyone's
    vmcnt_wait<Ring::PER_WAVE * (NS - 3)>();
    lds_hand_over();
    if (kt + 1 == tail_tile) {
      Ring::zero_tail(lds, (i + 1) % NS, tail_tile, a.kv_total, tid);
      lds_barrier();
    }
    // (4) request tile kt+NS-1 into the stage of tile kt-1; (5) next tile's key fragments
    ring.copy(kt + NS - 1, (i + NS - 1) % NS);
    load_kf((i + 1) % NS);
    // (6) softmax; register e of s holds key kt*32 + 16 (e / 8) + 8 half + (e % 8)
    const int key0 = kt * AT3_BKV;
    if (key0 + AT3_BKV > it.wave_lim) mask_tile(s, key0, half, it.my_lim);
    {
      // lazy reference: raised only when some query of the wave needs it (rare after the first tile)
      const float tm = tile_max_rel(s);
      if (__any(tm > thr)) {
        const float off = m_ref == -INFINITY ? 0.f : m_ref;                 // what negm subtracted
        const float m_new = m_ref == -INFINITY ? tm : fmaxf(m_ref, off + tm);
        const float up = m_new == -INFINITY ? 0.f : m_new - off;
        if (m_ref != -INFINITY && m_new > m_ref) {
          const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] -= up;
        m_ref = m_new;
        thr = m_new == -INFINITY ? -INFINITY : 8.f;
        const float nm = m_new == -INFINITY ? 0.f : -m_new;
#pragma unroll
        for (int e = 0; e < 16; ++e) negm[e] = nm;
      }
    }
    uint4 pf[2];
    {
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) w[e >> 1] = pack2_bf16(__builtin_amdgcn_exp2f(s[e]), __builtin_amdgcn_exp2f(s[e + 1]));
      // row sum of exactly the bf16 weights the value product uses: dot products with ones
      const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
#pragma unroll
      for (int k = 0; k < 8; ++k) l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[k]), one, l_run, false);
      pf[0] = make_uint4(w[0], w[1], w[2], w[3]);
      pf[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
    // (7) O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[db][j]),
                                                         __builtin_bit_cast(bf16x8_t, pf[j]), o[db], 0, 0, 0);
  }
  vmcnt_wait<0>();
  lds_barrier();
  if (a.kv_splits == 1) {
    store_output<D, NW>(smem, o, l_run, a, it, wave, lane);
  } else {   // unnormalised partial of this key range: accumulators (float4 q of lane l at (q*64 + l)*4),
             // then the reference max and the row-sum share of each lane
    float* dst = a.part + ((long)(it.item * a.kv_splits + it.split) * NW + wave) * AT3_PART;
#pragma unroll
    for (int q = 0; q < DB * 4; ++q)
      reinterpret_cast<float4*>(dst)[q * 64 + lane] =
          make_float4(o[q >> 2][4 * (q & 3)], o[q >> 2][4 * (q & 3) + 1], o[q >> 2][4 * (q & 3) + 2], o[q >> 2][4 * (q & 3) + 3]);
    dst[64 * 64 + lane] = m_ref;
    dst[65 * 64 + lane] = l_run;
  }
}

// Two key ranges inside one workgroup: NW query waves x 2 (waves NW .. 2 NW - 1 take the upper
// half of the block's key tiles, one tile more when the count is odd). With NW = 5 the ten waves sit
// three, three, two and two on the SIMDs, so the busiest SIMD issues three half-length chains (66
// tile steps at 44 tiles) instead of two full ones (88). Three waves per SIMD leave 168 registers per
// lane, so the block's query fragments (pre-scaled as in attn3_kernel) live in LDS, fragment-major,
// and each tile reads them with its key fragments in two bounded halves. Each key half streams its
// tiles through its own three-stage ring with attn3_kernel's copy / hand-over protocol; the rings
// share the workgroup's barriers, so every wave runs the same number of loop steps (a half that has
// run out of tiles skips the compute). At the end the upper half publishes its accumulators,
// reference and row-sum shares in LDS and the lower half merges them in a fixed order (lower, then
// upper: deterministic), normalises and stores. Every block must hold at least two key tiles (the
// launcher checks the first query block, whose limit is the least).
template <int D, int NS, int NW>
__global__ void __launch_bounds__(2 * NW * 64) attn3h_kernel(AttnArgs a) {
  using Ring = KvRing<D, NS, NW>;
  constexpr int SB = Ring::SB, DC = D / 16, DB = D / 32;
  constexpr int SROW = D + 8;
  constexpr int RINGS = 2 * NS * SB;
  constexpr int QBYTES = NW * DC * 64 * 16;                  // query fragments of the block
  constexpr int PART_ACC = DB * 4 * 64;                      // float4 accumulators of one wave's share
  constexpr int PART_BYTES = NW * (PART_ACC * 16 + 2 * 64 * 4);
  static_assert(D == 128, "ring, partials and output staging are sized for 128-wide heads");
  static_assert(NS >= 3, "the hand-over waits for the copies issued one tile earlier");
  static_assert(PART_BYTES + NW * 32 * SROW * 2 <= RINGS + QBYTES, "partials and output staging fit");
  __shared__ __attribute__((aligned(1024))) uint4 smem[(RINGS + QBYTES) / 16];
  char* lds = reinterpret_cast<char*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave >= NW ? 1 : 0;   // key half (wave-uniform)
  const int qw = wave - kh * NW;       // query wave inside the block
  const int half = lane >> 5, l32 = lane & 31;
  const AttnItem<NW> it(a, qw, l32, 1);
  if (!it.valid) return;   // workgroup-uniform
  const int nh = it.n_tiles / 2;
  const int t0 = kh ? nh : 0, t1 = kh ? it.n_tiles : nh;
  const int nt = t1 - t0, n_iter = it.n_tiles - nh;   // the upper half holds the odd tile
  char* rl = lds + kh * NS * SB;
  const Ring ring(a, it.bh, rl, qw, lane, t1);
  const int tail_tile = (a.kv_total % AT3_BKV) ? a.kv_total / AT3_BKV : -1;
  const int tail0 = tail_tile >= 0 && tail_tile < nh ? tail_tile : -1;
  const int tail1 = tail_tile >= nh && tail_tile < it.n_tiles ? tail_tile - nh : -1;
  const int my_tail = kh ? tail1 : tail0;
  const uint4* qlds = reinterpret_cast<const uint4*>(lds + RINGS) + qw * DC * 64 + lane;

  if (!kh) {   // the lower half stages the block's pre-scaled query fragments
    uint4 qf[DC];
    load_q_frags<D, NW>(a, it, half, qf);
    uint4* qd = reinterpret_cast<uint4*>(lds + RINGS) + qw * DC * 64 + lane;
#pragma unroll
    for (int cc = 0; cc < DC; ++cc) qd[cc * 64] = scale_bf16x8(qf[cc], a.scale_log2);
  }
  floatx16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = floatx16{};
  float m_ref = -INFINITY, l_run = 0.f, thr = -INFINITY;
  floatx16 negm = floatx16{};

  const int srow = swap_bits_2_3(l32);
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) ring.copy(t0 + t, t);
  vmcnt_wait<Ring::PER_WAVE * (NS - 2)>();
  lds_barrier();   // the copies of each half's first tile and the query fragments are visible
  if (my_tail == 0) Ring::zero_tail(rl, 0, tail_tile, a.kv_total, qw * 64 + lane);
  if (tail0 == 0 || tail1 == 0) lds_barrier();
  for (int i = 0; i < n_iter; ++i) {
    const int kt = t0 + i;
    const bool act = i < nt;   // wave-uniform: only the lower half can run out, one step early
    const char* sb = rl + (i % NS) * SB;
    const char* sk = sb + srow * (D * 2);
    floatx16 s = negm;
    if (act) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        uint4 kf[DC / 2], qf[DC / 2];
#pragma unroll
        for (int c2 = 0; c2 < DC / 2; ++c2) {
          const int cc = hb * (DC / 2) + c2;
          kf[c2] = *reinterpret_cast<const uint4*>(sk + (((2 * cc + half) ^ Ring::kswz(srow)) * 16));
          qf[c2] = qlds[cc * 64];
        }
#pragma unroll
        for (int c2 = 0; c2 < DC / 2; ++c2)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[c2]), __builtin_bit_cast(bf16x8_t, qf[c2]),
                                                      s, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    vmcnt_wait<Ring::PER_WAVE * (NS - 3)>();
    lds_hand_over();
    if (i + 1 == my_tail) Ring::zero_tail(rl, (i + 1) % NS, tail_tile, a.kv_total, qw * 64 + lane);
    if (i + 1 == tail0 || i + 1 == tail1) lds_barrier();
    ring.copy(kt + NS - 1, (i + NS - 1) % NS);
    if (act) {
      uint4 vf[DB][2];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = db * 32 + l32;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          vf[db][j] = *reinterpret_cast<const uint4*>(sb + Ring::KB + row * 64 + (((2 * j + half) ^ Ring::vswz(row)) * 16));
      }
      const int key0 = kt * AT3_BKV;
      if (key0 + AT3_BKV > it.wave_lim) mask_tile(s, key0, half, it.my_lim);
      {
        const float tm = tile_max_rel(s);
        if (__any(tm > thr)) {
          const float off = m_ref == -INFINITY ? 0.f : m_ref;
          const float m_new = m_ref == -INFINITY ? tm : fmaxf(m_ref, off + tm);
          const float up = m_new == -INFINITY ? 0.f : m_new - off;
          if (m_ref != -INFINITY && m_new > m_ref) {
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
              for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) s[e] -= up;
          m_ref = m_new;
          thr = m_new == -INFINITY ? -INFINITY : 8.f;
          const float nm = m_new == -INFINITY ? 0.f : -m_new;
#pragma unroll
          for (int e = 0; e < 16; ++e) negm[e] = nm;
        }
      }
      uint4 pf[2];
      {
        uint32_t w[8];
#pragma unroll
        for (int e = 0; e < 16; e += 2) w[e >> 1] = pack2_bf16(__builtin_amdgcn_exp2f(s[e]), __builtin_amdgcn_exp2f(s[e + 1]));
        const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
#pragma unroll
        for (int k = 0; k < 8; ++k) l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[k]), one, l_run, false);
        pf[0] = make_uint4(w[0], w[1], w[2], w[3]);
        pf[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[db][j]),
                                                           __builtin_bit_cast(bf16x8_t, pf[j]), o[db], 0, 0, 0);
    }
  }
  vmcnt_wait<0>();
  lds_barrier();
  // the upper half publishes (accumulator float4 q of lane l at q * 64 + l), the lower half merges
  float4* pacc = reinterpret_cast<float4*>(lds) + qw * PART_ACC;
  float* pml = reinterpret_cast<float*>(lds + NW * PART_ACC * 16) + qw * 128;
  if (kh) {
#pragma unroll
    for (int q = 0; q < DB * 4; ++q)
      pacc[q * 64 + lane] = make_float4(o[q >> 2][4 * (q & 3)], o[q >> 2][4 * (q & 3) + 1], o[q >> 2][4 * (q & 3) + 2],
                                        o[q >> 2][4 * (q & 3) + 3]);
    pml[lane] = m_ref;
    pml[64 + lane] = l_run;
  }
  lds_barrier();
  bf16_t* stage = reinterpret_cast<bf16_t*>(lds + PART_BYTES) + qw * 32 * SROW;
  if (!kh) {
    const float m1 = pml[lane], l1 = pml[64 + lane];
    const float mx = fmaxf(m_ref, m1);
    const float f0 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mx);
    const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mx);
    const float l = f0 * l_run + f1 * l1;
    const float l_tot = l + __shfl_xor(l, 32, 64);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int q = 0; q < DB * 4; ++q) {
      const float4 u = pacc[q * 64 + lane];
      const int db = q >> 2, e = 4 * (q & 3);
      stage[l32 * SROW + db * 32 + acc_row(e, lane)] = f32_to_bf16((f0 * o[db][e] + f1 * u.x) * inv);
      stage[l32 * SROW + db * 32 + acc_row(e + 1, lane)] = f32_to_bf16((f0 * o[db][e + 1] + f1 * u.y) * inv);
      stage[l32 * SROW + db * 32 + acc_row(e + 2, lane)] = f32_to_bf16((f0 * o[db][e + 2] + f1 * u.z) * inv);
      stage[l32 * SROW + db * 32 + acc_row(e + 3, lane)] = f32_to_bf16((f0 * o[db][e + 3] + f1 * u.w) * inv);
    }
  }
  lds_barrier();
  if (!kh) {
    constexpr int ROW_UNITS = D / 8;
    bf16_t* O = reinterpret_cast<bf16_t*>(a.O);
    for (int u = lane; u < 32 * ROW_UNITS; u += 64) {
      const int r = u / ROW_UNITS, cu = u % ROW_UNITS;
      const int qq = it.qblk + qw * 32 + r;
      if (qq < a.Lq_total)
        *reinterpret_cast<uint4*>(O + ((long)it.b * a.Lq_total + qq) * ((long)a.H * D) + (long)it.h * D + cu * 8) =
            reinterpret_cast<const uint4*>(stage + r * SROW)[cu];
    }
  }
}

// Merge of the key-split partials of one query block (one workgroup): every lane combines the
// values it held in each range, p-weighted by 2^(m_s - M) with M the largest reference, in range
// order (deterministic), then normalises and stores like the unsplit kernel. A range with no
// visible key for a query (reference -inf) contributes nothing.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64) attn_merge_kernel(AttnArgs a) {
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(16))) uint4 smem[NW * 32 * (D + 8) * 2 / 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const AttnItem<NW> it = AttnItem<NW>::block(a, (int)blockIdx.x, wave, lane & 31);
  const int S = a.kv_splits;
  const float* base = a.part + ((long)it.item * S * NW + wave) * AT3_PART;
  constexpr long SPLIT = (long)NW * AT3_PART;
  float m = -INFINITY;
  for (int sp = 0; sp < S; ++sp) m = fmaxf(m, base[sp * SPLIT + 64 * 64 + lane]);
  floatx16 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = floatx16{};
  float l = 0.f;
  for (int sp = 0; sp < S; ++sp) {
    const float* p = base + sp * SPLIT;
    float4 v[DB * 4];   // all of the range's values requested before any is used
#pragma unroll
    for (int q = 0; q < DB * 4; ++q) v[q] = reinterpret_cast<const float4*>(p)[q * 64 + lane];
    const float ms = p[64 * 64 + lane], ls = p[65 * 64 + lane];
    const float f = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - m);
    l += f * ls;
#pragma unroll
    for (int q = 0; q < DB * 4; ++q) {
      floatx16& acc = o[q >> 2];
      const int e = 4 * (q & 3);
      acc[e] += f * v[q].x;
      acc[e + 1] += f * v[q].y;
      acc[e + 2] += f * v[q].z;
      acc[e + 3] += f * v[q].w;
    }
  }
  store_output<D, NW>(smem, o, l, a, it, wave, lane);
}

// a.kv_splits ranges per query block; above one, the merge kernel follows
template <int D, int NS = 4, int NW = AT3_NW>
static hipError_t launch_attn3(const AttnArgs& a, hipStream_t s) {
  const int blocks = ((a.Lq_total + 32 * NW - 1) / (32 * NW)) * a.H * a.br;
  const int units = blocks * a.kv_splits;
  hipLaunchKernelGGL((attn3_kernel<D, NS, NW>), dim3(8 * ((units + 7) / 8)), dim3(NW * 64), 0, s, a);
  if (a.kv_splits > 1) hipLaunchKernelGGL((attn_merge_kernel<D, NW>), dim3(blocks), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

// Five query waves x two key halves (ten waves per workgroup), three-stage rings.
static hipError_t launch_attn3h(const AttnArgs& a, hipStream_t s) {
  const int blocks = ((a.Lq_total + 159) / 160) * a.H * a.br;
  hipLaunchKernelGGL((attn3h_kernel<128, 3, 5>), dim3(8 * ((blocks + 7) / 8)), dim3(640), 0, s, a);
  return hipGetLastError();
}

// Key split (flash-decoding style): only when the query blocks fill fewer than half of the 256 CUs
// and every range keeps at least four tiles; ranges up to the CU count, at most eight.
int attn_kv_splits(int Lq_total, int H, int br, int kv_total) {
  const int blocks = (Lq_total + 32 * AT3_NW - 1) / (32 * AT3_NW) * H * br;
  const int n_tiles = (kv_total + AT3_BKV - 1) / AT3_BKV;
  if (blocks <= 0 || blocks >= 128 || n_tiles < 8) return 1;
  const int sp = std::min(std::min(8, (256 + blocks - 1) / blocks), n_tiles / 4);
  return sp >= 2 ? sp : 1;
}

long attn_split_floats(int Lq_total, int H, int br, int kv_total) {
  const int sp = attn_kv_splits(Lq_total, H, br, kv_total);
  if (sp == 1) return 0;
  const long blocks = (Lq_total + 32 * AT3_NW - 1) / (32 * AT3_NW) * (long)H * br;
  return blocks * sp * AT3_NW * AT3_PART;
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
    // the copy kernel reads whole 32-key tiles of every value row: rows must hold them, and the
    // 32-bit buffer offsets must cover the head's block
    const long tiles_end = ((long)a.kv_total + 31) / 32 * 32;
    const bool copy_ok = a.v_stride >= tiles_end && a.v_stride % 8 == 0 &&
                         (long)a.d * a.v_stride * 2 < (1L << 31) && (long)a.kv_total * a.d * 2 < (1L << 31) &&
                         reinterpret_cast<uintptr_t>(a.K) % 16 == 0 && reinterpret_cast<uintptr_t>(a.Vt) % 16 == 0 &&
                         (a.k_bh_stride * 2) % 16 == 0 && (a.v_bh_stride * 2) % 16 == 0;
    AttnArgs b = a;
    b.kv_splits = attn_kv_splits(a.Lq_total, a.H, a.br, a.kv_total);
    if (b.kv_splits > 1 && (!a.part || a.part_elems < attn_split_floats(a.Lq_total, a.H, a.br, a.kv_total)))
      b.kv_splits = 1;   // no scratch for the partials: one range per block
    const long heads = (long)a.H * a.br;
    // five waves (160 queries) per block when four-wave blocks would overflow the 256 CUs and
    // five-wave blocks fit them in one round (e.g. 2 x 40 heads x 464 queries: 320 -> 240 blocks)
    const bool five = b.kv_splits == 1 && (a.Lq_total + 127) / 128 * heads > 256 && (a.Lq_total + 159) / 160 * heads <= 256;
    // the two-half kernel needs two key tiles in every block; the first block's limit is the least
    const bool halves = ((long)attn_limit(a, std::min(160, a.Lq_total) - 1) + AT3_BKV - 1) / AT3_BKV >= 2;
    if (copy_ok && a.d == 128 && five && halves) return launch_attn3h(b, s);
    if (copy_ok && a.d == 128 && five) return launch_attn3<128, 4, 5>(b, s);
    if (copy_ok && a.d == 128) return launch_attn3<128>(b, s);
    if (copy_ok && a.d == 64) return launch_attn3<64>(b, s);
    if (a.d == 128) return launch_t<bf16_t, 128>(a, s);
    if (a.d == 64) return launch_t<bf16_t, 64>(a, s);
  } else {
    if (a.d == 128) return launch_t<float, 128>(a, s);
    if (a.d == 64) return launch_t<float, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace wam
