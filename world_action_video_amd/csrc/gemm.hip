// Tiled MFMA GEMM for the linear layers of the DiT block: C = A W^T with fused epilogues.
//
// A [M][K] and W [N][K] are both k-contiguous, so every operand fragment is one (bf16) or two
// (fp32) 16-byte LDS reads. A workgroup is 4 waves (256 threads); each wave owns a WM x WN
// sub-tile built from 32x32 MFMA blocks. K is consumed in 128-byte tile rows (64 bf16 / 32 fp32),
// staged global -> registers -> LDS with two LDS buffers so the loads of tile k+1 overlap the
// MFMAs of tile k (one barrier per k-tile). LDS rows are 8 units of 16 bytes, XOR-swizzled by
// ((row / 2) mod 8): a 16-lane pass of a fragment read touches 16 consecutive rows at one logical
// unit, and pairs of rows differ in their half of a 256-byte bank line, so the swizzle must spread
// the 8 row pairs over the 8 units to keep the pass free of bank conflicts.
//
// Tiles are assigned XCD-aware: workgroup b runs on XCD b mod 8, and each XCD receives one
// contiguous range of tiles ordered M-fastest, so the workgroups that share a W tile (the
// streamed operand) share one XCD's L2.
#include "common.h"
#include "kernels.h"
#include <type_traits>

namespace wam {

template <typename T, int BM, int BN, int WM, int WN, int NW, int EPI>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
gemm_kernel(GemmArgs g) {
  constexpr int NT = NW * 64;
  constexpr int UNITS = 8;                 // 16-byte units per LDS tile row (128 bytes)
  constexpr int EPU = 16 / sizeof(T);      // elements per unit
  constexpr int BK = UNITS * EPU;          // k per tile: 64 (bf16) or 32 (fp32)
  constexpr int NWN = BN / WN;
  static_assert((BM / WM) * NWN == NW, "wave grid must cover the tile");
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_PER_T = BM * UNITS / NT, B_PER_T = BN * UNITS / NT;
  static_assert(A_PER_T * NT == BM * UNITS && B_PER_T * NT == BN * UNITS, "tile loads split evenly");
  static_assert((BK / 16) % 2 == 0, "an even number of k16 chunks per tile keeps the fragment sets aligned");
  static_assert((NT / UNITS) % 16 == 0, "every load of a thread keeps the same swizzle phase");
  constexpr int UPF = 8 / EPU;             // units per fragment: 1 (bf16) or 2 (fp32)
  constexpr int CHUNKS = BK / 16;
  __shared__ uint4 smem[2][(BM + BN) * UNITS];

  // ---- XCD-aware tile assignment
  const int Mt = (g.M + BM - 1) / BM, Nt = (g.N + BN - 1) / BN;
  const int T_all = Mt * Nt;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int per = T_all >> 3, rem = T_all & 7;
  const int cnt = per + (xcd < rem ? 1 : 0);
  if (kx >= cnt) return;
  const int tile = xcd * per + (xcd < rem ? xcd : rem) + kx;
  const int m0 = (tile % Mt) * BM, n0 = (tile / Mt) * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int half = lane >> 5, l32 = lane & 31;
  const int KT = g.K / BK;

  // Buffer resources over the whole operands: rows at or past M (N) fall outside num_records and
  // read as zero, so ragged tiles need no branches; those rows are never stored.
  const __amdgpu_buffer_rsrc_t ra_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.A), (short)0,
                                                                       (int)((long)g.M * g.lda * sizeof(T)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.W), (short)0,
                                                                       (int)((long)g.N * g.ldw * sizeof(T)), 0x00020000);
  // per-thread byte offsets of its 16-byte units (row r = tid/8 + i*NT/8, unit u = tid%8)
  const int lrow = tid >> 3, lunit = tid & 7;
  int offa[A_PER_T], offw[B_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) offa[i] = (int)(((long)(m0 + lrow + i * (NT / 8)) * g.lda + lunit * EPU) * sizeof(T));
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) offw[i] = (int)(((long)(n0 + lrow + i * (NT / 8)) * g.ldw + lunit * EPU) * sizeof(T));
  // every unit of this thread lands in the same swizzled column: unit ^ ((row / 2) mod 8)
  const int sbase = lrow * UNITS + (lunit ^ ((lrow >> 1) & 7));

  uint4 ra[A_PER_T], rb[B_PER_T];
  auto gload = [&](int kt) {
    const int koff = kt * BK * (int)sizeof(T);
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i)
      ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra_, offa[i], koff, 0));
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i)
      rb[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw_, offw[i], koff, 0));
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) smem[st][sbase + i * (NT / 8) * UNITS] = ra[i];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) smem[st][BM * UNITS + sbase + i * (NT / 8) * UNITS] = rb[i];
  };
  // fragment loads: rows of this wave's sub-tile; the swizzle phase of a row is (l32 / 2) mod 8
  auto fload = [&](const uint4* sa, const uint4* sb, int c, Frag<T>* fa, Frag<T>* fb) {
    const int u0 = (c * 16 + half * 8) / EPU;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * WM + i * 32 + l32;
      uint4* dst = reinterpret_cast<uint4*>(&fa[i]);
#pragma unroll
      for (int q = 0; q < UPF; ++q) dst[q] = sa[row * UNITS + ((u0 + q) ^ ((l32 >> 1) & 7))];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = wn * WN + j * 32 + l32;
      uint4* dst = reinterpret_cast<uint4*>(&fb[j]);
#pragma unroll
      for (int q = 0; q < UPF; ++q) dst[q] = sb[row * UNITS + ((u0 + q) ^ ((l32 >> 1) & 7))];
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx16{};

  // Pipeline: tile kt+1 is fetched into registers while tile kt computes; before the last chunk of
  // tile kt the registers go to the other LDS buffer and the workgroup synchronises, so the first
  // fragments of tile kt+1 are read while the last chunk of tile kt is still in the MFMA pipe.
  // The buffer written during tile kt was last read during tile kt-1, whose reads all completed
  // before the previous barrier.
  gload(0);
  sstore(0);
  __syncthreads();
  Frag<T> fa[2][TM], fb[2][TN];
  fload(smem[0], smem[0] + BM * UNITS, 0, fa[0], fb[0]);
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more) gload(kt + 1);
    const uint4* sa = smem[cur];
    const uint4* sb = sa + BM * UNITS;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const int fcur = c & 1;      // CHUNKS is even: chunk 0 of every tile uses fragment set 0
      if (c + 1 < CHUNKS) {
        fload(sa, sb, c + 1, fa[fcur ^ 1], fb[fcur ^ 1]);
      } else if (more) {
        sstore(cur ^ 1);
        __syncthreads();
        fload(smem[cur ^ 1], smem[cur ^ 1] + BM * UNITS, 0, fa[fcur ^ 1], fb[fcur ^ 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mfma_k16(acc[i][j], fa[fcur][i], fb[fcur][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue
  if constexpr (EPI == EPI_RESID || EPI == EPI_RESID_GATED) {
    // Residual updates read H (and the gate) before writing it: issue all loads of one 32-row block
    // first, then update, so the load latency is paid once per block rather than once per element.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float hv[16][TN], gv[16][TN];
      long hoff[16];
      bool ok[16];
      // (row within branch, chunk, position in chunk) of the block's first row: two divisions per
      // 32-row block; the rows below it advance with at most one wrap each (32 < chunk length).
      const int row0 = m0 + wm * WM + i * 32;
      int rb0 = 0, ch0 = 0, loc0 = 0;
      if constexpr (EPI == EPI_RESID_GATED) {
        rb0 = row0 % g.rm.rows_per_branch;
        ch0 = rb0 / g.rm.Lq;
        loc0 = rb0 - ch0 * g.rm.Lq;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = acc_row(r, lane);
        const int row = row0 + off;
        ok[r] = row < g.M;
        hoff[r] = (long)row * g.ldh;
        const float* grow = nullptr;
        if constexpr (EPI == EPI_RESID_GATED) {
          int rb = rb0 + off, ch = ch0, loc = loc0 + off;
          if (rb >= g.rm.rows_per_branch) { rb -= g.rm.rows_per_branch; ch = 0; loc = rb; }
          else if (loc >= g.rm.Lq) { loc -= g.rm.Lq; ++ch; }
          const int grp = loc < g.rm.Lv ? 0 : 1;
          grow = g.e6 + ((long)(ch * 2 + grp) * 6 + g.gate_idx) * g.D;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * WN + j * 32 + l32;
          const bool v = ok[r] && col < g.N;
          hv[r][j] = v ? g.H[hoff[r] + col] : 0.f;
          if constexpr (EPI == EPI_RESID_GATED) gv[r][j] = v ? grow[col] + g.mod[g.gate_idx * g.D + col] : 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn * WN + j * 32 + l32;
        if (col >= g.N) continue;
        const float bias = g.bias ? g.bias[col] : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (!ok[r]) continue;
          const float v = acc[i][j][r] + bias;
          if constexpr (EPI == EPI_RESID_GATED) g.H[hoff[r] + col] = hv[r][j] + gv[r][j] * v;
          else g.H[hoff[r] + col] = hv[r][j] + v;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn * WN + j * 32 + l32;
    if (col >= g.N) continue;
    const float bias = g.bias ? g.bias[col] : 0.f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + i * 32 + acc_row(r, lane);
        if (row >= g.M) continue;
        const float v = acc[i][j][r] + bias;
        if constexpr (EPI == EPI_STORE) {
          Elem<T>::store(reinterpret_cast<T*>(g.C) + (long)row * g.ldc + col, v);
        } else if constexpr (EPI == EPI_SWIGLU) {
          // gate column 2j in an even lane, its up column 2j+1 in the next lane (N even: both or neither
          // lane of a pair is past the edge, and both hold the same row)
          const float up = __shfl_xor(v, 1, 64);
          if (!(l32 & 1)) Elem<T>::store(reinterpret_cast<T*>(g.C) + (long)row * g.ldc + col / 2, silu_f(v) * up);
        } else if constexpr (EPI == EPI_GELU) {
          Elem<T>::store(reinterpret_cast<T*>(g.C) + (long)row * g.ldc + col, gelu_tanh_f(v));
        } else if constexpr (EPI == EPI_ROWSEL_F32) {
          const int b = row / g.rm.rows_per_branch, rb_ = row % g.rm.rows_per_branch;
          const int ch = rb_ / g.rm.Lq, loc = rb_ % g.rm.Lq;
          const int La = g.rm.Lq - g.rm.Lv;
          const int nch = g.rm.rows_per_branch / g.rm.Lq;
          if (g.sel_group == 0 && loc < g.rm.Lv) {
            reinterpret_cast<float*>(g.C)[((long)b * nch * g.rm.Lv + ch * g.rm.Lv + loc) * g.ldc + col] = v;
          } else if (g.sel_group == 1 && loc >= g.rm.Lv) {
            reinterpret_cast<float*>(g.C)[((long)b * nch * La + ch * La + (loc - g.rm.Lv)) * g.ldc + col] = v;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// 256x256 bf16 tile on 4 waves (one per SIMD), 128x128 per wave (4x4 MFMA blocks): half the LDS
// fragment traffic per MFMA of the 8-wave tile, which is what bounds the 8-wave kernel. Global data
// for tile kt+3 is fetched while tile kt computes (two register sets), tile kt+1 is written to the
// other LDS buffer one quarter per k16 chunk between the MFMA groups, and the workgroup synchronises
// before the last chunk so the next tile's first fragments load under it.
// Split-K: with `splits` > 1 each workgroup covers one contiguous range of k-tiles and writes fp32
// partial products to g.part[split][M][N]; splitk_reduce_kernel sums them in split order (fixed,
// deterministic) and applies the epilogue.
// ------------------------------------------------------------------------------------------------
static constexpr int EPI_PARTIAL = 16;   // internal: partial products of one split (fp32, or bf16 with part_bf16)

// Accumulators of a 32 TM x 32 TN wave tile in the transposed layout the epilogue reads (lane
// (l32, half) holds columns wcol + 4 half + 32 j + 8 g + 0..3 of block (i, j) in acc[i][j][4 g ..]).
// They start at zero, except for split 0 of a product whose partials are stored in bf16: those start
// at the bias, so the stored partial carries it and the finish adds none.
template <int EPI, int TM, int TN>
__device__ __forceinline__ void g4_acc_init(floatx16 (&acc)[TM][TN], const GemmArgs& g, int sp, int wcol, int half) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx16{};
  if constexpr (EPI == EPI_PARTIAL) {
    if (g.part_bf16 && sp == 0 && g.bias) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = wcol + 4 * half + 32 * j + 8 * gq;
          const float4 b = n < g.N ? *reinterpret_cast<const float4*>(g.bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            acc[i][j][4 * gq] = b.x; acc[i][j][4 * gq + 1] = b.y; acc[i][j][4 * gq + 2] = b.z; acc[i][j][4 * gq + 3] = b.w;
          }
        }
    }
  }
}

// Epilogue of the four-wave tiles (bf16 and MX operands alike): a wave's TM x TN blocks of 32 x 32 whose first row / column are wrow / wcol.
template <int EPI, int TM, int TN>
__device__ __forceinline__ void g4_epilogue_t(const GemmArgs& g, const floatx16 (&acc)[TM][TN], int wrow, int wcol,
                                              int sp, int l32, int half) {
  // ---- lane (l32, half) holds, for block (i, j), output row m = mb + 32 i and columns
  // nb + 32 j + 8 g + 0..3 in acc[i][j][4 g .. 4 g + 3] (g = 0..3). N % 4 == 0 (checked at launch), so
  // a run is either wholly inside the matrix or wholly outside.
  const int mb = wrow + l32, nb = wcol + 4 * half;
  auto run = [&](int i, int j, int gq) {
    return make_float4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
  };
  if constexpr (EPI == EPI_PARTIAL) {
    const long base = (long)sp * g.M * g.N;
    float* part = g.part + base;
    bf16_t* part16 = reinterpret_cast<bf16_t*>(g.part) + base;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mb + 32 * i;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = nb + 32 * j + 8 * gq;
          if (n >= g.N) continue;
          const float4 v = run(i, j, gq);
          if (g.part_bf16)
            *reinterpret_cast<uint2*>(part16 + (long)m * g.N + n) = make_uint2(pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w));
          else
            *reinterpret_cast<float4*>(part + (long)m * g.N + n) = v;
        }
    }
    return;
  }
  float4 bias[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int n = nb + 32 * j + 8 * gq;
      bias[j][gq] = (g.bias && n < g.N) ? *reinterpret_cast<const float4*>(g.bias + n) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  if constexpr (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mb + 32 * i;
      if (m >= g.M) continue;
      bf16_t* crow = reinterpret_cast<bf16_t*>(g.C) + (long)m * g.ldc;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = nb + 32 * j + 8 * gq;
          if (n >= g.N) continue;
          float4 v = run(i, j, gq);
          const float4 b = bias[j][gq];
          v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
          if constexpr (EPI == EPI_SWIGLU) {   // columns (n, n+1), (n+2, n+3): two outputs at n / 2
            *reinterpret_cast<uint32_t*>(crow + n / 2) = pack2_bf16(silu_f(v.x) * v.y, silu_f(v.z) * v.w);
            continue;
          }
          if constexpr (EPI == EPI_GELU) {
            v.x = gelu_tanh_f(v.x); v.y = gelu_tanh_f(v.y); v.z = gelu_tanh_f(v.z); v.w = gelu_tanh_f(v.w);
          }
          *reinterpret_cast<uint2*>(crow + n) = make_uint2(pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w));
        }
    }
  } else {   // EPI_RESID, EPI_RESID_GATED: fp32 residual rows, read-modify-write per run of four
    float4 gm[TN][4];
    if constexpr (EPI == EPI_RESID_GATED) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = nb + 32 * j + 8 * gq;
          gm[j][gq] = n < g.N ? *reinterpret_cast<const float4*>(g.mod + (long)g.gate_idx * g.D + n)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mb + 32 * i;
      if (m >= g.M) continue;
      float* hrow = g.H + (long)m * g.ldh;
      const float* grow = nullptr;
      if constexpr (EPI == EPI_RESID_GATED) {
        const int rb = m % g.rm.rows_per_branch;
        const int ch = rb / g.rm.Lq, grp = (rb % g.rm.Lq) < g.rm.Lv ? 0 : 1;
        grow = g.e6 + ((long)(ch * 2 + grp) * 6 + g.gate_idx) * g.D;
      }
      // per block: the four runs' loads first, then the updates
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        float4 hv[4], gv[4];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = nb + 32 * j + 8 * gq;
          const bool ok = n < g.N;
          hv[gq] = ok ? *reinterpret_cast<const float4*>(hrow + n) : make_float4(0.f, 0.f, 0.f, 0.f);
          if constexpr (EPI == EPI_RESID_GATED)
            gv[gq] = ok ? *reinterpret_cast<const float4*>(grow + n) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = nb + 32 * j + 8 * gq;
          if (n >= g.N) continue;
          float4 v = run(i, j, gq);
          const float4 b = bias[j][gq];
          v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
          float4 h = hv[gq];
          if constexpr (EPI == EPI_RESID_GATED) {
            const float4 ge = gv[gq], gmm = gm[j][gq];
            h.x += (ge.x + gmm.x) * v.x; h.y += (ge.y + gmm.y) * v.y; h.z += (ge.z + gmm.z) * v.z; h.w += (ge.w + gmm.w) * v.w;
          } else {
            h.x += v.x; h.y += v.y; h.z += v.z; h.w += v.w;
          }
          *reinterpret_cast<float4*>(hrow + n) = h;
        }
      }
    }
  }
}

template <int EPI, int TM, int TN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm4_kernel(GemmArgs g, int splits) {
  using T = bf16_t;
  // 2 x 2 waves of (32 TM) x (32 TN); BM + BN = 512 rows staged per k-tile in both shapes used
  // (256 x 256 and 192 x 320), i.e. 16 units of 16 bytes per thread, in four quarters of 4 units
  constexpr int BM = 64 * TM, BN = 64 * TN, WM = 32 * TM, WN = 32 * TN;
  constexpr int NT = 256, UNITS = 8, EPU = 8, BK = 64, CHUNKS = 4;
  constexpr int PA = BM * UNITS / NT, PW = BN * UNITS / NT, PER_T = PA + PW;   // units of A / W per thread
  constexpr int NMF = TM * TN;   // MFMAs per wave per k16 chunk
  static_assert(PER_T == 16 && NMF >= 12, "staging and schedule assume 512 tile rows and at least 12 blocks");
  // Rows are padded to 9 units (144 bytes): row r's unit u sits in bank group (r + u) mod 8, so eight
  // consecutive rows or eight units of one row never collide, and every fragment address of a chunk
  // is one per-lane base plus a compile-time offset (no per-chunk swizzle registers).
  constexpr int PITCH = UNITS + 1;
  __shared__ uint4 smem[2][(BM + BN) * PITCH];

  const int Mt = (g.M + BM - 1) / BM, Nt = (g.N + BN - 1) / BN;
  const int items = Mt * Nt * splits;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int per = items >> 3, rem = items & 7;
  if (kx >= per + (xcd < rem ? 1 : 0)) return;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + kx;
  const int mt = item % Mt, rest = item / Mt;
  const int sp = rest % splits, nt = rest / splits;
  const int m0 = mt * BM, n0 = nt * BN;
  const int KT_all = g.K / BK;
  const int kb = (int)((long)sp * KT_all / splits), ke = (int)((long)(sp + 1) * KT_all / splits);
  const int KT = ke - kb;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;

  const __amdgpu_buffer_rsrc_t ra_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.A), (short)0,
                                                                       (int)((long)g.M * g.lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.W), (short)0,
                                                                       (int)((long)g.N * g.ldw * 2), 0x00020000);
  const int lrow = tid >> 3, lunit = tid & 7;
  // unit i < PA: A rows m0 + lrow + 32 i; else W rows n0 + lrow + 32 (i - PA)
  int off[PER_T];
#pragma unroll
  for (int i = 0; i < PER_T; ++i)
    off[i] = i < PA ? (int)(((long)(m0 + lrow + i * 32) * g.lda + lunit * EPU) * 2)
                    : (int)(((long)(n0 + lrow + (i - PA) * 32) * g.ldw + lunit * EPU) * 2);
  const int sbase = lrow * PITCH + lunit;

  uint4 rg[2][PER_T];                      // [register set][unit]
  // quarter q of a tile: units 4q .. 4q+3 of the list
  auto gload_q = [&](int kt, int set, int q) {
    const int koff = (kb + min(kt, KT - 1)) * BK * 2;   // prefetches past the split re-read its last tile
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 4 * q + u;
      rg[set][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(i < PA ? ra_ : rw_, off[i], koff, 0));
    }
  };
  auto sstore_q = [&](int st, int set, int q) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 4 * q + u;
      smem[st][(i < PA ? i * 32 * PITCH : BM * PITCH + (i - PA) * 32 * PITCH) + sbase] = rg[set][i];
    }
  };
  auto fload = [&](int st, int c, uint4* fa, uint4* fb) {
    const uint4* sa = smem[st] + (wm * WM + l32) * PITCH + half;
    const uint4* sb = smem[st] + (BM + wn * WN + l32) * PITCH + half;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = sa[i * 32 * PITCH + 2 * c];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = sb[j * 32 * PITCH + 2 * c];
  };

  floatx16 acc[TM][TN];
  g4_acc_init<EPI, TM, TN>(acc, g, sp, n0 + wn * WN, half);

  // The loop body has no data-dependent branches: loads past the split's last k-tile read other
  // valid rows or fall outside the buffer range (returning zero), and stores/fragment loads into the
  // idle LDS buffer after the last tile are never consumed. This keeps both register sets in
  // registers instead of merging them through control flow.
  uint4 fa[2][TM], fb[2][TN];
#pragma unroll
  for (int q = 0; q < 4; ++q) gload_q(0, 0, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) gload_q(1, 1, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) sstore_q(0, 0, q);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) gload_q(2, 0, q);
  fload(0, 0, fa[0], fb[0]);
  __builtin_amdgcn_sched_barrier(0);   // keep the prologue's loads ahead of the first tile's

  // One k-tile from LDS buffer CUR; register set CUR^1 holds tile kt+1 and is refilled with kt+3.
  // CUR is a compile-time constant so both register sets keep fixed registers.
  // acc[i][j] holds the transposed 32x32 block (W rows x A rows): lane l then owns output row
  // m = .. + l % 32 and four runs of four consecutive columns, which the epilogue stores as vectors.
  auto mma = [&](int fc, int lo, int hi) {
#pragma unroll
    for (int q = lo; q < hi; ++q)
      acc[q / TN][q % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fb[fc][q % TN]),
                                                                    __builtin_bit_cast(bf16x8_t, fa[fc][q / TN]),
                                                                    acc[q / TN][q % TN], 0, 0, 0);
  };
  // Scheduling groups: one MFMA, then one memory instruction of the given class, so the LDS and
  // global traffic issues while the matrix core works instead of in a burst between MFMA groups.
  constexpr int SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100, SG_DS_WR = 0x200;
  constexpr int NRD = TM + TN;   // fragment reads per chunk
  auto tile = [&](int kt, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value, nset = cur ^ 1;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const int fc = c & 1;
      if (c + 1 < CHUNKS) {
        fload(cur, c + 1, fa[fc ^ 1], fb[fc ^ 1]);
        sstore_q(nset, nset, c);
        gload_q(kt + 3, nset, c);
        mma(fc, 0, NMF);
#pragma unroll
        for (int k = 0; k < NRD; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_WR, 1, 0);
        }
#pragma unroll
        for (int k = 0; k < NMF - NRD - 4; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // last chunk: eight of its MFMAs cover the tile's final LDS writes and global loads, the
        // barrier sits after them, and the rest cover the first fragment loads of the next tile
        sstore_q(nset, nset, c);
        gload_q(kt + 3, nset, c);
        mma(fc, 0, 8);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_WR, 1, 0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        fload(nset, 0, fa[fc ^ 1], fb[fc ^ 1]);
        mma(fc, 8, NMF);
#pragma unroll
        for (int k = 0; k < NMF - 8; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // The first tile is peeled: the loop is then entered after an even tile both from before it and
  // from its own end, so the wait counts the compiler derives for the loads in flight at its entry
  // match the steady state (entered from the prologue, they would wait for tile 2's loads at once).
  tile(0, std::integral_constant<int, 0>{});
  int kt = 1;
  for (; kt + 1 < KT; kt += 2) {
    tile(kt, std::integral_constant<int, 1>{});
    tile(kt + 1, std::integral_constant<int, 0>{});
  }
  if (kt < KT) tile(kt, std::integral_constant<int, 1>{});

  g4_epilogue_t<EPI, TM, TN>(g, acc, m0 + wm * WM, n0 + wn * WN, sp, l32, half);
}


// ------------------------------------------------------------------------------------------------
// 256 x 224 four-wave product: the waves stacked along M (64 rows x 224 columns each, 2 x 7 blocks of
// 32 x 32), the loads, LDS layout and pipeline of gemm4_kernel. For products whose 256-wide tiles
// leave CUs idle in their single round while 224-wide tiles still fit in one (e.g. 928 x 13824:
// 216 -> 248 workgroups, each with 7/8 of the work).
// ------------------------------------------------------------------------------------------------
template <int EPI>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm4w_kernel(GemmArgs g) {
  constexpr int BM = 256, BN = 224, WM = 64, TM = 2, TN = 7;
  constexpr int NT = 256, UNITS = 8, EPU = 8, BK = 64, CHUNKS = 4, PITCH = UNITS + 1;
  constexpr int PER_A = BM * UNITS / NT, PER_W = BN * UNITS / NT;   // 8 and 7 units per thread per tile
  __shared__ uint4 smem[2][(BM + BN) * PITCH];

  const int Mt = (g.M + BM - 1) / BM, Nt = (g.N + BN - 1) / BN;
  const int items = Mt * Nt;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int per = items >> 3, rem = items & 7;
  if (kx >= per + (xcd < rem ? 1 : 0)) return;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + kx;
  const int mt = item % Mt, nt = item / Mt;
  const int m0 = mt * BM, n0 = nt * BN;
  const int KT = g.K / BK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  const __amdgpu_buffer_rsrc_t ra_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.A), (short)0,
                                                                       (int)((long)g.M * g.lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.W), (short)0,
                                                                       (int)((long)g.N * g.ldw * 2), 0x00020000);
  const int lrow = tid >> 3, lunit = tid & 7;
  int offa[PER_A], offw[PER_W];
#pragma unroll
  for (int i = 0; i < PER_A; ++i) offa[i] = (int)(((long)(m0 + lrow + i * 32) * g.lda + lunit * EPU) * 2);
#pragma unroll
  for (int i = 0; i < PER_W; ++i) offw[i] = (int)(((long)(n0 + lrow + i * 32) * g.ldw + lunit * EPU) * 2);
  const int sbase = lrow * PITCH + lunit;

  uint4 rg[2][PER_A + PER_W];   // [register set][A units 0..7, W units 8..14]
  // quarter q of a tile: A units 2q, 2q+1 and W units 2q, 2q+1 (quarter 3 has one W unit)
  auto gload_q = [&](int kt, int set, int q) {
    const int koff = min(kt, KT - 1) * BK * 2;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * q + u;
      rg[set][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra_, offa[i], koff, 0));
      if (i < PER_W)
        rg[set][PER_A + i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw_, offw[i], koff, 0));
    }
  };
  auto sstore_q = [&](int st, int set, int q) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * q + u;
      smem[st][sbase + i * 32 * PITCH] = rg[set][i];
      if (i < PER_W) smem[st][BM * PITCH + sbase + i * 32 * PITCH] = rg[set][PER_A + i];
    }
  };
  auto fload = [&](int st, int c, uint4* fa, uint4* fb) {
    const uint4* sa = smem[st] + (wave * WM + l32) * PITCH + half;
    const uint4* sb = smem[st] + (BM + l32) * PITCH + half;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = sa[i * 32 * PITCH + 2 * c];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = sb[j * 32 * PITCH + 2 * c];
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx16{};

  uint4 fa[2][TM], fb[2][TN];
#pragma unroll
  for (int q = 0; q < 4; ++q) gload_q(0, 0, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) gload_q(1, 1, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) sstore_q(0, 0, q);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) gload_q(2, 0, q);
  fload(0, 0, fa[0], fb[0]);
  __builtin_amdgcn_sched_barrier(0);   // keep the prologue's loads ahead of the first tile's

  auto mma = [&](int fc, int lo, int hi) {
#pragma unroll
    for (int q = lo; q < hi; ++q)
      acc[q / TN][q % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fb[fc][q % TN]),
                                                                    __builtin_bit_cast(bf16x8_t, fa[fc][q / TN]),
                                                                    acc[q / TN][q % TN], 0, 0, 0);
  };
  constexpr int SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100, SG_DS_WR = 0x200;
  auto tile = [&](int kt, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value, nset = cur ^ 1;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const int fc = c & 1;
      if (c + 1 < CHUNKS) {
        fload(cur, c + 1, fa[fc ^ 1], fb[fc ^ 1]);
        sstore_q(nset, nset, c);
        gload_q(kt + 3, nset, c);
        mma(fc, 0, TM * TN);
        // 14 MFMAs: the 9 fragment reads between the first seven, then the writes and loads
#pragma unroll
        for (int k = 0; k < 5; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 2, 0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_WR, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 3, 0);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // last chunk: half of its MFMAs cover the tile's final LDS writes, the barrier sits in the
        // middle, and the other half cover the first fragment loads of the next tile
        sstore_q(nset, nset, c);
        gload_q(kt + 3, nset, c);
        mma(fc, 0, 7);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_WR, 1, 0);
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        fload(nset, 0, fa[fc ^ 1], fb[fc ^ 1]);
        mma(fc, 7, TM * TN);
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 3, 0);
#pragma unroll
        for (int k = 0; k < 6; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // The first tile is peeled: the loop is then entered after an even tile both from before it and
  // from its own end, so the wait counts the compiler derives for the loads in flight at its entry
  // match the steady state (entered from the prologue, they would wait for tile 2's loads at once).
  tile(0, std::integral_constant<int, 0>{});
  int kt = 1;
  for (; kt + 1 < KT; kt += 2) {
    tile(kt, std::integral_constant<int, 1>{});
    tile(kt + 1, std::integral_constant<int, 0>{});
  }
  if (kt < KT) tile(kt, std::integral_constant<int, 1>{});

  g4_epilogue_t<EPI, TM, TN>(g, acc, m0 + wave * WM, n0, 0, l32, half);
}

// ------------------------------------------------------------------------------------------------
// Products with fragment-packed weights. W [N][K] is stored once, ahead of the products, in the
// order the matrix instruction reads it: block (b, c) -- W rows 32 b .. 32 b + 31, k 16 c .. 16 c + 15
// -- is 64 lanes x 16 bytes, lane l holding row 32 b + l % 32 at k 16 c + 8 (l / 32) .. + 7, and the
// blocks of one 32-row band follow each other along k (so a band occupies the same 32 K * 2 bytes as
// its rows do unpacked). One wave's load of a weight fragment is then one contiguous 1 KB read.
//
// gemm4p_kernel: a tile of 32 TM rows x 128 TN columns on 4 waves side by side along N; each wave
// owns all 32 TM rows and 32 TN columns (TM x TN blocks of 32x32, v_mfma_f32_32x32x16_bf16, W block
// first as in gemm4_kernel, so the epilogues are shared). Every weight fragment is used by exactly
// one wave, which streams its own fragments from global memory straight into an 8-chunk register
// ring (two k-tiles ahead); only the activation tile is staged through LDS (global -> two register
// sets -> two LDS buffers, 144-byte padded rows, one barrier per k-tile). Per k16 chunk a CU then
// reads 4 x TM activation fragments from LDS and writes TM / 4 units per thread, against 8 reads and
// 4 writes per wave in gemm4_kernel: the LDS traffic that bounded that kernel drops by more than half,
// while the weight stream goes through the vector memory path in whole 1 KB lines.
// ------------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) pack_weight_kernel(const uint4* __restrict__ W, long ldw_units,
                                                          uint4* __restrict__ Wp, int N, int K) {
  const long total = (long)(N / 32) * (K / 16) * 64;
  const int KC = K / 16;
  for (long idx = (long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long)gridDim.x * 256) {
    const int lane = (int)(idx & 63);
    const long blk = idx >> 6;
    const int c = (int)(blk % KC), b = (int)(blk / KC);
    Wp[idx] = W[(long)(b * 32 + (lane & 31)) * ldw_units + 2 * c + (lane >> 5)];
  }
}

// bf16 outputs of gemm4p_kernel (store, GELU, bf16 split-K partials) leave through LDS: each wave
// writes one 32-row block row of its 32 TM x 32 TN tile into its own LDS rows (row-major, pitch
// 32 TN + 8 bf16), then stores it with 16 bytes per lane, consecutive lanes along a row, so a store
// instruction writes whole row segments instead of 16 bytes in each of 32 rows. When every workgroup
// finishes at once (the split products), this halves the time the output takes to drain.
// Whether a product takes this path depends on its arguments only, so all waves agree.
template <int EPI, int TM, int TN>
__device__ __forceinline__ bool g4p_staged_ok(const GemmArgs& g) {
  if constexpr (EPI == EPI_STORE || EPI == EPI_GELU)
    return g.ldc % 8 == 0 && reinterpret_cast<uintptr_t>(g.C) % 16 == 0;
  else if constexpr (EPI == EPI_PARTIAL)
    return g.part_bf16 && g.N % 8 == 0;
  else
    return false;
}

template <int EPI, int TM, int TN>
__device__ __forceinline__ void g4p_epilogue_staged(const GemmArgs& g, const floatx16 (&acc)[TM][TN], int m0, int wcol,
                                                    int sp, int wave, int lane, bf16_t* lds) {
  constexpr int WN = 32 * TN, SP = WN + 8, UPR = WN / 8;
  const int l32 = lane & 31, half = lane >> 5;
  bf16_t* stage = lds + wave * 32 * SP;
  float4 bias[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int n = wcol + 32 * j + 8 * gq + 4 * half;
      bias[j][gq] = (EPI != EPI_PARTIAL && g.bias && n < g.N) ? *reinterpret_cast<const float4*>(g.bias + n)
                                                             : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  bf16_t* out;
  long ld;
  if constexpr (EPI == EPI_PARTIAL) {
    out = reinterpret_cast<bf16_t*>(g.part) + (long)sp * g.M * g.N;
    ld = g.N;
  } else {
    out = reinterpret_cast<bf16_t*>(g.C);
    ld = g.ldc;
  }
  __syncthreads();   // every wave is done with the activation buffers the stage reuses
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float4 v = make_float4(acc[i][j][4 * gq], acc[i][j][4 * gq + 1], acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
        const float4 b = bias[j][gq];
        v.x += b.x; v.y += b.y; v.z += b.z; v.w += b.w;
        if constexpr (EPI == EPI_GELU) {
          v.x = gelu_tanh_f(v.x); v.y = gelu_tanh_f(v.y); v.z = gelu_tanh_f(v.z); v.w = gelu_tanh_f(v.w);
        }
        *reinterpret_cast<uint2*>(stage + l32 * SP + 32 * j + 8 * gq + 4 * half) =
            make_uint2(pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w));
      }
    // the wave reads back what its own lanes wrote: LDS operations of one wave complete in order
#pragma unroll
    for (int s = 0; s < (32 * UPR + 63) / 64; ++s) {
      const int u = lane + 64 * s;
      if (u < 32 * UPR) {
        const int r = u / UPR, cu = u % UPR;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + r * SP + 8 * cu);
        const int m = m0 + 32 * i + r, n = wcol + 8 * cu;
        if (m < g.M && n < g.N) *reinterpret_cast<uint4*>(out + (long)m * ld + n) = v;
      }
    }
  }
}

template <int EPI, int TM, int TN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm4p_kernel(GemmArgs g, int splits) {
  constexpr int BM = 32 * TM, WN = 32 * TN, BN = 4 * WN;
  constexpr int UNITS = 8, PITCH = UNITS + 1, BK = 64, CHUNKS = 4, RING = 8;
  constexpr int PA = BM * UNITS / 256;   // activation units (16 bytes) per thread per k-tile
  constexpr int NMF = TM * TN;           // MFMAs per wave per chunk
  static_assert(PA == TM && RING == 2 * CHUNKS, "tile staging and ring layout");
  __shared__ uint4 smem[2][BM * PITCH];

  const int Mt = (g.M + BM - 1) / BM, Nt = (g.N + BN - 1) / BN;
  const int items = Mt * Nt * splits;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int per = items >> 3, rem = items & 7;
  if (kx >= per + (xcd < rem ? 1 : 0)) return;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + kx;
  const int mt = item % Mt, rest = item / Mt;
  const int sp = rest % splits, nt = rest / splits;
  const int m0 = mt * BM, n0 = nt * BN;
  const int KT_all = g.K / BK, KC = g.K / 16;
  const int kb = (int)((long)sp * KT_all / splits), ke = (int)((long)(sp + 1) * KT_all / splits);
  const int KT = ke - kb;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;

  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.A), (short)0,
                                                                      (int)((long)g.M * g.lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.W), (short)0,
                                                                      (int)((long)g.N * g.K * 2), 0x00020000);
  // activation unit i: row m0 + lrow + 32 i, 16-byte unit lunit of the k-tile; rows past M and weight
  // bands past N lie outside the buffer ranges and read as zero
  const int lrow = tid >> 3, lunit = tid & 7;
  int aoff[PA];
#pragma unroll
  for (int i = 0; i < PA; ++i) aoff[i] = (int)(((long)(m0 + lrow + 32 * i) * g.lda + lunit * 8) * 2);
  const int sbase = lrow * PITCH + lunit;
  const int band0 = (n0 + wave * WN) / 32;
  int woff[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) woff[j] = ((band0 + j) * KC * 64 + lane) * 16;

  uint4 rg[2][PA];       // activation register sets
  uint4 fw[RING][TN];    // weight fragments of chunks c .. c + 7
  uint4 fa[2][TM];       // activation fragments, double-buffered per chunk
  auto gload_a = [&](int kt, int set, int c) {
    const int koff = (kb + min(kt, KT - 1)) * BK * 2;   // prefetches past the split re-read its last tile
#pragma unroll
    for (int i = 0; i < PA; ++i)
      if (i % CHUNKS == c)
        rg[set][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[i], koff, 0));
  };
  auto sstore_a = [&](int st, int set, int c) {
#pragma unroll
    for (int i = 0; i < PA; ++i)
      if (i % CHUNKS == c) smem[st][i * 32 * PITCH + sbase] = rg[set][i];
  };
  auto wload = [&](int slot, int kc, int j) {   // kc: chunk of this split (clamped to its last)
    const int koff = (4 * kb + min(kc, 4 * KT - 1)) * 1024;
    fw[slot][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[j], koff, 0));
  };
  auto fload = [&](int st, int c, uint4* f) {
    const uint4* sa = smem[st] + l32 * PITCH + half;
#pragma unroll
    for (int i = 0; i < TM; ++i) f[i] = sa[i * 32 * PITCH + 2 * c];
  };

  floatx16 acc[TM][TN];
  g4_acc_init<EPI, TM, TN>(acc, g, sp, n0 + wave * WN, half);

  // Prologue, in the order the loop keeps loads in flight (activation tiles 0 and 1, ring chunks
  // 0..3, activation tile 2, ring chunks 4..7), so that the waits the compiler derives at the loop's
  // entry match those of its steady state.
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) gload_a(0, 0, c);
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) gload_a(1, 1, c);
#pragma unroll
  for (int s = 0; s < RING / 2; ++s)
#pragma unroll
    for (int j = 0; j < TN; ++j) wload(s, s, j);
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) sstore_a(0, 0, c);
  __syncthreads();
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) gload_a(2, 0, c);
#pragma unroll
  for (int s = RING / 2; s < RING; ++s)
#pragma unroll
    for (int j = 0; j < TN; ++j) wload(s, s, j);
  fload(0, 0, fa[0]);
  __builtin_amdgcn_sched_barrier(0);

  auto mma_col = [&](int fc, int slot, int j) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fw[slot][j]),
                                                          __builtin_bit_cast(bf16x8_t, fa[fc][i]), acc[i][j], 0, 0, 0);
  };
  constexpr int SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100, SG_DS_WR = 0x200;
  constexpr int JB = (TN + 1) / 2;   // weight columns of the last chunk issued before the barrier
  // One k-tile: LDS buffer CUR holds tile kt; register set CUR^1 holds tile kt+1 (written to LDS
  // during this tile) and is refilled with kt+3; ring slots 4 CUR + c hold chunk 4 kt + c and are
  // refilled with the chunk eight ahead once its column's MFMAs have read them. After each MFMA one
  // memory instruction issues (the next chunk's fragment reads, the tile writes, then the loads).
  auto tile = [&](int kt, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value, nset = cur ^ 1;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const int fc = c & 1, slot = cur * CHUNKS + c, kc = kt * CHUNKS + c;
      const int na = (PA - c + CHUNKS - 1) / CHUNKS;   // activation units of this chunk
      if (c + 1 < CHUNKS) {
        fload(cur, c + 1, fa[fc ^ 1]);
        sstore_a(nset, nset, c);
        gload_a(kt + 3, nset, c);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          mma_col(fc, slot, j);
          wload(slot, kc + RING, j);
        }
#pragma unroll
        for (int k = 0; k < NMF; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          if (k < TM) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
          else if (k < TM + na) __builtin_amdgcn_sched_group_barrier(SG_DS_WR, 1, 0);
          else if (k < TM + 2 * na + TN) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        sstore_a(nset, nset, c);
        gload_a(kt + 3, nset, c);
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          mma_col(fc, slot, j);
          wload(slot, kc + RING, j);
        }
#pragma unroll
        for (int k = 0; k < TM * JB; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          if (k < na) __builtin_amdgcn_sched_group_barrier(SG_DS_WR, 1, 0);
          else if (k < 2 * na + JB) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        fload(nset, 0, fa[fc ^ 1]);
#pragma unroll
        for (int j = JB; j < TN; ++j) {
          mma_col(fc, slot, j);
          wload(slot, kc + RING, j);
        }
#pragma unroll
        for (int k = 0; k < TM * (TN - JB); ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          if (k < TM) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
          else if (k < TM + TN - JB) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // first tile peeled (the loop is entered after an even tile from both sides, as in gemm4_kernel)
  tile(0, std::integral_constant<int, 0>{});
  int kt = 1;
  for (; kt + 1 < KT; kt += 2) {
    tile(kt, std::integral_constant<int, 1>{});
    tile(kt + 1, std::integral_constant<int, 0>{});
  }
  if (kt < KT) tile(kt, std::integral_constant<int, 1>{});

  static_assert(4 * 32 * (32 * TN + 8) * 2 <= (int)sizeof(smem), "the staged epilogue reuses the activation buffers");
  if (g4p_staged_ok<EPI, TM, TN>(g))
    g4p_epilogue_staged<EPI, TM, TN>(g, acc, m0, n0 + wave * WN, sp, wave, lane, reinterpret_cast<bf16_t*>(&smem[0][0]));
  else
    g4_epilogue_t<EPI, TM, TN>(g, acc, m0, n0 + wave * WN, sp, l32, half);
}

// ------------------------------------------------------------------------------------------------
// MXFP8 256x256 four-wave product. Operands are fp8 e4m3 codes with one e8m0 (power-of-two) scale per
// 32 consecutive k of a row; v_mfma_scale_f32_32x32x64_f8f6f4 applies the scales in the product.
// A k-tile is 128 codes = 128 bytes per row, exactly the bytes of a bf16 k-tile, so the tile's LDS
// layout (144-byte padded rows) and the global -> register -> LDS staging are those of gemm4_kernel;
// one register set (the tile after next is requested while the next one is written to LDS).
// Per tile: two k64 steps, each as two chunks of 8 MFMAs (row blocks 0-1, then 2-3). Operand lanes
// (measured): lane l holds row l % 32; bytes 0-15 are k 16 h .. 16 h + 15 and bytes 16-31 are
// k 32 + 16 h .. (h = l / 32) of the step, i.e. both 32-k scale blocks, and lane l supplies the scale
// of block h of its row. The W block goes first (transposed accumulators, as in gemm4_kernel).
// W4: W holds MXFP4 (e2m1 nibbles, two k per byte, low nibble first): a k-tile is 64 bytes per row,
// and in the fp4 operand lane l holds k 32 h .. 32 h + 31 of the step as 16 contiguous bytes
// (measured), which is unit 2 s + h of the row's tile; the A (fp8) operand and the scales are as above.
// ------------------------------------------------------------------------------------------------
typedef int int8v_t __attribute__((ext_vector_type(8)));

template <int EPI, bool W4 = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm4mx_kernel(GemmArgs g, int splits) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, TM = 4, TN = 4;
  constexpr int NT = 256, UNITS = 8, BK = 128, PER_T = BM * UNITS / NT, PITCH = UNITS + 1;
  constexpr int UNITS_W = W4 ? 4 : 8, PITCH_W = UNITS_W + 1, PER_TW = BN * UNITS_W / NT, BKW = W4 ? 64 : 128;
  constexpr int WROWS = NT / UNITS_W;   // W rows one pass of the workgroup's loads covers
  __shared__ uint4 smem[2][BM * PITCH + BN * PITCH_W];

  const int Mt = (g.M + BM - 1) / BM, Nt = (g.N + BN - 1) / BN;
  const int items = Mt * Nt * splits;
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int per = items >> 3, rem = items & 7;
  if (kx >= per + (xcd < rem ? 1 : 0)) return;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + kx;
  const int mt = item % Mt, rest = item / Mt;
  const int sp = rest % splits, nt = rest / splits;
  const int m0 = mt * BM, n0 = nt * BN;
  const int KT_all = g.K / BK;
  const int kb = (int)((long)sp * KT_all / splits), ke = (int)((long)(sp + 1) * KT_all / splits);
  const int KT = ke - kb;
  const int kblocks = g.K / 32;   // scale bytes per row

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int half = lane >> 5, l32 = lane & 31;

  const __amdgpu_buffer_rsrc_t ra_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.A), (short)0,
                                                                       (int)((long)g.M * g.lda), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.W), (short)0,
                                                                       (int)((long)g.N * g.ldw), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsa_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.As), (short)0,
                                                                        (int)((long)g.M * kblocks), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsw_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(g.Ws), (short)0,
                                                                        (int)((long)g.N * kblocks), 0x00020000);
  const int lrow = tid >> 3, lunit = tid & 7;
  const int lroww = tid / UNITS_W, lunitw = tid % UNITS_W;
  int offa[PER_T], offw[PER_TW];
#pragma unroll
  for (int i = 0; i < PER_T; ++i) offa[i] = (int)((long)(m0 + lrow + i * 32) * g.lda + lunit * 16);
#pragma unroll
  for (int i = 0; i < PER_TW; ++i) offw[i] = (int)((long)(n0 + lroww + i * WROWS) * g.ldw + lunitw * 16);
  // this lane's scale rows: row block i of the wave's A rows, column block j of its W rows
  int soff_a[TM], soff_w[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) soff_a[i] = (m0 + wm * WM + i * 32 + l32) * kblocks;
#pragma unroll
  for (int j = 0; j < TN; ++j) soff_w[j] = (n0 + wn * WN + j * 32 + l32) * kblocks;
  const int sbase = lrow * PITCH + lunit;
  const int sbasew = BM * PITCH + lroww * PITCH_W + lunitw;

  constexpr int QW = PER_TW / 4;   // W units per quarter: 2 (fp8) or 1 (fp4)
  uint4 rg[PER_T], rgw[PER_TW];
  auto gload_q = [&](int kt, int q) {
    const int kc = kb + min(kt, KT - 1);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * q + u;
      rg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra_, offa[i], kc * BK, 0));
    }
#pragma unroll
    for (int u = 0; u < QW; ++u) {
      const int i = QW * q + u;
      rgw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw_, offw[i], kc * BKW, 0));
    }
  };
  auto sstore_q = [&](int st, int q) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 2 * q + u;
      smem[st][sbase + i * 32 * PITCH] = rg[i];
    }
#pragma unroll
    for (int u = 0; u < QW; ++u) {
      const int i = QW * q + u;
      smem[st][sbasew + i * WROWS * PITCH_W] = rgw[i];
    }
  };
  // the four 32-k scale bytes of tile kt for this lane's rows (one dword per row block)
  uint32_t sca[2][TM], scw[2][TN];
  auto sload = [&](int kt, uint32_t* a_, uint32_t* w_) {
    const int koff = (kb + min(kt, KT - 1)) * 4;
#pragma unroll
    for (int i = 0; i < TM; ++i) a_[i] = __builtin_amdgcn_raw_buffer_load_b32(rsa_, soff_a[i], koff, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) w_[j] = __builtin_amdgcn_raw_buffer_load_b32(rsw_, soff_w[j], koff, 0);
  };
  // fragments of chunk c: step s = c / 2, A row blocks 2 (c % 2), +1; W column blocks with the step
  uint4 fa[2][2][2], fb[2][TN][2];
  auto fload_a = [&](int st, int c, uint4 (&f)[2][2]) {
    const int s_ = c >> 1, i0 = 2 * (c & 1);
    const uint4* sa = smem[st] + (wm * WM + l32) * PITCH + half;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      f[ii][0] = sa[(i0 + ii) * 32 * PITCH + 4 * s_];
      f[ii][1] = sa[(i0 + ii) * 32 * PITCH + 4 * s_ + 2];
    }
  };
  auto fload_w = [&](int st, int s_, uint4 (&f)[TN][2]) {
    const uint4* sb = smem[st] + BM * PITCH + (wn * WN + l32) * PITCH_W + half;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (W4) {
        f[j][0] = sb[j * 32 * PITCH_W + 2 * s_];
      } else {
        f[j][0] = sb[j * 32 * PITCH_W + 4 * s_];
        f[j][1] = sb[j * 32 * PITCH_W + 4 * s_ + 2];
      }
    }
  };

  floatx16 acc[TM][TN];
  g4_acc_init<EPI, TM, TN>(acc, g, sp, n0 + wn * WN, half);

#pragma unroll
  for (int q = 0; q < 4; ++q) gload_q(0, q);
  sload(0, sca[0], scw[0]);
#pragma unroll
  for (int q = 0; q < 4; ++q) sstore_q(0, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) gload_q(1, q);
  __syncthreads();
  fload_a(0, 0, fa[0]);
  fload_w(0, 0, fb[0]);

  // tile kt from LDS buffer CUR with scale set CUR; rg holds tile kt+1, written to the other buffer
  // quarter by quarter and refilled with tile kt+2; scales of kt+1 are requested into the other set.
  // Scheduling groups (chunks 0-2): the chunk's LDS reads go out between its first four MFMAs, its
  // LDS writes and global loads between the last four, so they issue while the matrix core works.
  constexpr int SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100, SG_DS_WR = 0x200;
  auto tile = [&](int kt, auto cur_c) {
    constexpr int cur = decltype(cur_c)::value, nxt = cur ^ 1;
    sload(kt + 1, sca[nxt], scw[nxt]);
    auto chunk = [&](auto c_c) {
      constexpr int c = decltype(c_c)::value;
      const int s_ = c >> 1, i0 = 2 * (c & 1);
      const int fc = c & 1, fs = s_ & 1;
      if constexpr (c + 1 < 4) {
        fload_a(cur, c + 1, fa[fc ^ 1]);
        if constexpr (c == 1) fload_w(cur, 1, fb[fs ^ 1]);
      }
      sstore_q(nxt, c);
      gload_q(kt + 2, c);
      if constexpr (c + 1 == 4) {
        __syncthreads();
        fload_a(nxt, 0, fa[fc ^ 1]);
        fload_w(nxt, 0, fb[fs ^ 1]);
      }
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = i0 + ii;
        const int sa_ = (int)(sca[cur][i] >> (8 * (2 * s_ + half)));
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int sw_ = (int)(scw[cur][j] >> (8 * (2 * s_ + half)));
          const int8v_t av = __builtin_bit_cast(int8v_t, fa[fc][ii]);
          if constexpr (W4) {   // first operand e2m1 (format 4): its low four registers
            const uint4 w4 = fb[fs][j][0];
            const int8v_t wv = {(int)w4.x, (int)w4.y, (int)w4.z, (int)w4.w, 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, av, acc[i][j], 4, 0, 0, sw_, 0, sa_);
          } else {
            const int8v_t wv = __builtin_bit_cast(int8v_t, fb[fs][j]);
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, av, acc[i][j], 0, 0, 0, sw_, 0, sa_);
          }
        }
      }
      if constexpr (c + 1 == 4) {   // the next tile's first fragments go out between this chunk's MFMAs
        constexpr int RD = W4 ? 1 : 2;                    // 8 or 12 reads over six MFMAs
#pragma unroll
        for (int k = 0; k < 6; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RD, 0);
        }
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
      }
      if constexpr (c + 1 < 4) {
        constexpr int RD = c == 1 ? (W4 ? 2 : 3) : 1;   // LDS reads per early MFMA (4, 8 or 12 in all)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_RD, RD, 0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_DS_WR, 1, 0);
          __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    chunk(std::integral_constant<int, 0>{});
    chunk(std::integral_constant<int, 1>{});
    chunk(std::integral_constant<int, 2>{});
    chunk(std::integral_constant<int, 3>{});
  };
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    tile(kt, std::integral_constant<int, 0>{});
    tile(kt + 1, std::integral_constant<int, 1>{});
  }
  if (kt < KT) tile(kt, std::integral_constant<int, 0>{});
  g4_epilogue_t<EPI, TM, TN>(g, acc, m0 + wm * WM, n0 + wn * WN, sp, l32, half);
}

// Sum of the split partials in split order, plus bias, then the epilogue. One thread per 4 columns.
template <typename T, int EPI>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmArgs g, int splits) {
  const int row = blockIdx.y;
  const int c4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c4 >= g.N) return;
  float v[4];
  {
    const float4 p = *reinterpret_cast<const float4*>(g.part + (long)row * g.N + c4);
    v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
  }
  for (int s = 1; s < splits; ++s) {
    const float4 p = *reinterpret_cast<const float4*>(g.part + ((long)s * g.M + row) * g.N + c4);
    v[0] += p.x; v[1] += p.y; v[2] += p.z; v[3] += p.w;
  }
  if (g.bias) {
    const float4 b = *reinterpret_cast<const float4*>(g.bias + c4);
    v[0] += b.x; v[1] += b.y; v[2] += b.z; v[3] += b.w;
  }
  if constexpr (EPI == EPI_SWIGLU) {
    T* out = reinterpret_cast<T*>(g.C) + (long)row * g.ldc + c4 / 2;
    Elem<T>::store(out, silu_f(v[0]) * v[1]);
    Elem<T>::store(out + 1, silu_f(v[2]) * v[3]);
  } else if constexpr (EPI == EPI_STORE || EPI == EPI_GELU) {
    if constexpr (EPI == EPI_GELU) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = gelu_tanh_f(v[e]);
    }
    T* out = reinterpret_cast<T*>(g.C) + (long)row * g.ldc + c4;
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<uint2*>(out) = make_uint2(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]));
    } else {
      *reinterpret_cast<float4*>(out) = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
    float4* h = reinterpret_cast<float4*>(g.H + (long)row * g.ldh + c4);
    float4 hv = *h;
    if constexpr (EPI == EPI_RESID_GATED) {
      const int rb = row % g.rm.rows_per_branch;
      const int ch = rb / g.rm.Lq, grp = (rb % g.rm.Lq) < g.rm.Lv ? 0 : 1;
      const float4 ge = *reinterpret_cast<const float4*>(g.e6 + ((long)(ch * 2 + grp) * 6 + g.gate_idx) * g.D + c4);
      const float4 gm = *reinterpret_cast<const float4*>(g.mod + (long)g.gate_idx * g.D + c4);
      hv.x += (ge.x + gm.x) * v[0]; hv.y += (ge.y + gm.y) * v[1]; hv.z += (ge.z + gm.z) * v[2]; hv.w += (ge.w + gm.w) * v[3];
    } else {
      hv.x += v[0]; hv.y += v[1]; hv.z += v[2]; hv.w += v[3];
    }
    *h = hv;
  }
}

template <typename T, int BM, int BN, int WM, int WN, int NW>
static hipError_t launch_cfg(const GemmArgs& a, Epi epi, hipStream_t s) {
  if constexpr (BM * BN > 128 * 128) {
    if (epi == EPI_ROWSEL_F32) return hipErrorInvalidValue;  // output heads never use the large tiles
  }
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const dim3 grid(8 * ((tiles + 7) / 8)), block(NW * 64);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, NW, EPI_STORE>), grid, block, 0, s, a); break;
    case EPI_GELU: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, NW, EPI_GELU>), grid, block, 0, s, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, NW, EPI_SWIGLU>), grid, block, 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, NW, EPI_RESID>), grid, block, 0, s, a); break;
    case EPI_RESID_GATED:
      hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, NW, EPI_RESID_GATED>), grid, block, 0, s, a);
      break;
    case EPI_ROWSEL_F32:
      if constexpr (BM * BN <= 128 * 128)
        hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, NW, EPI_ROWSEL_F32>), grid, block, 0, s, a);
      break;
  }
  return hipGetLastError();
}

// Four-wave bf16 tiles: 256 x 256 (waves of 128 x 128) or 192 x 320 (waves of 96 x 160). Both stage
// 512 rows per k-tile; the planner takes the one whose busiest CU has less work (rounds of 256
// workgroups times the work of one), so M = 928 runs on 5 x 192 rows (3.4% padding) instead of 4 x 256
// (9.4%) at the same workgroup count.
struct G4Plan {
  int splits = 0;     // 0: shape not suited, 1: direct epilogue, else split-K partials
  bool t192 = false;  // 192 x 320 tiles
};

template <int EPI>
static void launch_g4(const GemmArgs& a, const G4Plan& p, hipStream_t s) {
  const int bm = p.t192 ? 192 : 256, bn = p.t192 ? 320 : 256;
  const int items = ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn) * p.splits;
  const dim3 grid(8 * ((items + 7) / 8)), block(256);
  if (p.t192)
    hipLaunchKernelGGL((gemm4_kernel<EPI, 3, 5>), grid, block, 0, s, a, p.splits);
  else
    hipLaunchKernelGGL((gemm4_kernel<EPI, 4, 4>), grid, block, 0, s, a, p.splits);
}

// bf16 four-wave path: direct epilogue when there are enough tiles to occupy the CUs, else split-K
// (about 240 workgroups) with a finishing row kernel. splits == 0 when the shape does not suit the
// kernel (the caller falls back to the 8-wave tiles).
static bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }
// vector epilogues: runs of four columns, 16-byte aligned fp32 rows, 8-byte aligned bf16 rows
static bool g4_vec_ok(const GemmArgs& a, Epi epi) {
  return a.N % 4 == 0 && (!a.bias || aligned16(a.bias)) &&
         (epi == EPI_STORE || epi == EPI_GELU || epi == EPI_SWIGLU
              ? (reinterpret_cast<uintptr_t>(a.C) % 8 == 0 && a.ldc % 4 == 0)
              : (aligned16(a.H) && a.ldh % 4 == 0)) &&
         (epi != EPI_RESID_GATED || (aligned16(a.e6) && aligned16(a.mod) && a.D % 4 == 0));
}
static G4Plan g4_plan(const GemmArgs& a, Epi epi) {
  G4Plan best;
  if (epi == EPI_ROWSEL_F32 || a.M < 256 || a.N < 256) return best;
  if (!g4_vec_ok(a, epi)) return best;
  const int KT = a.K / 64;
  long best_cost = 0;
  for (const bool t192 : {false, true}) {
    const int bm = t192 ? 192 : 256, bn = t192 ? 320 : 256;
    const long tiles = (long)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
    int splits = 1;
    if (tiles < 128 && a.part) {
      splits = (int)((240 + tiles - 1) / tiles);
      if (splits > 4) splits = 4;
      while (splits > 1 && (KT < 4 * splits || (long)splits * a.M * a.N > a.part_elems)) --splits;
    }
    const long rounds = (tiles * splits + 255) / 256;
    const long cost = rounds * bm * bn * ((KT + splits - 1) / splits);
    if (best.splits == 0 || cost < best_cost) {
      best.splits = splits;
      best.t192 = t192;
      best_cost = cost;
    }
  }
  return best;
}

// Fragment-packed weights: 160 x 384 tiles (waves of 160 x 96), 160 x 256 (waves of 160 x 64) or
// 128 x 512 (waves of 128 x 128), the one whose busiest CU has less work (the first on a tie), split
// over K as in g4_plan when there are fewer than 128 tiles. At 928 x 5120 x 5120 the 160 x 256 tiles
// have no partly filled column of tiles and split K in two instead of three, so the finish that sums
// the partials reads a third less.
// Every shape and every epilogue but the row gather runs here (a packed matrix has no unpacked copy
// to fall back on): rows past M and columns past N are masked.
struct G4pPlan {
  int splits = 0;     // 0: the packed kernel does not take this product
  int tile = 0;       // 0: 128 x 512, 1: 160 x 384, 2: 160 x 256
};
static constexpr int G4P_BM[3] = {128, 160, 160}, G4P_BN[3] = {512, 384, 256};
static G4pPlan g4p_plan(const GemmArgs& a, Epi epi) {
  G4pPlan best;
  if (epi == EPI_ROWSEL_F32 || a.M <= 0 || a.N % 32 || a.K % 64 || a.K <= 0 || !aligned16(a.W) ||
      (long)a.N * a.K * 2 >= (1L << 31) || (long)a.M * a.lda * 2 >= (1L << 31) || a.lda % 8 || !aligned16(a.A) ||
      !g4_vec_ok(a, epi))
    return best;
  const int KT = a.K / 64;
  long best_cost = 0;
  for (int tile = 0; tile < 3; ++tile) {
    const int bm = G4P_BM[tile], bn = G4P_BN[tile];
    const long tiles = (long)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
    int splits = 1;
    if (tiles < 128 && a.part) {
      splits = (int)((240 + tiles - 1) / tiles);
      if (splits > 4) splits = 4;
      while (splits > 1 && (KT < 4 * splits || (long)splits * a.M * a.N > a.part_elems)) --splits;
    }
    const long rounds = (tiles * splits + 255) / 256;
    const long cost = rounds * bm * bn * ((KT + splits - 1) / splits);
    // on a tie the plan with fewer K ranges wins: its finish reads fewer partials
    if (best.splits == 0 || cost < best_cost || (cost == best_cost && splits < best.splits)) {
      best.splits = splits;
      best.tile = tile;
      best_cost = cost;
    }
  }
  return best;
}

template <int EPI>
static void launch_g4p(const GemmArgs& a, const G4pPlan& p, hipStream_t s) {
  const int bm = G4P_BM[p.tile], bn = G4P_BN[p.tile];
  const long items = (long)((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn) * p.splits;
  const dim3 grid((unsigned)(8 * ((items + 7) / 8))), block(256);
  if (p.tile == 1)
    hipLaunchKernelGGL((gemm4p_kernel<EPI, 5, 3>), grid, block, 0, s, a, p.splits);
  else if (p.tile == 2)
    hipLaunchKernelGGL((gemm4p_kernel<EPI, 5, 2>), grid, block, 0, s, a, p.splits);
  else
    hipLaunchKernelGGL((gemm4p_kernel<EPI, 4, 4>), grid, block, 0, s, a, p.splits);
}

static void launch_reduce(const GemmArgs& a, Epi epi, int splits, hipStream_t s);

static hipError_t launch_gemm_packed(const GemmArgs& a, Epi epi, hipStream_t s) {
  const G4pPlan p = g4p_plan(a, epi);
  if (p.splits == 0) return hipErrorInvalidValue;
  if (p.splits > 1) {
    launch_g4p<EPI_PARTIAL>(a, p, s);
    launch_reduce(a, epi, p.splits, s);
  } else {
    switch (epi) {
      case EPI_STORE: launch_g4p<EPI_STORE>(a, p, s); break;
      case EPI_GELU: launch_g4p<EPI_GELU>(a, p, s); break;
      case EPI_SWIGLU: launch_g4p<EPI_SWIGLU>(a, p, s); break;
      case EPI_RESID: launch_g4p<EPI_RESID>(a, p, s); break;
      case EPI_RESID_GATED: launch_g4p<EPI_RESID_GATED>(a, p, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_pack_weight(const void* W, long ldw, int N, int K, void* Wp, hipStream_t s) {
  if (N <= 0 || K <= 0 || N % 32 || K % 64 || ldw < K || ldw % 8 || !aligned16(W) || !aligned16(Wp))
    return hipErrorInvalidValue;
  const long total = (long)(N / 32) * (K / 16) * 64;
  const long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(W), ldw / 8, reinterpret_cast<uint4*>(Wp), N, K);
  return hipGetLastError();
}

static void launch_g4_direct(const GemmArgs& a, Epi epi, const G4Plan& p, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: launch_g4<EPI_STORE>(a, p, s); break;
    case EPI_GELU: launch_g4<EPI_GELU>(a, p, s); break;
    case EPI_SWIGLU: launch_g4<EPI_SWIGLU>(a, p, s); break;
    case EPI_RESID: launch_g4<EPI_RESID>(a, p, s); break;
    case EPI_RESID_GATED: launch_g4<EPI_RESID_GATED>(a, p, s); break;
    default: break;
  }
}

static void launch_reduce(const GemmArgs& a, Epi epi, int splits, hipStream_t s) {
  const dim3 grid((a.N / 4 + 255) / 256, a.M);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((splitk_reduce_kernel<bf16_t, EPI_STORE>), grid, dim3(256), 0, s, a, splits); break;
    case EPI_GELU: hipLaunchKernelGGL((splitk_reduce_kernel<bf16_t, EPI_GELU>), grid, dim3(256), 0, s, a, splits); break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL((splitk_reduce_kernel<bf16_t, EPI_SWIGLU>), grid, dim3(256), 0, s, a, splits);
      break;
    case EPI_RESID: hipLaunchKernelGGL((splitk_reduce_kernel<bf16_t, EPI_RESID>), grid, dim3(256), 0, s, a, splits); break;
    case EPI_RESID_GATED:
      hipLaunchKernelGGL((splitk_reduce_kernel<bf16_t, EPI_RESID_GATED>), grid, dim3(256), 0, s, a, splits);
      break;
    default: break;
  }
}

// 224-wide tiles when the 256-wide ones fill between half and all of the CUs in one round and the
// 224-wide ones still fit in one round: every workgroup then has 7/8 of the work
static bool use_wide_rows(const GemmArgs& a, Epi epi) {
  if (epi != EPI_STORE && epi != EPI_GELU) return false;
  const long mt = (a.M + 255) / 256;
  const long t256 = mt * ((a.N + 255) / 256), t224 = mt * ((a.N + 223) / 224);
  return t256 >= 128 && t256 < 256 && t224 <= 256;
}

static bool try_gemm4(const GemmArgs& a, Epi epi, hipStream_t s, hipError_t* err) {
  const G4Plan plan = g4_plan(a, epi);
  if (plan.splits == 0) return false;
  if (plan.splits == 1 && use_wide_rows(a, epi)) {
    const long items = (long)((a.M + 255) / 256) * ((a.N + 223) / 224);
    const dim3 grid((unsigned)(8 * ((items + 7) / 8))), block(256);
    if (epi == EPI_GELU)
      hipLaunchKernelGGL((gemm4w_kernel<EPI_GELU>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((gemm4w_kernel<EPI_STORE>), grid, block, 0, s, a);
  } else if (plan.splits == 1) {
    launch_g4_direct(a, epi, plan, s);
  } else {
    launch_g4<EPI_PARTIAL>(a, plan, s);
    launch_reduce(a, epi, plan.splits, s);
  }
  *err = hipGetLastError();
  return true;
}

hipError_t launch_gemm(const GemmArgs& a, DType dt, Epi epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.w_packed) return dt == DT_BF16 && !a.As ? launch_gemm_packed(a, epi, s) : hipErrorInvalidValue;
  if (a.As) return dt == DT_BF16 ? launch_gemm_mx(a, epi, s) : hipErrorInvalidValue;   // MXFP8 operands
  if (epi == EPI_SWIGLU && a.N % 2) return hipErrorInvalidValue;   // (gate, up) column pairs
  // buffer descriptors address each operand with 32-bit byte offsets
  const long esz = dt == DT_BF16 ? 2 : 4;
  if ((long)a.M * a.lda * esz >= (1L << 31) || (long)a.N * a.ldw * esz >= (1L << 31)) return hipErrorInvalidValue;
  // Tile choice (measured on MI355X over the step's shapes): bf16 products with M, N >= 256 take the
  // four-wave kernel with 256x256 or 192x320 tiles (split over K when it has fewer than 128 tiles), or
  // 256x224 tiles when those fill one round; the rest take 256x128 /
  // 128x256 tiles with 8 waves of 64x64, and smaller tiles for tiny shapes.
  if (dt == DT_BF16) {
    hipError_t e4;
    if (try_gemm4(a, epi, s, &e4)) return e4;
    if (epi != EPI_ROWSEL_F32 && a.M >= 256 && a.N >= 128) return launch_cfg<bf16_t, 256, 128, 64, 64, 8>(a, epi, s);
    if (epi != EPI_ROWSEL_F32 && a.M >= 128 && a.N >= 256) return launch_cfg<bf16_t, 128, 256, 64, 64, 8>(a, epi, s);
    if (a.N >= 128 && a.M >= 128) return launch_cfg<bf16_t, 128, 128, 64, 64, 4>(a, epi, s);
    return launch_cfg<bf16_t, 64, 64, 32, 32, 4>(a, epi, s);
  }
  if (a.N >= 128 && a.M >= 128) return launch_cfg<float, 128, 128, 64, 64, 4>(a, epi, s);
  return launch_cfg<float, 64, 64, 32, 32, 4>(a, epi, s);
}

// ------------------------------------------------------------------------------------------------
// Split-K finish fused with the row stage that follows the product: one workgroup (256 threads) per
// output row sums the fp32 partials in split order, adds the bias, applies the epilogue and then, with
// the whole row in registers, the LayerNorm (POST_NORM) or the q/k RMSNorm with head-major scatter
// (POST_QK). Row statistics are block reductions in a fixed order (deterministic).
// ------------------------------------------------------------------------------------------------
constexpr int FIN_G = 8;   // float4 groups per thread (template G <= FIN_G): rows of up to 8192 columns
// Stands in for a missing bias, so that the finish adds a bias unconditionally (no branch between
// its loads).
__device__ float fin_zero_row[FIN_G * 1024];

__device__ __forceinline__ float4 keep_if(bool c, float4 a) {   // component selects, never a memory select
  return make_float4(c ? a.x : 0.f, c ? a.y : 0.f, c ? a.z : 0.f, c ? a.w : 0.f);
}

template <int EPI, int POST, int SPLITS, int G, bool PB>   // PB: bf16 partials (else fp32)
__global__ void __launch_bounds__(256) splitk_finish_kernel(GemmArgs g, PostArgs p) {
  __shared__ float red[4];
  const int m = blockIdx.x, t = threadIdx.x;
  const int nv = g.N / 4;
  const long pstride = (long)g.M * g.N;
  // Every load of the row (partials, bias, residual, gate) is issued before any arithmetic, with no
  // control flow between them, so their latencies overlap: lanes past the row's end read its last quad
  // (the values are dropped), and a missing bias is read from a zero row.
  float4 v[G], hv[G], gv[G];
  int qc[G];
#pragma unroll
  for (int k = 0; k < G; ++k) qc[k] = min(t + 256 * k, nv - 1);
  // fp32 partials: the bias is added here; bf16 partials (the block's fused path): split 0's carries it
  const float* bsrc = g.bias ? g.bias : fin_zero_row;
  const float* grow = nullptr;
  if constexpr (EPI == EPI_RESID_GATED) {
    const int rb = m % g.rm.rows_per_branch;
    const int ch = rb / g.rm.Lq, grp = (rb % g.rm.Lq) < g.rm.Lv ? 0 : 1;
    grow = g.e6 + ((long)(ch * 2 + grp) * 6 + g.gate_idx) * g.D;
  }
  {
    using Raw = std::conditional_t<PB, uint2, float4>;
    const Raw* pp = reinterpret_cast<const Raw*>(g.part) + (long)m * nv;   // one quad per element
    const long qstride = pstride / 4;                                        // quads per split
    Raw raw[G][SPLITS];
    float4 bv[G], ge[G], gm[G];
#pragma unroll
    for (int k = 0; k < G; ++k) {
#pragma unroll
      for (int sp = 0; sp < SPLITS; ++sp) raw[k][sp] = pp[sp * qstride + qc[k]];
      if constexpr (!PB) bv[k] = reinterpret_cast<const float4*>(bsrc)[qc[k]];
      if constexpr (EPI != EPI_STORE) hv[k] = reinterpret_cast<const float4*>(g.H + (long)m * g.ldh)[qc[k]];
      if constexpr (EPI == EPI_RESID_GATED) {
        ge[k] = reinterpret_cast<const float4*>(grow)[qc[k]];
        gm[k] = reinterpret_cast<const float4*>(g.mod + (long)g.gate_idx * g.D)[qc[k]];
      }
    }
    auto widen = [](const Raw& r) {
      if constexpr (PB)   // four bf16 values, widened exactly
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
      else
        return r;
    };
#pragma unroll
    for (int k = 0; k < G; ++k) {
      float4 a = widen(raw[k][0]);   // partials summed in split order
#pragma unroll
      for (int sp = 1; sp < SPLITS; ++sp) {
        const float4 b = widen(raw[k][sp]);
        a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
      }
      if constexpr (!PB) { a.x += bv[k].x; a.y += bv[k].y; a.z += bv[k].z; a.w += bv[k].w; }
      const bool in = t + 256 * k < nv;
      v[k] = keep_if(in, a);
      if constexpr (EPI != EPI_STORE) hv[k] = keep_if(in, hv[k]);
      else hv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (EPI == EPI_RESID_GATED)
        gv[k] = keep_if(in, make_float4(ge[k].x + gm[k].x, ge[k].y + gm[k].y, ge[k].z + gm[k].z, ge[k].w + gm[k].w));
      else
        gv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int k = 0; k < G; ++k) {
    const int q = t + 256 * k;
    if (q >= nv) continue;
    float4 a = v[k];
    if constexpr (EPI == EPI_STORE) {
      // the stage reads what the unfused path would have stored: bf16-rounded outputs
      a.x = bf16_to_f32(f32_to_bf16(a.x)); a.y = bf16_to_f32(f32_to_bf16(a.y));
      a.z = bf16_to_f32(f32_to_bf16(a.z)); a.w = bf16_to_f32(f32_to_bf16(a.w));
    } else {
      float4 h = hv[k];
      if constexpr (EPI == EPI_RESID_GATED) {
        const float4 gg = gv[k];
        h.x += gg.x * a.x; h.y += gg.y * a.y; h.z += gg.z * a.z; h.w += gg.w * a.w;
      } else {
        h.x += a.x; h.y += a.y; h.z += a.z; h.w += a.w;
      }
      *reinterpret_cast<float4*>(g.H + (long)m * g.ldh + 4 * q) = h;
      a = h;
    }
    v[k] = a;
  }
  if constexpr (POST == POST_NORM) {
    // y = (v - mean) rstd mv + av with mv = 1 + scale (+ layer offset) and av = shift (+ offset), or
    // mv = w, av = b (affine): both are loaded before the reductions, so their latency hides there
    const NormArgs& na = p.na;
    float4 mv[G], av[G];
    {
      const float4 *sh = nullptr, *sc = nullptr, *sh2 = nullptr, *sc2 = nullptr;
      if (na.mode != NORM_AFFINE) {
        const int rb = m % na.rm.rows_per_branch;
        const int ch = rb / na.rm.Lq, grp = (rb % na.rm.Lq) < na.rm.Lv ? 0 : 1;
        if (na.mode == NORM_ADALN) {
          const float* e6 = na.e6 + (long)(ch * 2 + grp) * 6 * na.D;
          sh = reinterpret_cast<const float4*>(e6 + (long)na.shift_idx * na.D);
          sc = reinterpret_cast<const float4*>(e6 + (long)na.scale_idx * na.D);
          sh2 = reinterpret_cast<const float4*>(na.mod + (long)na.shift_idx * na.D);
          sc2 = reinterpret_cast<const float4*>(na.mod + (long)na.scale_idx * na.D);
        } else {
          const float* e = na.e6 + (long)(ch * 2 + grp) * na.D;
          sh = sc = reinterpret_cast<const float4*>(e);
          sh2 = reinterpret_cast<const float4*>(na.mod);
          sc2 = reinterpret_cast<const float4*>(na.mod + na.D);
        }
      }
      if (na.mode == NORM_AFFINE) {
#pragma unroll
        for (int k = 0; k < G; ++k) {
          mv[k] = reinterpret_cast<const float4*>(na.w)[qc[k]];
          av[k] = reinterpret_cast<const float4*>(na.b)[qc[k]];
        }
      } else {
        float4 pa[G], pb[G], ra[G], rb2[G];
#pragma unroll
        for (int k = 0; k < G; ++k) {
          pa[k] = sh[qc[k]]; pb[k] = sh2[qc[k]]; ra[k] = sc[qc[k]]; rb2[k] = sc2[qc[k]];
        }
#pragma unroll
        for (int k = 0; k < G; ++k) {
          mv[k] = make_float4(1.f + (ra[k].x + rb2[k].x), 1.f + (ra[k].y + rb2[k].y), 1.f + (ra[k].z + rb2[k].z),
                              1.f + (ra[k].w + rb2[k].w));
          av[k] = make_float4(pa[k].x + pb[k].x, pa[k].y + pb[k].y, pa[k].z + pb[k].z, pa[k].w + pb[k].w);
        }
      }
    }
    float s1 = 0.f;
#pragma unroll
    for (int k = 0; k < G; ++k) s1 += (v[k].x + v[k].y) + (v[k].z + v[k].w);
    const float mean = na.rms ? 0.f : block_sum<256>(s1, red) / (float)g.N;
    float s2 = 0.f;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      if (t + 256 * k >= nv) continue;
      const float d0 = v[k].x - mean, d1 = v[k].y - mean, d2 = v[k].z - mean, d3 = v[k].w - mean;
      s2 += (d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3);
    }
    const float rstd = 1.f / sqrtf(block_sum<256>(s2, red) / (float)g.N + na.eps);
    bf16_t* y = reinterpret_cast<bf16_t*>(na.Y) + (long)m * na.D;
    auto modulate = [&](int k) {
      const float4 o = make_float4((v[k].x - mean) * rstd, (v[k].y - mean) * rstd, (v[k].z - mean) * rstd,
                                   (v[k].w - mean) * rstd);
      return make_float4(o.x * mv[k].x + av[k].x, o.y * mv[k].y + av[k].y, o.z * mv[k].z + av[k].z,
                         o.w * mv[k].w + av[k].w);
    };
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int q = t + 256 * k;
      if (na.mxq && 256 * k < nv) {   // MXFP8 copy of the stored (bf16-rounded) row; whole waves call it
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (q < nv) {
          o = modulate(k);
          reinterpret_cast<uint2*>(y)[q] = make_uint2(pack2_bf16(o.x, o.y), pack2_bf16(o.z, o.w));
          o = make_float4(bf16_round(o.x), bf16_round(o.y), bf16_round(o.z), bf16_round(o.w));
        }
        mx_store_quad(o, q < nv, na.mxq + (long)m * na.D, na.mxs + (long)m * (na.D / 32), q);
        continue;
      }
      if (q >= nv) continue;
      const float4 o = modulate(k);
      reinterpret_cast<uint2*>(y)[q] = make_uint2(pack2_bf16(o.x, o.y), pack2_bf16(o.z, o.w));
    }
  } else {   // POST_QK
    const QkNormArgs& qa = p.qa;
    float4 gn[G];   // the gain, loaded before the reduction
#pragma unroll
    for (int k = 0; k < G; ++k) gn[k] = reinterpret_cast<const float4*>(qa.gain)[qc[k]];   // lanes past the end store nothing
    float s2 = 0.f;
#pragma unroll
    for (int k = 0; k < G; ++k) s2 += (v[k].x * v[k].x + v[k].y * v[k].y) + (v[k].z * v[k].z + v[k].w * v[k].w);
    const float rstd = 1.f / sqrtf(block_sum<256>(s2, red) / (float)g.N + qa.eps);
    const int b = m / qa.rows_per_branch, rb = m % qa.rows_per_branch;
    bf16_t* dst = reinterpret_cast<bf16_t*>(qa.dst);
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int q = t + 256 * k;
      if (q >= nv) continue;
      const int c0 = 4 * q, hh = c0 / qa.d, j = c0 % qa.d;
      bf16_t* o = dst + (long)(b * qa.H + hh) * qa.dst_bh_stride + (long)(qa.dst_row0 + rb) * qa.d + j;
      *reinterpret_cast<uint2*>(o) = make_uint2(pack2_bf16(v[k].x * rstd * gn[k].x, v[k].y * rstd * gn[k].y),
                                                pack2_bf16(v[k].z * rstd * gn[k].z, v[k].w * rstd * gn[k].w));
    }
  }
}

hipError_t launch_split_finish(const GemmArgs& a, Epi epi, const PostArgs& post, int splits, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (splits < 2 || splits > 4 || a.N % 4 || a.N > 256 * 4 * FIN_G) return hipErrorInvalidValue;
  const bool norm_ok = post.mode == POST_NORM && (epi == EPI_RESID || epi == EPI_RESID_GATED);
  if (!norm_ok && !(post.mode == POST_QK && epi == EPI_STORE)) return hipErrorInvalidValue;
  const dim3 grid(a.M), block(256);
  const int groups = (a.N / 4 + 255) / 256;   // float4 groups per thread
#define WAM_FINISH_GP(E, P, S, B)                                                                                \
  if (groups <= 1) hipLaunchKernelGGL((splitk_finish_kernel<E, P, S, 1, B>), grid, block, 0, s, a, post);      \
  else if (groups <= 5) hipLaunchKernelGGL((splitk_finish_kernel<E, P, S, 5, B>), grid, block, 0, s, a, post); \
  else hipLaunchKernelGGL((splitk_finish_kernel<E, P, S, FIN_G, B>), grid, block, 0, s, a, post);
#define WAM_FINISH_G(E, P, S)        \
  if (a.part_bf16) {                 \
    WAM_FINISH_GP(E, P, S, true)     \
  } else {                           \
    WAM_FINISH_GP(E, P, S, false)    \
  }
#define WAM_FINISH(E, P)                  \
  switch (splits) {                       \
    case 2: WAM_FINISH_G(E, P, 2) break;  \
    case 3: WAM_FINISH_G(E, P, 3) break;  \
    default: WAM_FINISH_G(E, P, 4) break; \
  }
  if (post.mode == POST_NORM) {
    if (epi == EPI_RESID) {
      WAM_FINISH(EPI_RESID, POST_NORM)
    } else {
      WAM_FINISH(EPI_RESID_GATED, POST_NORM)
    }
  } else {
    WAM_FINISH(EPI_STORE, POST_QK)
  }
#undef WAM_FINISH
#undef WAM_FINISH_G
#undef WAM_FINISH_GP
  return hipGetLastError();
}

static int mx_splits(const GemmArgs& a);
static bool mx_operands_ok(const GemmArgs& a);
static void launch_g4mx_partial(const GemmArgs& a, int splits, hipStream_t s);

hipError_t launch_gemm_post(const GemmArgs& a, DType dt, Epi epi, const PostArgs& post, hipStream_t s) {
  if (post.mode == POST_NONE || a.M <= 0 || a.N <= 0) return launch_gemm(a, dt, epi, s);
  bool fused = dt == DT_BF16 && a.N <= 256 * 4 * FIN_G;
  if (post.mode == POST_NORM)
    fused = fused && (epi == EPI_RESID || epi == EPI_RESID_GATED) && post.na.X == a.H && post.na.D == a.N &&
            post.na.M == a.M && aligned16(post.na.Y) && (post.na.mode != NORM_AFFINE || (aligned16(post.na.w) && aligned16(post.na.b))) &&
            (post.na.mode == NORM_AFFINE || (aligned16(post.na.e6) && aligned16(post.na.mod)));
  else
    fused = fused && epi == EPI_STORE && post.qa.rope == nullptr && post.qa.D == a.N && post.qa.M == a.M &&
            post.qa.d % 4 == 0 && aligned16(post.qa.gain) && reinterpret_cast<uintptr_t>(post.qa.dst) % 8 == 0;
  G4Plan p4;
  G4pPlan pp;
  if (fused && !a.As) {
    if (a.w_packed)
      pp = g4p_plan(a, epi);
    else
      p4 = g4_plan(a, epi);
  }
  const int plan = !fused ? 0 : a.As ? (mx_operands_ok(a) ? mx_splits(a) : 0) : a.w_packed ? pp.splits : p4.splits;
  if (plan > 1) {
    // The partials of this fused path are stored in bf16, each rounded once (about the single
    // rounding a bf16 projection output gets), and summed in fp32 by the finish: half the bytes
    // written at the product's end and read back by the finish.
    GemmArgs b = a;
    b.part_bf16 = 1;
    if (b.As)
      launch_g4mx_partial(b, plan, s);
    else if (b.w_packed)
      launch_g4p<EPI_PARTIAL>(b, pp, s);
    else
      launch_g4<EPI_PARTIAL>(b, p4, s);
    return launch_split_finish(b, epi, post, plan, s);
  }
  hipError_t e = launch_gemm(a, dt, epi, s);
  if (e != hipSuccess) return e;
  return post.mode == POST_NORM ? launch_norm(post.na, dt, s) : launch_qk_norm_rope(post.qa, dt, s);
}

// MXFP8 quantisation (OCP microscaling, 32-element blocks along a row): shared exponent
// e = floor(log2(amax)) - 8 (8 = exponent of e4m3's largest power of two), clamped to >= -127; the
// codes are e4m3 of x * 2^-e (exact scaling) saturated to +-448 and rounded to nearest even by the
// conversion instruction; the scale byte is e + 127. LPB lanes share a block, each with 16 bytes of
// it (8 bf16 or 4 float values), so a wave's loads and stores cover contiguous bytes; the block
// maximum is a butterfly over the LPB lanes.
template <typename T>
__global__ void __launch_bounds__(256) mx_quantize_kernel(const T* src, long ld, int rows, int cols, uint8_t* codes,
                                                          long ldq, uint8_t* scales) {
  constexpr int LPB = sizeof(T) == 2 ? 4 : 8, VALS = 32 / LPB;
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long blk = gid / LPB;
  const int part = (int)(gid % LPB);
  const int nb = cols / 32;
  const bool live = blk < (long)rows * nb;   // whole groups of LPB lanes agree (LPB divides 256)
  const int r = live ? (int)(blk / nb) : 0, b = live ? (int)(blk % nb) : 0;
  float v[VALS];
  if (live) {
    const uint4 w = *reinterpret_cast<const uint4*>(src + (long)r * ld + b * 32 + part * VALS);
    if constexpr (sizeof(T) == 2) {
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(ww[k] << 16);
        v[2 * k + 1] = __uint_as_float(ww[k] & 0xffff0000u);
      }
    } else {
      v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y); v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < VALS; ++i) v[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < VALS; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < LPB; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (!live) return;
  const int e = mx_block_exponent(amax);
  const float inv = mx_inv_scale(e);
  uint8_t* out = codes + (long)r * ldq + b * 32 + part * VALS;
  if constexpr (VALS == 8) {
    *reinterpret_cast<uint2*>(out) = make_uint2(mx_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv),
                                                mx_pack4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv));
  } else {
    *reinterpret_cast<uint32_t*>(out) = mx_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  }
  if (part == 0) scales[(long)r * nb + b] = (uint8_t)(e + 127);
}

// e2m1 code of |y| <= 6 (y already scaled), nearest with ties to even: the midpoints 0.25, 0.75, 1.25,
// 1.75, 2.5, 3.5, 5 go to the neighbour with mantissa bit 0
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t m = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.f ? 6u : 7u;
  return m | (__float_as_uint(y) >> 31 << 3);
}

// MXFP4 weights: as mx_quantize_kernel with the block exponent floor(log2 amax) - 2 (2 = exponent of
// e2m1's largest power of two), values saturated to +-6; each lane packs its values two per byte.
template <typename T>
__global__ void __launch_bounds__(256) mx4_quantize_kernel(const T* src, long ld, int rows, int cols, uint8_t* codes,
                                                           long ldq, uint8_t* scales) {
  constexpr int LPB = sizeof(T) == 2 ? 4 : 8, VALS = 32 / LPB;
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long blk = gid / LPB;
  const int part = (int)(gid % LPB);
  const int nb = cols / 32;
  const bool live = blk < (long)rows * nb;
  const int r = live ? (int)(blk / nb) : 0, b = live ? (int)(blk % nb) : 0;
  float v[VALS];
  if (live) {
    const uint4 w = *reinterpret_cast<const uint4*>(src + (long)r * ld + b * 32 + part * VALS);
    if constexpr (sizeof(T) == 2) {
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(ww[k] << 16);
        v[2 * k + 1] = __uint_as_float(ww[k] & 0xffff0000u);
      }
    } else {
      v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y); v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < VALS; ++i) v[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < VALS; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = 1; o < LPB; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (!live) return;
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xff);
  const int e = ebits == 0 ? -127 : max(ebits - 127 - 2, -127);
  const float inv = mx_inv_scale(e);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < VALS; ++i) word |= e2m1_code(fminf(fmaxf(v[i] * inv, -6.f), 6.f)) << (4 * i);
  uint8_t* out = codes + (long)r * ldq + b * 16 + part * (VALS / 2);
  if constexpr (VALS == 8)
    *reinterpret_cast<uint32_t*>(out) = word;
  else
    *reinterpret_cast<uint16_t*>(out) = (uint16_t)word;
  if (part == 0) scales[(long)r * nb + b] = (uint8_t)(e + 127);
}

hipError_t launch_mx4_quantize(const void* src, long ld_src, DType dt, int rows, int cols, uint8_t* codes, long ldq,
                               uint8_t* scales, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 32 || ldq % 16 || ldq < cols / 2 || reinterpret_cast<uintptr_t>(codes) % 16 ||
      reinterpret_cast<uintptr_t>(src) % 16 || ld_src % (dt == DT_BF16 ? 8 : 4))
    return hipErrorInvalidValue;
  const long lanes = (long)rows * (cols / 32) * (dt == DT_BF16 ? 4 : 8);
  const dim3 grid((unsigned)((lanes + 255) / 256)), block(256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL((mx4_quantize_kernel<bf16_t>), grid, block, 0, s, reinterpret_cast<const bf16_t*>(src), ld_src,
                       rows, cols, codes, ldq, scales);
  else
    hipLaunchKernelGGL((mx4_quantize_kernel<float>), grid, block, 0, s, reinterpret_cast<const float*>(src), ld_src,
                       rows, cols, codes, ldq, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(const void* src, long ld_src, DType dt, int rows, int cols, uint8_t* codes, long ldq,
                              uint8_t* scales, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 32 || ldq % 16 || reinterpret_cast<uintptr_t>(codes) % 16 || reinterpret_cast<uintptr_t>(src) % 16 ||
      ld_src % (dt == DT_BF16 ? 8 : 4))
    return hipErrorInvalidValue;
  const long lanes = (long)rows * (cols / 32) * (dt == DT_BF16 ? 4 : 8);
  const dim3 grid((unsigned)((lanes + 255) / 256)), block(256);
  if (dt == DT_BF16)
    hipLaunchKernelGGL((mx_quantize_kernel<bf16_t>), grid, block, 0, s, reinterpret_cast<const bf16_t*>(src), ld_src,
                       rows, cols, codes, ldq, scales);
  else
    hipLaunchKernelGGL((mx_quantize_kernel<float>), grid, block, 0, s, reinterpret_cast<const float*>(src), ld_src,
                       rows, cols, codes, ldq, scales);
  return hipGetLastError();
}

// Splits over K of the MXFP8 product: as the bf16 product, about 240 workgroups when there are fewer
// than 128 tiles and a partial buffer, each split at least two 128-k tiles.
static int mx_splits(const GemmArgs& a) {
  const long tiles = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
  const int KT = a.K / 128;
  int splits = 1;
  if (tiles < 128 && a.part) {
    splits = (int)((240 + tiles - 1) / tiles);
    if (splits > 4) splits = 4;
    while (splits > 1 && (KT < 2 * splits || (long)splits * a.M * a.N > a.part_elems)) --splits;
  }
  return splits;
}

static bool mx_operands_ok(const GemmArgs& a) {
  return a.K % 128 == 0 && a.N % 4 == 0 && a.As && a.Ws && (long)a.M * a.lda < (1L << 31) &&
         (long)a.N * a.ldw < (1L << 31) && a.lda % 16 == 0 && a.ldw % 16 == 0 && aligned16(a.A) && aligned16(a.W) &&
         reinterpret_cast<uintptr_t>(a.As) % 4 == 0 && reinterpret_cast<uintptr_t>(a.Ws) % 4 == 0;
}

static void launch_g4mx_partial(const GemmArgs& a, int splits, hipStream_t s) {
  const long tiles = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
  const int units = (int)tiles * splits;
  if (a.w_fp4)
    hipLaunchKernelGGL((gemm4mx_kernel<EPI_PARTIAL, true>), dim3(8 * ((units + 7) / 8)), dim3(256), 0, s, a, splits);
  else
    hipLaunchKernelGGL((gemm4mx_kernel<EPI_PARTIAL>), dim3(8 * ((units + 7) / 8)), dim3(256), 0, s, a, splits);
}

hipError_t launch_gemm_mx(const GemmArgs& a, Epi epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!mx_operands_ok(a) || epi == EPI_ROWSEL_F32) return hipErrorInvalidValue;
  if (epi == EPI_SWIGLU && a.N % 2) return hipErrorInvalidValue;
  const bool vec_ok = (!a.bias || aligned16(a.bias)) &&
                      (epi == EPI_STORE || epi == EPI_GELU || epi == EPI_SWIGLU
                           ? (reinterpret_cast<uintptr_t>(a.C) % 8 == 0 && a.ldc % 4 == 0)
                           : (aligned16(a.H) && a.ldh % 4 == 0)) &&
                      (epi != EPI_RESID_GATED || (aligned16(a.e6) && aligned16(a.mod) && a.D % 4 == 0));
  if (!vec_ok) return hipErrorInvalidValue;
  const long tiles = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
  const int splits = mx_splits(a);
  if (splits > 1) {   // fp32 partials summed in split order
    launch_g4mx_partial(a, splits, s);
    launch_reduce(a, epi, splits, s);
    return hipGetLastError();
  }
  const dim3 grid(8 * (((int)tiles + 7) / 8)), block(256);
#define WAM_MX_CASE(E)                                                                             \
  case E:                                                                                          \
    if (a.w_fp4) hipLaunchKernelGGL((gemm4mx_kernel<E, true>), grid, block, 0, s, a, 1);           \
    else hipLaunchKernelGGL((gemm4mx_kernel<E>), grid, block, 0, s, a, 1);                         \
    break;
  switch (epi) {
    WAM_MX_CASE(EPI_STORE)
    WAM_MX_CASE(EPI_GELU)
    WAM_MX_CASE(EPI_SWIGLU)
    WAM_MX_CASE(EPI_RESID)
    WAM_MX_CASE(EPI_RESID_GATED)
    default: return hipErrorInvalidValue;
  }
#undef WAM_MX_CASE
  return hipGetLastError();
}

}  // namespace wam
