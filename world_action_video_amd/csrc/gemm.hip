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

hipError_t launch_gemm(const GemmArgs& a, DType dt, Epi epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  // buffer descriptors address each operand with 32-bit byte offsets
  const long esz = dt == DT_BF16 ? 2 : 4;
  if ((long)a.M * a.lda * esz >= (1L << 31) || (long)a.N * a.ldw * esz >= (1L << 31)) return hipErrorInvalidValue;
  // Tile choice (measured on MI355X over the step's shapes): the 256x256 tile with 8 waves (128x64 per
  // wave) when it yields enough tiles to cover most of the 256 CUs; otherwise 256x128 / 128x256 tiles
  // with 8 waves of 64x64, which double the tile count at M = 928 or 464; smaller tiles for tiny shapes.
  if (dt == DT_BF16) {
    const long t256 = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
    if (epi != EPI_ROWSEL_F32 && a.M >= 256 && a.N >= 256 && t256 >= 192)
      return launch_cfg<bf16_t, 256, 256, 128, 64, 8>(a, epi, s);
    if (epi != EPI_ROWSEL_F32 && a.M >= 256 && a.N >= 128) return launch_cfg<bf16_t, 256, 128, 64, 64, 8>(a, epi, s);
    if (epi != EPI_ROWSEL_F32 && a.M >= 128 && a.N >= 256) return launch_cfg<bf16_t, 128, 256, 64, 64, 8>(a, epi, s);
    if (a.N >= 128 && a.M >= 128) return launch_cfg<bf16_t, 128, 128, 64, 64, 4>(a, epi, s);
    return launch_cfg<bf16_t, 64, 64, 32, 32, 4>(a, epi, s);
  }
  if (a.N >= 128 && a.M >= 128) return launch_cfg<float, 128, 128, 64, 64, 4>(a, epi, s);
  return launch_cfg<float, 64, 64, 32, 32, 4>(a, epi, s);
}

}  // namespace wam
