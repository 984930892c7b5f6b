// Tiled MFMA GEMM for the linear layers of the DiT block: C = A W^T with fused epilogues.
//
// A [M][K] and W [N][K] are both k-contiguous, so every operand fragment is one (bf16) or two
// (fp32) 16-byte LDS reads. A workgroup is 4 waves (256 threads); each wave owns a WM x WN
// sub-tile built from 32x32 MFMA blocks. K is consumed in 128-byte tile rows (64 bf16 / 32 fp32),
// staged global -> registers -> LDS with two LDS buffers so the loads of tile k+1 overlap the
// MFMAs of tile k (one barrier per k-tile). LDS rows are 8 units of 16 bytes, XOR-swizzled by
// (row mod 8) so the 32 rows of a fragment read land on distinct banks.
//
// Tiles are assigned XCD-aware: workgroup b runs on XCD b mod 8, and each XCD receives one
// contiguous range of tiles ordered M-fastest, so the workgroups that share a W tile (the
// streamed operand) share one XCD's L2.
#include "common.h"
#include "kernels.h"

namespace wam {

template <typename T, int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
gemm_kernel(GemmArgs g) {
  constexpr int UNITS = 8;                 // 16-byte units per LDS tile row (128 bytes)
  constexpr int EPU = 16 / sizeof(T);      // elements per unit
  constexpr int BK = UNITS * EPU;          // k per tile: 64 (bf16) or 32 (fp32)
  constexpr int NWN = BN / WN;
  static_assert((BM / WM) * NWN == 4, "4 waves per workgroup");
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_PER_T = BM * UNITS / 256, B_PER_T = BN * UNITS / 256;
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
  const T* A = reinterpret_cast<const T*>(g.A);
  const T* W = reinterpret_cast<const T*>(g.W);
  const int KT = g.K / BK;

  uint4 ra[A_PER_T], rb[B_PER_T];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int u = tid + 256 * i, row = u >> 3, unit = u & 7;
      const int gm = m0 + row;
      ra[i] = (gm < g.M) ? *reinterpret_cast<const uint4*>(A + (long)gm * g.lda + (long)kt * BK + unit * EPU)
                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int u = tid + 256 * i, row = u >> 3, unit = u & 7;
      const int gn = n0 + row;
      rb[i] = (gn < g.N) ? *reinterpret_cast<const uint4*>(W + (long)gn * g.ldw + (long)kt * BK + unit * EPU)
                         : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int u = tid + 256 * i, row = u >> 3, unit = u & 7;
      smem[st][row * UNITS + (unit ^ (row & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int u = tid + 256 * i, row = u >> 3, unit = u & 7;
      smem[st][(BM + row) * UNITS + (unit ^ (row & 7))] = rb[i];
    }
  };

  floatx16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx16{};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) gload(kt + 1);
    const uint4* sa = smem[kt & 1];
    const uint4* sb = sa + BM * UNITS;
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const int u0 = (c * 16 + half * 8) / EPU;
      Frag<T> fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 32 + l32;
        uint4* dst = reinterpret_cast<uint4*>(&fa[i]);
#pragma unroll
        for (int q = 0; q < UPF; ++q) dst[q] = sa[row * UNITS + ((u0 + q) ^ (row & 7))];
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WN + j * 32 + l32;
        uint4* dst = reinterpret_cast<uint4*>(&fb[j]);
#pragma unroll
        for (int q = 0; q < UPF; ++q) dst[q] = sb[row * UNITS + ((u0 + q) ^ (row & 7))];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mfma_k16(acc[i][j], fa[i], fb[j]);
    }
    if (kt + 1 < KT) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue
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
        } else if constexpr (EPI == EPI_RESID) {
          g.H[(long)row * g.ldh + col] += v;
        } else if constexpr (EPI == EPI_RESID_GATED) {
          const int rb_ = row % g.rm.rows_per_branch;
          const int ch = rb_ / g.rm.Lq, grp = (rb_ % g.rm.Lq) < g.rm.Lv ? 0 : 1;
          const float gate = g.e6[((long)(ch * 2 + grp) * 6 + g.gate_idx) * g.D + col] + g.mod[g.gate_idx * g.D + col];
          g.H[(long)row * g.ldh + col] += gate * v;
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

template <typename T, int BM, int BN, int WM, int WN>
static hipError_t launch_cfg(const GemmArgs& a, Epi epi, hipStream_t s) {
  if constexpr (BM >= 256) {
    if (epi == EPI_ROWSEL_F32) return hipErrorInvalidValue;  // output heads never use the large tile
  }
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const dim3 grid(8 * ((tiles + 7) / 8)), block(256);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_STORE>), grid, block, 0, s, a); break;
    case EPI_GELU: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_GELU>), grid, block, 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_RESID>), grid, block, 0, s, a); break;
    case EPI_RESID_GATED:
      hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_RESID_GATED>), grid, block, 0, s, a);
      break;
    case EPI_ROWSEL_F32:
      if constexpr (BM < 256) hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI_ROWSEL_F32>), grid, block, 0, s, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, DType dt, Epi epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (dt == DT_BF16) {
    const long big = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
    if (epi != EPI_ROWSEL_F32 && a.N >= 256 && a.M >= 256 && big >= 192) return launch_cfg<bf16_t, 256, 256, 128, 128>(a, epi, s);
    if (a.N >= 128 && a.M >= 128) return launch_cfg<bf16_t, 128, 128, 64, 64>(a, epi, s);
    return launch_cfg<bf16_t, 64, 64, 32, 32>(a, epi, s);
  }
  if (a.N >= 128 && a.M >= 128) return launch_cfg<float, 128, 128, 64, 64>(a, epi, s);
  return launch_cfg<float, 64, 64, 32, 32>(a, epi, s);
}

}  // namespace wam
