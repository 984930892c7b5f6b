// Shared device helpers for the gfx950 (CDNA4) kernels of the chunk-causal DiT step.
//
// Element types: bf16 values are carried as raw 16-bit patterns (uint16_t) in memory and
// converted with round-to-nearest-even; the fp32 debug build of every kernel uses float.
// Matrix products go through the 32x32 MFMA family in "k16 chunks": a chunk of 16 consecutive
// k-values, of which lane half h (lanes 32h..32h+31) supplies elements 8h..8h+7. For bf16 that is
// one v_mfma_f32_32x32x16_bf16; for fp32 it is eight v_mfma_f32_32x32x2_f32, the t-th consuming
// element t of each half's eight -- the same contraction with the k-order permuted identically on
// both operands.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wam {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// two fp32 -> packed bf16 pair (low half = a), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const float2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// ---- MXFP8 (OCP microscaling: fp8 e4m3 codes, one e8m0 scale per 32 consecutive values of a row) ----
// Shared exponent e = floor(log2(amax)) - 8 (8 = exponent of e4m3's largest power of two), clamped to
// >= -127; codes = e4m3(x * 2^-e) saturated to +-448, nearest even; scale byte e + 127.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xff);   // 0 for zero and fp32 subnormals
  return ebits == 0 ? -127 : max(ebits - 127 - 8, -127);
}

__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// four values (already multiplied by 2^-e) -> four e4m3 bytes, little-endian in one word
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float bf16_round(float x) { return bf16_to_f32(f32_to_bf16(x)); }

// Columns 4q .. 4q+3 of a row, held by one lane; the 8 lanes of an aligned group hold one 32-column
// block and share its scale (butterfly maximum). Every lane of the wave calls this (act = the lane
// holds data); codes / scales point at the row.
__device__ __forceinline__ void mx_store_quad(float4 o, bool act, uint8_t* codes, uint8_t* scales, int q) {
  float amax = act ? fmaxf(fmaxf(fabsf(o.x), fabsf(o.y)), fmaxf(fabsf(o.z), fabsf(o.w))) : 0.f;
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
  if (!act) return;
  const int e = mx_block_exponent(amax);
  const float inv = mx_inv_scale(e);
  reinterpret_cast<uint32_t*>(codes)[q] = mx_pack4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  if ((q & 7) == 0) scales[q >> 3] = (uint8_t)(e + 127);
}

// Generic element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16_t* p, float v) { *p = f32_to_bf16(v); }
  static __device__ __forceinline__ float to_f(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f(float v) { return f32_to_bf16(v); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};

// A k16 fragment: the eight elements one lane contributes to a 32x32 MFMA chunk.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> { uint4 v; };            // 8 x bf16 = 16 bytes
template <> struct Frag<float> { uint4 v[2]; };          // 8 x f32  = 32 bytes

__device__ __forceinline__ void mfma_k16(floatx16& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  bf16x8_t av = __builtin_bit_cast(bf16x8_t, a.v);
  bf16x8_t bv = __builtin_bit_cast(bf16x8_t, b.v);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
}

__device__ __forceinline__ void mfma_k16(floatx16& acc, const Frag<float>& a, const Frag<float>& b) {
  const float* af = reinterpret_cast<const float*>(&a.v[0]);
  const float* bf = reinterpret_cast<const float*>(&b.v[0]);
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(af[t], bf[t], acc, 0, 0, 0);
}

// Pack eight fp32 values (already in k order) into a fragment.
__device__ __forceinline__ void pack_frag(Frag<bf16_t>& f, const float* x) {
  f.v = make_uint4(pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3]), pack2_bf16(x[4], x[5]), pack2_bf16(x[6], x[7]));
}
__device__ __forceinline__ void pack_frag(Frag<float>& f, const float* x) {
  f.v[0] = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
  f.v[1] = make_uint4(__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7]));
}

// Output layout of a 32x32 MFMA accumulator: lane l, register r holds
// row = 8*(r/4) + 4*(l/32) + (r%4), column = l%32.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Wave-wide (64 lanes) reductions by butterfly shuffles; every lane gets the result.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum for blockDim.x = NT threads (multiple of 64); deterministic order.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red /* >= NT/64 floats of LDS */) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  return s;
}

// GELU, tanh form: 0.5 x (1 + tanh(u)) with u = sqrt(2/pi) (x + 0.044715 x^3), evaluated through the
// identity 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)): one v_exp_f32 and one v_rcp_f32 (about 1e-7
// relative). Saturates correctly: exp -> inf gives 0, exp -> 0 gives x.
__device__ __forceinline__ float gelu_tanh_f(float x) {
  const float c2 = -2.f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float e = __builtin_amdgcn_exp2f(c2 * (x + 0.044715f * x * x * x));
  return x * __builtin_amdgcn_rcpf(1.f + e);
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.f + expf(-x)); }

}  // namespace wam
