// Shared device helpers for the gfx950 kernels: vector types, bf16
// conversion, MFMA wrappers and the NF4 block decoder.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Round two floats to bfloat16 (nearest, ties to even: v_cvt_pk_bf16_f32) and
// pack them, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  return (uint16_t)(pack_bf16x2(a, 0.0f) & 0xFFFFu);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane s supplies the address of 4 consecutive bf16 values S[s][0..3]; lane i
// receives O[i][k] = S[(i >> 2) + 4k][i & 3].  So if lane s points at row
// base + (s >> 2), column cbase + 4 (s & 3) of a row-major tile, lane i gets
// column cbase + i of rows base .. base + 3: an MFMA operand whose contraction
// runs down the rows.
typedef short lsf_v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr4(const uint16_t* base, int off) {
  const lsf_v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) lsf_v4s*)(base + off));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The 16 NF4 levels (QLoRA's NormalFloat-4 values), fp32.
__device__ __forceinline__ float nf4_level(int i) {
  constexpr float L[16] = {
      -1.0f, -0.6961928009986877f, -0.5250730514526367f, -0.39491748809814453f,
      -0.28444138169288635f, -0.18477343022823334f, -0.09105003625154495f, 0.0f,
      0.07958029955625534f, 0.16093020141124725f, 0.24611230194568634f, 0.33791524171829224f,
      0.44070982933044434f, 0.5626170039176941f, 0.7229568362236023f, 1.0f};
  return L[i];
}

// Absmax of a block stored with an 8-bit code: fp32(fp32(code * scale) + offset),
// two roundings, never contracted into an fma.
__device__ __forceinline__ float dq_absmax_value(uint32_t code, float scale, float offset) {
#pragma clang fp contract(off)
  const float p = (float)code * scale;
  return p + offset;
}

// Byte planes of one block's scaled table e_i = bf16(level_i * absmax):
// lo[k] holds the low bytes of e_{4k..4k+3}, hi[k] the high bytes.  A code is
// then looked up with byte permutes instead of a per-element multiply.
struct Nf4Table {
  uint32_t lo[4], hi[4];
};

__device__ __forceinline__ Nf4Table nf4_table(float absmax) {
  uint32_t p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = pack_bf16x2(nf4_level(2 * j) * absmax, nf4_level(2 * j + 1) * absmax);
  Nf4Table t;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t.lo[k] = __builtin_amdgcn_perm(p[2 * k + 1], p[2 * k], 0x06040200u);
    t.hi[k] = __builtin_amdgcn_perm(p[2 * k + 1], p[2 * k], 0x07050301u);
  }
  return t;
}

// Look up four codes (one per byte of n, values 0..15).  Returns the low bytes
// and the high bytes of the four bf16 entries, byte i for code i.
__device__ __forceinline__ void nf4_lookup4(const Nf4Table& t, uint32_t n, uint32_t& lo, uint32_t& hi) {
  const uint32_t s = n & 0x07070707u;
  const uint32_t b = n & 0x08080808u;
  const uint32_t m = (b << 5) - (b >> 3);  // 0xFF in every byte whose code is >= 8
  const uint32_t lo_a = __builtin_amdgcn_perm(t.lo[1], t.lo[0], s);
  const uint32_t lo_b = __builtin_amdgcn_perm(t.lo[3], t.lo[2], s);
  const uint32_t hi_a = __builtin_amdgcn_perm(t.hi[1], t.hi[0], s);
  const uint32_t hi_b = __builtin_amdgcn_perm(t.hi[3], t.hi[2], s);
  lo = (lo_b & m) | (lo_a & ~m);
  hi = (hi_b & m) | (hi_a & ~m);
}

// Decode one packed dword (8 codes, element 2j in the high nibble of byte j)
// into 8 bf16 values in natural order: out[j] = elements 2j (low half), 2j+1.
__device__ __forceinline__ void nf4_decode8(const Nf4Table& t, uint32_t w, uint32_t out[4]) {
  uint32_t le, he, lo_, ho;
  nf4_lookup4(t, (w >> 4) & 0x0F0F0F0Fu, le, he);  // elements 0,2,4,6
  nf4_lookup4(t, w & 0x0F0F0F0Fu, lo_, ho);        // elements 1,3,5,7
  const uint32_t e01 = __builtin_amdgcn_perm(he, le, 0x05010400u);  // e0 | e2
  const uint32_t e23 = __builtin_amdgcn_perm(he, le, 0x07030602u);  // e4 | e6
  const uint32_t o01 = __builtin_amdgcn_perm(ho, lo_, 0x05010400u); // e1 | e3
  const uint32_t o23 = __builtin_amdgcn_perm(ho, lo_, 0x07030602u); // e5 | e7
  out[0] = __builtin_amdgcn_perm(o01, e01, 0x05040100u);  // e0 | e1
  out[1] = __builtin_amdgcn_perm(o01, e01, 0x07060302u);  // e2 | e3
  out[2] = __builtin_amdgcn_perm(o23, e23, 0x05040100u);  // e4 | e5
  out[3] = __builtin_amdgcn_perm(o23, e23, 0x07060302u);  // e6 | e7
}

// dg and du of one element from the input gradient v of a = silu(g) u, with
// no contraction into fused multiply-adds, so every kernel that applies it
// gets the same bits.
__device__ __forceinline__ void swiglu_grad(float v, float gv, float uv, float& dg, float& du) {
#pragma clang fp contract(off)
  const float sg = 1.0f / (1.0f + __expf(-gv));
  dg = v * uv * sg * (1.0f + gv * (1.0f - sg));
  du = v * gv * sg;
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace lsf
