// NF4 quantise and dequantise kernels.
//
// Quantise: 16 lanes own one 64-element block (a float4 each), reduce max|w|
// across the 16 lanes, divide each element by the absmax with IEEE fp32
// division and count how many fp32 midpoints of the 16 levels lie strictly
// below it (a tie goes to the lower level).  Codes are packed two per byte,
// the first element in the high nibble.
//
// Dequantise: a thread owns 32 consecutive elements (16 packed bytes, one
// absmax) and decodes them with the same table routine the GEMMs use, so the
// bytes this kernel writes are exactly the bf16 weights the GEMMs multiply.
// The output goes through LDS so that every store instruction of a wave
// writes 1 KB of contiguous memory.
#include "common.h"
#include "kernels.h"

namespace lsf {
namespace {

struct Mid {
  float t[15];
};
constexpr Mid make_mid() {
  constexpr float L[16] = {
      -1.0f, -0.6961928009986877f, -0.5250730514526367f, -0.39491748809814453f,
      -0.28444138169288635f, -0.18477343022823334f, -0.09105003625154495f, 0.0f,
      0.07958029955625534f, 0.16093020141124725f, 0.24611230194568634f, 0.33791524171829224f,
      0.44070982933044434f, 0.5626170039176941f, 0.7229568362236023f, 1.0f};
  Mid m{};
  for (int k = 0; k < 15; ++k) m.t[k] = (L[k] + L[k + 1]) * 0.5f;  // fp32 sum, exact halving
  return m;
}
constexpr Mid kMid = make_mid();

__device__ __forceinline__ uint32_t code_of(float x) {
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 15; ++k) c += (x > kMid.t[k]) ? 1u : 0u;
  return c;
}

__global__ __launch_bounds__(256) void nf4_quantize_kernel(const float* __restrict__ w, int64_t nblocks,
                                                           uint8_t* __restrict__ packed,
                                                           float* __restrict__ absmax) {
  const int sub = threadIdx.x & 15;
  const int64_t groups_per_grid = (int64_t)gridDim.x * (blockDim.x >> 4);
  for (int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 4) + (threadIdx.x >> 4); b < nblocks + 0;
       b += groups_per_grid) {
    const float4 v = reinterpret_cast<const float4*>(w + b * 64)[sub];
    float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
    uint32_t c0 = 7, c1 = 7, c2 = 7, c3 = 7;
    if (m > 0.0f) {
      c0 = code_of(v.x / m);
      c1 = code_of(v.y / m);
      c2 = code_of(v.z / m);
      c3 = code_of(v.w / m);
    }
    // elements 4*sub .. 4*sub+3 -> bytes 2*sub, 2*sub+1 (little-endian u16)
    const uint16_t out = (uint16_t)(((c0 << 4) | c1) | (((c2 << 4) | c3) << 8));
    reinterpret_cast<uint16_t*>(packed + b * 32)[sub] = out;
    if (sub == 0) absmax[b] = m;
  }
}

// A thread decodes 32 weights (64 output bytes) into LDS; the wave then writes
// its 4 KB of output with four fully contiguous 16-byte-per-lane stores.
__device__ __forceinline__ void stage_and_store(const uint32_t (&o)[16], bool live, int64_t base, int64_t nunits,
                                                u32x4* __restrict__ out16, u32x4* stage) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (live) {
#pragma unroll
    for (int k = 0; k < 4; ++k) stage[tid * 4 + k] = u32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = k * 64 + lane;             // 16-byte chunk of this wave's output
    const int64_t unit = base + wv * 64 + (c >> 2);
    if (unit < nunits) out16[(base + wv * 64) * 4 + c] = stage[wv * 256 + c];
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void nf4_dequantize_kernel(const uint8_t* __restrict__ packed,
                                                             const float* __restrict__ absmax, int64_t nunits,
                                                             uint16_t* __restrict__ out) {
  __shared__ u32x4 stage[256 * 4];
  for (int64_t base = (int64_t)blockIdx.x * 256; base < nunits; base += (int64_t)gridDim.x * 256) {
    const int64_t u = base + threadIdx.x;
    const bool live = u < nunits;
    uint32_t o[16] = {};
    if (live) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(packed + u * 16);
      const Nf4Table t = nf4_table(absmax[u >> 1]);
      nf4_decode8(t, q.x, reinterpret_cast<uint32_t(&)[4]>(o[0]));
      nf4_decode8(t, q.y, reinterpret_cast<uint32_t(&)[4]>(o[4]));
      nf4_decode8(t, q.z, reinterpret_cast<uint32_t(&)[4]>(o[8]));
      nf4_decode8(t, q.w, reinterpret_cast<uint32_t(&)[4]>(o[12]));
    }
    stage_and_store(o, live, base, nunits, reinterpret_cast<u32x4*>(out), stage);
  }
}

// Second-level code of the absmax values: one workgroup per group of 256
// blocks; offset = min, scale = (max - min) / 255 (IEEE division), code =
// clamp(rint((a - min) / scale), 0, 255), ties to even.
__global__ __launch_bounds__(256) void dq_encode_kernel(const float* __restrict__ absmax, int64_t nb,
                                                        uint8_t* __restrict__ codes, float2* __restrict__ s2) {
  __shared__ float red_lo[4], red_hi[4];
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = b < nb;
  const float a = live ? absmax[b] : 0.0f;
  float lo = live ? a : INFINITY, hi = live ? a : -INFINITY;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
  }
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red_lo[wid] = lo; red_hi[wid] = hi; }
  __syncthreads();
  lo = fminf(fminf(red_lo[0], red_lo[1]), fminf(red_lo[2], red_lo[3]));
  hi = fmaxf(fmaxf(red_hi[0], red_hi[1]), fmaxf(red_hi[2], red_hi[3]));
  const float scale = __fdiv_rn(__fsub_rn(hi, lo), 255.0f);
  if (live) {
    uint32_t c = 0;
    if (scale > 0.0f) {
      const float q = rintf(__fdiv_rn(__fsub_rn(a, lo), scale));
      c = (uint32_t)fminf(fmaxf(q, 0.0f), 255.0f);
    }
    codes[b] = (uint8_t)c;
  }
  if (threadIdx.x == 0) s2[blockIdx.x] = make_float2(scale, lo);
}

__global__ __launch_bounds__(256) void nf4dq_dequantize_kernel(const uint8_t* __restrict__ packed,
                                                               const uint8_t* __restrict__ absq,
                                                               const float2* __restrict__ s2, int64_t nunits,
                                                               uint16_t* __restrict__ out) {
  __shared__ u32x4 stage[256 * 4];
  for (int64_t base = (int64_t)blockIdx.x * 256; base < nunits; base += (int64_t)gridDim.x * 256) {
    const int64_t u = base + threadIdx.x;
    const bool live = u < nunits;
    uint32_t o[16] = {};
    if (live) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(packed + u * 16);
      const int64_t blk = u >> 1;
      const float2 so = s2[blk >> 8];
      const Nf4Table t = nf4_table(dq_absmax_value(absq[blk], so.x, so.y));
      nf4_decode8(t, q.x, reinterpret_cast<uint32_t(&)[4]>(o[0]));
      nf4_decode8(t, q.y, reinterpret_cast<uint32_t(&)[4]>(o[4]));
      nf4_decode8(t, q.z, reinterpret_cast<uint32_t(&)[4]>(o[8]));
      nf4_decode8(t, q.w, reinterpret_cast<uint32_t(&)[4]>(o[12]));
    }
    stage_and_store(o, live, base, nunits, reinterpret_cast<u32x4*>(out), stage);
  }
}

}  // namespace

hipError_t dq_encode_launch(const float* absmax, int64_t nblocks, uint8_t* codes, float* scale2, hipStream_t s) {
  if (nblocks <= 0) return hipSuccess;
  const int64_t groups = (nblocks + 255) / 256;
  hipLaunchKernelGGL(dq_encode_kernel, dim3((unsigned)groups), dim3(256), 0, s, absmax, nblocks, codes,
                     reinterpret_cast<float2*>(scale2));
  return hipGetLastError();
}

hipError_t nf4dq_dequantize_launch(const uint8_t* packed, const uint8_t* absq, const float* scale2, int64_t n,
                                   uint16_t* out, hipStream_t s) {
  const int64_t units = n / 32;
  if (units == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((units + 255) / 256, 65536);
  hipLaunchKernelGGL(nf4dq_dequantize_kernel, dim3(grid), dim3(256), 0, s, packed, absq,
                     reinterpret_cast<const float2*>(scale2), units, out);
  return hipGetLastError();
}

hipError_t nf4_quantize_launch(const float* w, int64_t n, uint8_t* packed, float* absmax, hipStream_t s) {
  const int64_t nblocks = n / 64;
  if (nblocks == 0) return hipSuccess;
  const int64_t want = (nblocks + 15) / 16;
  const int grid = (int)std::min<int64_t>(want, 65536);
  hipLaunchKernelGGL(nf4_quantize_kernel, dim3(grid), dim3(256), 0, s, w, nblocks, packed, absmax);
  return hipGetLastError();
}

hipError_t nf4_dequantize_launch(const uint8_t* packed, const float* absmax, int64_t n, uint16_t* out,
                                 hipStream_t s) {
  const int64_t units = n / 32;
  if (units == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((units + 255) / 256, 65536);
  hipLaunchKernelGGL(nf4_dequantize_kernel, dim3(grid), dim3(256), 0, s, packed, absmax, units, out);
  return hipGetLastError();
}

}  // namespace lsf
