// AdamW over one flat fp32 array of adapter parameters, with optional clipping
// of the global gradient norm.  HBM-bound: 16 bytes read and 12 written per
// value, 16-byte vector accesses, one pass.  The norm is a two-stage reduction
// over a grid whose size depends only on n, summed in a fixed order, so the
// result does not depend on scheduling.
#include <algorithm>
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace lsf {
namespace {

constexpr int kNormBlocks = 1024;

__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = warp_sum(v);
  const int wid = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wid] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// Stage 1: partial sums of squares; block b covers a grid-strided set of float4s.
__global__ __launch_bounds__(256) void sumsq_part_kernel(const float* __restrict__ g, int64_t n,
                                                         float* __restrict__ part) {
  __shared__ float red[4];
  const int64_t n4 = n / 4;
  const float4* g4 = reinterpret_cast<const float4*>(g);
  float s = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 x = g4[i];
    s += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const float x = g[n4 * 4 + threadIdx.x];
    s += x * x;
  }
  s = block_sum256(s, red);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// Stage 2: the norm and the clipping factor min(1, max_norm / (norm + 1e-6)).
__global__ __launch_bounds__(256) void norm_finish_kernel(const float* __restrict__ part, int nparts, float max_norm,
                                                          float* __restrict__ factor, float* __restrict__ norm_out) {
  __shared__ float red[4];
  float s = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += 256) s += part[i];
  s = block_sum256(s, red);
  if (threadIdx.x == 0) {
    const float nrm = sqrtf(s);
    *factor = max_norm > 0.0f ? fminf(1.0f, max_norm / (nrm + 1e-6f)) : 1.0f;
    if (norm_out != nullptr) *norm_out = nrm;
  }
}

struct AdamwArgs {
  float lr, beta1, beta2, eps, decay;  // decay = lr * weight_decay
  float step_size;                     // lr / (1 - beta1^t)
  float inv_sqrt_bc2;                  // 1 / sqrt(1 - beta2^t)
};

__device__ __forceinline__ void adamw1(float& p, float g, float& m, float& v, const AdamwArgs& a) {
  p = p - a.decay * p;
  m = a.beta1 * m + (1.0f - a.beta1) * g;
  v = a.beta2 * v + (1.0f - a.beta2) * (g * g);
  const float denom = sqrtf(v) * a.inv_sqrt_bc2 + a.eps;
  p = p - a.step_size * (m / denom);
}

__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v, int64_t n,
                                                    AdamwArgs a, const float* __restrict__ factor) {
  const float f = factor != nullptr ? *factor : 1.0f;
  const int64_t n4 = n / 4;
  float4* p4 = reinterpret_cast<float4*>(p);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  float4* m4 = reinterpret_cast<float4*>(m);
  float4* v4 = reinterpret_cast<float4*>(v);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 pp = p4[i], mm = m4[i], vv = v4[i];
    const float4 gg = g4[i];
    adamw1(pp.x, gg.x * f, mm.x, vv.x, a);
    adamw1(pp.y, gg.y * f, mm.y, vv.y, a);
    adamw1(pp.z, gg.z * f, mm.z, vv.z, a);
    adamw1(pp.w, gg.w * f, mm.w, vv.w, a);
    p4[i] = pp;
    m4[i] = mm;
    v4[i] = vv;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t i = n4 * 4 + threadIdx.x;
    float pp = p[i], mm = m[i], vv = v[i];
    adamw1(pp, g[i] * f, mm, vv, a);
    p[i] = pp;
    m[i] = mm;
    v[i] = vv;
  }
}

// ---------------------------------------------------------------------------
// AdamW with 8-bit moment states (block-wise dynamic code).  Each block of
// kQBlock values has one fp32 absmax per moment; a value is stored as the
// nearest entry of a fixed code of [-1, 1] (m, int8 offset from the zero entry)
// or [0, 1] (v, uint8) after division by the absmax.  Code values are
// +-(0.1 + 0.9 (j + 1) / 2^F) / 10^E: E leading zero bits after the sign, an
// indicator bit, F fraction bits (signed: 7 bits, F = 6 - E; unsigned: 8 bits,
// F = 7 - E), and 0.  The update runs in fp32 with every operation rounded (no
// contraction) so that its codes can be reproduced exactly.

constexpr int kQBlock = 2048;                      // values per absmax block
constexpr int kTabS = 255, kTabU = 256;            // signed / unsigned code sizes
constexpr int kTabOff = kNormBlocks + 64;          // tables start in the workspace (floats)
constexpr int kTabFloats = 256 + 256 + 256 + 256;  // TS, TU, midS, midU (padded)

__device__ __forceinline__ double code_value(int bits, int k) {
  // k-th smallest positive value (0-based) of the code with `bits` magnitude bits
  const int lg = 31 - __clz(k + 1);  // floor(log2(k + 1))
  const int e = bits - 1 - lg;        // decade
  const int f = bits - 1 - e;         // fraction bits
  const int j = k + 1 - (1 << f);
  constexpr double p10[8] = {1.0, 10.0, 100.0, 1000.0, 1e4, 1e5, 1e6, 1e7};
  return (0.1 + 0.9 * (double)(j + 1) / (double)(1 << f)) / p10[e];
}

// One workgroup of 256 threads: the two sorted code tables and their fp32
// midpoints, into tab[0..255] (signed, 255 used), tab[256..511] (unsigned),
// tab[512..767] (signed midpoints, 254), tab[768..1023] (unsigned, 255).
__global__ __launch_bounds__(256) void dyn_tables_kernel(float* __restrict__ tab) {
  __shared__ float ts[kTabS], tu[kTabU];
  const int i = threadIdx.x;
  if (i < 127) {
    const float v = (float)code_value(7, i);
    ts[128 + i] = v;
    ts[126 - i] = -v;
  }
  if (i == 127) ts[127] = 0.0f;
  if (i < 255) tu[1 + i] = (float)code_value(8, i);
  if (i == 255) tu[0] = 0.0f;
  __syncthreads();
  if (i < kTabS) tab[i] = ts[i];
  tab[256 + i] = tu[i];
  if (i < kTabS - 1) tab[512 + i] = (ts[i] + ts[i + 1]) * 0.5f;
  if (i < kTabU - 1) tab[768 + i] = (tu[i] + tu[i + 1]) * 0.5f;
}

// Number of entries of mid[0..len) strictly below y.
__device__ __forceinline__ int count_below(const float* mid, int len, float y) {
  int lo = 0, hi = len;
  while (lo < hi) {
    const int h = (lo + hi) >> 1;
    if (mid[h] < y) lo = h + 1;
    else hi = h;
  }
  return lo;
}

struct Adamw8Args {
  float beta1, beta2, omb1, omb2, eps, decay, step_size, inv_sqrt_bc2;
};

// One workgroup per block of kQBlock values, 8 per thread.
__global__ __launch_bounds__(256) void adamw8_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                     int8_t* __restrict__ qm, uint8_t* __restrict__ qv,
                                                     float* __restrict__ am, float* __restrict__ av, int64_t n,
                                                     Adamw8Args a, const float* __restrict__ factor,
                                                     const float* __restrict__ tab) {
#pragma clang fp contract(off)
  __shared__ float ts[256], tu[256], ms[256], mu[256];
  __shared__ float red_m[4], red_v[4];
  const int tid = threadIdx.x;
  ts[tid] = tab[tid];
  tu[tid] = tab[256 + tid];
  ms[tid] = tab[512 + tid];
  mu[tid] = tab[768 + tid];
  const int64_t blk = blockIdx.x;
  const int64_t i0 = blk * kQBlock + (int64_t)tid * 8;
  const float f = factor != nullptr ? *factor : 1.0f;
  const float am0 = am[blk], av0 = av[blk];
  __syncthreads();
  float pv[8], gv[8], m1[8], v1[8];
  int8_t cm[8];
  uint8_t cv[8];
  const bool full = i0 + 8 <= n;
  if (full) {
    const float4* p4 = reinterpret_cast<const float4*>(p + i0);
    const float4* g4 = reinterpret_cast<const float4*>(g + i0);
    const float4 pa = p4[0], pb = p4[1], ga = g4[0], gb = g4[1];
    pv[0] = pa.x; pv[1] = pa.y; pv[2] = pa.z; pv[3] = pa.w; pv[4] = pb.x; pv[5] = pb.y; pv[6] = pb.z; pv[7] = pb.w;
    gv[0] = ga.x; gv[1] = ga.y; gv[2] = ga.z; gv[3] = ga.w; gv[4] = gb.x; gv[5] = gb.y; gv[6] = gb.z; gv[7] = gb.w;
    const u32x2 cmw = *reinterpret_cast<const u32x2*>(qm + i0);
    const u32x2 cvw = *reinterpret_cast<const u32x2*>(qv + i0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cm[e] = (int8_t)(((e < 4 ? cmw.x : cmw.y) >> (8 * (e & 3))) & 0xFF);
      cv[e] = (uint8_t)(((e < 4 ? cvw.x : cvw.y) >> (8 * (e & 3))) & 0xFF);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool live = i0 + e < n;
      pv[e] = live ? p[i0 + e] : 0.0f;
      gv[e] = live ? g[i0 + e] : 0.0f;
      cm[e] = live ? qm[i0 + e] : (int8_t)0;
      cv[e] = live ? qv[i0 + e] : (uint8_t)0;
    }
  }
  float lm = 0.0f, lv = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float g1 = gv[e] * f;
    const float m0 = ts[(int)cm[e] + 127] * am0;
    const float v0 = tu[cv[e]] * av0;
    const float p1 = pv[e] - a.decay * pv[e];
    m1[e] = a.beta1 * m0 + a.omb1 * g1;
    v1[e] = a.beta2 * v0 + a.omb2 * (g1 * g1);
    const float den = sqrtf(v1[e]) * a.inv_sqrt_bc2 + a.eps;
    pv[e] = p1 - a.step_size * (m1[e] / den);
    if (i0 + e < n) {
      lm = fmaxf(lm, fabsf(m1[e]));
      lv = fmaxf(lv, v1[e]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lm = fmaxf(lm, __shfl_xor(lm, o, 64));
    lv = fmaxf(lv, __shfl_xor(lv, o, 64));
  }
  if ((tid & 63) == 0) {
    red_m[tid >> 6] = lm;
    red_v[tid >> 6] = lv;
  }
  __syncthreads();
  const float bm = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  const float bv = fmaxf(fmaxf(red_v[0], red_v[1]), fmaxf(red_v[2], red_v[3]));
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    cm[e] = (int8_t)(bm > 0.0f ? count_below(ms, kTabS - 1, m1[e] / bm) - 127 : 0);
    cv[e] = (uint8_t)(bv > 0.0f ? count_below(mu, kTabU - 1, v1[e] / bv) : 0);
  }
  if (full) {
    float4* p4 = reinterpret_cast<float4*>(p + i0);
    p4[0] = make_float4(pv[0], pv[1], pv[2], pv[3]);
    p4[1] = make_float4(pv[4], pv[5], pv[6], pv[7]);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      w[e >> 2] |= (uint32_t)(uint8_t)cm[e] << (8 * (e & 3));
      w[2 + (e >> 2)] |= (uint32_t)cv[e] << (8 * (e & 3));
    }
    *reinterpret_cast<u32x2*>(qm + i0) = u32x2{w[0], w[1]};
    *reinterpret_cast<u32x2*>(qv + i0) = u32x2{w[2], w[3]};
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (i0 + e < n) {
        p[i0 + e] = pv[e];
        qm[i0 + e] = cm[e];
        qv[i0 + e] = cv[e];
      }
  }
  if (tid == 0) {
    am[blk] = bm;
    av[blk] = bv;
  }
}

}  // namespace

size_t adamw_ws_bytes() { return (size_t)(kNormBlocks + 64) * sizeof(float); }
size_t adamw8_ws_bytes() { return (size_t)(kTabOff + kTabFloats) * sizeof(float); }
int64_t adamw8_blocks(int64_t n) { return (n + kQBlock - 1) / kQBlock; }

hipError_t adamw8_update(float* p, const float* g, int8_t* qm, uint8_t* qv, float* am, float* av, int64_t n,
                         float lr, float beta1, float beta2, float eps, float weight_decay, float max_grad_norm,
                         int step, float* grad_norm, float* ws, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool need_norm = max_grad_norm > 0.0f || grad_norm != nullptr;
  float* part = ws;
  float* factor = ws + kNormBlocks;
  if (need_norm) {
    const int64_t blocks = (n / 4 + 255) / 256;
    const int nb = (int)std::max<int64_t>(1, std::min<int64_t>(blocks, kNormBlocks));
    hipLaunchKernelGGL(sumsq_part_kernel, dim3(nb), dim3(256), 0, s, g, n, part);
    hipLaunchKernelGGL(norm_finish_kernel, dim3(1), dim3(256), 0, s, part, nb, max_grad_norm, factor, grad_norm);
  }
  float* tab = ws + kTabOff;
  hipLaunchKernelGGL(dyn_tables_kernel, dim3(1), dim3(256), 0, s, tab);
  // b^t by repeated multiplication in fp64 (bit-reproducible anywhere)
  double b1t = beta1, b2t = beta2;
  for (int i = 1; i < step; ++i) {
    b1t *= (double)beta1;
    b2t *= (double)beta2;
  }
  Adamw8Args a;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.omb1 = 1.0f - beta1;
  a.omb2 = 1.0f - beta2;
  a.eps = eps;
  a.decay = (float)((double)lr * (double)weight_decay);
  a.step_size = (float)((double)lr / (1.0 - b1t));
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - b2t));
  hipLaunchKernelGGL(adamw8_kernel, dim3((unsigned)adamw8_blocks(n)), dim3(256), 0, s, p, g, qm, qv, am, av, n, a,
                     max_grad_norm > 0.0f ? (const float*)factor : nullptr, (const float*)tab);
  return hipGetLastError();
}

hipError_t adamw_update(float* p, const float* g, float* m, float* v, int64_t n, float lr, float beta1, float beta2,
                        float eps, float weight_decay, float max_grad_norm, int step, float* grad_norm, float* ws,
                        hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool need_norm = max_grad_norm > 0.0f || grad_norm != nullptr;
  float* part = ws;
  float* factor = ws + kNormBlocks;
  if (need_norm) {
    const int64_t blocks = (n / 4 + 255) / 256;
    const int nb = (int)std::max<int64_t>(1, std::min<int64_t>(blocks, kNormBlocks));
    hipLaunchKernelGGL(sumsq_part_kernel, dim3(nb), dim3(256), 0, s, g, n, part);
    hipLaunchKernelGGL(norm_finish_kernel, dim3(1), dim3(256), 0, s, part, nb, max_grad_norm, factor, grad_norm);
  }
  AdamwArgs a;
  a.lr = lr;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.eps = eps;
  a.decay = (float)((double)lr * (double)weight_decay);
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  a.step_size = (float)((double)lr / bc1);
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  const int64_t blocks = (n / 4 + 255) / 256;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(blocks, 8192));
  hipLaunchKernelGGL(adamw_kernel, dim3(grid), dim3(256), 0, s, p, g, m, v, n, a,
                     max_grad_norm > 0.0f ? (const float*)factor : nullptr);
  return hipGetLastError();
}

}  // namespace lsf
