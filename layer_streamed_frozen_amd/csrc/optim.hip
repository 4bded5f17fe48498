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

}  // namespace

size_t adamw_ws_bytes() { return (size_t)(kNormBlocks + 64) * sizeof(float); }

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
