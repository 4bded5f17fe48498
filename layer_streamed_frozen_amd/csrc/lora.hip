// LoRA side paths that are not folded into the base GEMMs.
//
// lora_down: the rank-r projections U = s X A^T (forward) and dU = s dY B
// (backward).  Skinny [M, K] x [K, r] products on MFMA: a workgroup owns 16
// rows and 16 adapter columns of one section; its four waves split the
// contraction and their partial tiles are summed in a fixed order in LDS.
//
// lora_grad: the adapter gradients dA = dU^T X and dB = s dY^T U, reductions
// over the tokens.  A lane owns one input/output feature and all r adapter
// columns; the four waves of a workgroup take interleaved token rows and are
// summed in a fixed order, then added (+=) into the fp32 gradient.  No atomics,
// so the result is the same bits on every run.
#include "common.h"
#include "kernels.h"

namespace lsf {
namespace {

__global__ __launch_bounds__(256) void lora_down_kernel(LoraDown a) {
  __shared__ float red[4][16][17];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.x * 16;
  const int sec = blockIdx.y;
  const int j0 = blockIdx.z * 16;
  const float* mat = a.mat[sec];
  f32x4 acc = {0, 0, 0, 0};
  if (mat != nullptr) {
    const int m = m0 + lr;
    const int j = j0 + lr;
    const uint16_t* xrow = a.X + (int64_t)min(m, a.M - 1) * a.ldx + a.xoff[sec];
    const int Ks = a.ksec[sec] > 0 ? a.ksec[sec] : a.K;
    const int steps = Ks / 32;
    for (int st = wid; st < steps; st += 4) {
      const int k = st * 32 + lg * 8;
      u32x4 xa = *reinterpret_cast<const u32x4*>(xrow + k);
      if (m >= a.M) xa = u32x4{0, 0, 0, 0};
      float v[8];
      if (j < a.r) {
        if (!a.bside) {
          const float4* src = reinterpret_cast<const float4*>(mat + (int64_t)j * a.K + k);
          const float4 p = src[0], q = src[1];
          v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w; v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = mat[(int64_t)(k + e) * a.r + j];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
      }
      const u32x4 bb = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                        pack_bf16x2(v[6], v[7])};
      acc = mfma16x16x32(xa, bb, acc);
    }
  }
  // acc[i] = C[row lg*4 + i][col lr]
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wid][lg * 4 + i][lr] = acc[i];
  __syncthreads();
  if (tid < 256) {
    const int row = tid >> 4, col = tid & 15;
    const float v = ((red[0][row][col] + red[1][row][col]) + red[2][row][col]) + red[3][row][col];
    const int m = m0 + row, j = j0 + col;
    if (m < a.M && j < a.r) a.U[(int64_t)m * a.ldu + sec * a.r + j] = a.scale * v;
  }
}

struct GradBatch {
  LoraGradSec s[3];
};

template <int R>
__global__ __launch_bounds__(256) void lora_grad_kernel(GradBatch gb, int T) {
  __shared__ float red[4][R][64];
  const LoraGradSec& g = gb.s[blockIdx.y];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int q = blockIdx.x * 64 + lane;
  if (blockIdx.x * 64 >= g.nq) return;  // whole workgroup idle for this section
  const bool live = q < g.nq;
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0.0f;
  for (int t = wid; t < T; t += 4) {
    const float qv = live ? bf16_to_f32(g.Q[(int64_t)t * g.ldq + g.qoff + q]) : 0.0f;
    const float* prow = g.P + (int64_t)t * g.ldp + g.pcol0;
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] = fmaf(prow[j], qv, acc[j]);
  }
#pragma unroll
  for (int j = 0; j < R; ++j) red[wid][j][lane] = acc[j];
  __syncthreads();
  if (wid == 0 && live) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float v = ((red[0][j][lane] + red[1][j][lane]) + red[2][j][lane]) + red[3][j][lane];
      float* dst = g.transposed ? g.out + (int64_t)q * R + j : g.out + (int64_t)j * g.nq + q;
      *dst += g.scale * v;
    }
  }
}

}  // namespace

hipError_t lora_down(const LoraDown& a, hipStream_t s) {
  if (a.M <= 0 || a.nsec <= 0) return hipSuccess;
  dim3 grid((a.M + 15) / 16, a.nsec, (a.r + 15) / 16);
  hipLaunchKernelGGL(lora_down_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t lora_grad(const LoraGradSec* secs, int nsec, int T, int r, hipStream_t s) {
  if (nsec <= 0 || T <= 0) return hipSuccess;
  GradBatch gb{};
  int maxq = 0;
  for (int i = 0; i < nsec; ++i) {
    gb.s[i] = secs[i];
    maxq = std::max(maxq, secs[i].nq);
  }
  dim3 grid((maxq + 63) / 64, nsec);
  switch (r) {
    case 4: hipLaunchKernelGGL(lora_grad_kernel<4>, grid, dim3(256), 0, s, gb, T); break;
    case 8: hipLaunchKernelGGL(lora_grad_kernel<8>, grid, dim3(256), 0, s, gb, T); break;
    case 16: hipLaunchKernelGGL(lora_grad_kernel<16>, grid, dim3(256), 0, s, gb, T); break;
    case 32: hipLaunchKernelGGL(lora_grad_kernel<32>, grid, dim3(256), 0, s, gb, T); break;
    case 64: hipLaunchKernelGGL(lora_grad_kernel<64>, grid, dim3(256), 0, s, gb, T); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lsf
