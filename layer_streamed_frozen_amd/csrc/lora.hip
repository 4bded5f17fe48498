// LoRA side paths that are not folded into the base GEMMs, on MFMA.
//
// lora_down: the rank-r projections U = X A^T (forward) and dU = s dY B
// (backward): [M, K] x [K, r] with r <= 64 and K up to 28672.  The
// contraction is cut into at most 16 chunks (multiples of 256, one 256-column
// step each up to K = 4096, so most workgroups wait for one round of loads
// only); a workgroup
// owns 64 rows and one chunk of one section, stages the chunk's adapter
// matrix 256 columns at a time in LDS as bf16 [r][256] and runs
// v_mfma_f32_16x16x32_bf16 over it, loading the next 256 columns while it
// multiplies these.  The per-chunk partial products are then summed in a fixed
// order by a second kernel.
//
// lora_grad: the adapter gradients dA = dU^T X and dB = s dY^T U, reductions
// over the tokens: Out[j, k] += scale * sum_t P[t, j] Q[t, k] (or = when the
// section asks to overwrite: the first accumulation of a step).  The dA and dB
// sections of a projection group share one launch.  A workgroup
// owns 64 columns k, all r rows j and one share of the tokens; each wave takes
// a quarter of that share in 32-row chunks, staged in its own LDS region so the
// MFMA operands can run along the token axis (P transposed, Q read down its
// rows with transposing loads), loading chunk i+1 while it multiplies chunk i.  The four wave tiles are summed in a fixed order; the
// token shares, when there are several, are summed in order by a second
// kernel (the tokens are split only when the launch would otherwise have fewer
// than 256 busy workgroups), and the result is added (+=) into the fp32
// gradient.  No atomics: the same inputs give the same bits on every run.
#include "common.h"
#include "kernels.h"

namespace lsf {
namespace {

constexpr int KC = 256;       // contraction columns lora_down stages per step
constexpr int MS_LD = KC + 8; // LDS row stride (bf16) of the staged adapter chunk

__device__ __forceinline__ int off_r8(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

__host__ __device__ __forceinline__ int sec_k(const LoraDown& a, int sec) {
  return a.ksec[sec] > 0 ? a.ksec[sec] : a.K;
}

// Workgroup (row block, section * nch_max + chunk): rows blockIdx.x * 64 ..
// + 64, contraction columns [c * kc, (c + 1) * kc) of the section, 256 at a
// time.
template <int R, bool BSIDE>
__global__ __launch_bounds__(256) void lora_down_part_kernel(LoraDown a, int nch_max, int kc) {
  __shared__ __attribute__((aligned(16))) uint16_t Ms[64 * MS_LD];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int sec = blockIdx.y / nch_max, c = blockIdx.y % nch_max;
  const int Ks = sec_k(a, sec);
  const int kbeg = c * kc;
  const float* mat = a.mat[sec];
  if (kbeg >= Ks || mat == nullptr) return;  // uniform over the workgroup
  const int kend = min(Ks, kbeg + kc);
  const int nsub = (kend - kbeg + KC - 1) / KC;
  // Load order: the adapter sub-chunk (16-byte vectors), then this lane's X
  // fragments; they are converted and stored only after the previous
  // sub-chunk's MFMAs, so the loads overlap them.  Addresses are clamped into
  // range and unused values zeroed afterwards: loads under a branch would each
  // be waited for on the spot.
  constexpr int SMAX = (R * KC / 4 + 255) / 256;  // float4 per thread
  const int m = blockIdx.x * 64 + wid * 16 + lr;
  const uint16_t* xrow = a.X + (int64_t)min(m, a.M - 1) * a.ldx + a.xoff[sec] + lg * 8;
  float4 sv[SMAX];
  u32x4 xa[KC / 32];
  auto load = [&](int k0, int kn) {
    const int n4 = R * kn / 4;
#pragma unroll
    for (int u = 0; u < SMAX; ++u) {
      const int idx = min(tid + 256 * u, n4 - 1);
      if constexpr (!BSIDE) {
        const int q4 = kn / 4, j = idx / q4, k = (idx - j * q4) * 4;
        sv[u] = *reinterpret_cast<const float4*>(mat + (int64_t)j * Ks + k0 + k);
      } else {
        sv[u] = reinterpret_cast<const float4*>(mat + (int64_t)k0 * R)[idx];
      }
    }
#pragma unroll
    for (int st = 0; st < KC / 32; ++st)
      xa[st] = *reinterpret_cast<const u32x4*>(xrow + k0 + (st * 32 < kn ? st * 32 : 0));
  };
  constexpr int jt_n = (R + 15) / 16;
  f32x4 acc[jt_n];
#pragma unroll
  for (int jt = 0; jt < jt_n; ++jt) acc[jt] = f32x4{0, 0, 0, 0};
  load(kbeg, min(KC, kend - kbeg));
  for (int sc = 0; sc < nsub; ++sc) {
    const int k0 = kbeg + sc * KC;
    const int kn = min(KC, kend - k0);  // a multiple of 32
    if (sc > 0) __syncthreads();         // the previous sub-chunk's reads of Ms are done
    // the sub-chunk as bf16 [j][k] (B-side: element f of it is B[k0 + f / R][f % R])
    const int n4 = R * kn / 4;
#pragma unroll
    for (int u = 0; u < SMAX; ++u) {
      const int idx = tid + 256 * u;
      if (idx < n4) {
        if constexpr (!BSIDE) {
          const int q4 = kn / 4, j = idx / q4, k = (idx - j * q4) * 4;
          *reinterpret_cast<uint2*>(Ms + j * MS_LD + k) =
              make_uint2(pack_bf16x2(sv[u].x, sv[u].y), pack_bf16x2(sv[u].z, sv[u].w));
        } else {
          const int k = (4 * idx) / R, j = 4 * idx - k * R;  // R is a multiple of 4: one row k
          Ms[j * MS_LD + k] = f32_to_bf16(sv[u].x);
          Ms[(j + 1) * MS_LD + k] = f32_to_bf16(sv[u].y);
          Ms[(j + 2) * MS_LD + k] = f32_to_bf16(sv[u].z);
          Ms[(j + 3) * MS_LD + k] = f32_to_bf16(sv[u].w);
        }
      }
    }
    u32x4 xc[KC / 32];
#pragma unroll
    for (int st = 0; st < KC / 32; ++st) xc[st] = xa[st];
    __syncthreads();
    if (sc + 1 < nsub) load(k0 + KC, min(KC, kend - k0 - KC));
    // No branches around the MFMAs: steps past the sub-chunk, rows past M and
    // adapter rows past R multiply zeros.
#pragma unroll
    for (int st = 0; st < KC / 32; ++st) {
      const uint32_t xkeep = (st * 32 < kn && m < a.M) ? 0xffffffffu : 0u;
      const u32x4 x = {xc[st].x & xkeep, xc[st].y & xkeep, xc[st].z & xkeep, xc[st].w & xkeep};
      const int k = (st * 32 < kn ? st * 32 : 0) + lg * 8;
#pragma unroll
      for (int jt = 0; jt < jt_n; ++jt) {
        const int j = jt * 16 + lr;
        const u32x4 v = *reinterpret_cast<const u32x4*>(Ms + min(j, R - 1) * MS_LD + k);
        const uint32_t keep = (j < R) ? 0xffffffffu : 0u;
        const u32x4 bb = {v.x & keep, v.y & keep, v.z & keep, v.w & keep};
        acc[jt] = mfma16x16x32(x, bb, acc[jt]);
      }
    }
  }
  float* out = a.part + (size_t)(sec * nch_max + c) * a.M * R;
  const int mb = blockIdx.x * 64 + wid * 16 + lg * 4;
#pragma unroll
  for (int jt = 0; jt < jt_n; ++jt) {
    const int j = jt * 16 + lr;
    if (j >= R) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (mb + i < a.M) out[(size_t)(mb + i) * R + j] = acc[jt][i];
  }
}

__global__ __launch_bounds__(256) void lora_down_reduce_kernel(LoraDown a, int nch_max, int kc) {
  const int64_t total = (int64_t)a.M * a.nsec * a.r;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int j = (int)(i % a.r);
    const int64_t rest = i / a.r;
    const int sec = (int)(rest % a.nsec);
    const int64_t t = rest / a.nsec;
    float v = 0.0f;
    if (a.mat[sec] != nullptr) {
      const int nch = (sec_k(a, sec) + kc - 1) / kc;
      const size_t stride = (size_t)a.M * a.r;
      const float* p = a.part + (size_t)sec * nch_max * stride + (size_t)t * a.r + j;
      // eight loads in flight, then the adds in chunk order
      for (int c0 = 0; c0 < nch; c0 += 8) {
        float q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) q[u] = (c0 + u < nch) ? p[(size_t)(c0 + u) * stride] : 0.0f;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (c0 + u < nch) v += q[u];
      }
    }
    a.U[t * a.ldu + sec * a.r + j] = a.scale * v;
  }
}

struct GradBatch {
  LoraGradSec s[kLoraGradSecs];
};

constexpr int PS_LD = 40;  // LDS row stride (bf16) of the transposed P chunk

// This wave's LDS accesses so far are complete, and neither the compiler nor
// the hardware moves later ones ahead of them.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup (column tile, section, token split z): tokens
// [z * 4 * cpw * 32, (z + 1) * 4 * cpw * 32).  With one split the result is
// added into the gradient directly; with several, each split writes its
// partial [z][section][R][maxq] and lora_grad_reduce_kernel adds their sum.
template <int R>
__global__ __launch_bounds__(256) void lora_grad_kernel(GradBatch gb, int T, int cpw, float* part, int maxq) {
  __shared__ __attribute__((aligned(16))) uint16_t Qs[4][32 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[4][R * PS_LD];
  __shared__ float red[4][R][65];
  const LoraGradSec& g = gb.s[blockIdx.y];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int k0 = blockIdx.x * 64;
  if (k0 >= g.nq) return;  // uniform over the workgroup
  constexpr int JT = R / 16 > 0 ? R / 16 : 1;
  f32x4 acc[JT][4];
#pragma unroll
  for (int a = 0; a < JT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0, 0, 0, 0};
  // Each wave works on its own 32-token chunks and its own LDS regions, so
  // between staging and reading a chunk it only has to wait for its own LDS
  // writes (LDS operations of one wave complete in order); the global loads of
  // the next chunk are issued before the current one is read.
  u32x4 qv[4];
  float pv[R / 2];
  auto load = [&](int ci) {
    const int t0 = (((int)blockIdx.z * 4 + wid) * cpw + ci) * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = lane + 64 * i;
      const int row = idx >> 3, ch = idx & 7;
      const int t = t0 + row, k = k0 + ch * 8;
      qv[i] = u32x4{0, 0, 0, 0};
      if (t < T && k < g.nq) qv[i] = *reinterpret_cast<const u32x4*>(g.Q + (int64_t)t * g.ldq + g.qoff + k);
    }
    const int t = lane >> 1, jh = (lane & 1) * (R / 2);
    const bool ok = t0 + t < T;
    const float* prow = g.P + (int64_t)(t0 + t) * g.ldp + g.pcol0 + jh;
#pragma unroll
    for (int e = 0; e < R / 2; ++e) pv[e] = ok ? prow[e] : 0.0f;
  };
  if (cpw > 0) load(0);
  for (int ci = 0; ci < cpw; ++ci) {
    // Q chunk: 32 tokens x 64 columns; P chunk transposed to [j][t] bf16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = lane + 64 * i;
      *reinterpret_cast<u32x4*>(Qs[wid] + off_r8(idx >> 3, idx & 7)) = qv[i];
    }
    {
      const int t = lane >> 1, jh = (lane & 1) * (R / 2);
#pragma unroll
      for (int e = 0; e < R / 2; ++e) Ps[wid][(jh + e) * PS_LD + t] = f32_to_bf16(pv[e]);
    }
    if (ci + 1 < cpw) load(ci + 1);
    wave_lds_sync();
    u32x4 af[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
      af[jt] = (jt * 16 + lr < R) ? *reinterpret_cast<const u32x4*>(Ps[wid] + (jt * 16 + lr) * PS_LD + lg * 8)
                                  : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      // column nf*16 + lr, tokens lg*8 .. lg*8 + 7: two transposing reads
      const int col = nf * 16 + 4 * (lr & 3);
      const int row = lg * 8 + (lr >> 2);
      const u32x2 lo = lds_read_tr4(Qs[wid], off_r8(row, col >> 3) + (col & 7));
      const u32x2 hi = lds_read_tr4(Qs[wid], off_r8(row + 4, col >> 3) + (col & 7));
      const u32x4 bf = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) acc[jt][nf] = mfma16x16x32(af[jt], bf, acc[jt][nf]);
    }
    wave_lds_sync();  // this chunk's reads are done before the next one is staged
  }
  // acc[jt][nf][i] = partial Out[jt*16 + lg*4 + i][nf*16 + lr]
#pragma unroll
  for (int jt = 0; jt < JT; ++jt)
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = jt * 16 + lg * 4 + i;
        if (j < R) red[wid][j][nf * 16 + lr] = acc[jt][nf][i];
      }
  __syncthreads();
  for (int o = tid; o < R * 64; o += 256) {
    const int j = o >> 6, kk = o & 63;
    const int k = k0 + kk;
    if (k >= g.nq) continue;
    const float v = ((red[0][j][kk] + red[1][j][kk]) + red[2][j][kk]) + red[3][j][kk];
    if (part != nullptr) {
      part[(((size_t)blockIdx.z * gridDim.y + blockIdx.y) * R + j) * maxq + k] = v;
    } else {
      float* dst = g.transposed ? g.out + (int64_t)k * R + j : g.out + (int64_t)j * g.nq + k;
      *dst = (g.overwrite ? 0.0f : *dst) + g.scale * v;
    }
  }
}

// Out += scale * (sum over the token splits, in order) of the partials.
template <int R>
__global__ __launch_bounds__(256) void lora_grad_reduce_kernel(GradBatch gb, int nsec, int nz, const float* part,
                                                               int maxq) {
  const int64_t total = (int64_t)nsec * R * maxq;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int k = (int)(i % maxq);
    const int64_t rest = i / maxq;
    const int j = (int)(rest % R);
    const int sec = (int)(rest / R);
    const LoraGradSec& g = gb.s[sec];
    if (k >= g.nq) continue;
    const size_t stride = (size_t)nsec * R * maxq;
    const float* p = part + ((size_t)sec * R + j) * maxq + k;
    float q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) q[u] = (u < nz) ? p[u * stride] : 0.0f;  // nz <= 8 loads in flight
    float v = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < nz) v += q[u];
    float* dst = g.transposed ? g.out + (int64_t)k * R + j : g.out + (int64_t)j * g.nq + k;
    *dst = (g.overwrite ? 0.0f : *dst) + g.scale * v;
  }
}

template <int R>
void launch_down(const LoraDown& a, dim3 grid, int nch_max, int kc, hipStream_t s) {
  if (a.bside) hipLaunchKernelGGL((lora_down_part_kernel<R, true>), grid, dim3(256), 0, s, a, nch_max, kc);
  else hipLaunchKernelGGL((lora_down_part_kernel<R, false>), grid, dim3(256), 0, s, a, nch_max, kc);
}

// Chunk length (a multiple of 256) that cuts the longest section into at
// most kLoraDownChunks chunks, and the chunk count of that section.
int down_chunk(const LoraDown& a, int* nch_max) {
  int kmax = 0;
  for (int i = 0; i < a.nsec; ++i) kmax = std::max(kmax, sec_k(a, i));
  const int kc = KC * std::max(1, (kmax + kLoraDownChunks * KC - 1) / (kLoraDownChunks * KC));
  *nch_max = std::max(1, (kmax + kc - 1) / kc);
  return kc;
}

}  // namespace

hipError_t lora_down(const LoraDown& a, hipStream_t s) {
  if (a.M <= 0 || a.nsec <= 0) return hipSuccess;
  if (a.r < 4 || a.r > 64 || (a.r & (a.r - 1)) != 0 || a.part == nullptr || a.U == nullptr)
    return hipErrorInvalidValue;
  int nch_max = 0;
  const int kc = down_chunk(a, &nch_max);
  if ((size_t)a.nsec * nch_max * a.M * a.r > a.part_floats) return hipErrorInvalidValue;
  dim3 grid((a.M + 63) / 64, a.nsec * nch_max);
  switch (a.r) {
    case 4: launch_down<4>(a, grid, nch_max, kc, s); break;
    case 8: launch_down<8>(a, grid, nch_max, kc, s); break;
    case 16: launch_down<16>(a, grid, nch_max, kc, s); break;
    case 32: launch_down<32>(a, grid, nch_max, kc, s); break;
    case 64: launch_down<64>(a, grid, nch_max, kc, s); break;
    default: return hipErrorInvalidValue;
  }
  if (a.U == nullptr) return hipErrorInvalidValue;
  const int64_t total = (int64_t)a.M * a.nsec * a.r;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 2048);
  hipLaunchKernelGGL(lora_down_reduce_kernel, dim3(blocks), dim3(256), 0, s, a, nch_max, kc);
  return hipGetLastError();
}

template <int R>
hipError_t launch_grad(const GradBatch& gb, int nsec, int T, int maxq, float* part, size_t part_floats,
                       hipStream_t s) {
  const int tiles = (maxq + 63) / 64;
  const int chunks = (T + 31) / 32;
  int busy = 0;  // workgroups with columns to work on (sections narrower than maxq leave some idle)
  for (int i = 0; i < nsec; ++i) busy += (gb.s[i].nq + 63) / 64;
  // token splits: only as many as it takes to give at least 256 busy
  // workgroups, at least two 32-token chunks per wave, and partials that fit
  // the scratch
  int nz = std::max(1, std::min(std::min(8, (256 + busy - 1) / std::max(busy, 1)), chunks / 8));
  while (nz > 1 && (part == nullptr || (size_t)nz * nsec * R * maxq > part_floats)) --nz;
  const int cpw = (chunks + 4 * nz - 1) / (4 * nz);
  nz = (chunks + 4 * cpw - 1) / (4 * cpw);
  dim3 grid(tiles, nsec, nz);
  hipLaunchKernelGGL(lora_grad_kernel<R>, grid, dim3(256), 0, s, gb, T, cpw, nz > 1 ? part : nullptr, maxq);
  if (nz > 1) {
    const int64_t total = (int64_t)nsec * R * maxq;
    const int blocks = (int)std::min<int64_t>((total + 255) / 256, 2048);
    hipLaunchKernelGGL(lora_grad_reduce_kernel<R>, dim3(blocks), dim3(256), 0, s, gb, nsec, nz, part, maxq);
  }
  return hipGetLastError();
}

hipError_t lora_grad(const LoraGradSec* secs, int nsec, int T, int r, float* part, size_t part_floats,
                     hipStream_t s) {
  if (nsec <= 0 || T <= 0) return hipSuccess;
  if (nsec > kLoraGradSecs) return hipErrorInvalidValue;
  GradBatch gb{};
  int maxq = 0;
  for (int i = 0; i < nsec; ++i) {
    gb.s[i] = secs[i];
    maxq = std::max(maxq, secs[i].nq);
  }
  switch (r) {
    case 4: return launch_grad<4>(gb, nsec, T, maxq, part, part_floats, s);
    case 8: return launch_grad<8>(gb, nsec, T, maxq, part, part_floats, s);
    case 16: return launch_grad<16>(gb, nsec, T, maxq, part, part_floats, s);
    case 32: return launch_grad<32>(gb, nsec, T, maxq, part, part_floats, s);
    case 64: return launch_grad<64>(gb, nsec, T, maxq, part, part_floats, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lsf
