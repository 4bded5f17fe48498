// Bandwidth-bound kernels: RMSNorm forward/backward, RoPE, embedding gather,
// cross-entropy, fills.  Rows are processed by one 256-thread workgroup with
// 16-byte vector accesses; reductions go lane -> wave (shuffles) -> workgroup
// (LDS, fixed order), so results do not depend on scheduling.
#include "common.h"
#include "kernels.h"

namespace lsf {
namespace {

// Sum over the 256 threads of a workgroup, the same order every time.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = warp_sum(v);
  const int wid = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wid] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ __forceinline__ void unpack8(const u32x4& q, float f[8]) {
  f[0] = bf16lo(q.x); f[1] = bf16hi(q.x); f[2] = bf16lo(q.y); f[3] = bf16hi(q.y);
  f[4] = bf16lo(q.z); f[5] = bf16hi(q.z); f[6] = bf16lo(q.w); f[7] = bf16hi(q.w);
}
__device__ __forceinline__ u32x4 pack8(const float f[8]) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

// Rows of up to kRowRegs * 2048 elements stay in registers between the two
// passes (sum of squares or dot product, then the output), so every input
// byte is read from memory once; longer rows are read twice.
constexpr int kRowRegs = 4;

__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w, int H, float eps,
                                                          uint16_t* __restrict__ y, float* __restrict__ rstd) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * H;
  const bool keep = H <= 256 * 8 * kRowRegs;
  u32x4 xs[kRowRegs];
  float ss = 0.0f;
  int it = 0;
  for (int i = threadIdx.x * 8; i < H; i += 256 * 8, ++it) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(xr + i);
    if (keep) {
#pragma unroll
      for (int j = 0; j < kRowRegs; ++j)
        if (j == it) xs[j] = q;
    }
    float f[8];
    unpack8(q, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  it = 0;
  for (int i = threadIdx.x * 8; i < H; i += 256 * 8, ++it) {
    u32x4 q;
    if (keep) {
#pragma unroll
      for (int j = 0; j < kRowRegs; ++j)
        if (j == it) q = xs[j];
    } else {
      q = *reinterpret_cast<const u32x4*>(xr + i);
    }
    float f[8], g[8];
    unpack8(q, f);
    unpack8(*reinterpret_cast<const u32x4*>(w + i), g);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = f[e] * r * g[e];
    *reinterpret_cast<u32x4*>(y + row * H + i) = pack8(f);
  }
  if (threadIdx.x == 0 && rstd != nullptr) rstd[row] = r;
}

__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const uint16_t* __restrict__ dy,
                                                          const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w,
                                                          const float* __restrict__ rstd,
                                                          const uint16_t* __restrict__ resid, int H,
                                                          uint16_t* __restrict__ dx) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int64_t base = row * H;
  const bool keep = H <= 256 * 8 * kRowRegs;
  u32x4 as[kRowRegs], cs[kRowRegs];
  float dot = 0.0f;
  int it = 0;
  for (int i = threadIdx.x * 8; i < H; i += 256 * 8, ++it) {
    const u32x4 qa = *reinterpret_cast<const u32x4*>(dy + base + i);
    const u32x4 qc = *reinterpret_cast<const u32x4*>(x + base + i);
    if (keep) {
#pragma unroll
      for (int j = 0; j < kRowRegs; ++j)
        if (j == it) { as[j] = qa; cs[j] = qc; }
    }
    float a[8], b[8], c[8];
    unpack8(qa, a);
    unpack8(*reinterpret_cast<const u32x4*>(w + i), b);
    unpack8(qc, c);
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fmaf(a[e] * b[e], c[e], dot);
  }
  dot = block_sum(dot, red);
  const float r = rstd[row];
  const float k = r * r * r * dot / (float)H;
  it = 0;
  for (int i = threadIdx.x * 8; i < H; i += 256 * 8, ++it) {
    u32x4 qa, qc;
    if (keep) {
#pragma unroll
      for (int j = 0; j < kRowRegs; ++j)
        if (j == it) { qa = as[j]; qc = cs[j]; }
    } else {
      qa = *reinterpret_cast<const u32x4*>(dy + base + i);
      qc = *reinterpret_cast<const u32x4*>(x + base + i);
    }
    float a[8], b[8], c[8], o[8];
    unpack8(qa, a);
    unpack8(*reinterpret_cast<const u32x4*>(w + i), b);
    unpack8(qc, c);
    if (resid != nullptr) unpack8(*reinterpret_cast<const u32x4*>(resid + base + i), o);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += r * (a[e] * b[e]) - c[e] * k;
    *reinterpret_cast<u32x4*>(dx + base + i) = pack8(o);
  }
}

__global__ void rope_table_kernel(int seq, int half, float theta, float2* tab) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= seq * half) return;
  const int pos = idx / half, i = idx - pos * half;
  const double inv = pow((double)theta, -2.0 * (double)i / (double)(2 * half));
  const double ang = (double)pos * inv;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

// One thread: 8 consecutive pairs (i, i + d/2) of one head of one token.
__global__ __launch_bounds__(256) void rope_apply_kernel(uint16_t* __restrict__ qk, int64_t ld, int T, int seq,
                                                         int nheads, int d, const float2* __restrict__ tab,
                                                         int inverse) {
  const int half = d >> 1, groups = half >> 3;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)T * nheads * groups;
  if (idx >= total) return;
  const int gi = (int)(idx % groups);
  const int64_t th = idx / groups;
  const int h = (int)(th % nheads);
  const int t = (int)(th / nheads);
  const int pos = t % seq;
  uint16_t* p = qk + (int64_t)t * ld + (int64_t)h * d + gi * 8;
  float a[8], b[8];
  unpack8(*reinterpret_cast<const u32x4*>(p), a);
  unpack8(*reinterpret_cast<const u32x4*>(p + half), b);
  const float sgn = inverse ? -1.0f : 1.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 cs = tab[pos * half + gi * 8 + e];
    const float s = sgn * cs.y;
    const float x1 = a[e], x2 = b[e];
    a[e] = x1 * cs.x - x2 * s;
    b[e] = x2 * cs.x + x1 * s;
  }
  *reinterpret_cast<u32x4*>(p) = pack8(a);
  *reinterpret_cast<u32x4*>(p + half) = pack8(b);
}

// One row per workgroup.  An id outside [0, V) reads nothing: its row is
// zero and *status (if given) is set to 1 (every writer stores the same value).
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ ids, const uint16_t* __restrict__ E,
                                                    int H, int V, uint16_t* __restrict__ x, int32_t* status) {
  const int64_t t = blockIdx.x;
  const int id = ids[t];
  const bool ok = id >= 0 && id < V;
  u32x4* dst = reinterpret_cast<u32x4*>(x + t * H);
  if (!ok) {
    if (status != nullptr && threadIdx.x == 0) *status = 1;
    for (int i = threadIdx.x; i < H / 8; i += 256) dst[i] = u32x4{0, 0, 0, 0};
    return;
  }
  const u32x4* src = reinterpret_cast<const u32x4*>(E + (int64_t)id * H);
  for (int i = threadIdx.x; i < H / 8; i += 256) dst[i] = src[i];
}

// Cross-entropy rows: one 1024-thread workgroup per row of V fp32 logits (16
// waves per row keep enough loads in flight; a row of the 128256-entry
// vocabulary is 501 KB), 16-byte loads when the row is 16-byte aligned.
constexpr int kCeThreads = 1024;

__device__ __forceinline__ void lse_push(float x, float& m, float& s) {
  if (x > m) {
    s = s * __expf(m - x) + 1.0f;
    m = x;
  } else {
    s += __expf(x - m);
  }
}

// Log-sum-exp of one row: a running (max, sum of exp) per thread, merged
// lane -> wave -> workgroup in a fixed order.
__device__ __forceinline__ float row_lse(const float* __restrict__ z, int V) {
  __shared__ float sm[kCeThreads / 64], ss[kCeThreads / 64];
  float m = -INFINITY, s = 0.0f;
  if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0) {
    const float4* z4 = reinterpret_cast<const float4*>(z);
    for (int v = threadIdx.x; v < V / 4; v += kCeThreads) {
      const float4 x = z4[v];
      const float mx = fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w));
      if (mx > m) {
        s *= __expf(m - mx);
        m = mx;
      }
      s += (__expf(x.x - m) + __expf(x.y - m)) + (__expf(x.z - m) + __expf(x.w - m));
    }
  } else {
    for (int v = threadIdx.x; v < V; v += kCeThreads) lse_push(z[v], m, s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    const float mm = fmaxf(m, m2);
    s = (m == -INFINITY ? 0.0f : s * __expf(m - mm)) + (m2 == -INFINITY ? 0.0f : s2 * __expf(m2 - mm));
    m = mm;
  }
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[wid] = m; ss[wid] = s; }
  __syncthreads();
  float M = sm[0];
#pragma unroll
  for (int w = 1; w < kCeThreads / 64; ++w) M = fmaxf(M, sm[w]);
  float S = 0.0f;
#pragma unroll
  for (int w = 0; w < kCeThreads / 64; ++w) S += ss[w] * __expf(sm[w] - M);
  return M + __logf(S);
}

// d[v] = bf16(c * (exp(z[v] - lse) - [v == label])) over one row, or zeros
// when the row has no label; 8-byte stores when the rows are aligned.
__device__ __forceinline__ void grad_row(const float* __restrict__ z, int V, float lse, int label, bool valid,
                                         float c, uint16_t* __restrict__ d) {
  if ((V & 3) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0 && (reinterpret_cast<uintptr_t>(d) & 7) == 0) {
    const float4* z4 = reinterpret_cast<const float4*>(z);
    u32x2* d4 = reinterpret_cast<u32x2*>(d);
    for (int v = threadIdx.x; v < V / 4; v += kCeThreads) {
      float g[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (valid) {
        const float4 x = z4[v];
        const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) g[e] = (__expf(xs[e] - lse) - (4 * v + e == label ? 1.0f : 0.0f)) * c;
      }
      d4[v] = u32x2{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
    }
  } else {
    for (int v = threadIdx.x; v < V; v += kCeThreads) {
      float g = 0.0f;
      if (valid) g = (__expf(z[v] - lse) - (v == label ? 1.0f : 0.0f)) * c;
      d[v] = f32_to_bf16(g);
    }
  }
}

// Next-token label of row t (the id one position on) and whether row t has
// one: the last position of each sequence is unlabelled, and so is a row whose
// label lies outside [0, V) (the embedding gather reports such ids).
__device__ __forceinline__ int row_label(const int32_t* __restrict__ ids, int64_t t, int seq, int V, bool& valid) {
  valid = (t % seq) < seq - 1;
  const int label = valid ? ids[t + 1] : 0;
  if (label < 0 || label >= V) {
    valid = false;
    return 0;
  }
  return label;
}

// One workgroup per row of logits: the loss term and softmax minus one-hot, scaled.
__global__ __launch_bounds__(kCeThreads) void ce_row_kernel(const float* __restrict__ logits,
                                                            const int32_t* __restrict__ ids, int seq, int V,
                                                            float coef, uint16_t* __restrict__ dlogits,
                                                            float* __restrict__ row_loss) {
  const int64_t t = blockIdx.x;
  const float* z = logits + t * V;
  bool valid;
  const int label = row_label(ids, t, seq, V, valid);
  const float lse = row_lse(z, V);
  if (threadIdx.x == 0) row_loss[t] = valid ? (lse - z[label]) : 0.0f;
  grad_row(z, V, lse, label, valid, coef, dlogits + t * V);
}

// Row statistics for sequence log-probabilities: lse[t] and the log-probability
// of row t's label (0 for unlabelled rows).
__global__ __launch_bounds__(kCeThreads) void ce_stats_kernel(const float* __restrict__ logits,
                                                       const int32_t* __restrict__ ids, int seq, int V,
                                                       float* __restrict__ lse_out, float* __restrict__ row_logp) {
  const int64_t t = blockIdx.x;
  const float* z = logits + t * V;
  bool valid;
  const int label = row_label(ids, t, seq, V, valid);
  const float lse = row_lse(z, V);
  if (threadIdx.x == 0) {
    lse_out[t] = lse;
    row_logp[t] = valid ? (z[label] - lse) : 0.0f;
  }
}

// One workgroup per sequence: the sum of its seq row values, fixed order.
__global__ __launch_bounds__(256) void seq_sum_kernel(const float* __restrict__ x, int seq, float* __restrict__ out) {
  __shared__ float red[4];
  const float* r = x + (int64_t)blockIdx.x * seq;
  float s = 0.0f;
  for (int i = threadIdx.x; i < seq; i += 256) s += r[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) out[blockIdx.x] = s;
}

// DPO over P pairs (sequences 0..P-1 chosen, P..2P-1 rejected):
// h_p = (lp[p] - ref[p]) - (lp[P+p] - ref[P+p]), loss = mean_p softplus(-beta h_p).
// coef[s] is -dloss/dlp[s] times loss_scale, the factor on (softmax - onehot)
// in the rows of sequence s.  One thread, pairs summed in order.
__global__ void dpo_coef_kernel(const float* __restrict__ lp, const float* __restrict__ ref, int P, float beta,
                                float loss_scale, float* __restrict__ coef, float* __restrict__ loss) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  float acc = 0.0f;
  for (int p = 0; p < P; ++p) {
    const float h = (lp[p] - ref[p]) - (lp[P + p] - ref[P + p]);
    const float x = -beta * h;
    acc += fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));  // softplus(x)
    const float sig = 1.0f / (1.0f + expf(beta * h));  // sigmoid(-beta h)
    const float c = beta * sig / (float)P * loss_scale;
    coef[p] = c;
    coef[P + p] = -c;
  }
  *loss = acc / (float)P;
}

// dlogits of a sequence-level loss: coef[sequence] (softmax - onehot) on labelled rows.
__global__ __launch_bounds__(kCeThreads) void ce_grad_kernel(const float* __restrict__ logits,
                                                             const int32_t* __restrict__ ids,
                                                             const float* __restrict__ lse_in,
                                                             const float* __restrict__ coef, int seq, int V,
                                                             uint16_t* __restrict__ dlogits) {
  const int64_t t = blockIdx.x;
  bool valid;
  const int label = row_label(ids, t, seq, V, valid);
  grad_row(logits + t * V, V, lse_in[t], label, valid, coef[t / seq], dlogits + t * V);
}

__global__ __launch_bounds__(256) void mean_kernel(const float* __restrict__ x, int n, float inv, float* out) {
  __shared__ float red[4];
  float s = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) s += x[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) *out = s * inv;
}

__global__ void fill_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

// 16-byte stores of one 32-bit pattern over n16 vectors.
__global__ void fill_pattern_kernel(u32x4* p, int64_t n16, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = u32x4{v, v, v, v};
}

// A fixed-length wait: `iters` sleeps of about 64 x 127 clocks each, whatever
// else runs.  It reads and writes nothing.
__global__ void delay_kernel(int iters) {
  for (int i = 0; i < iters; ++i) __builtin_amdgcn_s_sleep(127);
}

}  // namespace

hipError_t rmsnorm_fwd(const uint16_t* x, const uint16_t* w, int T, int H, float eps, uint16_t* y, float* rstd,
                       hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_fwd_kernel, dim3(T), dim3(256), 0, s, x, w, H, eps, y, rstd);
  return hipGetLastError();
}

hipError_t rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* w, const float* rstd,
                       const uint16_t* resid, int T, int H, uint16_t* dx, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3(T), dim3(256), 0, s, dy, x, w, rstd, resid, H, dx);
  return hipGetLastError();
}

hipError_t rope_table(int seq, int d, float theta, float2* tab, hipStream_t s) {
  const int n = seq * (d / 2);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, seq, d / 2, theta, tab);
  return hipGetLastError();
}

hipError_t rope_apply(uint16_t* qk, int64_t ld, int T, int seq, int n_heads_total, int d, const float2* tab,
                      bool inverse, hipStream_t s) {
  const int64_t total = (int64_t)T * n_heads_total * (d / 16);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_apply_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, qk, ld, T, seq,
                     n_heads_total, d, tab, inverse ? 1 : 0);
  return hipGetLastError();
}

hipError_t embed_gather(const int32_t* ids, const uint16_t* E, int T, int H, int V, uint16_t* x, int32_t* status,
                        hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel, dim3(T), dim3(256), 0, s, ids, E, H, V, x, status);
  return hipGetLastError();
}

hipError_t cross_entropy(const float* logits, const int32_t* ids, int batch, int seq, int V, float loss_scale,
                         uint16_t* dlogits, float* row_loss, float* loss, hipStream_t s) {
  const int T = batch * seq;
  const int count = batch * (seq - 1);
  const float coef = count > 0 ? loss_scale / (float)count : 0.0f;
  hipLaunchKernelGGL(ce_row_kernel, dim3(T), dim3(kCeThreads), 0, s, logits, ids, seq, V, coef, dlogits, row_loss);
  hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(256), 0, s, row_loss, T, count > 0 ? 1.0f / (float)count : 0.0f,
                     loss);
  return hipGetLastError();
}

hipError_t seq_logprobs(const float* logits, const int32_t* ids, int batch, int seq, int V, float* lse,
                        float* row_logp, float* lp, hipStream_t s) {
  const int T = batch * seq;
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(ce_stats_kernel, dim3(T), dim3(kCeThreads), 0, s, logits, ids, seq, V, lse, row_logp);
  hipLaunchKernelGGL(seq_sum_kernel, dim3(batch), dim3(256), 0, s, row_logp, seq, lp);
  return hipGetLastError();
}

hipError_t dpo_head_grad(const float* logits, const int32_t* ids, const float* lse, const float* lp_pi,
                         const float* lp_ref, int batch, int seq, int V, float beta, float loss_scale, float* coef,
                         float* loss, uint16_t* dlogits, hipStream_t s) {
  const int P = batch / 2;
  hipLaunchKernelGGL(dpo_coef_kernel, dim3(1), dim3(64), 0, s, lp_pi, lp_ref, P, beta, loss_scale, coef, loss);
  if (dlogits != nullptr)
    hipLaunchKernelGGL(ce_grad_kernel, dim3(batch * seq), dim3(kCeThreads), 0, s, logits, ids, lse, coef, seq, V,
                       dlogits);
  return hipGetLastError();
}

hipError_t fill_pattern(void* p, int64_t bytes, uint32_t v, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(p) % 16 != 0) return hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int grid = (int)std::min<int64_t>((n16 + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_pattern_kernel, dim3(grid), dim3(256), 0, s, static_cast<u32x4*>(p), n16, v);
  return hipGetLastError();
}

hipError_t delay(int iters, hipStream_t s) {
  if (iters <= 0) return hipSuccess;
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, s, iters);
  return hipGetLastError();
}

hipError_t zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_kernel, dim3(grid), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace lsf
