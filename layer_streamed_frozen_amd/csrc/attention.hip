// Causal grouped-query attention, head_dim 128, on gfx950 MFMA.
//
// Forward: one workgroup per (64-query block, query head, sequence); four
// waves own 16 query rows each.  Key/value blocks of 64 rows are staged in
// LDS; S = Q K^T and O += P V run on v_mfma_f32_16x16x32_bf16 with an online
// (running max / running sum) softmax in fp32.  The log-sum-exp of every row
// is kept for the backward pass.
//
// Backward (recomputes P from Q, K and the saved log-sum-exp):
//   pass 0: Dsum[q] = sum_d dO[q, d] O[q, d]
//   pass 1: per (64-key block, query head): dV_h = P^T dO, dK_h = dS^T Q,
//           written as fp32 partials per query head;
//   pass 2: per (64-query block, query head): dQ = dS K;
//   pass 3: dK, dV of a kv head = the sum of its query heads' partials,
//           in a fixed order (no atomics).
// with dS = P (dP - Dsum), dP = dO V^T, and the 1/sqrt(d) scale.
#include "common.h"
#include "kernels.h"

namespace lsf {
namespace {

constexpr int HD = 128, BLK = 64, NTHR = 256;
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ int swz16(int row) { return (row & 15) ^ (((row >> 4) & 1) << 2); }
__device__ __forceinline__ int off_r16(int row, int chunk) { return row * 128 + ((chunk ^ swz16(row)) << 3); }
__device__ __forceinline__ int off_r8(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

// Stage rows [r0, r0 + 64) of a [rows, ld] bf16 matrix (columns col0 .. col0+127)
// into a 64 x 128 LDS tile; rows at or past `rows` are zero.
__device__ __forceinline__ void load_tile(const uint16_t* src, int64_t ld, int64_t col0, int r0, int rows,
                                          uint16_t* lds, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + NTHR * i;
    const int row = idx >> 4, ch = idx & 15;
    u32x4 v = {0, 0, 0, 0};
    if (r0 + row < rows) v = *reinterpret_cast<const u32x4*>(src + (int64_t)(r0 + row) * ld + col0 + ch * 8);
    *reinterpret_cast<u32x4*>(lds + off_r16(row, ch)) = v;
  }
}

__device__ __forceinline__ u32x4 frag_row(const uint16_t* lds, int row, int chunk) {
  return *reinterpret_cast<const u32x4*>(lds + off_r16(row, chunk));
}
// Operand whose contraction runs down the tile rows: rows row0..row0+7 of column col.
__device__ __forceinline__ u32x4 frag_gather(const uint16_t* lds, int col, int row0) {
  const int ch = col >> 3, e = col & 7;
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t lo = lds[off_r16(row0 + 2 * p, ch) + e];
    const uint32_t hi = lds[off_r16(row0 + 2 * p + 1, ch) + e];
    w[p] = lo | (hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Global row fragment: row `row` (or zeros past `rows`), dims s*32 + lg*8 .. +8.
__device__ __forceinline__ u32x4 gfrag(const uint16_t* base, int64_t ld, int row, int rows, int s, int lg) {
  if (row >= rows) return u32x4{0, 0, 0, 0};
  return *reinterpret_cast<const u32x4*>(base + (int64_t)row * ld + s * 32 + lg * 8);
}

// Write a wave's 16 x 64 C-layout fragment set as bf16 into a row-major
// (R8-swizzled) 16 x 64 LDS block.
__device__ __forceinline__ void store_c16x64(uint16_t* lds, const f32x4 (&v)[4], int lr, int lg) {
#pragma unroll
  for (int nf = 0; nf < 4; ++nf)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lg * 4 + i, col = nf * 16 + lr;
      lds[off_r8(row, col >> 3) + (col & 7)] = f32_to_bf16(v[nf][i]);
    }
}

__global__ __launch_bounds__(NTHR) void attn_fwd_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BLK * HD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BLK * HD];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[4][16 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (a.nq / a.nkv);
  const int seq = a.seq;
  const int64_t rowbase = (int64_t)b * seq;
  const uint16_t* Qg = a.qkv + rowbase * a.ldqkv + (int64_t)h * HD;
  const uint16_t* Kg = a.qkv + rowbase * a.ldqkv + (int64_t)(a.nq + kvh) * HD;
  const uint16_t* Vg = a.qkv + rowbase * a.ldqkv + (int64_t)(a.nq + a.nkv + kvh) * HD;
  const int qw = qb * BLK + wid * 16;
  const float c = LOG2E / sqrtf((float)HD);

  u32x4 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = gfrag(Qg, a.ldqkv, qw + lr, seq, s, lg);

  f32x4 o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4{0, 0, 0, 0};
  float mrow[4], lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { mrow[i] = -INFINITY; lrow[i] = 0.0f; }

  const int nkb = min(qb + 1, (seq + BLK - 1) / BLK);
  for (int kb = 0; kb < nkb; ++kb) {
    load_tile(Kg, a.ldqkv, 0, kb * BLK, seq, Ks, tid);
    load_tile(Vg, a.ldqkv, 0, kb * BLK, seq, Vs, tid);
    __syncthreads();
    f32x4 S[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      S[nf] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) S[nf] = mfma16x16x32(qf[s], frag_row(Ks, nf * 16 + lr, s * 4 + lg), S[nf]);
    }
    float mloc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = qw + lg * 4 + i;
      mloc[i] = -INFINITY;
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int kv = kb * BLK + nf * 16 + lr;
        const float v = (kv <= q && kv < seq) ? S[nf][i] * c : -INFINITY;
        S[nf][i] = v;
        mloc[i] = fmaxf(mloc[i], v);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mloc[i] = fmaxf(mloc[i], __shfl_xor(mloc[i], off, 64));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mn = fmaxf(mrow[i], mloc[i]);
      const float alpha = (mrow[i] == -INFINITY) ? 0.0f : exp2f(mrow[i] - mn);
      float rs = 0.0f;
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const float p = (S[nf][i] == -INFINITY) ? 0.0f : exp2f(S[nf][i] - mn);
        S[nf][i] = p;
        rs += p;
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) rs += __shfl_xor(rs, off, 64);
      lrow[i] = lrow[i] * alpha + rs;
      mrow[i] = mn;
#pragma unroll
      for (int n = 0; n < 8; ++n) o[n][i] *= alpha;
    }
    store_c16x64(Ps[wid], S, lr, lg);
    __syncthreads();
    u32x4 pa[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) pa[s2] = *reinterpret_cast<const u32x4*>(Ps[wid] + off_r8(lr, s2 * 4 + lg));
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) o[n] = mfma16x16x32(pa[s2], frag_gather(Vs, n * 16 + lr, s2 * 32 + lg * 8), o[n]);
    __syncthreads();
  }
  uint16_t* Og = a.o + rowbase * ((int64_t)a.nq * HD) + (int64_t)h * HD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = qw + lg * 4 + i;
    if (q >= seq) continue;
    const float inv = 1.0f / lrow[i];
#pragma unroll
    for (int n = 0; n < 8; ++n) Og[(int64_t)q * a.nq * HD + n * 16 + lr] = f32_to_bf16(o[n][i] * inv);
    if (lr == 0) a.lse[((int64_t)b * a.nq + h) * seq + q] = (mrow[i] + log2f(lrow[i])) / LOG2E;
  }
}

// Dsum[b, h, q] = sum_d dO * O   (one wave per (token, head), 2 dims per lane)
__global__ __launch_bounds__(NTHR) void attn_dsum_kernel(AttnArgs a) {
  const int64_t gw = ((int64_t)blockIdx.x * NTHR + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t T = (int64_t)a.batch * a.seq;
  if (gw >= T * a.nq) return;
  const int64_t t = gw / a.nq;
  const int h = (int)(gw - t * a.nq);
  const int64_t off = t * ((int64_t)a.nq * HD) + (int64_t)h * HD + lane * 2;
  const uint32_t d = *reinterpret_cast<const uint32_t*>(a.dout + off);
  const uint32_t o = *reinterpret_cast<const uint32_t*>(a.o + off);
  float v = bf16lo(d) * bf16lo(o) + bf16hi(d) * bf16hi(o);
  v = warp_sum(v);
  if (lane == 0) {
    const int b = (int)(t / a.seq), q = (int)(t % a.seq);
    a.Dsum[((int64_t)b * a.nq + h) * a.seq + q] = v;
  }
}

struct BwdScratch {
  float* dkp;  // [batch*seq, nq, 128] partial dK per query head
  float* dvp;
};

__global__ __launch_bounds__(NTHR) void attn_bwd_kv_kernel(AttnArgs a, BwdScratch sc) {
  __shared__ __attribute__((aligned(16))) uint16_t Qs[BLK * HD];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[BLK * HD];
  __shared__ __attribute__((aligned(16))) uint16_t Pt[4][16 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t Dt[4][16 * 64];
  __shared__ float lse_s[BLK], ds_s[BLK];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int kb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (a.nq / a.nkv);
  const int seq = a.seq;
  const int64_t rowbase = (int64_t)b * seq;
  const int64_t ldo = (int64_t)a.nq * HD;
  const uint16_t* Qg = a.qkv + rowbase * a.ldqkv + (int64_t)h * HD;
  const uint16_t* Kg = a.qkv + rowbase * a.ldqkv + (int64_t)(a.nq + kvh) * HD;
  const uint16_t* Vg = a.qkv + rowbase * a.ldqkv + (int64_t)(a.nq + a.nkv + kvh) * HD;
  const uint16_t* dOg = a.dout + rowbase * ldo + (int64_t)h * HD;
  const float* lse = a.lse + ((int64_t)b * a.nq + h) * seq;
  const float* Ds = a.Dsum + ((int64_t)b * a.nq + h) * seq;
  const int kw = kb * BLK + wid * 16;
  const float c = LOG2E / sqrtf((float)HD);

  u32x4 kf[4], vf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kf[s] = gfrag(Kg, a.ldqkv, kw + lr, seq, s, lg);
    vf[s] = gfrag(Vg, a.ldqkv, kw + lr, seq, s, lg);
  }
  f32x4 dk[8], dv[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) { dk[n] = f32x4{0, 0, 0, 0}; dv[n] = f32x4{0, 0, 0, 0}; }

  const int nqb = (seq + BLK - 1) / BLK;
  for (int qb = kb; qb < nqb; ++qb) {
    load_tile(Qg, a.ldqkv, 0, qb * BLK, seq, Qs, tid);
    load_tile(dOg, ldo, 0, qb * BLK, seq, dOs, tid);
    if (tid < BLK) {
      const int q = qb * BLK + tid;
      lse_s[tid] = (q < seq) ? lse[q] * LOG2E : 0.0f;
      ds_s[tid] = (q < seq) ? Ds[q] : 0.0f;
    }
    __syncthreads();
    f32x4 St[4], dPt[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      St[nf] = f32x4{0, 0, 0, 0};
      dPt[nf] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        St[nf] = mfma16x16x32(kf[s], frag_row(Qs, nf * 16 + lr, s * 4 + lg), St[nf]);
        dPt[nf] = mfma16x16x32(vf[s], frag_row(dOs, nf * 16 + lr, s * 4 + lg), dPt[nf]);
      }
    }
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int ql = nf * 16 + lr;
      const int q = qb * BLK + ql;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kv = kw + lg * 4 + i;
        const bool ok = kv <= q && q < seq && kv < seq;
        const float p = ok ? exp2f(St[nf][i] * c - lse_s[ql]) : 0.0f;
        St[nf][i] = p;
        dPt[nf][i] = p * (dPt[nf][i] - ds_s[ql]);
      }
    }
    store_c16x64(Pt[wid], St, lr, lg);
    store_c16x64(Dt[wid], dPt, lr, lg);
    __syncthreads();
    u32x4 pa[2], da[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      pa[s2] = *reinterpret_cast<const u32x4*>(Pt[wid] + off_r8(lr, s2 * 4 + lg));
      da[s2] = *reinterpret_cast<const u32x4*>(Dt[wid] + off_r8(lr, s2 * 4 + lg));
    }
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        dv[n] = mfma16x16x32(pa[s2], frag_gather(dOs, n * 16 + lr, s2 * 32 + lg * 8), dv[n]);
        dk[n] = mfma16x16x32(da[s2], frag_gather(Qs, n * 16 + lr, s2 * 32 + lg * 8), dk[n]);
      }
    __syncthreads();
  }
  const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kv = kw + lg * 4 + i;
    if (kv >= seq) continue;
    const int64_t base = ((rowbase + kv) * a.nq + h) * HD;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      sc.dkp[base + n * 16 + lr] = dk[n][i] * scale;
      sc.dvp[base + n * 16 + lr] = dv[n][i];
    }
  }
}

__global__ __launch_bounds__(NTHR) void attn_bwd_q_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BLK * HD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BLK * HD];
  __shared__ __attribute__((aligned(16))) uint16_t Dt[4][16 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (a.nq / a.nkv);
  const int seq = a.seq;
  const int64_t rowbase = (int64_t)b * seq;
  const int64_t ldo = (int64_t)a.nq * HD;
  const uint16_t* Qg = a.qkv + rowbase * a.ldqkv + (int64_t)h * HD;
  const uint16_t* Kg = a.qkv + rowbase * a.ldqkv + (int64_t)(a.nq + kvh) * HD;
  const uint16_t* Vg = a.qkv + rowbase * a.ldqkv + (int64_t)(a.nq + a.nkv + kvh) * HD;
  const uint16_t* dOg = a.dout + rowbase * ldo + (int64_t)h * HD;
  const float* lse = a.lse + ((int64_t)b * a.nq + h) * seq;
  const float* Ds = a.Dsum + ((int64_t)b * a.nq + h) * seq;
  const int qw = qb * BLK + wid * 16;
  const float c = LOG2E / sqrtf((float)HD);

  u32x4 qf[4], of[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qf[s] = gfrag(Qg, a.ldqkv, qw + lr, seq, s, lg);
    of[s] = gfrag(dOg, ldo, qw + lr, seq, s, lg);
  }
  float l2[4], dd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = qw + lg * 4 + i;
    l2[i] = (q < seq) ? lse[q] * LOG2E : 0.0f;
    dd[i] = (q < seq) ? Ds[q] : 0.0f;
  }
  f32x4 dq[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) dq[n] = f32x4{0, 0, 0, 0};
  const int nkb = min(qb + 1, (seq + BLK - 1) / BLK);
  for (int kb = 0; kb < nkb; ++kb) {
    load_tile(Kg, a.ldqkv, 0, kb * BLK, seq, Ks, tid);
    load_tile(Vg, a.ldqkv, 0, kb * BLK, seq, Vs, tid);
    __syncthreads();
    f32x4 S[4], dP[4];
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      S[nf] = f32x4{0, 0, 0, 0};
      dP[nf] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        S[nf] = mfma16x16x32(qf[s], frag_row(Ks, nf * 16 + lr, s * 4 + lg), S[nf]);
        dP[nf] = mfma16x16x32(of[s], frag_row(Vs, nf * 16 + lr, s * 4 + lg), dP[nf]);
      }
    }
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int kv = kb * BLK + nf * 16 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = qw + lg * 4 + i;
        const bool ok = kv <= q && q < seq && kv < seq;
        const float p = ok ? exp2f(S[nf][i] * c - l2[i]) : 0.0f;
        dP[nf][i] = p * (dP[nf][i] - dd[i]);
      }
    }
    store_c16x64(Dt[wid], dP, lr, lg);
    __syncthreads();
    u32x4 da[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) da[s2] = *reinterpret_cast<const u32x4*>(Dt[wid] + off_r8(lr, s2 * 4 + lg));
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) dq[n] = mfma16x16x32(da[s2], frag_gather(Ks, n * 16 + lr, s2 * 32 + lg * 8), dq[n]);
    __syncthreads();
  }
  const float scale = 1.0f / sqrtf((float)HD);
  uint16_t* dQg = a.dqkv + rowbase * a.ldqkv + (int64_t)h * HD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = qw + lg * 4 + i;
    if (q >= seq) continue;
#pragma unroll
    for (int n = 0; n < 8; ++n) dQg[(int64_t)q * a.ldqkv + n * 16 + lr] = f32_to_bf16(dq[n][i] * scale);
  }
}

// dK, dV of kv head g = sum over its query heads, fixed order.
__global__ __launch_bounds__(NTHR) void attn_kv_reduce_kernel(AttnArgs a, BwdScratch sc) {
  const int64_t T = (int64_t)a.batch * a.seq;
  const int64_t total = T * a.nkv * HD;
  const int grp = a.nq / a.nkv;
  for (int64_t i = (int64_t)blockIdx.x * NTHR + threadIdx.x; i < total; i += (int64_t)gridDim.x * NTHR) {
    const int d = (int)(i % HD);
    const int64_t r = i / HD;
    const int g = (int)(r % a.nkv);
    const int64_t t = r / a.nkv;
    float sk = 0.0f, sv = 0.0f;
    for (int j = 0; j < grp; ++j) {
      const int64_t src = (t * a.nq + g * grp + j) * HD + d;
      sk += sc.dkp[src];
      sv += sc.dvp[src];
    }
    a.dqkv[t * a.ldqkv + (int64_t)(a.nq + g) * HD + d] = f32_to_bf16(sk);
    a.dqkv[t * a.ldqkv + (int64_t)(a.nq + a.nkv + g) * HD + d] = f32_to_bf16(sv);
  }
}

}  // namespace

hipError_t attention_fwd(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.seq + BLK - 1) / BLK, a.nq, a.batch);
  hipLaunchKernelGGL(attn_fwd_kernel, grid, dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

// Scratch: the caller passes it through a.Dsum's neighbour: dK/dV partials
// live right after Dsum (see attention_bwd_scratch_floats).
hipError_t attention_bwd(const AttnArgs& a, hipStream_t s) {
  const int64_t T = (int64_t)a.batch * a.seq;
  BwdScratch sc;
  sc.dkp = a.Dsum + (int64_t)a.batch * a.nq * a.seq;
  sc.dvp = sc.dkp + T * a.nq * HD;
  {
    const int64_t waves = T * a.nq;
    hipLaunchKernelGGL(attn_dsum_kernel, dim3((unsigned)((waves * 64 + NTHR - 1) / NTHR)), dim3(NTHR), 0, s, a);
  }
  dim3 grid((a.seq + BLK - 1) / BLK, a.nq, a.batch);
  hipLaunchKernelGGL(attn_bwd_kv_kernel, grid, dim3(NTHR), 0, s, a, sc);
  hipLaunchKernelGGL(attn_bwd_q_kernel, grid, dim3(NTHR), 0, s, a);
  const int64_t total = T * a.nkv * HD;
  const int blocks = (int)std::min<int64_t>((total + NTHR - 1) / NTHR, 8192);
  hipLaunchKernelGGL(attn_kv_reduce_kernel, dim3(blocks), dim3(NTHR), 0, s, a, sc);
  return hipGetLastError();
}

}  // namespace lsf
