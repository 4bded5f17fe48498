// Causal grouped-query attention, head_dim 128, on gfx950 MFMA.
//
// Every product whose output feeds another product is computed transposed, so
// that its C fragments are already the B operand of the next MFMA and P and
// dS never leave the registers: a 16x16 C fragment gives lane l the column
// l % 16 at rows 4 (l / 16) + 0..3; two of them (rows 32c .. 32c + 31) make
// the 8 contraction values of lane group l / 16 in the order
// {32c + 4g + 0..3, 32c + 16 + 4g + 0..3}.  The matching A operand is read
// from a row-major LDS tile with two transposing loads (ds_read_b64_tr_b16)
// at those row groups.
//
// Forward: one workgroup per (64-query block, query head, sequence); four
// waves own 16 query rows each.  Key/value blocks of 64 rows are prefetched
// into registers and double-buffered in LDS.  S^T = K Q^T, online softmax in
// fp32 per query (column), O^T += V^T P^T.  The log-sum-exp of every row is
// kept for the backward pass.
//
// Backward (recomputes P from Q, K and the saved log-sum-exp):
//   pass 0: Dsum[q] = sum_d dO[q, d] O[q, d]
//   pass 1: per (64-key block, query head): S = Q K^T, dP = dO V^T,
//           dV_h^T = dO^T P, dK_h^T = Q^T dS, written as fp32 partials per
//           query head;
//   pass 2: per (64-query block, query head): S^T, dP^T, dQ^T = K^T dS^T;
//   pass 3: dK, dV of a kv head = the sum of its query heads' partials,
//           in a fixed order (no atomics).
// with dS = P (dP - Dsum), and the 1/sqrt(d) scale.
#include "common.h"
#include "kernels.h"

namespace lsf {
namespace {

constexpr int HD = 128, BLK = 64, NTHR = 256;
constexpr float LOG2E = 1.4426950408889634f;

// Tile rows of 128 bf16 (16 chunks of 16 B), chunk' = chunk ^ swz16(row).
// The tiles are read two ways: 16-byte fragments (one chunk from each of 16
// rows) and transposing 8-byte reads (chunks 2j, 2j+1 from each of 8 rows), and
// written as whole rows.  swz16 = 13 r0 ^ 8 r1 ^ 2 r2 (XOR of the row bits'
// multiples) was chosen by timing these three patterns on gfx950 for a set of
// XOR-linear swizzles: it is the fastest for all three at once (transposing
// reads 2 cycles per instruction instead of 4 with r & 15, fragment reads
// and row stores unchanged).
__device__ __forceinline__ int swz16(int row) {
  return ((row & 1) ? 13 : 0) ^ (((row >> 1) & 1) << 3) ^ (((row >> 2) & 1) << 1);
}
__device__ __forceinline__ int off_r16(int row, int chunk) { return row * 128 + ((chunk ^ swz16(row)) << 3); }

// A 64 x 128 bf16 tile (rows r0 .. r0 + 63 of a [rows, ld] matrix; zeros at or
// past `rows`) held as four 16-byte chunks per thread between its global load
// and its LDS store.
struct TileRegs {
  u32x4 v[4];
};

__device__ __forceinline__ void tile_load(const uint16_t* src, int64_t ld, int r0, int rows, int tid, TileRegs& t) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + NTHR * i;
    const int row = idx >> 4, ch = idx & 15;
    t.v[i] = (r0 + row < rows) ? *reinterpret_cast<const u32x4*>(src + (int64_t)(r0 + row) * ld + ch * 8)
                               : u32x4{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void tile_store(const TileRegs& t, uint16_t* lds, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + NTHR * i;
    *reinterpret_cast<u32x4*>(lds + off_r16(idx >> 4, idx & 15)) = t.v[i];
  }
}

// Row fragment of an LDS tile: row `row`, 8 values of chunk `chunk`.
__device__ __forceinline__ u32x4 frag_row(const uint16_t* lds, int row, int chunk) {
  return *reinterpret_cast<const u32x4*>(lds + off_r16(row, chunk));
}

// Operand whose contraction runs down the tile rows: lane l gets column
// col0 + l % 16 at rows r0 + 4g + 0..3 and r0 + 16 + 4g + 0..3, g = l / 16.
__device__ __forceinline__ u32x4 frag_tr(const uint16_t* lds, int col0, int r0, int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  const int col = col0 + 4 * (lr & 3);
  const int row = r0 + lg * 4 + (lr >> 2);
  const u32x2 lo = lds_read_tr4(lds, off_r16(row, col >> 3) + (col & 7));
  const u32x2 hi = lds_read_tr4(lds, off_r16(row + 16, col >> 3) + (col & 7));
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// B operand from two C fragments (contraction rows 32c .. 32c + 31).
__device__ __forceinline__ u32x4 c_to_b(const f32x4& f0, const f32x4& f1) {
  return u32x4{pack_bf16x2(f0[0], f0[1]), pack_bf16x2(f0[2], f0[3]), pack_bf16x2(f1[0], f1[1]),
               pack_bf16x2(f1[2], f1[3])};
}

// Global row fragment: row `row` (or zeros past `rows`), dims s*32 + lg*8 .. +8.
__device__ __forceinline__ u32x4 gfrag(const uint16_t* base, int64_t ld, int row, int rows, int s, int lg) {
  if (row >= rows) return u32x4{0, 0, 0, 0};
  return *reinterpret_cast<const u32x4*>(base + (int64_t)row * ld + s * 32 + lg * 8);
}

__global__ __launch_bounds__(NTHR) void attn_fwd_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BLK * HD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BLK * HD];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int seq = a.seq;
  const int nqb = (seq + BLK - 1) / BLK;
  const int qb = nqb - 1 - (int)blockIdx.x;  // the longest rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (a.nq / a.nkv);
  const int64_t rowbase = (int64_t)b * seq;
  const uint16_t* Qg = a.qkv + rowbase * a.ldqkv + (int64_t)h * HD;
  const uint16_t* Kg = a.qkv + rowbase * a.ldqkv + (int64_t)(a.nq + kvh) * HD;
  const uint16_t* Vg = a.qkv + rowbase * a.ldqkv + (int64_t)(a.nq + a.nkv + kvh) * HD;
  const int qw = qb * BLK + wid * 16;
  const int q = qw + lr;  // this lane's query (its softmax column)
  const float c = LOG2E / sqrtf((float)HD);

  u32x4 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s] = gfrag(Qg, a.ldqkv, q, seq, s, lg);

  f32x4 o[8];  // O^T: o[n][i] = O[q][16 n + 4 lg + i]
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = f32x4{0, 0, 0, 0};
  float mrow = -INFINITY, lrow = 0.0f;

  const int nkb = min(qb + 1, nqb);
  TileRegs kr, vr;
  tile_load(Kg, a.ldqkv, 0, seq, tid, kr);
  tile_load(Vg, a.ldqkv, 0, seq, tid, vr);
  tile_store(kr, Ks[0], tid);
  tile_store(vr, Vs[0], tid);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    const bool pre = kb + 1 < nkb;
    if (pre) {
      tile_load(Kg, a.ldqkv, (kb + 1) * BLK, seq, tid, kr);
      tile_load(Vg, a.ldqkv, (kb + 1) * BLK, seq, tid, vr);
    }
    f32x4 st[4];  // S^T: st[nf][i] = S[q][kb*64 + 16 nf + 4 lg + i]
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      st[nf] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) st[nf] = mfma16x16x32(frag_row(Ks[cur], nf * 16 + lr, s * 4 + lg), qf[s], st[nf]);
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kv = kb * BLK + nf * 16 + lg * 4 + i;
        const float v = (kv <= q && kv < seq) ? st[nf][i] * c : -INFINITY;
        st[nf][i] = v;
        mloc = fmaxf(mloc, v);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float mn = fmaxf(mrow, mloc);
    const float alpha = (mrow == -INFINITY) ? 0.0f : exp2f(mrow - mn);
    float rs = 0.0f;
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (st[nf][i] == -INFINITY) ? 0.0f : exp2f(st[nf][i] - mn);
        st[nf][i] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    lrow = lrow * alpha + rs;
    mrow = mn;
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] *= alpha;
    const u32x4 pb0 = c_to_b(st[0], st[1]), pb1 = c_to_b(st[2], st[3]);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      o[n] = mfma16x16x32(frag_tr(Vs[cur], n * 16, 0, lane), pb0, o[n]);
      o[n] = mfma16x16x32(frag_tr(Vs[cur], n * 16, 32, lane), pb1, o[n]);
    }
    if (pre) {
      tile_store(kr, Ks[cur ^ 1], tid);
      tile_store(vr, Vs[cur ^ 1], tid);
    }
    __syncthreads();
  }
  if (q < seq) {
    uint16_t* Og = a.o + (rowbase + q) * ((int64_t)a.nq * HD) + (int64_t)h * HD;
    const float inv = 1.0f / lrow;
#pragma unroll
    for (int n = 0; n < 8; ++n)
      *reinterpret_cast<u32x2*>(Og + n * 16 + lg * 4) =
          u32x2{pack_bf16x2(o[n][0] * inv, o[n][1] * inv), pack_bf16x2(o[n][2] * inv, o[n][3] * inv)};
    if (lg == 0) a.lse[((int64_t)b * a.nq + h) * seq + q] = (mrow + log2f(lrow)) / LOG2E;
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
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BLK * HD];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[2][BLK * HD];
  __shared__ float lse_s[2][BLK], ds_s[2][BLK];
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
  const int kv = kw + lr;  // this lane's key (column of S, dP)
  const float c = LOG2E / sqrtf((float)HD);

  u32x4 kf[4], vf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kf[s] = gfrag(Kg, a.ldqkv, kv, seq, s, lg);
    vf[s] = gfrag(Vg, a.ldqkv, kv, seq, s, lg);
  }
  f32x4 dk[8], dv[8];  // dK^T, dV^T: dk[n][i] = dK[kv][16 n + 4 lg + i]
#pragma unroll
  for (int n = 0; n < 8; ++n) { dk[n] = f32x4{0, 0, 0, 0}; dv[n] = f32x4{0, 0, 0, 0}; }

  const int nqb = (seq + BLK - 1) / BLK;
  TileRegs qr, orr;
  auto stage_scalars = [&](int qb, int buf) {
    if (tid < BLK) {
      const int qq = qb * BLK + tid;
      lse_s[buf][tid] = (qq < seq) ? lse[qq] * LOG2E : 0.0f;
      ds_s[buf][tid] = (qq < seq) ? Ds[qq] : 0.0f;
    }
  };
  tile_load(Qg, a.ldqkv, kb * BLK, seq, tid, qr);
  tile_load(dOg, ldo, kb * BLK, seq, tid, orr);
  tile_store(qr, Qs[0], tid);
  tile_store(orr, dOs[0], tid);
  stage_scalars(kb, 0);
  __syncthreads();
  for (int qb = kb; qb < nqb; ++qb) {
    const int cur = (qb - kb) & 1;
    const bool pre = qb + 1 < nqb;
    f32x4 st[4], dpt[4];  // S, dP: st[nf][i] = S[qb*64 + 16 nf + 4 lg + i][kv]
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      st[nf] = f32x4{0, 0, 0, 0};
      dpt[nf] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        st[nf] = mfma16x16x32(frag_row(Qs[cur], nf * 16 + lr, s * 4 + lg), kf[s], st[nf]);
        dpt[nf] = mfma16x16x32(frag_row(dOs[cur], nf * 16 + lr, s * 4 + lg), vf[s], dpt[nf]);
      }
    }
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ql = nf * 16 + lg * 4 + i;
        const int qq = qb * BLK + ql;
        const bool ok = kv <= qq && qq < seq && kv < seq;
        const float p = ok ? exp2f(st[nf][i] * c - lse_s[cur][ql]) : 0.0f;
        st[nf][i] = p;
        dpt[nf][i] = p * (dpt[nf][i] - ds_s[cur][ql]);
      }
    const u32x4 pb0 = c_to_b(st[0], st[1]), pb1 = c_to_b(st[2], st[3]);
    const u32x4 db0 = c_to_b(dpt[0], dpt[1]), db1 = c_to_b(dpt[2], dpt[3]);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      dv[n] = mfma16x16x32(frag_tr(dOs[cur], n * 16, 0, lane), pb0, dv[n]);
      dv[n] = mfma16x16x32(frag_tr(dOs[cur], n * 16, 32, lane), pb1, dv[n]);
      dk[n] = mfma16x16x32(frag_tr(Qs[cur], n * 16, 0, lane), db0, dk[n]);
      dk[n] = mfma16x16x32(frag_tr(Qs[cur], n * 16, 32, lane), db1, dk[n]);
    }
    if (pre) {
      // The next tiles are loaded here rather than before the MFMAs: holding
      // them in registers across the block took the kernel to 260 registers,
      // one workgroup per CU; at 228 two fit, 22% faster at 2048 tokens.
      tile_load(Qg, a.ldqkv, (qb + 1) * BLK, seq, tid, qr);
      tile_load(dOg, ldo, (qb + 1) * BLK, seq, tid, orr);
      tile_store(qr, Qs[cur ^ 1], tid);
      tile_store(orr, dOs[cur ^ 1], tid);
      stage_scalars(qb + 1, cur ^ 1);
    }
    __syncthreads();
  }
  if (kv < seq) {
    const float scale = 1.0f / sqrtf((float)HD);
    const int64_t base = ((rowbase + kv) * a.nq + h) * HD;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      *reinterpret_cast<f32x4*>(sc.dkp + base + n * 16 + lg * 4) = dk[n] * scale;
      *reinterpret_cast<f32x4*>(sc.dvp + base + n * 16 + lg * 4) = dv[n];
    }
  }
}

__global__ __launch_bounds__(NTHR) void attn_bwd_q_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BLK * HD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BLK * HD];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int seq = a.seq;
  const int nqb = (seq + BLK - 1) / BLK;
  const int qb = nqb - 1 - (int)blockIdx.x;  // the longest rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / (a.nq / a.nkv);
  const int64_t rowbase = (int64_t)b * seq;
  const int64_t ldo = (int64_t)a.nq * HD;
  const uint16_t* Qg = a.qkv + rowbase * a.ldqkv + (int64_t)h * HD;
  const uint16_t* Kg = a.qkv + rowbase * a.ldqkv + (int64_t)(a.nq + kvh) * HD;
  const uint16_t* Vg = a.qkv + rowbase * a.ldqkv + (int64_t)(a.nq + a.nkv + kvh) * HD;
  const uint16_t* dOg = a.dout + rowbase * ldo + (int64_t)h * HD;
  const int qw = qb * BLK + wid * 16;
  const int q = qw + lr;  // this lane's query (column of S^T, dP^T)
  const float c = LOG2E / sqrtf((float)HD);

  u32x4 qf[4], of[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qf[s] = gfrag(Qg, a.ldqkv, q, seq, s, lg);
    of[s] = gfrag(dOg, ldo, q, seq, s, lg);
  }
  const float l2 = (q < seq) ? a.lse[((int64_t)b * a.nq + h) * seq + q] * LOG2E : 0.0f;
  const float dd = (q < seq) ? a.Dsum[((int64_t)b * a.nq + h) * seq + q] : 0.0f;
  f32x4 dq[8];  // dQ^T: dq[n][i] = dQ[q][16 n + 4 lg + i]
#pragma unroll
  for (int n = 0; n < 8; ++n) dq[n] = f32x4{0, 0, 0, 0};
  const int nkb = min(qb + 1, nqb);
  TileRegs kr, vr;
  tile_load(Kg, a.ldqkv, 0, seq, tid, kr);
  tile_load(Vg, a.ldqkv, 0, seq, tid, vr);
  tile_store(kr, Ks[0], tid);
  tile_store(vr, Vs[0], tid);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    const bool pre = kb + 1 < nkb;
    if (pre) {
      tile_load(Kg, a.ldqkv, (kb + 1) * BLK, seq, tid, kr);
      tile_load(Vg, a.ldqkv, (kb + 1) * BLK, seq, tid, vr);
    }
    f32x4 st[4], dpt[4];  // S^T, dP^T: st[nf][i] = S[q][kb*64 + 16 nf + 4 lg + i]
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      st[nf] = f32x4{0, 0, 0, 0};
      dpt[nf] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        st[nf] = mfma16x16x32(frag_row(Ks[cur], nf * 16 + lr, s * 4 + lg), qf[s], st[nf]);
        dpt[nf] = mfma16x16x32(frag_row(Vs[cur], nf * 16 + lr, s * 4 + lg), of[s], dpt[nf]);
      }
    }
#pragma unroll
    for (int nf = 0; nf < 4; ++nf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kv = kb * BLK + nf * 16 + lg * 4 + i;
        const bool ok = kv <= q && q < seq && kv < seq;
        const float p = ok ? exp2f(st[nf][i] * c - l2) : 0.0f;
        dpt[nf][i] = p * (dpt[nf][i] - dd);
      }
    const u32x4 db0 = c_to_b(dpt[0], dpt[1]), db1 = c_to_b(dpt[2], dpt[3]);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      dq[n] = mfma16x16x32(frag_tr(Ks[cur], n * 16, 0, lane), db0, dq[n]);
      dq[n] = mfma16x16x32(frag_tr(Ks[cur], n * 16, 32, lane), db1, dq[n]);
    }
    if (pre) {
      tile_store(kr, Ks[cur ^ 1], tid);
      tile_store(vr, Vs[cur ^ 1], tid);
    }
    __syncthreads();
  }
  if (q < seq) {
    const float scale = 1.0f / sqrtf((float)HD);
    uint16_t* dQg = a.dqkv + (rowbase + q) * a.ldqkv + (int64_t)h * HD;
#pragma unroll
    for (int n = 0; n < 8; ++n)
      *reinterpret_cast<u32x2*>(dQg + n * 16 + lg * 4) = u32x2{pack_bf16x2(dq[n][0] * scale, dq[n][1] * scale),
                                                              pack_bf16x2(dq[n][2] * scale, dq[n][3] * scale)};
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

// Scratch: the dK / dV partials live right after Dsum, at a 64-float boundary.
hipError_t attention_bwd(const AttnArgs& a, hipStream_t s) {
  const int64_t T = (int64_t)a.batch * a.seq;
  BwdScratch sc;
  sc.dkp = a.Dsum + attention_dsum_floats(a.batch, a.nq, a.seq);
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
