// Fused NF4-dequant bf16 MFMA GEMMs for gfx950.
//
// Forward (NT):  C[M, N] = A[M, K] . deq(W)[N, K]^T  (+ LoRA, + epilogue)
// Backward (NN): C[M, N] = A[M, K] . deq(W)[K, N]    (the input gradient
//                dX = dY W through the frozen weight; W gets no gradient)
//
// The frozen weight is never materialised in HBM: every 128x64 (NT) or
// 64x128 (NN) weight tile is read as packed 4-bit codes plus one fp32 absmax
// per 64-element block, decoded in registers to exactly the bf16 values
// nf4_dequantize writes (bf16_rne(level * absmax)), and staged in LDS for the
// MFMA.  The LoRA side path is folded in as extra contraction steps: the
// rank-r activations U (already scaled) and the adapter matrix form a 64-wide
// extension of A and W, so the scaled add happens inside the accumulator.
//
// Tiling: BM x 128 C tiles (BM = 128 or 256), 64-deep k tiles, waves of 64x64
// (2 across N, BM/64 down M), v_mfma_f32_16x16x32_bf16, LDS double-buffered.
// A 256-row tile decodes each weight once for twice the rows.  The forward
// loop keeps two register stages (prefetch distance 2) and places the decode
// of the next tile in the same basic block as the MFMAs of the current one.  The input-gradient
// GEMM reads its B operand with transposing LDS loads (ds_read_b64_tr_b16)
// because its contraction runs down the weight's rows.  Split-K over grid.z
// with a fixed-order reduction keeps results deterministic.
#include "common.h"
#include "kernels.h"
#include "weight_decode.h"

#include <atomic>

namespace lsf {
namespace {

constexpr int BN = 128, BK = 64;

template <int BM>
struct Cfg {
  static constexpr int NTHR = BM * 2;            // one 64x64 wave tile per 64 rows x 64 columns
  static constexpr int A_ELEMS = BM * BK;
  static constexpr int STAGE = A_ELEMS + BK * BN;
  static constexpr int UNIT = (BN * BK) / NTHR;  // weights each thread decodes per tile: 32 or 16
  static constexpr int MIN_BLOCKS = 512 / NTHR;  // eight waves per CU
};

// LDS layouts (in bf16 elements).  R8: 64 bf16 per row (8 chunks of 16 B),
// chunk' = chunk ^ (row & 7).  R16: 128 bf16 per row (16 chunks), chunk' =
// chunk ^ swz16(row), for the weight tile of the input-gradient GEMM.  gfx950's
// LDS has 64 banks (256 bytes per cycle) and serves each 32-lane half of a
// wave separately; 8-byte reads, the transposing ones included, are free of
// bank conflicts when no 8-byte slot (mod 256 B) repeats within a half.  The
// transposing reads here take chunks 2j, 2j+1 of rows {0-3, 8-11} (or {4-7,
// 12-15}) of a 16-row group, so swz16 gives those 8 rows 8 distinct values of
// its upper three bits (r3, r0, r1); its low bit (r0) keeps the decode stores
// at the fastest rate measured for them.  Measured with LDS pattern probes:
// transposing reads 2 cycles per instruction (4 with the earlier r & 15).
__device__ __forceinline__ int swz16(int row) {
  return (((row >> 3) & 1) << 3) | ((row & 1) << 2) | (((row >> 1) & 1) << 1) | (row & 1);
}
__device__ __forceinline__ int off_r8(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }
__device__ __forceinline__ int off_r16(int row, int chunk) { return row * 128 + ((chunk ^ swz16(row)) << 3); }

__device__ __forceinline__ u32x4 lds_read16(const uint16_t* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(uint16_t* base, int off, const u32x4& v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}

__device__ __forceinline__ u32x4 gload16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 gload8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// Row of the weight that feeds physical tile column c (NT).
__device__ __forceinline__ int64_t nt_wrow(const GemmArgs& g, int ntile, int c) {
  if (g.pair_I > 0) {
    const int j = ntile * 64 + (c >> 5) * 16 + (c & 15);
    return ((c >> 4) & 1) ? (int64_t)g.pair_I + j : (int64_t)j;
  }
  return (int64_t)ntile * BN + c;
}

struct Stage {
  u32x4 a[4];
  u32x4 b[4];
  float absmax;
};

template <int BM, bool NN, int FMT>
__device__ __forceinline__ void load_main(const GemmArgs& g, int m0, int ntile, int k0, int tid, Stage& st) {
  using C = Cfg<BM>;
  // A tile: BM rows x 64 k, 4 chunks of 16 B per thread.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + C::NTHR * i;
    const int row = idx >> 3, ch = idx & 7;
    // Rows past M read row M-1: each C row depends on its own A row only and
    // rows past M are never stored, so the load needs no branch.
    const int gm = min(m0 + row, g.M - 1);
    st.a[i] = gload16(g.A + (int64_t)gm * g.lda + k0 + ch * 8);
  }
  if constexpr (FMT == FMT_BF16) {
    constexpr int PER = 1024 / C::NTHR;  // 16-byte chunks of the weight tile per thread
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + C::NTHR * i;
      if constexpr (!NN) {
        const int row = idx >> 3, ch = idx & 7;
        st.b[i] = gload16(g.W.bf16 + nt_wrow(g, ntile, row) * g.W.ld + k0 + ch * 8);
      } else {
        const int row = idx >> 4, ch = idx & 15;
        st.b[i] = gload16(g.W.bf16 + (int64_t)(k0 + row) * g.W.ld + ntile * BN + ch * 8);
      }
    }
  } else {
    constexpr int U = C::UNIT;
    int64_t e;
    if constexpr (!NN) {
      const int per_row = BK / U;  // units per weight row
      const int row = tid / per_row, q = tid % per_row;
      e = nt_wrow(g, ntile, row) * g.W.ld + k0 + q * U;
    } else {
      const int per_row = BN / U;
      const int row = tid / per_row, q = tid % per_row;
      e = (int64_t)(k0 + row) * g.W.ld + ntile * BN + q * U;
    }
    if constexpr (U == 32) st.b[0] = gload16(g.W.packed + (e >> 1));
    else {
      const u32x2 v = gload8(g.W.packed + (e >> 1));
      st.b[0] = u32x4{v.x, v.y, 0, 0};
    }
    st.absmax = block_absmax_t<FMT>(g.W, e);
  }
}

template <int BM, bool NN, int FMT>
__device__ __forceinline__ void store_main(const Stage& st, int tid, uint16_t* As, uint16_t* Bs) {
  using C = Cfg<BM>;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + C::NTHR * i;
    lds_write16(As, off_r8(idx >> 3, idx & 7), st.a[i]);
  }
  if constexpr (FMT == FMT_BF16) {
    constexpr int PER = 1024 / C::NTHR;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + C::NTHR * i;
      if constexpr (!NN) lds_write16(Bs, off_r8(idx >> 3, idx & 7), st.b[i]);
      else lds_write16(Bs, off_r16(idx >> 4, idx & 15), st.b[i]);
    }
  } else {
    constexpr int U = C::UNIT;
    constexpr int NW = U / 8;  // packed dwords per thread
    const Nf4Table t = nf4_table(st.absmax);
    const uint32_t q[4] = {st.b[0].x, st.b[0].y, st.b[0].z, st.b[0].w};
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      uint32_t o[4];
      nf4_decode8(t, q[i], o);
      const u32x4 v = {o[0], o[1], o[2], o[3]};
      if constexpr (!NN) {
        const int per_row = BK / U;
        const int row = tid / per_row, qq = tid % per_row;
        lds_write16(Bs, off_r8(row, qq * NW + i), v);
      } else {
        const int per_row = BN / U;
        const int row = tid / per_row, qq = tid % per_row;
        lds_write16(Bs, off_r16(row, qq * NW + i), v);
      }
    }
  }
}

// LoRA extension tile number `xt` written straight into LDS.
template <int BM, bool NN>
__device__ void store_ext(const GemmArgs& g, int m0, int ntile, int xt, int tid, uint16_t* As, uint16_t* Bs) {
  const LoraExt& x = g.ext;
  const int jb = xt * BK;
  {  // A: BM rows x 64 columns of U, scaled, rounded to bf16
    const int row = tid >> 1, h = tid & 1;
    const int gm = m0 + row;
    uint32_t w[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      float v[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int j = jb + h * 32 + p * 2 + q;
        v[q] = (gm < g.M && j < x.kx) ? x.uscale * x.u[(int64_t)gm * x.ldu + j] : 0.0f;
      }
      w[p] = pack_bf16x2(v[0], v[1]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds_write16(As, off_r8(row, h * 4 + i), u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]});
  }
  if (tid >= 256) return;
  if constexpr (!NN) {  // B: tile row c = weight row, column = U column j
    const int row = tid >> 1, h = tid & 1;
    const int64_t wr = nt_wrow(g, ntile, row);
    int sec = 0;
    for (int s = 1; s < x.nsec; ++s)
      if (wr >= x.row_off[s]) sec = s;
    const float* bm = x.mat[sec];
    const int64_t lr = wr - x.row_off[sec];
    uint32_t w[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      float v[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int j = jb + h * 32 + p * 2 + q;
        const int jl = j - sec * x.r;
        v[q] = (bm != nullptr && j < x.kx && jl >= 0 && jl < x.r) ? bm[lr * x.r + jl] : 0.0f;
      }
      w[p] = pack_bf16x2(v[0], v[1]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds_write16(Bs, off_r8(row, h * 4 + i), u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]});
  } else {  // B: tile row = U column j (contraction), columns = output n
    const int row = tid >> 2, seg = tid & 3;
    const int j = jb + row;
    const int sec = (x.r > 0) ? j / x.r : 0;
    const float* am = (j < x.kx && sec < x.nsec) ? x.mat[sec] : nullptr;
    const int n0 = ntile * BN + seg * 32;
    uint32_t w[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      float v0 = 0.0f, v1 = 0.0f;
      if (am != nullptr) {
        const float* src = am + (int64_t)(j - sec * x.r) * x.ldmat + n0 + p * 2;
        v0 = src[0];
        v1 = src[1];
      }
      w[p] = pack_bf16x2(v0, v1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds_write16(Bs, off_r16(row, seg * 4 + i), u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]});
  }
}

template <bool NN>
__device__ __forceinline__ void compute_tile(const uint16_t* As, const uint16_t* Bs, int lane, int wm, int wn,
                                             f32x4 (&acc)[4][4]) {
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    u32x4 af[4], bf[4];
#pragma unroll
    for (int mf = 0; mf < 4; ++mf) af[mf] = lds_read16(As, off_r8(wm * 64 + mf * 16 + lr, s * 4 + lg));
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      if constexpr (!NN) {
        bf[nf] = lds_read16(Bs, off_r8(wn * 64 + nf * 16 + lr, s * 4 + lg));
      } else {
        // Contraction runs down the tile rows: two transposing 8-byte reads
        // give this lane (column nbase + lr) rows c..c+3 and c+4..c+7.
        const int col = wn * 64 + nf * 16 + 4 * (lr & 3);
        const int row = s * 32 + lg * 8 + (lr >> 2);
        const u32x2 lo = lds_read_tr4(Bs, off_r16(row, col >> 3) + (col & 7));
        const u32x2 hi = lds_read_tr4(Bs, off_r16(row + 4, col >> 3) + (col & 7));
        bf[nf] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    }
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mfma16x16x32(af[mf], bf[nf], acc[mf][nf]);
  }
}

// One 64-deep k tile of MFMAs from (As, Bs) and, in the same basic block, the
// decode + LDS store of the next tile (staged in st) into (An, Bn), so the
// compiler can issue the decode's VALU work between the MFMAs.  (Explicit
// MFMA/VALU interleaving hints measured 2-4% slower than its own schedule.)
template <int BM, bool NN, int FMT>
__device__ __forceinline__ void compute_and_stage(const uint16_t* As, const uint16_t* Bs, const Stage& st, int tid,
                                                  uint16_t* An, uint16_t* Bn, int lane, int wm, int wn,
                                                  f32x4 (&acc)[4][4]) {
  compute_tile<NN>(As, Bs, lane, wm, wn, acc);
  store_main<BM, NN, FMT>(st, tid, An, Bn);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// This wave's LDS accesses so far are complete, and neither the compiler nor
// the hardware moves later ones ahead of them.
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// SwiGLU backward with the accumulator tile passed through LDS.  Each wave
// writes 32 rows of its 64 x 64 tile at a time into its own 8 KB of the stage
// buffers (idle once the k loop has ended), then every lane takes 8
// consecutive columns of one row, so the gate/up reads and the dg/du writes
// are 16-byte accesses, 128 contiguous bytes per 8 lanes.  Rows past M load a
// clamped row and store nothing.  Same arithmetic per element as the direct
// form, so the same bits.
__device__ void swiglu_bwd_staged(const GemmArgs& g, const EpiArgs& e, const f32x4 (&acc)[4][4], int m0, int ntile,
                                  int lane, int wm, int wn, float* red) {
  const int lr = lane & 15, lg = lane >> 4;
  float* my = red + (wm * 2 + wn) * (32 * 64);
  const int cq = (lane & 7) * 8;
  const int n = ntile * BN + wn * 64 + cq;
  uint16_t* C = static_cast<uint16_t*>(e.C);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int mf = 0; mf < 2; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
#pragma unroll
        for (int i = 0; i < 4; ++i) my[(mf * 16 + lg * 4 + i) * 64 + nf * 16 + lr] = acc[2 * h + mf][nf][i];
    wave_lds_fence();
    u32x4 gq[4], uq[4];
    float4 v0[4], v1[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = p * 8 + (lane >> 3);
      const int64_t m = min(m0 + wm * 64 + h * 32 + r, g.M - 1);
      gq[p] = *reinterpret_cast<const u32x4*>(e.g + m * e.ldgu + n);
      uq[p] = *reinterpret_cast<const u32x4*>(e.u + m * e.ldgu + n);
      v0[p] = *reinterpret_cast<const float4*>(my + r * 64 + cq);
      v1[p] = *reinterpret_cast<const float4*>(my + r * 64 + cq + 4);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int m = m0 + wm * 64 + h * 32 + p * 8 + (lane >> 3);
      const float v[8] = {v0[p].x, v0[p].y, v0[p].z, v0[p].w, v1[p].x, v1[p].y, v1[p].z, v1[p].w};
      u32x4 dgo, duo;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float dg0, du0, dg1, du1;
        swiglu_grad(v[2 * q], bf16lo(gq[p][q]), bf16lo(uq[p][q]), dg0, du0);
        swiglu_grad(v[2 * q + 1], bf16hi(gq[p][q]), bf16hi(uq[p][q]), dg1, du1);
        dgo[q] = pack_bf16x2(dg0, dg1);
        duo[q] = pack_bf16x2(du0, du1);
      }
      if (m < g.M) {
        *reinterpret_cast<u32x4*>(C + (int64_t)m * e.ldc + n) = dgo;
        *reinterpret_cast<u32x4*>(C + (int64_t)m * e.ldc + g.N + n) = duo;
      }
    }
    wave_lds_fence();
  }
}

template <bool NN, int EPI>
__device__ void epilogue(const GemmArgs& g, const EpiArgs& e, const f32x4 (&acc)[4][4], int m0, int ntile,
                         int lane, int wm, int wn, int z, uint16_t* lds_base) {
  const int lr = lane & 15, lg = lane >> 4;
  if constexpr (NN && EPI == EPI_SWIGLU_BWD) {
    swiglu_bwd_staged(g, e, acc, m0, ntile, lane, wm, wn, reinterpret_cast<float*>(lds_base));
    return;
  }
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
      for (int np = 0; np < 2; ++np) {
        const int j = ntile * 64 + (2 * wn + np) * 16 + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wm * 64 + mf * 16 + lg * 4 + i;
          if (m >= g.M) continue;
          const float gv = acc[mf][2 * np][i], uv = acc[mf][2 * np + 1][i];
          static_cast<uint16_t*>(e.C)[(int64_t)m * e.ldc + j] = f32_to_bf16(silu(gv) * uv);
          if (e.g != nullptr) {
            e.g[(int64_t)m * e.ldgu + j] = f32_to_bf16(gv);
            e.u[(int64_t)m * e.ldgu + j] = f32_to_bf16(uv);
          }
        }
      }
    return;
  }
#pragma unroll
  for (int mf = 0; mf < 4; ++mf)
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int n = ntile * BN + wn * 64 + nf * 16 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 64 + mf * 16 + lg * 4 + i;
        if (m >= g.M) continue;
        const float v = acc[mf][nf][i];
        if constexpr (EPI == EPI_F32) {
          static_cast<float*>(e.C)[(int64_t)z * g.M * g.N + (int64_t)m * e.ldc + n] = v;
        } else if constexpr (EPI == EPI_BF16) {
          static_cast<uint16_t*>(e.C)[(int64_t)m * e.ldc + n] = f32_to_bf16(v);
        } else if constexpr (EPI == EPI_RESID_BF16) {
          static_cast<uint16_t*>(e.C)[(int64_t)m * e.ldc + n] =
              f32_to_bf16(bf16_to_f32(e.R[(int64_t)m * e.ldr + n]) + v);
        }
      }
    }
}

template <int BM, bool NN, int FMT, int EPI>
__global__ __launch_bounds__(Cfg<BM>::NTHR, Cfg<BM>::MIN_BLOCKS) void gemm_kernel(GemmArgs g, EpiArgs e) {
  using C = Cfg<BM>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int mt = (g.M + BM - 1) / BM, nt = g.N / BN;
  const int total = mt * nt;
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);  // keep an XCD on neighbouring tiles
  const int mtile = t % mt, ntile = t / mt;
  const int m0 = mtile * BM;

  const int z = blockIdx.z;
  const int kch = g.K / BK;
  const int per = (kch + g.splits - 1) / g.splits;
  const int kb = z * per;
  const int ke = min(kch, kb + per);
  const int nmain = max(0, ke - kb);
  const int next = (z == g.splits - 1 && g.ext.kx > 0) ? (g.ext.kx + BK - 1) / BK : 0;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  uint16_t* b0 = lds[0];
  uint16_t* b1 = lds[1];
  if constexpr (NN || FMT == FMT_BF16) {
    // Input-gradient GEMM, and any GEMM over an unquantised bf16 weight (its
    // tile arrives as 16-byte chunks, twice the registers of packed codes):
    // one register stage.
    Stage st;
    if (nmain > 0) {
      load_main<BM, NN, FMT>(g, m0, ntile, kb * BK, tid, st);
      store_main<BM, NN, FMT>(st, tid, b0, b0 + C::A_ELEMS);
    }
    __syncthreads();
    for (int i = 0; i < nmain; ++i) {
      const bool pre = i + 1 < nmain;
      if (pre) load_main<BM, NN, FMT>(g, m0, ntile, (kb + i + 1) * BK, tid, st);
      uint16_t* cur = lds[i & 1];
      compute_tile<NN>(cur, cur + C::A_ELEMS, lane, wm, wn, acc);
      if (pre) store_main<BM, NN, FMT>(st, tid, lds[(i + 1) & 1], lds[(i + 1) & 1] + C::A_ELEMS);
      __syncthreads();
    }
  } else {
    // Forward GEMM: two register stages and two LDS buffers.  Iteration i
    // computes tile i from buffer i&1 while the decode of tile i+1 (loaded
    // one iteration earlier) fills the other buffer and tile i+2 loads.
    Stage s0, s1;
    if (nmain > 0) load_main<BM, NN, FMT>(g, m0, ntile, kb * BK, tid, s0);
    if (nmain > 1) load_main<BM, NN, FMT>(g, m0, ntile, (kb + 1) * BK, tid, s1);
    if (nmain > 0) store_main<BM, NN, FMT>(s0, tid, b0, b0 + C::A_ELEMS);
    __syncthreads();
    int it = 0;
    for (; it + 1 < nmain; it += 2) {
      if (it + 2 < nmain) load_main<BM, NN, FMT>(g, m0, ntile, (kb + it + 2) * BK, tid, s0);
      compute_and_stage<BM, NN, FMT>(b0, b0 + C::A_ELEMS, s1, tid, b1, b1 + C::A_ELEMS, lane, wm, wn, acc);
      __syncthreads();
      if (it + 2 < nmain) {
        if (it + 3 < nmain) load_main<BM, NN, FMT>(g, m0, ntile, (kb + it + 3) * BK, tid, s1);
        compute_and_stage<BM, NN, FMT>(b1, b1 + C::A_ELEMS, s0, tid, b0, b0 + C::A_ELEMS, lane, wm, wn, acc);
      } else {
        compute_tile<NN>(b1, b1 + C::A_ELEMS, lane, wm, wn, acc);
      }
      __syncthreads();
    }
    if (it < nmain) {  // odd tile count: the last tile sits in b0
      compute_tile<NN>(b0, b0 + C::A_ELEMS, lane, wm, wn, acc);
      __syncthreads();
    }
  }
  // LoRA extension steps (last split only)
  for (int xt = 0; xt < next; ++xt) {
    store_ext<BM, NN>(g, m0, ntile, xt, tid, b0, b0 + C::A_ELEMS);
    __syncthreads();
    compute_tile<NN>(b0, b0 + C::A_ELEMS, lane, wm, wn, acc);
    __syncthreads();
  }
  epilogue<NN, EPI>(g, e, acc, m0, ntile, lane, wm, wn, z, &lds[0][0]);
}

template <int BM, bool NN, int EPI>
hipError_t launch_fmt(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  const int mt = (g.M + BM - 1) / BM, nt = g.N / BN;
  dim3 grid(mt * nt, 1, g.splits), block(Cfg<BM>::NTHR);
  switch (g.W.fmt) {
    case FMT_NF4: hipLaunchKernelGGL((gemm_kernel<BM, NN, FMT_NF4, EPI>), grid, block, 0, s, g, e); break;
    case FMT_BF16: hipLaunchKernelGGL((gemm_kernel<BM, NN, FMT_BF16, EPI>), grid, block, 0, s, g, e); break;
    case FMT_NF4_DQ: hipLaunchKernelGGL((gemm_kernel<BM, NN, FMT_NF4_DQ, EPI>), grid, block, 0, s, g, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BM, bool NN>
hipError_t launch_bm(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  switch (e.kind) {
    case EPI_F32: return launch_fmt<BM, NN, EPI_F32>(g, e, s);
    case EPI_BF16: return launch_fmt<BM, NN, EPI_BF16>(g, e, s);
    case EPI_RESID_BF16:
      if constexpr (!NN) return launch_fmt<BM, NN, EPI_RESID_BF16>(g, e, s);
      break;
    case EPI_SWIGLU:
      if constexpr (!NN) return launch_fmt<BM, NN, EPI_SWIGLU>(g, e, s);
      break;
    case EPI_SWIGLU_BWD:
      if constexpr (NN) {
        // 16-byte accesses to g, u and both halves of C
        const bool al = ((uintptr_t)e.C | (uintptr_t)e.g | (uintptr_t)e.u) % 16 == 0 && e.ldc % 8 == 0 &&
                        e.ldgu % 8 == 0 && g.N % 8 == 0;
        if (!al) return hipErrorInvalidValue;
        return launch_fmt<BM, NN, EPI_SWIGLU_BWD>(g, e, s);
      }
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <bool NN>
hipError_t launch(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  return gemm_tile_rows(g.M, g.N, NN) == 256 ? launch_bm<256, NN>(g, e, s) : launch_bm<128, NN>(g, e, s);
}

__global__ void splitk_reduce_kernel(const float* part, int splits, int M, int N, EpiArgs e) {
  const int64_t MN = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += (int64_t)gridDim.x * blockDim.x) {
    float q[8];
#pragma unroll
    for (int zz = 0; zz < 8; ++zz) q[zz] = (zz < splits) ? part[zz * MN + i] : 0.0f;  // splits <= 8
    float v = q[0];
#pragma unroll
    for (int zz = 1; zz < 8; ++zz)
      if (zz < splits) v += q[zz];
    const int64_t m = i / N, n = i - m * N;
    switch (e.kind) {
      case EPI_F32: static_cast<float*>(e.C)[m * e.ldc + n] = v; break;
      case EPI_BF16: static_cast<uint16_t*>(e.C)[m * e.ldc + n] = f32_to_bf16(v); break;
      case EPI_RESID_BF16:
        static_cast<uint16_t*>(e.C)[m * e.ldc + n] = f32_to_bf16(bf16_to_f32(e.R[m * e.ldr + n]) + v);
        break;
      case EPI_SWIGLU_BWD: {
        float dg, du;
        swiglu_grad(v, bf16_to_f32(e.g[m * e.ldgu + n]), bf16_to_f32(e.u[m * e.ldgu + n]), dg, du);
        uint16_t* C = static_cast<uint16_t*>(e.C);
        C[m * e.ldc + n] = f32_to_bf16(dg);
        C[m * e.ldc + N + n] = f32_to_bf16(du);
        break;
      }
      default: break;
    }
  }
}

// The same reduction four elements of one row at a time: 16-byte loads of
// every partial and 8-byte bf16 stores (the scalar form moves 4 bytes per lane
// and load).  The same fp32 adds in the same order per element, so the same
// bits.  Needs N % 4 == 0 and the aligned pointers and strides the host checks.
__device__ __forceinline__ void add4(float4& v, const float4& q) {
  v.x += q.x;
  v.y += q.y;
  v.z += q.z;
  v.w += q.w;
}
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return uint2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

template <int EPI>
__global__ void splitk_reduce4_kernel(const float* part, int splits, int M, int N, EpiArgs e) {
  const int64_t MN = (int64_t)M * N, n4 = MN / 4;
  for (int64_t i4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i4 < n4; i4 += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = i4 * 4;
    float4 q[8];
#pragma unroll
    for (int zz = 0; zz < 8; ++zz)  // splits <= 8
      q[zz] = (zz < splits) ? *reinterpret_cast<const float4*>(part + zz * MN + i) : float4{0, 0, 0, 0};
    float4 v = q[0];
#pragma unroll
    for (int zz = 1; zz < 8; ++zz)
      if (zz < splits) add4(v, q[zz]);
    const int64_t m = i / N, n = i - m * N;
    if constexpr (EPI == EPI_F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(e.C) + m * e.ldc + n) = v;
    } else if constexpr (EPI == EPI_BF16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(e.C) + m * e.ldc + n) = pack4_bf16(v.x, v.y, v.z, v.w);
    } else if constexpr (EPI == EPI_RESID_BF16) {
      const uint2 r = *reinterpret_cast<const uint2*>(e.R + m * e.ldr + n);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(e.C) + m * e.ldc + n) =
          pack4_bf16(bf16lo(r.x) + v.x, bf16hi(r.x) + v.y, bf16lo(r.y) + v.z, bf16hi(r.y) + v.w);
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {
      const uint2 gq = *reinterpret_cast<const uint2*>(e.g + m * e.ldgu + n);
      const uint2 uq = *reinterpret_cast<const uint2*>(e.u + m * e.ldgu + n);
      float dg[4], du[4];
      swiglu_grad(v.x, bf16lo(gq.x), bf16lo(uq.x), dg[0], du[0]);
      swiglu_grad(v.y, bf16hi(gq.x), bf16hi(uq.x), dg[1], du[1]);
      swiglu_grad(v.z, bf16lo(gq.y), bf16lo(uq.y), dg[2], du[2]);
      swiglu_grad(v.w, bf16hi(gq.y), bf16hi(uq.y), dg[3], du[3]);
      uint16_t* C = static_cast<uint16_t*>(e.C);
      *reinterpret_cast<uint2*>(C + m * e.ldc + n) = pack4_bf16(dg[0], dg[1], dg[2], dg[3]);
      *reinterpret_cast<uint2*>(C + m * e.ldc + N + n) = pack4_bf16(du[0], du[1], du[2], du[3]);
    }
  }
}

}  // namespace

// Measured on MI355X at 512 and 2048 tokens: 256-row tiles are faster for the
// input-gradient GEMMs with N <= 4096 (q|k|v, o, gate|up), for forward GEMMs
// with N <= 4096 (o, down) and for the very wide forward gate|up (N = 28672: 6%
// less time, each weight tile decoded once per 256 rows); the forward q|k|v
// (N = 6144) and the input gradient of down (N = 14336: 6% less time) are
// faster with 128-row tiles.
int gemm_tile_rows(int M, int N, bool nn) {
  if (M < 256) return 128;
  if (nn) return N >= 8192 ? 128 : 256;
  return (N <= 4096 || N >= 16384) ? 256 : 128;
}

namespace {
std::atomic<bool> g_wide_enabled{true};
}  // namespace

void set_gemm_wide(bool enable) { g_wide_enabled.store(enable, std::memory_order_relaxed); }

hipError_t gemm_nt(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  if (g_wide_enabled.load(std::memory_order_relaxed) && gemm_wide_applies(g, e)) return gemm_nt_wide(g, e, s);
  return launch<false>(g, e, s);
}
hipError_t gemm_nn(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  if (g_wide_enabled.load(std::memory_order_relaxed) && gemm_wide_nn_applies(g, e)) return gemm_nn_wide(g, e, s);
  return launch<true>(g, e, s);
}

hipError_t splitk_reduce(const float* part, int splits, int M, int N, const EpiArgs& e, hipStream_t s) {
  if (splits < 1 || splits > 8) return hipErrorInvalidValue;
  const int64_t MN = (int64_t)M * N;
  // Four elements per thread where every access of the epilogue is aligned.
  auto al = [](const void* p, int64_t ld, int bytes) {
    return p == nullptr || ((uintptr_t)p % bytes == 0 && ld % 4 == 0);
  };
  bool vec = N % 4 == 0 && (uintptr_t)part % 16 == 0;
  switch (e.kind) {
    case EPI_F32: vec = vec && al(e.C, e.ldc, 16); break;
    case EPI_BF16: vec = vec && al(e.C, e.ldc, 8); break;
    case EPI_RESID_BF16: vec = vec && al(e.C, e.ldc, 8) && al(e.R, e.ldr, 8); break;
    case EPI_SWIGLU_BWD: vec = vec && al(e.C, e.ldc, 8) && al(e.g, e.ldgu, 8) && al(e.u, e.ldgu, 8); break;
    default: vec = false; break;
  }
  if (vec) {
    const int blocks = (int)std::min<int64_t>((MN / 4 + 255) / 256, 4096);
    switch (e.kind) {
      case EPI_F32: hipLaunchKernelGGL(splitk_reduce4_kernel<EPI_F32>, dim3(blocks), dim3(256), 0, s, part, splits, M, N, e); break;
      case EPI_BF16: hipLaunchKernelGGL(splitk_reduce4_kernel<EPI_BF16>, dim3(blocks), dim3(256), 0, s, part, splits, M, N, e); break;
      case EPI_RESID_BF16:
        hipLaunchKernelGGL(splitk_reduce4_kernel<EPI_RESID_BF16>, dim3(blocks), dim3(256), 0, s, part, splits, M, N, e);
        break;
      default:
        hipLaunchKernelGGL(splitk_reduce4_kernel<EPI_SWIGLU_BWD>, dim3(blocks), dim3(256), 0, s, part, splits, M, N, e);
        break;
    }
    return hipGetLastError();
  }
  const int blocks = (int)std::min<int64_t>((MN + 255) / 256, 4096);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, part, splits, M, N, e);
  return hipGetLastError();
}

}  // namespace lsf
