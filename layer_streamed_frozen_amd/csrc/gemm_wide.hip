// Wide NF4 GEMMs for gfx950 ("ping-pong" kernels).  Forward, used when the
// output has many tiles (the gate|up projection; q|k|v from 2048 tokens), and
// as split-K with fp32 partial sums for long contractions over few tiles (the
// down projection): C[M, N] = A[M, K] . deq(W)[N, K]^T  (+ LoRA, + epilogue);
// and the input gradient of gate|up and down: C = A . deq(W)[K, N].
//
// Same arithmetic as the general kernel in gemm.hip (every weight decoded to
// bf16_rne(level * absmax), bf16 MFMA with fp32 accumulation, the k order of
// the contraction unchanged, LoRA as extra contraction steps after the main
// ones), so both kernels give bitwise-identical results; only the schedule
// differs:
//
// * TM x TN C tile (512 x 128 by default, 256 x 256 selectable), 512 threads
//   = two groups of four waves.  The hardware places wave w and wave w+4 of a
//   workgroup on the same SIMD, so every SIMD holds one wave of each group.
//   Each wave owns 128 rows x 64 columns (8 x 4 fragments of
//   v_mfma_f32_16x16x32_bf16); group g owns rows g*TM/2 .. + TM/2.
// * 32-deep k tiles in a ring of four LDS stages (40 or 32 KB each).  The
//   groups run half a tile apart (ping-pong): while one group issues its 32
//   MFMAs, the other runs its memory phase: issue the LDS-DMA of its half of
//   A three tiles ahead (global_load_lds_dwordx4, no register round trip) and
//   load the packed codes and absmax of the tile five ahead into registers,
//   read its own fragments of the current tile, wait for the loads of two
//   phases ago, and decode its half of the weight tile three ahead into LDS.
//   A workgroup barrier between the phases swaps the roles; the one ending a
//   memory phase waits only for the fragment reads (LDS operations of a wave
//   complete in issue order), so the decoded tile's stores land during the
//   compute phase, and the barrier ending the compute phase waits for them.
// * Every memory phase issues the same vector-memory operations: the LDS-DMA
//   of A (past the last tile it repeats the last tile into a stage nobody
//   reads again), then the code and absmax loads.  Loads complete in issue
//   order, so after this phase's own loads `s_waitcnt vmcnt(2n)`, n the
//   operations of one phase, means "everything issued two phases ago has
//   landed": the codes decoded now and the A tile read in the next phase.
//   Every LDS-DMA is an explicit instruction and the two register loads read
//   different arrays, so no phase issues fewer than n; more would only make
//   the wait stricter.  Reusing a stage is safe: the stage written in phase t
//   (tile t+3) held tile t-1, whose fragment reads both groups finished
//   before the barriers that ended their phases t-1.
//   Barriers carry no memory-model fence: a release fence would wait for
//   every LDS-DMA in flight.
// * The input-gradient kernel below keeps its fragment reads ahead of its
//   loads (see its comment).
#include "common.h"
#include "kernels.h"
#include "weight_decode.h"

#include <algorithm>
#include <atomic>

namespace lsf {
namespace {

// C tile TM x TN with TM * TN = 65536 (8 waves of 128 x 64): 256 x 256, or
// 512 x 128 when the rows fit one tile (every weight is then decoded once,
// half the decode work per MFMA of the square tile; the A tile doubles).
constexpr int WBK = 32, WNST = 4;
template <int TM>
struct WCfg {
  static constexpr int TN = 65536 / TM;
  static constexpr int ATILE = TM * WBK;        // bf16 elements of the A tile
  static constexpr int BTILE = TN * WBK;        // and of the B tile
  static constexpr int STAGE = ATILE + BTILE;   // 32 KB (256 x 256) or 40 KB (512 x 128)
  static constexpr int NCW = TN / 64;           // waves across N in one group
  static constexpr int DMA = TM / 128;          // LDS-DMA instructions of A per wave and phase
  static constexpr int DEC = TN * WBK / 512;    // weights each thread decodes per tile: 16 or 8
};

// k tiles (32 deep) of each split but the last: whole 64-blocks, the same k
// ranges as the general kernel's split-K, so both sum the same partials.
__host__ __device__ __forceinline__ int wide_split_tiles(int K, int splits) {
  return 2 * ((K / 64 + splits - 1) / splits);
}

// Tile rows of 32 bf16 (4 chunks of 16 B), chunk' = chunk ^ ((row >> 1) & 3):
// the 8 lanes of a 16-byte read phase hit 8 distinct 16-byte bank groups.
__device__ __forceinline__ int woff(int row, int ch) { return row * 32 + ((ch ^ ((row >> 1) & 3)) << 3); }

// s_waitcnt with only the vector-memory counter constrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x3f70 | N);
}

// This wave's LDS accesses so far are complete, and neither the compiler nor
// the hardware moves later ones ahead of them (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier: this wave's LDS reads and writes complete (lgkmcnt 0),
// then s_barrier.  The empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void wbar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier that lets this wave's last NW LDS stores stay in flight:
// LDS operations of one wave complete in issue order, so lgkmcnt(NW) after
// NW trailing stores means every earlier LDS read has returned.  The stores
// finish before the next wbar() (lgkmcnt 0), and their stage is read only
// after that.  NW must not exceed the number of LDS stores issued after the
// last LDS read.
template <int NW>
__device__ __forceinline__ void wbar_stores() {
  static_assert(NW >= 0 && NW < 16, "lgkmcnt immediate");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0xc07f & ~0x0f00) | (NW << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// Weight row feeding tile column c of column tile `ntile` (TN columns); in
// pair mode gate row j and up row pair_I + j sit 16 columns apart, so one
// lane holds both in its accumulators.
template <int TN>
__device__ __forceinline__ int64_t wide_wrow(const GemmArgs& g, int ntile, int c) {
  if (g.pair_I > 0) {
    const int j = ntile * (TN / 2) + (c >> 5) * 16 + (c & 15);
    return ((c >> 4) & 1) ? (int64_t)g.pair_I + j : (int64_t)j;
  }
  return (int64_t)ntile * TN + c;
}

// Vector-memory operations of one memory phase: the LDS-DMA of A, the codes,
// and the absmax (one load for fp32 absmax; code + group pair for NF4_DQ).
template <int TM, int FMT>
constexpr int phase_vm_ops() { return WCfg<TM>::DMA + (FMT == FMT_NF4_DQ ? 3 : 2); }

// One thread's packed codes of one tile (16 or 8 weights) and its block's absmax.
template <int DEC>
struct CodeSet {
  u32x2 c;
  float am;
};

// Codes of tile t from this thread's code pointer cp, and the absmax of their
// 64-block from its absmax pointer ap (tiles 2j and 2j + 1 share block j).
// Both pointers are per-thread values computed before the k loop, so no kernel
// argument is reloaded inside it (a scalar reload there costs a wait for every
// LDS read in flight).
template <int DEC>
__device__ __forceinline__ CodeSet<DEC> load_codes(const uint8_t* cp, const float* ap, int t) {
  CodeSet<DEC> s;
  if constexpr (DEC == 16) {
    s.c = *reinterpret_cast<const u32x2*>(cp + t * 16);
  } else {
    s.c.x = *reinterpret_cast<const uint32_t*>(cp + t * 16);
    s.c.y = 0;
  }
  s.am = ap[t >> 1];
  return s;
}

__device__ __forceinline__ float wsilu(float x) { return x / (1.0f + __expf(-x)); }

template <int TM, int FMT, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_wide_kernel(GemmArgs g, EpiArgs e) {
  using C = WCfg<TM>;
  constexpr int TN = C::TN, DEC = C::DEC;
  __shared__ __attribute__((aligned(16))) uint16_t lds[WNST * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid >> 2, q = wid & 3, tg = tid & 255;
  const int lr = lane & 15, lg = lane >> 4;
  // wave (grp, q): rows wr .. wr + 128, columns wc .. wc + 64 of the tile
  const int wr = grp * (TM / 2) + (q / C::NCW) * 128, wc = (q % C::NCW) * 64;
  // Split-K only for fp32 partial sums (the split index z and the k range
  // stay compile-time zero and whole otherwise).
  constexpr bool SPLIT = EPI == EPI_F32;
  const int splits = SPLIT ? g.splits : 1;
  const int mt = (g.M + TM - 1) / TM, nt = g.N / TN, tiles = mt * nt, total = tiles * splits;
  int t0 = blockIdx.x;
  // Neighbouring work items on one XCD; split z is the slow index, so an XCD
  // mostly works on one k range of A.
  if ((total & 7) == 0) t0 = (t0 & 7) * (total >> 3) + (t0 >> 3);
  const int z = SPLIT ? t0 / tiles : 0, tile = t0 - z * tiles;
  const int mtile = tile % mt, ntile = tile / mt;
  const int m0 = mtile * TM;
  // This split's k tiles: whole 64-blocks, the same ranges as the general kernel.
  const int per = SPLIT ? wide_split_tiles(g.K, splits) : g.K / WBK;
  const int kt0 = z * per;
  const int nk = min(g.K / WBK - kt0, per);

  // LDS-DMA of A: wave (grp, q) moves rows grp*TM/2 + q*TM/8 + j*16 + lane/4,
  // 16 bytes each, into consecutive 16-byte slots; the source chunk is the
  // one the swizzle puts in that slot.  Rows past M repeat row M-1 (their C
  // rows are never stored).
  const uint16_t* asrc[C::DMA];
  int adst[C::DMA];
#pragma unroll
  for (int j = 0; j < C::DMA; ++j) {
    const int rbase = grp * (TM / 2) + q * (TM / 8) + j * 16;
    const int row = rbase + (lane >> 2);
    const int lch = (lane & 3) ^ ((row >> 1) & 3);
    asrc[j] = g.A + (int64_t)min(m0 + row, g.M - 1) * g.lda + (int64_t)kt0 * WBK + lch * 8;
    adst[j] = rbase * 32;
  }
  // Decode share: tile column dcol and DEC consecutive k of it per tile.
  const int dcol = grp * (TN / 2) + tg / (WBK / DEC), dk = tg % (WBK / DEC);
  const int64_t e0 = wide_wrow<TN>(g, ntile, dcol) * g.W.ld + (int64_t)kt0 * WBK + dk * DEC;  // at tile 0
  const uint8_t* cp = g.W.packed + (e0 >> 1);
  const float* ap = g.W.absmax + (e0 >> 6);  // rows are whole 64-blocks (K % 64 == 0)
  static_assert(FMT == FMT_NF4, "the wide kernel reads fp32 absmax");

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  auto issue_a = [&](int tsrc, int tdst) {
    uint16_t* st = lds + (tdst & 3) * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::DMA; ++j) lds_dma16(asrc[j] + tsrc * WBK, st + adst[j]);
  };
  auto decode_b = [&](int t, const u32x2& c, const Nf4Table& tb) {
    uint16_t* bs = lds + (t & 3) * C::STAGE + C::ATILE;
    uint32_t o0[4];
    nf4_decode8(tb, c.x, o0);
    *reinterpret_cast<u32x4*>(bs + woff(dcol, (DEC / 8) * dk)) = u32x4{o0[0], o0[1], o0[2], o0[3]};
    if constexpr (DEC == 16) {
      uint32_t o1[4];
      nf4_decode8(tb, c.y, o1);
      *reinterpret_cast<u32x4*>(bs + woff(dcol, 2 * dk + 1)) = u32x4{o1[0], o1[1], o1[2], o1[3]};
    }
  };

  // Prologue: tiles 0..2 in LDS, the codes of tiles 3 and 4 in registers.
  CodeSet<DEC> cs[3];
  {
    CodeSet<DEC> pc[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      issue_a(t, t);
      pc[t] = load_codes<DEC>(cp, ap, t);
    }
    cs[0] = load_codes<DEC>(cp, ap, 3);
    cs[1] = load_codes<DEC>(cp, ap, 4);
    cs[2] = cs[1];
    wait_vm<0>();
#pragma unroll
    for (int t = 0; t < 3; ++t) decode_b(t, pc[t].c, nf4_table(pc[t].am));
  }
  Nf4Table tb = nf4_table(cs[0].am);  // tile 3 shares its 64-block with tile 2
  wbar();
  if (grp == 1) wbar();  // group 1 runs half a tile behind

  // One k tile: the memory phase, the barrier, the compute phase, the barrier.
  // The codes of tile t+3 are in `cdec`; tile t+5 loads into `cld`.
  auto step = [&](int t, CodeSet<DEC>& cdec, CodeSet<DEC>& cld) {
    __builtin_amdgcn_sched_barrier(0);
    // The LDS-DMA of tile t+3 and the codes of tile t+5 go out first (their
    // stage was last read in the previous phase, before the barrier), then
    // the fragment reads of tile t, which landed two phases ago: their LDS
    // latency overlaps the decode instead of ending the phase.  Waiting for
    // the loads of two phases ago only after issuing this phase's keeps the
    // loads from queueing behind that wait (2-4% faster than waiting first).
    issue_a(min(t + 3, nk - 1), t + 3);
    __builtin_amdgcn_sched_barrier(0);
    cld = load_codes<DEC>(cp, ap, min(t + 5, nk - 1));
    __builtin_amdgcn_sched_barrier(0);
    u32x4 af[8], bf[4];
    {
      const uint16_t* st = lds + (t & 3) * C::STAGE;
#pragma unroll
      for (int mf = 0; mf < 8; ++mf)
        af[mf] = *reinterpret_cast<const u32x4*>(st + woff(wr + mf * 16 + lr, lg));
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
        bf[nf] = *reinterpret_cast<const u32x4*>(st + C::ATILE + woff(wc + nf * 16 + lr, lg));
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<2 * phase_vm_ops<TM, FMT>()>();  // tile t+3's codes (loaded two phases ago)
    __builtin_amdgcn_sched_barrier(0);
    if (((t + 3) & 1) == 0) tb = nf4_table(cdec.am);  // first half of a 64-block
    decode_b(t + 3, cdec.c, tb);
    __builtin_amdgcn_sched_barrier(0);
    wbar_stores<DEC / 8>();  // the decoded stores land during the compute phase
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mfma16x16x32(af[mf], bf[nf], acc[mf][nf]);
    __builtin_amdgcn_sched_barrier(0);
    wbar();
  };
  int t = 0;
  for (; t + 3 <= nk; t += 3) {
    step(t, cs[0], cs[2]);
    step(t + 1, cs[1], cs[0]);
    step(t + 2, cs[2], cs[1]);
  }
  if (t < nk) step(t, cs[0], cs[2]);
  if (t + 1 < nk) step(t + 1, cs[1], cs[0]);
  if (grp == 0) wbar();
  // The last phases re-issued LDS-DMA into stages nobody reads; let them land
  // before the LDS is reused or released.
  wait_vm<0>();
  wbar();

  // LoRA extension: 32-wide steps of [uscale * U | adapter B] in stage 0;
  // each unit is one row and 16 of the step's 32 columns.
  const LoraExt& x = g.ext;
  const int next = (x.kx > 0 && z == splits - 1) ? (x.kx + WBK - 1) / WBK : 0;  // last split only
  uint16_t* As = lds;
  uint16_t* Bs = lds + C::ATILE;
  for (int xt = 0; xt < next; ++xt) {
#pragma unroll
    for (int u0 = 0; u0 < 2 * TM; u0 += 512) {
      const int row = (u0 + tid) >> 1, h = tid & 1;
      const int jb = xt * WBK + h * 16;
      const int gm = m0 + row;
      uint32_t w[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        float v[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int j = jb + 2 * p + k;
          v[k] = (gm < g.M && j < x.kx) ? x.uscale * x.u[(int64_t)gm * x.ldu + j] : 0.0f;
        }
        w[p] = pack_bf16x2(v[0], v[1]);
      }
      *reinterpret_cast<u32x4*>(As + woff(row, 2 * h)) = u32x4{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4*>(As + woff(row, 2 * h + 1)) = u32x4{w[4], w[5], w[6], w[7]};
    }
    if (tid < 2 * TN) {
      const int row = tid >> 1, h = tid & 1;
      const int jb = xt * WBK + h * 16;
      const int64_t wrow = wide_wrow<TN>(g, ntile, row);
      int sec = 0;
      for (int s = 1; s < x.nsec; ++s)
        if (wrow >= x.row_off[s]) sec = s;
      const float* bm = x.mat[sec];
      const int64_t lrow = wrow - x.row_off[sec];
      uint32_t w[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        float v[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int j = jb + 2 * p + k;
          const int jl = j - sec * x.r;
          v[k] = (bm != nullptr && j < x.kx && jl >= 0 && jl < x.r) ? bm[lrow * x.r + jl] : 0.0f;
        }
        w[p] = pack_bf16x2(v[0], v[1]);
      }
      *reinterpret_cast<u32x4*>(Bs + woff(row, 2 * h)) = u32x4{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4*>(Bs + woff(row, 2 * h + 1)) = u32x4{w[4], w[5], w[6], w[7]};
    }
    wbar();
    u32x4 af[8], bf[4];
#pragma unroll
    for (int mf = 0; mf < 8; ++mf) af[mf] = *reinterpret_cast<const u32x4*>(As + woff(wr + mf * 16 + lr, lg));
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) bf[nf] = *reinterpret_cast<const u32x4*>(Bs + woff(wc + nf * 16 + lr, lg));
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mfma16x16x32(af[mf], bf[nf], acc[mf][nf]);
    wbar();
  }

  // Epilogue.  Lane holds C[m0 + wr + mf*16 + lg*4 + i][tile column wc + nf*16 + lr].
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
      for (int np = 0; np < 2; ++np) {
        const int j = ntile * (TN / 2) + ((wc >> 6) * 2 + np) * 16 + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wr + mf * 16 + lg * 4 + i;
          if (m >= g.M) continue;
          const float gv = acc[mf][2 * np][i], uv = acc[mf][2 * np + 1][i];
          static_cast<uint16_t*>(e.C)[(int64_t)m * e.ldc + j] = f32_to_bf16(wsilu(gv) * uv);
          if (e.g != nullptr) {
            e.g[(int64_t)m * e.ldgu + j] = f32_to_bf16(gv);
            e.u[(int64_t)m * e.ldgu + j] = f32_to_bf16(uv);
          }
        }
      }
  } else {  // EPI_BF16, EPI_RESID_BF16, EPI_F32 (split z's partial sums)
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int n = ntile * TN + wc + nf * 16 + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wr + mf * 16 + lg * 4 + i;
          if (m >= g.M) continue;
          const float v = acc[mf][nf][i];
          if constexpr (EPI == EPI_F32) {
            static_cast<float*>(e.C)[(int64_t)z * g.M * g.N + (int64_t)m * e.ldc + n] = v;
          } else if constexpr (EPI == EPI_RESID_BF16) {
            static_cast<uint16_t*>(e.C)[(int64_t)m * e.ldc + n] =
                f32_to_bf16(bf16_to_f32(e.R[(int64_t)m * e.ldr + n]) + v);
          } else {
            static_cast<uint16_t*>(e.C)[(int64_t)m * e.ldc + n] = f32_to_bf16(v);
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Input-gradient variant: C[M, N] = A[M, K] . deq(W)[K, N], W stored [K][N]
// (the frozen weight's own layout: the contraction runs down its rows).  The
// schedule is the forward kernel's (two groups half a tile apart, A by
// LDS-DMA three tiles ahead, codes five ahead, four LDS stages); the weight
// tile is 32 k rows x TN columns, decoded along its rows (each k row has its
// own absmax blocks, so every decode builds its table) into a row-major LDS
// tile, and each wave reads its B operand from it with transposing loads
// (ds_read_b64_tr_b16), 4 k rows per load.  Same k order and MFMA as the
// general kernel's input-gradient GEMM, so both give the same bits.

// B tile rows of TN bf16 (TN / 8 chunks of 16 B), chunk' = chunk ^ nn_swz(row):
// the transposing reads take chunks 2j, 2j+1 of rows {0-3, 8-11} (or {4-7,
// 12-15}) of a 16-row group, and nn_swz gives those 8 rows 8 distinct values
// of its upper three bits, so no 8-byte slot repeats within a 32-lane half
// (gfx950 serves each half at 256 bytes per cycle).
__device__ __forceinline__ int nn_swz(int row) {
  return (((row >> 3) & 1) << 3) | ((row & 1) << 2) | (((row >> 1) & 1) << 1) | (row & 1);
}
template <int TN>
__device__ __forceinline__ int nboff(int row, int chunk) { return row * TN + ((chunk ^ nn_swz(row)) << 3); }

template <int TM, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_wide_nn_kernel(GemmArgs g, EpiArgs e) {
  using C = WCfg<TM>;
  constexpr int TN = C::TN;
  constexpr int CPR = TN / 8;              // 16-byte chunks per B row
  constexpr int NDEC = TN * WBK / 512;     // weights each thread decodes per tile: 8 or 16
  constexpr int NC = NDEC / 8;             // its chunks
  __shared__ __attribute__((aligned(16))) uint16_t lds[WNST * C::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid >> 2, q = wid & 3, tg = tid & 255;
  const int lr = lane & 15, lg = lane >> 4;
  const int wr = grp * (TM / 2) + (q / C::NCW) * 128, wc = (q % C::NCW) * 64;
  constexpr bool SPLIT = EPI == EPI_F32;
  const int splits = SPLIT ? g.splits : 1;
  const int mt = (g.M + TM - 1) / TM, nt = g.N / TN, tiles = mt * nt, total = tiles * splits;
  int t0 = blockIdx.x;
  if ((total & 7) == 0) t0 = (t0 & 7) * (total >> 3) + (t0 >> 3);
  const int z = SPLIT ? t0 / tiles : 0, tile = t0 - z * tiles;
  const int mtile = tile % mt, ntile = tile / mt;
  const int m0 = mtile * TM;
  const int per = SPLIT ? wide_split_tiles(g.K, splits) : g.K / WBK;
  const int kt0 = z * per;
  const int nk = min(g.K / WBK - kt0, per);

  const uint16_t* asrc[C::DMA];
  int adst[C::DMA];
#pragma unroll
  for (int j = 0; j < C::DMA; ++j) {
    const int rbase = grp * (TM / 2) + q * (TM / 8) + j * 16;
    const int row = rbase + (lane >> 2);
    const int lch = (lane & 3) ^ ((row >> 1) & 3);
    asrc[j] = g.A + (int64_t)min(m0 + row, g.M - 1) * g.lda + (int64_t)kt0 * WBK + lch * 8;
    adst[j] = rbase * 32;
  }
  // Decode share: group grp decodes k rows 16 grp .. + 16 of every B tile;
  // thread tg takes row drow, chunks dch .. dch + NC (NDEC columns, inside
  // one 64-column absmax block).
  const int drow = 16 * grp + tg / (CPR / NC), dch = (tg % (CPR / NC)) * NC;
  const int64_t e0 = ((int64_t)kt0 * WBK + drow) * g.W.ld + (int64_t)ntile * TN + dch * 8;
  const uint8_t* cp = g.W.packed + (e0 >> 1);
  const float* ap = g.W.absmax + (e0 >> 6);
  const int64_t cstride = (int64_t)WBK * g.W.ld / 2, astride = (int64_t)WBK * g.W.ld / 64;  // per k tile

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  auto issue_a = [&](int tsrc, int tdst) {
    uint16_t* st = lds + (tdst & 3) * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::DMA; ++j) lds_dma16(asrc[j] + tsrc * WBK, st + adst[j]);
  };
  auto ld_codes = [&](int t) {
    CodeSet<NDEC> cs;
    const uint8_t* p = cp + t * cstride;
    if constexpr (NDEC == 16) {
      cs.c = *reinterpret_cast<const u32x2*>(p);
    } else {
      cs.c.x = *reinterpret_cast<const uint32_t*>(p);
      cs.c.y = 0;
    }
    cs.am = ap[t * astride];
    return cs;
  };
  auto decode_b = [&](int t, const CodeSet<NDEC>& cs) {
    uint16_t* bs = lds + (t & 3) * C::STAGE + C::ATILE;
    const Nf4Table tb = nf4_table(cs.am);
    uint32_t o[4];
    nf4_decode8(tb, cs.c.x, o);
    *reinterpret_cast<u32x4*>(bs + nboff<TN>(drow, dch)) = u32x4{o[0], o[1], o[2], o[3]};
    if constexpr (NDEC == 16) {
      nf4_decode8(tb, cs.c.y, o);
      *reinterpret_cast<u32x4*>(bs + nboff<TN>(drow, dch + 1)) = u32x4{o[0], o[1], o[2], o[3]};
    }
  };
  // This wave's B operand of tile stage `bs`: column wc + nf*16 + lr, k rows
  // lg*8 .. + 8, from two transposing loads.
  auto read_b = [&](const uint16_t* bs, u32x4 (&bf)[4]) {
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int col = wc + nf * 16 + 4 * (lr & 3);
      const int row = lg * 8 + (lr >> 2);
      const u32x2 lo = lds_read_tr4(bs, nboff<TN>(row, col >> 3) + (col & 7));
      const u32x2 hi = lds_read_tr4(bs, nboff<TN>(row + 4, col >> 3) + (col & 7));
      bf[nf] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  };

  CodeSet<NDEC> cs[3];
  {
    CodeSet<NDEC> pc[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      issue_a(t, t);
      pc[t] = ld_codes(t);
    }
    cs[0] = ld_codes(3);
    cs[1] = ld_codes(4);
    cs[2] = cs[1];
    wait_vm<0>();
#pragma unroll
    for (int t = 0; t < 3; ++t) decode_b(t, pc[t]);
  }
  wbar();
  if (grp == 1) wbar();

  auto step = [&](int t, CodeSet<NDEC>& cdec, CodeSet<NDEC>& cld) {
    __builtin_amdgcn_sched_barrier(0);
    // Unlike the forward kernel, the fragment reads go out before this
    // phase's LDS-DMA: the compiler waits for every LDS-DMA in flight before
    // a transposing LDS read that follows one, which serialises the phase.
    u32x4 af[8], bf[4];
    {
      const uint16_t* st = lds + (t & 3) * C::STAGE;
#pragma unroll
      for (int mf = 0; mf < 8; ++mf)
        af[mf] = *reinterpret_cast<const u32x4*>(st + woff(wr + mf * 16 + lr, lg));
      read_b(st + C::ATILE, bf);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<phase_vm_ops<TM, FMT_NF4>()>();
    issue_a(min(t + 3, nk - 1), t + 3);
    __builtin_amdgcn_sched_barrier(0);
    cld = ld_codes(min(t + 5, nk - 1));
    __builtin_amdgcn_sched_barrier(0);
    decode_b(t + 3, cdec);
    __builtin_amdgcn_sched_barrier(0);
    wbar_stores<NDEC / 8>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mfma16x16x32(af[mf], bf[nf], acc[mf][nf]);
    __builtin_amdgcn_sched_barrier(0);
    wbar();
  };
  int t = 0;
  for (; t + 3 <= nk; t += 3) {
    step(t, cs[0], cs[2]);
    step(t + 1, cs[1], cs[0]);
    step(t + 2, cs[2], cs[1]);
  }
  if (t < nk) step(t, cs[0], cs[2]);
  if (t + 1 < nk) step(t + 1, cs[1], cs[0]);
  if (grp == 0) wbar();
  wait_vm<0>();
  wbar();

  // LoRA extension (last split only): 32-wide steps of [U | adapter A rows].
  const LoraExt& x = g.ext;
  const int next = (x.kx > 0 && z == splits - 1) ? (x.kx + WBK - 1) / WBK : 0;
  uint16_t* As = lds;
  uint16_t* Bs = lds + C::ATILE;
  for (int xt = 0; xt < next; ++xt) {
#pragma unroll
    for (int u0 = 0; u0 < 2 * TM; u0 += 512) {
      const int row = (u0 + tid) >> 1, h = tid & 1;
      const int jb = xt * WBK + h * 16;
      const int gm = m0 + row;
      uint32_t w[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        float v[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int j = jb + 2 * p + k;
          v[k] = (gm < g.M && j < x.kx) ? x.uscale * x.u[(int64_t)gm * x.ldu + j] : 0.0f;
        }
        w[p] = pack_bf16x2(v[0], v[1]);
      }
      *reinterpret_cast<u32x4*>(As + woff(row, 2 * h)) = u32x4{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4*>(As + woff(row, 2 * h + 1)) = u32x4{w[4], w[5], w[6], w[7]};
    }
#pragma unroll
    for (int u0 = 0; u0 < WBK * CPR; u0 += 512) {
      const int idx = u0 + tid, row = idx / CPR, ch = idx % CPR;
      const int j = xt * WBK + row;
      const int sec = x.r > 0 ? j / x.r : 0;
      const float* am = (j < x.kx && sec < x.nsec) ? x.mat[sec] : nullptr;
      const int64_t n0 = (int64_t)ntile * TN + ch * 8;
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float v0 = 0.0f, v1 = 0.0f;
        if (am != nullptr) {
          const float* src = am + (int64_t)(j - sec * x.r) * x.ldmat + n0 + 2 * p;
          v0 = src[0];
          v1 = src[1];
        }
        w[p] = pack_bf16x2(v0, v1);
      }
      *reinterpret_cast<u32x4*>(Bs + nboff<TN>(row, ch)) = u32x4{w[0], w[1], w[2], w[3]};
    }
    wbar();
    u32x4 af[8], bf[4];
#pragma unroll
    for (int mf = 0; mf < 8; ++mf) af[mf] = *reinterpret_cast<const u32x4*>(As + woff(wr + mf * 16 + lr, lg));
    read_b(Bs, bf);
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mfma16x16x32(af[mf], bf[nf], acc[mf][nf]);
    wbar();
  }

  // Epilogue.  Lane holds C[m0 + wr + mf*16 + lg*4 + i][ntile*TN + wc + nf*16 + lr].
  if constexpr (EPI == EPI_SWIGLU_BWD) {
    // Through LDS (free once the k loop is over): each wave stages 32 rows
    // of its 128 x 64 tile at a time in its own 32 x 68 fp32 block (8.5 KB),
    // then every lane takes 8 consecutive columns of one row, so the gate/up
    // reads and the dg/du writes are 16-byte accesses, 128 contiguous bytes
    // per 8 lanes.  Rows past M read a clamped row and store nothing.
    constexpr int SLD = 68;
    static_assert(8 * 32 * SLD * 4 <= WNST * C::STAGE * 2, "staging fits the LDS ring");
    float* my = reinterpret_cast<float*>(lds) + wid * (32 * SLD);
    const int cq = (lane & 7) * 8;
    const int n = ntile * TN + wc + cq;
    uint16_t* Cp = static_cast<uint16_t*>(e.C);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
      for (int mf = 0; mf < 2; ++mf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf)
#pragma unroll
          for (int i = 0; i < 4; ++i) my[(mf * 16 + lg * 4 + i) * SLD + nf * 16 + lr] = acc[2 * h + mf][nf][i];
      wave_lds_sync();
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = p * 8 + (lane >> 3);
        const int m = m0 + wr + h * 32 + r;
        const int64_t mc = min(m, g.M - 1);
        const u32x4 gq = *reinterpret_cast<const u32x4*>(e.g + mc * e.ldgu + n);
        const u32x4 uq = *reinterpret_cast<const u32x4*>(e.u + mc * e.ldgu + n);
        const float4 v0 = *reinterpret_cast<const float4*>(my + r * SLD + cq);
        const float4 v1 = *reinterpret_cast<const float4*>(my + r * SLD + cq + 4);
        const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        u32x4 dgo, duo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float dg0, du0, dg1, du1;
          swiglu_grad(v[2 * k], bf16lo(gq[k]), bf16lo(uq[k]), dg0, du0);
          swiglu_grad(v[2 * k + 1], bf16hi(gq[k]), bf16hi(uq[k]), dg1, du1);
          dgo[k] = pack_bf16x2(dg0, dg1);
          duo[k] = pack_bf16x2(du0, du1);
        }
        if (m < g.M) {
          *reinterpret_cast<u32x4*>(Cp + (int64_t)m * e.ldc + n) = dgo;
          *reinterpret_cast<u32x4*>(Cp + (int64_t)m * e.ldc + g.N + n) = duo;
        }
      }
      wave_lds_sync();
    }
    return;
  }
#pragma unroll
  for (int mf = 0; mf < 8; ++mf)
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
      const int n = ntile * TN + wc + nf * 16 + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wr + mf * 16 + lg * 4 + i;
        if (m >= g.M) continue;
        const float v = acc[mf][nf][i];
        if constexpr (EPI == EPI_F32) {
          static_cast<float*>(e.C)[(int64_t)z * g.M * g.N + (int64_t)m * e.ldc + n] = v;
        } else {
          static_cast<uint16_t*>(e.C)[(int64_t)m * e.ldc + n] = f32_to_bf16(v);
        }
      }
    }
}

template <int TM>
hipError_t launch_wide_nn(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  constexpr int TN = WCfg<TM>::TN;
  const dim3 grid(((g.M + TM - 1) / TM) * (g.N / TN) * g.splits), block(512);
  switch (e.kind) {
    case EPI_BF16: hipLaunchKernelGGL((gemm_wide_nn_kernel<TM, EPI_BF16>), grid, block, 0, s, g, e); break;
    case EPI_F32: hipLaunchKernelGGL((gemm_wide_nn_kernel<TM, EPI_F32>), grid, block, 0, s, g, e); break;
    case EPI_SWIGLU_BWD: hipLaunchKernelGGL((gemm_wide_nn_kernel<TM, EPI_SWIGLU_BWD>), grid, block, 0, s, g, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int TM>
hipError_t launch_wide(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  constexpr int TN = WCfg<TM>::TN;
  const dim3 grid(((g.M + TM - 1) / TM) * (g.N / TN) * g.splits), block(512);
  switch (e.kind) {
    case EPI_BF16: hipLaunchKernelGGL((gemm_wide_kernel<TM, FMT_NF4, EPI_BF16>), grid, block, 0, s, g, e); break;
    case EPI_RESID_BF16:
      hipLaunchKernelGGL((gemm_wide_kernel<TM, FMT_NF4, EPI_RESID_BF16>), grid, block, 0, s, g, e);
      break;
    case EPI_F32: hipLaunchKernelGGL((gemm_wide_kernel<TM, FMT_NF4, EPI_F32>), grid, block, 0, s, g, e); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_wide_kernel<TM, FMT_NF4, EPI_SWIGLU>), grid, block, 0, s, g, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tile rows of the wide kernel: 512 (x 128 columns), which decodes each
// weight half as often as 256 x 256 tiles and measured faster at 512 and 2048
// tokens (gate|up 150 vs 156 us and 582 vs 594 us).
int wide_tile_rows(const GemmArgs&) { return 512; }

}  // namespace

namespace {

// What the wide kernel can run: whole column tiles (and halves of them in
// pair mode), 64-deep absmax blocks, 16-byte aligned A rows, 8-byte aligned
// codes; with split-K (fp32 partial sums, ldc = N) at least 8 of its 32-deep
// k tiles in every split.
bool wide_capable(const GemmArgs& g, const EpiArgs& e) {
  if (g.splits < 1 || g.M < 256 || g.N % 256 != 0) return false;
  // fp32 absmax only: with the double-quantised absmax (two more loads in
  // flight per code set) the kernel no longer fits its 256 registers.
  if (g.W.fmt != FMT_NF4) return false;
  if (g.K % 64 != 0 || g.W.ld != g.K || g.lda % 8 != 0) return false;
  if (((uintptr_t)g.A & 15) != 0 || ((uintptr_t)g.W.packed & 7) != 0) return false;
  if (g.pair_I > 0 && (g.pair_I * 2 != g.N || g.pair_I % 128 != 0)) return false;
  if (g.splits > 1) {
    if (e.kind != EPI_F32 || g.pair_I > 0 || e.ldc != g.N) return false;
    const int per = wide_split_tiles(g.K, g.splits);
    return per >= 8 && g.K / WBK - (g.splits - 1) * per >= 8;
  }
  if (e.kind == EPI_SWIGLU) return g.pair_I > 0;
  return (e.kind == EPI_BF16 || e.kind == EPI_RESID_BF16) && g.pair_I == 0;
}

}  // namespace

// Forward GEMMs with long contractions (K >= 8192: down) and fewer than 192
// tiles of 512 x 128 run split-K on the wide kernel: as many splits (up to 8)
// as keep the tiles times splits within the 256 compute units.  Measured on
// MI355X: down 95.5 vs 103 us at 512 tokens (8 splits), 276 vs 332 us at 2048
// (2 splits); q|k|v and o (K = 4096) stay faster on the general kernel (at
// 512 tokens q|k|v 71.7 us there against 73 - 108 us with 2 - 6 wide splits,
// o 46.6 against 49.5 - 78.6 us with 2 - 8).
int wide_splits(const GemmArgs& g) {
  if (g.M < 256 || g.K < 8192 || g.N >= 16384 || g.N % 256 != 0 || g.pair_I > 0) return 0;
  const int tiles = ((g.M + 511) / 512) * (g.N / 128);
  if (tiles >= 192) return 0;
  EpiArgs pe;
  pe.kind = EPI_F32;
  pe.ldc = g.N;
  GemmArgs t = g;
  for (int s = std::min(8, 256 / tiles); s > 1; --s) {
    t.splits = s;
    if (wide_capable(t, pe)) return s;
  }
  return 0;
}

// Without split-K the wide kernel is chosen for N >= 16384 (gate|up), or when
// there are at least 192 of its tiles, three quarters of the 256 compute units
// (q|k|v from 2048 tokens: 144 vs 174 us there, measured), and K >= 2048: with
// short contractions its prologue dominates (measured 1.7x slower than the
// general kernel at K = 512).  With split-K, where wide_splits chose it.
bool gemm_wide_applies(const GemmArgs& g, const EpiArgs& e) {
  if (!wide_capable(g, e)) return false;
  if (g.splits > 1) return wide_splits(g) == g.splits;
  if (g.K < 2048) return false;
  return g.N >= 16384 || (int64_t)((g.M + 255) / 256) * (g.N / 256) >= 192;
}

namespace {

// What the wide input-gradient kernel can run: W stored [K][N] with whole
// column tiles (N a multiple of 256 covers both tile shapes and the 64-column
// absmax blocks), 64-deep k steps, 16-byte aligned A rows, 8-byte aligned
// codes; fp32 partial sums (ldc = N, every split at least 8 k tiles) with
// split-K, else a bf16 or SwiGLU-backward epilogue.
bool wide_nn_capable(const GemmArgs& g, const EpiArgs& e) {
  if (g.splits < 1 || g.M < 256 || g.N % 256 != 0 || g.pair_I != 0) return false;
  if (g.W.fmt != FMT_NF4 || g.W.ld != g.N || g.K % 64 != 0 || g.K < 256 || g.lda % 8 != 0) return false;
  if (((uintptr_t)g.A & 15) != 0 || ((uintptr_t)g.W.packed & 7) != 0) return false;
  if (g.splits > 1) {
    if (e.kind != EPI_F32 || e.ldc != g.N) return false;
    const int per = wide_split_tiles(g.K, g.splits);
    return per >= 8 && g.K / WBK - (g.splits - 1) * per >= 8;
  }
  if (e.kind == EPI_SWIGLU_BWD)  // 16-byte accesses to g, u and both halves of C
    return e.g != nullptr && e.u != nullptr && ((uintptr_t)e.C | (uintptr_t)e.g | (uintptr_t)e.u) % 16 == 0 &&
           e.ldc % 8 == 0 && e.ldgu % 8 == 0;
  return e.kind == EPI_BF16;
}

}  // namespace

// Input-gradient GEMMs with a long contraction or a wide output (K or N at
// least 8192: gate|up, down) run on the wide kernel: without split-K from 192
// of its 512 x 128 tiles on, else with as many splits (up to 8) as keep tiles
// times splits within the 256 compute units.
int wide_nn_splits(const GemmArgs& g) {
  if (g.M < 256 || (g.K < 8192 && g.N < 8192) || g.N % 256 != 0) return 0;
  const int tiles = ((g.M + 511) / 512) * (g.N / 128);
  if (tiles >= 192) return 1;
  EpiArgs pe;
  pe.kind = EPI_F32;
  pe.ldc = g.N;
  GemmArgs t = g;
  for (int s = std::min(8, 256 / tiles); s > 1; --s) {
    t.splits = s;
    if (wide_nn_capable(t, pe)) return s;
  }
  return 0;
}

bool gemm_wide_nn_applies(const GemmArgs& g, const EpiArgs& e) {
  return wide_nn_capable(g, e) && wide_nn_splits(g) == g.splits;
}

namespace {
std::atomic<int64_t> g_wide_launches{0};
std::atomic<int> g_wide_tile{0};  // 0: by shape; 256 or 512: forced (diagnostics)
}  // namespace

int64_t gemm_wide_launches() { return g_wide_launches.load(std::memory_order_relaxed); }
void set_gemm_wide_tile(int rows) { g_wide_tile.store(rows, std::memory_order_relaxed); }

hipError_t gemm_nn_wide(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  if (!gemm_wide_nn_applies(g, e)) return hipErrorInvalidValue;
  g_wide_launches.fetch_add(1, std::memory_order_relaxed);
  const int forced = g_wide_tile.load(std::memory_order_relaxed);
  const int tm = forced != 0 ? forced : wide_tile_rows(g);
  return tm == 512 ? launch_wide_nn<512>(g, e, s) : launch_wide_nn<256>(g, e, s);
}

hipError_t gemm_nt_wide(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  if (!gemm_wide_applies(g, e)) return hipErrorInvalidValue;
  g_wide_launches.fetch_add(1, std::memory_order_relaxed);
  const int forced = g_wide_tile.load(std::memory_order_relaxed);
  const int tm = forced != 0 ? forced : wide_tile_rows(g);
  return tm == 512 ? launch_wide<512>(g, e, s) : launch_wide<256>(g, e, s);
}

}  // namespace lsf
