// Wide forward NF4 GEMM for gfx950, used when the output has many 256 x 256
// tiles (the gate|up projection; q|k|v from 2048 tokens):
// C[M, N] = A[M, K] . deq(W)[N, K]^T  (+ LoRA, + epilogue).
//
// Same arithmetic as the general kernel in gemm.hip (every weight decoded to
// bf16_rne(level * absmax), bf16 MFMA with fp32 accumulation, the k order of
// the contraction unchanged, LoRA as extra contraction steps after the main
// ones), so both kernels give bitwise-identical results; only the schedule
// differs:
//
// * 256 x 256 C tile, 512 threads = two groups of four waves.  The hardware
//   places wave w and wave w+4 of a workgroup on the same SIMD, so every SIMD
//   holds one wave of each group.  Wave (g, q) owns rows g*128..+128 and
//   columns q*64..+64 (8 x 4 fragments of v_mfma_f32_16x16x32_bf16).
// * 32-deep k tiles in a ring of four LDS stages (32 KB each).  The groups run
//   half a tile apart (ping-pong): while one group issues its 32 MFMAs, the
//   other runs its memory phase: read its own fragments of the current tile,
//   wait for the LDS-DMA issued two phases ago, issue the LDS-DMA of A three
//   tiles ahead (global_load_lds_dwordx4, no register round trip), load the
//   packed codes of the tile five ahead into registers, and decode its half
//   of the weight tile three ahead into LDS; the fragment reads complete
//   meanwhile instead of ending the phase.  A workgroup barrier between the
//   phases swaps the roles.
// * Every memory phase issues the same vector-memory operations, the two
//   LDS-DMA first (past the last tile they repeat it into a stage nobody reads
//   again), then the code and absmax loads.  Loads complete in issue order, so
//   `s_waitcnt vmcnt(4)` before this phase's own loads means "the LDS-DMA of
//   two phases ago has landed"; it stays safe if the compiler emits more loads
//   per phase (it then waits longer) or merges the two register loads into
//   one (the last operation of the older phase is still a register load).
//   The fragment reads of tile t may precede that wait: the DMA of tile t was
//   waited for one phase earlier and two barriers have passed since.
//   Barriers carry no memory-model fence: a release fence would wait for
//   every LDS-DMA in flight.
#include "common.h"
#include "kernels.h"
#include "weight_decode.h"

#include <atomic>

namespace lsf {
namespace {

constexpr int WBM = 256, WBN = 256, WBK = 32, WNST = 4;
constexpr int WTILE = WBM * WBK;  // bf16 elements of one A (or B) tile
constexpr int WSTAGE = 2 * WTILE;  // A tile then B tile: 32 KB

// Tile rows of 32 bf16 (4 chunks of 16 B), chunk' = chunk ^ ((row >> 1) & 3):
// the 8 lanes of a 16-byte read phase hit 8 distinct 16-byte bank groups.
__device__ __forceinline__ int woff(int row, int ch) { return row * 32 + ((ch ^ ((row >> 1) & 3)) << 3); }

// s_waitcnt with only the vector-memory counter constrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x3f70 | N);
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

__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// Weight row feeding tile column c (0..255) of column tile `ntile`; in pair
// mode gate row j and up row pair_I + j sit 16 columns apart, so one lane
// holds both in its accumulators.
__device__ __forceinline__ int64_t wide_wrow(const GemmArgs& g, int ntile, int c) {
  if (g.pair_I > 0) {
    const int j = ntile * (WBN / 2) + (c >> 5) * 16 + (c & 15);
    return ((c >> 4) & 1) ? (int64_t)g.pair_I + j : (int64_t)j;
  }
  return (int64_t)ntile * WBN + c;
}

// Vector-memory operations of one memory phase: two LDS-DMA of A, the codes,
// and the absmax (one load for fp32 absmax; code + group pair for NF4_DQ).
template <int FMT>
constexpr int phase_vm_ops() { return FMT == FMT_NF4_DQ ? 5 : 4; }

template <int FMT>
struct CodeSet {
  u32x2 c;
  float am;
};

template <int FMT>
__device__ __forceinline__ CodeSet<FMT> load_codes(const WeightRef& w, const uint8_t* cp, int64_t e0, int t) {
  CodeSet<FMT> s;
  s.c = *reinterpret_cast<const u32x2*>(cp + t * 16);
  s.am = block_absmax_t<FMT>(w, e0 + (int64_t)t * WBK);
  return s;
}

__device__ __forceinline__ float wsilu(float x) { return x / (1.0f + __expf(-x)); }

template <int FMT, int EPI>
__global__ __launch_bounds__(512, 1) void gemm_wide_kernel(GemmArgs g, EpiArgs e) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[WNST * WSTAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid >> 2, q = wid & 3, tg = tid & 255;
  const int lr = lane & 15, lg = lane >> 4;
  const int mt = (g.M + WBM - 1) / WBM, nt = g.N / WBN, total = mt * nt;
  int t0 = blockIdx.x;
  if ((total & 7) == 0) t0 = (t0 & 7) * (total >> 3) + (t0 >> 3);  // neighbouring tiles on one XCD
  const int mtile = t0 % mt, ntile = t0 / mt;
  const int m0 = mtile * WBM;
  const int nk = g.K / WBK;

  // LDS-DMA of A: wave (grp, q) moves rows grp*128 + q*32 + j*16 + lane/4,
  // 16 bytes each, into consecutive 16-byte slots; the source chunk is the
  // one the swizzle puts in that slot.  Rows past M repeat row M-1 (their C
  // rows are never stored).
  const uint16_t* asrc[2];
  int adst[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rbase = grp * 128 + q * 32 + j * 16;
    const int row = rbase + (lane >> 2);
    const int lch = (lane & 3) ^ ((row >> 1) & 3);
    asrc[j] = g.A + (int64_t)min(m0 + row, g.M - 1) * g.lda + lch * 8;
    adst[j] = rbase * 32;
  }
  // Decode share: tile column dcol, k half dh (16 weights per tile).
  const int dcol = grp * 128 + (tg >> 1), dh = tg & 1;
  const int64_t e0 = wide_wrow(g, ntile, dcol) * g.W.ld + dh * 16;  // element index at tile 0
  const uint8_t* cp = g.W.packed + (e0 >> 1);

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  auto issue_a = [&](int tsrc, int tdst) {
    uint16_t* st = lds + (tdst & 3) * WSTAGE;
#pragma unroll
    for (int j = 0; j < 2; ++j) lds_dma16(asrc[j] + tsrc * WBK, st + adst[j]);
  };
  auto decode_b = [&](int t, const u32x2& c, const Nf4Table& tb) {
    uint16_t* bs = lds + (t & 3) * WSTAGE + WTILE;
    uint32_t o0[4], o1[4];
    nf4_decode8(tb, c.x, o0);
    nf4_decode8(tb, c.y, o1);
    *reinterpret_cast<u32x4*>(bs + woff(dcol, 2 * dh)) = u32x4{o0[0], o0[1], o0[2], o0[3]};
    *reinterpret_cast<u32x4*>(bs + woff(dcol, 2 * dh + 1)) = u32x4{o1[0], o1[1], o1[2], o1[3]};
  };

  // Prologue: tiles 0..2 in LDS, the codes of tiles 3 and 4 in registers.
  CodeSet<FMT> cs[3];
  {
    CodeSet<FMT> pc[3];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      issue_a(t, t);
      pc[t] = load_codes<FMT>(g.W, cp, e0, t);
    }
    cs[0] = load_codes<FMT>(g.W, cp, e0, 3);
    cs[1] = load_codes<FMT>(g.W, cp, e0, 4);
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
  auto step = [&](int t, CodeSet<FMT>& cdec, CodeSet<FMT>& cld) {
    __builtin_amdgcn_sched_barrier(0);
    // Fragment reads first: tile t landed two phases ago, and their LDS
    // latency then overlaps the loads and the decode instead of ending the
    // phase (this order also keeps the kernel within 256 registers).
    u32x4 af[8], bf[4];
    {
      const uint16_t* st = lds + (t & 3) * WSTAGE;
#pragma unroll
      for (int mf = 0; mf < 8; ++mf)
        af[mf] = *reinterpret_cast<const u32x4*>(st + woff(grp * 128 + mf * 16 + lr, lg));
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
        bf[nf] = *reinterpret_cast<const u32x4*>(st + WTILE + woff(q * 64 + nf * 16 + lr, lg));
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<phase_vm_ops<FMT>()>();
    issue_a(min(t + 3, nk - 1), t + 3);
    __builtin_amdgcn_sched_barrier(0);  // the LDS-DMA goes out before the register loads
    cld = load_codes<FMT>(g.W, cp, e0, min(t + 5, nk - 1));
    __builtin_amdgcn_sched_barrier(0);
    if (((t + 3) & 1) == 0) tb = nf4_table(cdec.am);  // first half of a 64-block
    decode_b(t + 3, cdec.c, tb);
    __builtin_amdgcn_sched_barrier(0);
    wbar();
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

  // LoRA extension: 32-wide steps of [uscale * U | adapter B] in stage 0.
  const LoraExt& x = g.ext;
  const int next = x.kx > 0 ? (x.kx + WBK - 1) / WBK : 0;
  for (int xt = 0; xt < next; ++xt) {
    const int row = tid >> 1, h = tid & 1;
    const int jb = xt * WBK + h * 16;
    uint16_t* As = lds;
    uint16_t* Bs = lds + WTILE;
    {
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
    {
      const int64_t wr = wide_wrow(g, ntile, row);
      int sec = 0;
      for (int s = 1; s < x.nsec; ++s)
        if (wr >= x.row_off[s]) sec = s;
      const float* bm = x.mat[sec];
      const int64_t lrow = wr - x.row_off[sec];
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
    for (int mf = 0; mf < 8; ++mf) af[mf] = *reinterpret_cast<const u32x4*>(As + woff(grp * 128 + mf * 16 + lr, lg));
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) bf[nf] = *reinterpret_cast<const u32x4*>(Bs + woff(q * 64 + nf * 16 + lr, lg));
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mfma16x16x32(af[mf], bf[nf], acc[mf][nf]);
    wbar();
  }

  // Epilogue.  Lane holds C[m0 + grp*128 + mf*16 + lg*4 + i][tile column q*64 + nf*16 + lr].
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
      for (int np = 0; np < 2; ++np) {
        const int j = ntile * (WBN / 2) + (q * 2 + np) * 16 + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + grp * 128 + mf * 16 + lg * 4 + i;
          if (m >= g.M) continue;
          const float gv = acc[mf][2 * np][i], uv = acc[mf][2 * np + 1][i];
          static_cast<uint16_t*>(e.C)[(int64_t)m * e.ldc + j] = f32_to_bf16(wsilu(gv) * uv);
          if (e.g != nullptr) {
            e.g[(int64_t)m * e.ldgu + j] = f32_to_bf16(gv);
            e.u[(int64_t)m * e.ldgu + j] = f32_to_bf16(uv);
          }
        }
      }
  } else {  // EPI_BF16
#pragma unroll
    for (int mf = 0; mf < 8; ++mf)
#pragma unroll
      for (int nf = 0; nf < 4; ++nf) {
        const int n = ntile * WBN + q * 64 + nf * 16 + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + grp * 128 + mf * 16 + lg * 4 + i;
          if (m >= g.M) continue;
          const float v = acc[mf][nf][i];
          static_cast<uint16_t*>(e.C)[(int64_t)m * e.ldc + n] = f32_to_bf16(v);
        }
      }
  }
}

template <int FMT>
hipError_t launch_wide_fmt(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  const dim3 grid(((g.M + WBM - 1) / WBM) * (g.N / WBN)), block(512);
  switch (e.kind) {
    case EPI_BF16: hipLaunchKernelGGL((gemm_wide_kernel<FMT, EPI_BF16>), grid, block, 0, s, g, e); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_wide_kernel<FMT, EPI_SWIGLU>), grid, block, 0, s, g, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// The wide kernel needs whole 256-column tiles (and 128-row halves of them in
// pair mode), 64-deep absmax blocks, 16-byte aligned A rows, 8-byte aligned
// codes, and no split-K.  It is chosen for N >= 16384 (gate|up), or when
// there are at least 192 of its 256 x 256 tiles, three quarters of the 256
// compute units (q|k|v from 2048 tokens: 144 vs 174 us there, measured), and
// K >= 2048: with short contractions its prologue dominates (measured 1.7x
// slower than the general kernel at K = 512).
bool gemm_wide_applies(const GemmArgs& g, const EpiArgs& e) {
  if (g.splits != 1 || g.M < 256 || g.N % WBN != 0) return false;
  if (g.N < 16384 && (int64_t)((g.M + WBM - 1) / WBM) * (g.N / WBN) < 192) return false;
  // fp32 absmax only: with the double-quantised absmax (two more loads in
  // flight per code set) the kernel no longer fits its 256 registers.
  if (g.W.fmt != FMT_NF4) return false;
  if (g.K % 64 != 0 || g.K < 2048 || g.W.ld != g.K || g.lda % 8 != 0) return false;
  if (((uintptr_t)g.A & 15) != 0 || ((uintptr_t)g.W.packed & 7) != 0) return false;
  if (g.pair_I > 0 && (g.pair_I * 2 != g.N || g.pair_I % (WBN / 2) != 0)) return false;
  if (e.kind == EPI_SWIGLU) return g.pair_I > 0;
  return e.kind == EPI_BF16 && g.pair_I == 0;
}

namespace {
std::atomic<int64_t> g_wide_launches{0};
}  // namespace

int64_t gemm_wide_launches() { return g_wide_launches.load(std::memory_order_relaxed); }

hipError_t gemm_nt_wide(const GemmArgs& g, const EpiArgs& e, hipStream_t s) {
  if (!gemm_wide_applies(g, e)) return hipErrorInvalidValue;
  g_wide_launches.fetch_add(1, std::memory_order_relaxed);
  return launch_wide_fmt<FMT_NF4>(g, e, s);
}

}  // namespace lsf
