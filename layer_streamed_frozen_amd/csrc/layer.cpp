// One Llama-style decoder layer over a frozen NF4 base with LoRA adapters:
// forward, and the backward that first recomputes the forward from the layer
// input (the per-layer checkpoint) and then walks it in reverse.
#include "layer.h"

#include <algorithm>

namespace lsf {
namespace {

constexpr size_t AL = 256;
size_t up(size_t v) { return (v + AL - 1) / AL * AL; }

struct Sizes {
  int64_t T, H, I, Dq, Nqkv, r, nq, seq, batch;
  Sizes(const lsf_layer_cfg& c)
      : T((int64_t)c.batch * c.seq), H(c.hidden), I(c.intermediate), Dq((int64_t)c.n_heads * c.head_dim),
        Nqkv((int64_t)(c.n_heads + 2 * c.n_kv_heads) * c.head_dim), r(c.rank), nq(c.n_heads), seq(c.seq),
        batch(c.batch) {}
  int64_t maxN() const { return std::max(std::max(H, I), std::max(Dq, Nqkv)); }
};

const lsf_lora_proj* proj(const lsf_layer_lora* l, int i) {
  if (l == nullptr || !l->enabled) return nullptr;
  const lsf_lora_proj* p = &l->q + i;
  return p->A != nullptr ? p : nullptr;
}
enum { PQ = 0, PK, PV, PO, PG, PU, PD };

}  // namespace

size_t LayerWs::bytes(const lsf_layer_cfg& c) {
  Sizes z(c);
  size_t b = 0;
  b += up(z.T * z.H * 2) * 6;                 // h1, att(<=), x2, h2, dh, dx2 (att/dob sized by Dq below)
  b += up(z.T * z.Dq * 2) * 2;                // att, dob
  b += up(z.T * z.Nqkv * 2) * 2;              // qkv, dqkv
  b += up(z.T * z.I * 2) * 3;                 // g, u, a
  b += up(z.T * z.I * 2 * 2);                 // dgu
  b += up(z.T * z.H * 2);                     // y scratch
  b += up(z.T * 4) * 2;                       // rstd1, rstd2
  b += up(z.batch * z.nq * z.seq * 4);        // lse
  b += up(z.T * 3 * z.r * 4) + up(z.T * z.r * 4) * 2 + up(z.T * 2 * z.r * 4);  // U's
  b += up(z.T * 3 * z.r * 4);                 // dU
  b += up(z.seq * (c.head_dim / 2) * 8);      // rope table
  b += up((attention_dsum_floats(z.batch, z.nq, z.seq) + 2 * z.T * z.nq * 128) * 4);  // attention bwd scratch
  b += up((size_t)8 * z.T * z.maxN() * 4);    // split-K partials
  b += up(lora_part_floats(z.T, 3, (int)z.r) * 4);  // LoRA down-projection partials
  return b + AL;
}

LayerWs LayerWs::carve(const lsf_layer_cfg& c, void* base) {
  Sizes z(c);
  uintptr_t p = ((uintptr_t)base + AL - 1) / AL * AL;
  auto take = [&](size_t n) {
    void* r = (void*)p;
    p += up(n);
    return r;
  };
  LayerWs w{};
  w.h1 = (uint16_t*)take(z.T * z.H * 2);
  w.x2 = (uint16_t*)take(z.T * z.H * 2);
  w.h2 = (uint16_t*)take(z.T * z.H * 2);
  w.dh = (uint16_t*)take(z.T * z.H * 2);
  w.dx2 = (uint16_t*)take(z.T * z.H * 2);
  take(z.T * z.H * 2);  // spare (keeps bytes() an upper bound)
  w.att = (uint16_t*)take(z.T * z.Dq * 2);
  w.dob = (uint16_t*)take(z.T * z.Dq * 2);
  w.qkv = (uint16_t*)take(z.T * z.Nqkv * 2);
  w.dqkv = (uint16_t*)take(z.T * z.Nqkv * 2);
  w.g = (uint16_t*)take(z.T * z.I * 2);
  w.u = (uint16_t*)take(z.T * z.I * 2);
  w.a = (uint16_t*)take(z.T * z.I * 2);
  w.dgu = (uint16_t*)take(z.T * z.I * 2 * 2);
  w.y = (uint16_t*)take(z.T * z.H * 2);
  w.rstd1 = (float*)take(z.T * 4);
  w.rstd2 = (float*)take(z.T * 4);
  w.lse = (float*)take(z.batch * z.nq * z.seq * 4);
  w.Uqkv = (float*)take(z.T * 3 * z.r * 4);
  w.Uo = (float*)take(z.T * z.r * 4);
  w.Ud = (float*)take(z.T * z.r * 4);
  w.Ugu = (float*)take(z.T * 2 * z.r * 4);
  w.dU = (float*)take(z.T * 3 * z.r * 4);
  w.rope = (float2*)take(z.seq * (c.head_dim / 2) * 8);
  w.attn_scratch = (float*)take((attention_dsum_floats(z.batch, z.nq, z.seq) + 2 * z.T * z.nq * 128) * 4);
  w.part_floats = (size_t)8 * z.T * z.maxN();
  w.part = (float*)take(w.part_floats * 4);
  w.lpart_floats = lora_part_floats(z.T, 3, (int)z.r);
  w.lpart = (float*)take(w.lpart_floats * 4);
  return w;
}

size_t LayerWs::saved_bytes(const lsf_layer_cfg& c) {
  Sizes z(c);
  size_t b = up(z.T * z.H * 2) * 3;                 // h1, x2, h2
  b += up(z.T * z.Nqkv * 2) + up(z.T * z.Dq * 2);    // qkv (rotated), att
  b += up(z.T * z.I * 2) * 3;                        // g, u, a
  b += up(z.batch * z.nq * z.seq * 4) + up(z.T * 4) * 2;  // lse, rstd1, rstd2
  b += up(z.T * 3 * z.r * 4) + up(z.T * z.r * 4) * 2 + up(z.T * 2 * z.r * 4);  // U's
  return b;
}

LayerWs LayerWs::with_saved(const lsf_layer_cfg& c, void* base) const {
  Sizes z(c);
  uintptr_t p = (uintptr_t)base;
  auto take = [&](size_t n) {
    void* r = (void*)p;
    p += up(n);
    return r;
  };
  LayerWs w = *this;
  w.h1 = (uint16_t*)take(z.T * z.H * 2);
  w.x2 = (uint16_t*)take(z.T * z.H * 2);
  w.h2 = (uint16_t*)take(z.T * z.H * 2);
  w.qkv = (uint16_t*)take(z.T * z.Nqkv * 2);
  w.att = (uint16_t*)take(z.T * z.Dq * 2);
  w.g = (uint16_t*)take(z.T * z.I * 2);
  w.u = (uint16_t*)take(z.T * z.I * 2);
  w.a = (uint16_t*)take(z.T * z.I * 2);
  w.lse = (float*)take(z.batch * z.nq * z.seq * 4);
  w.rstd1 = (float*)take(z.T * 4);
  w.rstd2 = (float*)take(z.T * 4);
  w.Uqkv = (float*)take(z.T * 3 * z.r * 4);
  w.Uo = (float*)take(z.T * z.r * 4);
  w.Ud = (float*)take(z.T * z.r * 4);
  w.Ugu = (float*)take(z.T * 2 * z.r * 4);
  return w;
}

size_t LayerWs::u_bytes(const lsf_layer_cfg& c) {
  Sizes z(c);
  return up(z.T * 3 * z.r * 4) + up(z.T * z.r * 4) * 2 + up(z.T * 2 * z.r * 4);
}

LayerWs LayerWs::with_u(const lsf_layer_cfg& c, void* base) const {
  Sizes z(c);
  uintptr_t p = (uintptr_t)base;
  auto take = [&](size_t n) {
    void* r = (void*)p;
    p += up(n);
    return r;
  };
  LayerWs w = *this;
  w.Uqkv = (float*)take(z.T * 3 * z.r * 4);
  w.Uo = (float*)take(z.T * z.r * 4);
  w.Ud = (float*)take(z.T * z.r * 4);
  w.Ugu = (float*)take(z.T * 2 * z.r * 4);
  return w;
}

WeightRef weight_ref(const lsf_weight& w, int fmt, int64_t ld) {
  WeightRef r;
  r.fmt = fmt;
  r.ld = ld;
  if (fmt == FMT_BF16) {
    r.bf16 = static_cast<const uint16_t*>(w.data);
  } else if (fmt == FMT_NF4_DQ) {
    r.packed = static_cast<const uint8_t*>(w.data);
    r.absq = static_cast<const uint8_t*>(w.scale);
    r.dq2 = w.scale2;
  } else {
    r.packed = static_cast<const uint8_t*>(w.data);
    r.absmax = static_cast<const float*>(w.scale);
  }
  return r;
}

int choose_splits(int tiles, int K) {
  int s = 1;
  while (s < 8 && tiles * s < 256 && K / (s * 2) >= 512 && (K / 64) % (s * 2) == 0) s *= 2;
  return s;
}

hipError_t run_gemm(bool nn, GemmArgs g, const EpiArgs& e, float* part, size_t part_floats, hipStream_t s) {
  const int bm = gemm_tile_rows(g.M, g.N, nn);
  const int tiles = ((g.M + bm - 1) / bm) * (g.N / 128);
  int splits = 1;
  if (e.kind != EPI_SWIGLU && part != nullptr) {
    const int ws = nn ? wide_nn_splits(g) : wide_splits(g);
    splits = ws > 0 ? ws : choose_splits(tiles, g.K);
  }
  while (splits > 1 && (size_t)splits * g.M * g.N > part_floats) --splits;
  g.splits = splits;
  if (splits == 1) return nn ? gemm_nn(g, e, s) : gemm_nt(g, e, s);
  EpiArgs pe;
  pe.kind = EPI_F32;
  pe.C = part;
  pe.ldc = g.N;
  hipError_t err = nn ? gemm_nn(g, pe, s) : gemm_nt(g, pe, s);
  if (err != hipSuccess) return err;
  return splitk_reduce(part, splits, g.M, g.N, e, s);
}

#define CK(x)                               \
  do {                                      \
    hipError_t e_ = (x);                    \
    if (e_ != hipSuccess) return e_;        \
  } while (0)

static hipError_t timed_gemm(const LayerWs& ws, int kind, bool nn, const GemmArgs& g, const EpiArgs& e,
                             hipStream_t s) {
  if (ws.probe) CK(ws.probe->begin(kind, s));
  CK(run_gemm(nn, g, e, ws.part, ws.part_floats, s));
  if (ws.probe) CK(ws.probe->end(kind, s));
  return hipSuccess;
}

hipError_t layer_forward(const lsf_layer_cfg& c, const lsf_layer_weights& w, const lsf_layer_lora* lora,
                         const uint16_t* x, uint16_t* y, const LayerWs& ws, bool save, bool rope_ready,
                         hipStream_t s) {
  Sizes z(c);
  const int T = (int)z.T, H = (int)z.H, I = (int)z.I, r = (int)z.r;
  const int fmt = w.format;
  const float sc = c.lora_scale;
  if (!rope_ready) CK(rope_table(c.seq, c.head_dim, c.rope_theta, ws.rope, s));

  // attention block
  CK(rmsnorm_fwd(x, w.norm1, T, H, c.rms_eps, ws.h1, ws.rstd1, s));
  GemmArgs g;
  g.M = T;
  {
    const lsf_lora_proj* pq[3] = {proj(lora, PQ), proj(lora, PK), proj(lora, PV)};
    const bool any = pq[0] || pq[1] || pq[2];
    if (any && !ws.u_ready) {
      LoraDown d;
      d.part = ws.lpart; d.part_floats = ws.lpart_floats;
      d.M = T; d.K = H; d.X = ws.h1; d.ldx = H; d.nsec = 3; d.r = r;
      for (int i = 0; i < 3; ++i) d.mat[i] = pq[i] ? pq[i]->A : nullptr;
      d.scale = 1.0f; d.U = ws.Uqkv; d.ldu = 3 * r;
      CK(lora_down(d, s));
    }
    g.N = (int)z.Nqkv; g.K = H; g.A = ws.h1; g.lda = H;
    g.W = weight_ref(w.qkv, fmt, H);
    if (any) {
      g.ext.kx = 3 * r; g.ext.u = ws.Uqkv; g.ext.ldu = 3 * r; g.ext.uscale = sc; g.ext.nsec = 3; g.ext.r = r;
      for (int i = 0; i < 3; ++i) g.ext.mat[i] = pq[i] ? pq[i]->B : nullptr;
      g.ext.row_off[0] = 0;
      g.ext.row_off[1] = c.n_heads * c.head_dim;
      g.ext.row_off[2] = (c.n_heads + c.n_kv_heads) * c.head_dim;
      g.ext.row_off[3] = (int)z.Nqkv;
    }
    EpiArgs e; e.kind = EPI_BF16; e.C = ws.qkv; e.ldc = z.Nqkv;
    CK(timed_gemm(ws, LSF_K_QKV_FWD, false, g, e, s));
  }
  CK(rope_apply(ws.qkv, z.Nqkv, T, c.seq, c.n_heads + c.n_kv_heads, c.head_dim, ws.rope, false, s));
  {
    AttnArgs a;
    a.batch = c.batch; a.seq = c.seq; a.nq = c.n_heads; a.nkv = c.n_kv_heads;
    a.qkv = ws.qkv; a.ldqkv = z.Nqkv; a.o = ws.att; a.lse = ws.lse;
    if (ws.probe) CK(ws.probe->begin(LSF_K_ATTN_FWD, s));
    CK(attention_fwd(a, s));
    if (ws.probe) CK(ws.probe->end(LSF_K_ATTN_FWD, s));
  }
  {
    const lsf_lora_proj* po = proj(lora, PO);
    g = GemmArgs(); g.M = T;
    if (po) {
      if (!ws.u_ready) {
        LoraDown d;
        d.part = ws.lpart; d.part_floats = ws.lpart_floats;
        d.M = T; d.K = (int)z.Dq; d.X = ws.att; d.ldx = z.Dq; d.nsec = 1; d.r = r; d.mat[0] = po->A;
        d.scale = 1.0f; d.U = ws.Uo; d.ldu = r;
        CK(lora_down(d, s));
      }
      g.ext.kx = r; g.ext.u = ws.Uo; g.ext.ldu = r; g.ext.uscale = sc; g.ext.nsec = 1; g.ext.r = r;
      g.ext.mat[0] = po->B; g.ext.row_off[1] = H;
    }
    g.N = H; g.K = (int)z.Dq; g.A = ws.att; g.lda = z.Dq; g.W = weight_ref(w.o, fmt, z.Dq);
    EpiArgs e; e.kind = EPI_RESID_BF16; e.C = ws.x2; e.ldc = H; e.R = x; e.ldr = H;
    CK(timed_gemm(ws, LSF_K_O_FWD, false, g, e, s));
  }
  // MLP block
  CK(rmsnorm_fwd(ws.x2, w.norm2, T, H, c.rms_eps, ws.h2, ws.rstd2, s));
  {
    const lsf_lora_proj* pg[2] = {proj(lora, PG), proj(lora, PU)};
    const bool any = pg[0] || pg[1];
    g = GemmArgs(); g.M = T;
    if (any) {
      if (!ws.u_ready) {
        LoraDown d;
        d.part = ws.lpart; d.part_floats = ws.lpart_floats;
        d.M = T; d.K = H; d.X = ws.h2; d.ldx = H; d.nsec = 2; d.r = r;
        for (int i = 0; i < 2; ++i) d.mat[i] = pg[i] ? pg[i]->A : nullptr;
        d.scale = 1.0f; d.U = ws.Ugu; d.ldu = 2 * r;
        CK(lora_down(d, s));
      }
      g.ext.kx = 2 * r; g.ext.u = ws.Ugu; g.ext.ldu = 2 * r; g.ext.uscale = sc; g.ext.nsec = 2; g.ext.r = r;
      for (int i = 0; i < 2; ++i) g.ext.mat[i] = pg[i] ? pg[i]->B : nullptr;
      g.ext.row_off[1] = I; g.ext.row_off[2] = 2 * I;
    }
    g.N = 2 * I; g.K = H; g.A = ws.h2; g.lda = H; g.W = weight_ref(w.gate_up, fmt, H); g.pair_I = I;
    EpiArgs e; e.kind = EPI_SWIGLU; e.C = ws.a; e.ldc = I;
    if (save) { e.g = ws.g; e.u = ws.u; e.ldgu = I; }
    CK(timed_gemm(ws, LSF_K_GATEUP_FWD, false, g, e, s));
  }
  {
    const lsf_lora_proj* pd = proj(lora, PD);
    if (pd && !ws.u_ready) {
      LoraDown d;
      d.part = ws.lpart; d.part_floats = ws.lpart_floats;
      d.M = T; d.K = I; d.X = ws.a; d.ldx = I; d.nsec = 1; d.r = r; d.mat[0] = pd->A;
      d.scale = 1.0f; d.U = ws.Ud; d.ldu = r;
      CK(lora_down(d, s));
    }
    if (y != nullptr) {
      g = GemmArgs(); g.M = T;
      if (pd) {
        g.ext.kx = r; g.ext.u = ws.Ud; g.ext.ldu = r; g.ext.uscale = sc; g.ext.nsec = 1; g.ext.r = r;
        g.ext.mat[0] = pd->B; g.ext.row_off[1] = H;
      }
      g.N = H; g.K = I; g.A = ws.a; g.lda = I; g.W = weight_ref(w.down, fmt, I);
      EpiArgs e; e.kind = EPI_RESID_BF16; e.C = y; e.ldc = H; e.R = ws.x2; e.ldr = H;
      CK(timed_gemm(ws, LSF_K_DOWN_FWD, false, g, e, s));
    }
  }
  return hipSuccess;
}

namespace {

// dU = s * dY_sec B_sec for up to three column sections of dY.
hipError_t lora_dU(const uint16_t* dY, int64_t ld, int T, int r, float sc, int nsec, const lsf_lora_proj* const* p,
                   const int* xoff, const int* ksec, float* dU, const LayerWs& ws, hipStream_t s) {
  LoraDown d;
  d.part = ws.lpart;
  d.part_floats = ws.lpart_floats;
  d.M = T; d.X = dY; d.ldx = ld; d.nsec = nsec; d.r = r; d.bside = true; d.scale = sc; d.U = dU;
  d.ldu = nsec * r;
  d.K = ksec[0];
  for (int i = 0; i < nsec; ++i) {
    d.mat[i] = p[i] ? p[i]->B : nullptr;
    d.xoff[i] = xoff[i];
    d.ksec[i] = ksec[i];
  }
  return lora_down(d, s);
}

// dA_sec += dU_sec^T X  and  dB_sec += s dY_sec^T U_sec, every section of the
// group in one launch.
hipError_t lora_grads(int slot, int T, int r, float sc, int nsec, const lsf_lora_proj* const* p, const float* dU,
                      const uint16_t* X, int64_t ldx, int nx, const float* U, const uint16_t* dY, int64_t ldy,
                      const int* yoff, const int* ny, const LayerWs& ws, hipStream_t s) {
  LoraGradSec gs[2 * 3];
  int n = 0;
  for (int i = 0; i < nsec; ++i) {
    if (!p[i]) continue;
    if (p[i]->dA) {
      LoraGradSec& q = gs[n++];
      q.P = dU; q.ldp = nsec * r; q.pcol0 = i * r; q.Q = X; q.ldq = ldx; q.qoff = 0; q.nq = nx;
      q.out = p[i]->dA; q.transposed = false; q.scale = 1.0f; q.overwrite = ws.grads_overwrite;
    }
    if (p[i]->dB) {
      LoraGradSec& q = gs[n++];
      q.P = U; q.ldp = nsec * r; q.pcol0 = i * r; q.Q = dY; q.ldq = ldy; q.qoff = yoff[i]; q.nq = ny[i];
      q.out = p[i]->dB; q.transposed = true; q.scale = sc; q.overwrite = ws.grads_overwrite;
    }
  }
  hipError_t e;
  if (ws.grad_after[slot] && (e = hipStreamWaitEvent(s, ws.grad_after[slot], 0)) != hipSuccess) return e;
  if ((e = lora_grad(gs, n, T, r, ws.part, ws.part_floats, s)) != hipSuccess) return e;
  if (ws.grad_done[slot]) return hipEventRecord(ws.grad_done[slot], s);
  return hipSuccess;
}

}  // namespace

hipError_t layer_backward(const lsf_layer_cfg& c, const lsf_layer_weights& w, const lsf_layer_lora* lora,
                          const uint16_t* x, const uint16_t* dy, uint16_t* dx, const LayerWs& ws, bool rope_ready,
                          hipStream_t s, bool recompute) {
  Sizes z(c);
  const int T = (int)z.T, H = (int)z.H, I = (int)z.I, r = (int)z.r;
  const int fmt = w.format;
  const float sc = c.lora_scale;
  // Recompute the forward from the checkpoint, keeping what the backward reads.
  if (recompute) CK(layer_forward(c, w, lora, x, nullptr, ws, true, rope_ready, s));
  else if (!rope_ready) CK(rope_table(c.seq, c.head_dim, c.rope_theta, ws.rope, s));

  // down projection: dA = dY W_down (+ LoRA), then SwiGLU backward in the epilogue
  {
    const lsf_lora_proj* p[1] = {proj(lora, PD)};
    const int xo[1] = {0}, ks[1] = {H};
    if (p[0]) CK(lora_dU(dy, H, T, r, sc, 1, p, xo, ks, ws.dU, ws, s));
    GemmArgs g; g.M = T; g.N = I; g.K = H; g.A = dy; g.lda = H; g.W = weight_ref(w.down, fmt, I);
    if (p[0]) {
      g.ext.kx = r; g.ext.u = ws.dU; g.ext.ldu = r; g.ext.nsec = 1; g.ext.r = r; g.ext.mat[0] = p[0]->A;
      g.ext.ldmat = I;
    }
    EpiArgs e; e.kind = EPI_SWIGLU_BWD; e.C = ws.dgu; e.ldc = 2 * (int64_t)I; e.g = ws.g; e.u = ws.u; e.ldgu = I;
    CK(timed_gemm(ws, LSF_K_DOWN_BWD, true, g, e, s));
    if (p[0]) {
      const int yo[1] = {0}, ny[1] = {H};
      CK(lora_grads(0, T, r, sc, 1, p, ws.dU, ws.a, I, I, ws.Ud, dy, H, yo, ny, ws, s));
    }
  }
  // gate|up: dh2 = dG W_gate + dU W_up (+ LoRA)
  {
    const lsf_lora_proj* p[2] = {proj(lora, PG), proj(lora, PU)};
    const bool any = p[0] || p[1];
    const int xo[2] = {0, I}, ks[2] = {I, I};
    if (any) CK(lora_dU(ws.dgu, 2 * (int64_t)I, T, r, sc, 2, p, xo, ks, ws.dU, ws, s));
    GemmArgs g; g.M = T; g.N = H; g.K = 2 * I; g.A = ws.dgu; g.lda = 2 * (int64_t)I;
    g.W = weight_ref(w.gate_up, fmt, H);
    if (any) {
      g.ext.kx = 2 * r; g.ext.u = ws.dU; g.ext.ldu = 2 * r; g.ext.nsec = 2; g.ext.r = r;
      for (int i = 0; i < 2; ++i) g.ext.mat[i] = p[i] ? p[i]->A : nullptr;
      g.ext.ldmat = H;
    }
    EpiArgs e; e.kind = EPI_BF16; e.C = ws.dh; e.ldc = H;
    CK(timed_gemm(ws, LSF_K_GATEUP_BWD, true, g, e, s));
    if (any) {
      const int yo[2] = {0, I}, ny[2] = {I, I};
      CK(lora_grads(1, T, r, sc, 2, p, ws.dU, ws.h2, H, H, ws.Ugu, ws.dgu, 2 * (int64_t)I, yo, ny, ws, s));
    }
  }
  CK(rmsnorm_bwd(ws.dh, ws.x2, w.norm2, ws.rstd2, dy, T, H, ws.dx2, s));
  // o projection
  {
    const lsf_lora_proj* p[1] = {proj(lora, PO)};
    const int xo[1] = {0}, ks[1] = {H};
    if (p[0]) CK(lora_dU(ws.dx2, H, T, r, sc, 1, p, xo, ks, ws.dU, ws, s));
    GemmArgs g; g.M = T; g.N = (int)z.Dq; g.K = H; g.A = ws.dx2; g.lda = H; g.W = weight_ref(w.o, fmt, z.Dq);
    if (p[0]) {
      g.ext.kx = r; g.ext.u = ws.dU; g.ext.ldu = r; g.ext.nsec = 1; g.ext.r = r; g.ext.mat[0] = p[0]->A;
      g.ext.ldmat = z.Dq;
    }
    EpiArgs e; e.kind = EPI_BF16; e.C = ws.dob; e.ldc = z.Dq;
    CK(timed_gemm(ws, LSF_K_O_BWD, true, g, e, s));
    if (p[0]) {
      const int yo[1] = {0}, ny[1] = {H};
      CK(lora_grads(2, T, r, sc, 1, p, ws.dU, ws.att, z.Dq, (int)z.Dq, ws.Uo, ws.dx2, H, yo, ny, ws, s));
    }
  }
  // attention
  {
    AttnArgs a;
    a.batch = c.batch; a.seq = c.seq; a.nq = c.n_heads; a.nkv = c.n_kv_heads;
    a.qkv = ws.qkv; a.ldqkv = z.Nqkv; a.o = ws.att; a.lse = ws.lse; a.dout = ws.dob; a.Dsum = ws.attn_scratch;
    a.dqkv = ws.dqkv;
    if (ws.probe) CK(ws.probe->begin(LSF_K_ATTN_BWD, s));
    CK(attention_bwd(a, s));
    if (ws.probe) CK(ws.probe->end(LSF_K_ATTN_BWD, s));
  }
  CK(rope_apply(ws.dqkv, z.Nqkv, T, c.seq, c.n_heads + c.n_kv_heads, c.head_dim, ws.rope, true, s));
  // q|k|v projection
  {
    const lsf_lora_proj* p[3] = {proj(lora, PQ), proj(lora, PK), proj(lora, PV)};
    const bool any = p[0] || p[1] || p[2];
    const int qd = c.n_heads * c.head_dim, kd = c.n_kv_heads * c.head_dim;
    const int xo[3] = {0, qd, qd + kd}, ks[3] = {qd, kd, kd};
    if (any) CK(lora_dU(ws.dqkv, z.Nqkv, T, r, sc, 3, p, xo, ks, ws.dU, ws, s));
    GemmArgs g; g.M = T; g.N = H; g.K = (int)z.Nqkv; g.A = ws.dqkv; g.lda = z.Nqkv;
    g.W = weight_ref(w.qkv, fmt, H);
    if (any) {
      g.ext.kx = 3 * r; g.ext.u = ws.dU; g.ext.ldu = 3 * r; g.ext.nsec = 3; g.ext.r = r;
      for (int i = 0; i < 3; ++i) g.ext.mat[i] = p[i] ? p[i]->A : nullptr;
      g.ext.ldmat = H;
    }
    EpiArgs e; e.kind = EPI_BF16; e.C = ws.dh; e.ldc = H;
    CK(timed_gemm(ws, LSF_K_QKV_BWD, true, g, e, s));
    if (any) {
      const int ny[3] = {qd, kd, kd};
      CK(lora_grads(3, T, r, sc, 3, p, ws.dU, ws.h1, H, H, ws.Uqkv, ws.dqkv, z.Nqkv, xo, ny, ws, s));
    }
  }
  return rmsnorm_bwd(ws.dh, x, w.norm1, ws.rstd1, ws.dx2, T, H, dx, s);
}

}  // namespace lsf
