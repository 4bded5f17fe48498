// Host-side launchers of the gfx950 kernels (internal to liblsf.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsf {

enum { FMT_NF4 = 0, FMT_BF16 = 1, FMT_NF4_DQ = 2 };

// A frozen weight as the GEMMs read it.  Row length `ld` = in-features.
struct WeightRef {
  int fmt = FMT_NF4;
  const uint8_t* packed = nullptr;  // NF4 / NF4_DQ codes
  const float* absmax = nullptr;    // NF4 fp32 absmax
  const uint8_t* absq = nullptr;    // NF4_DQ uint8 absmax codes
  const float* dq2 = nullptr;       // NF4_DQ second-level (scale, offset) pairs
  const uint16_t* bf16 = nullptr;   // BF16 weights
  int64_t ld = 0;
};

// LoRA folded into the GEMM as extra contraction steps.
//  NT (forward):  C[m, n] += sum_j (uscale * U[m, j]) * Bsec(n)[n - row_off[sec], j - sec*r]
//  NN (backward): C[m, k] += sum_j U[m, j] * Asec(j)[j - sec*r, k]
// with j running over the nsec*r columns of U.  Missing sections (mat NULL)
// contribute nothing.
struct LoraExt {
  int kx = 0;  // nsec * r, 0 = no extension
  const float* u = nullptr;
  int ldu = 0;
  float uscale = 1.0f;
  int nsec = 0, r = 0;
  const float* mat[3] = {nullptr, nullptr, nullptr};
  int row_off[4] = {0, 0, 0, 0};  // NT: W-row offset of every section, row_off[nsec] = end
  int64_t ldmat = 0;              // NN: row length of A_sec
};

struct GemmArgs {
  int M = 0, N = 0, K = 0;  // C is M x N, main contraction K
  const uint16_t* A = nullptr;
  int64_t lda = 0;
  WeightRef W;
  LoraExt ext;
  int pair_I = 0;  // NT only: >0 pairs gate row j with up row pair_I + j
  int splits = 1;  // K splits (grid.z); the extension runs in the last split
};

enum EpiKind {
  EPI_BF16 = 0,        // C = bf16(acc)
  EPI_RESID_BF16 = 1,  // C = bf16(R + acc)
  EPI_SWIGLU = 2,      // NT pair mode: a = bf16(silu(g) u), optional g, u
  EPI_SWIGLU_BWD = 3,  // NN: dA -> dg, du using saved g, u
  EPI_F32 = 4,         // C = acc (fp32)
};

struct EpiArgs {
  int kind = EPI_BF16;
  void* C = nullptr;
  int64_t ldc = 0;
  const uint16_t* R = nullptr;  // residual
  int64_t ldr = 0;
  uint16_t* g = nullptr;        // EPI_SWIGLU: saved gate (optional); EPI_SWIGLU_BWD: input gate
  uint16_t* u = nullptr;        // same for up
  int64_t ldgu = 0;
};

// Rows of the C tile (128 or 256) a GEMM of M x N uses; columns are 128.
int gemm_tile_rows(int M, int N, bool nn);
// C = A W^T (+ LoRA), W rows map to C columns.
hipError_t gemm_nt(const GemmArgs& g, const EpiArgs& e, hipStream_t s);
// The ping-pong kernel for forward NF4 GEMMs (gate|up; with split-K also
// q|k|v, o and down at a few hundred tokens); gemm_nt uses it by itself where
// gemm_wide_applies.
bool gemm_wide_applies(const GemmArgs& g, const EpiArgs& e);
// Split count (2..8) with which the wide kernel serves a forward GEMM of few
// tiles as split-K, or 0.  Depends on the shape only, so the general kernel
// given the same count sums the same partials in the same order.
int wide_splits(const GemmArgs& g);
void set_gemm_wide(bool enable);  // process-wide; default on
void set_gemm_wide_tile(int rows);  // 0: tile rows by shape; 256 or 512: forced (diagnostics)
int64_t gemm_wide_launches();      // wide-kernel launches so far
hipError_t gemm_nt_wide(const GemmArgs& g, const EpiArgs& e, hipStream_t s);
// The same schedule for input-gradient GEMMs (gate|up and down backward);
// gemm_nn uses it by itself where gemm_wide_nn_applies.  wide_nn_splits: the
// split count (1 = none) it serves a shape with, or 0; like wide_splits it
// depends on the shape only.
bool gemm_wide_nn_applies(const GemmArgs& g, const EpiArgs& e);
int wide_nn_splits(const GemmArgs& g);
hipError_t gemm_nn_wide(const GemmArgs& g, const EpiArgs& e, hipStream_t s);
// C = A W (+ LoRA), contraction over W rows.
hipError_t gemm_nn(const GemmArgs& g, const EpiArgs& e, hipStream_t s);
// Sum `splits` (1..8) fp32 partials [splits, M, N] in fixed order and apply e.
hipError_t splitk_reduce(const float* part, int splits, int M, int N, const EpiArgs& e, hipStream_t s);

// NF4
hipError_t nf4_quantize_launch(const float* w, int64_t n, uint8_t* packed, float* absmax, hipStream_t s);
hipError_t nf4_dequantize_launch(const uint8_t* packed, const float* absmax, int64_t n, uint16_t* out,
                                 hipStream_t s);
// Double quantisation: 8-bit absmax codes and (scale, offset) per 256 blocks.
hipError_t dq_encode_launch(const float* absmax, int64_t nblocks, uint8_t* codes, float* scale2, hipStream_t s);
hipError_t nf4dq_dequantize_launch(const uint8_t* packed, const uint8_t* absq, const float* scale2, int64_t n,
                                   uint16_t* out, hipStream_t s);

// LoRA side paths.
//  down_fwd: U[m, sec*r + j] = scale * sum_k X[m, k] * A_sec[j, k]  (all sections read X)
//  down_bwd: U[m, sec*r + j] = scale * sum_{n in sec} X[m, xoff_sec + n] * B_sec[n, j]
// The contraction is cut into at most kLoraDownChunks chunks per section;
// lora_down writes one partial product per chunk into part and their ordered
// sum into U.
constexpr int kLoraDownChunks = 16;
struct LoraDown {
  int M = 0, K = 0;  // K: columns of X read per section
  const uint16_t* X = nullptr;
  int64_t ldx = 0;
  int nsec = 0, r = 0;
  const float* mat[3] = {nullptr, nullptr, nullptr};
  int xoff[3] = {0, 0, 0};
  int ksec[3] = {0, 0, 0};  // B-side: rows of B_sec (columns of X) per section; 0 = K
  float scale = 1.0f;
  float* U = nullptr;
  int ldu = 0;
  bool bside = false;  // false: A-side [r, K]; true: B-side [K, r]
  float* part = nullptr;  // the per-chunk partial products (lora_part_floats of them)
  size_t part_floats = 0;
};
// Floats of partials lora_down writes for M rows, nsec sections of rank r.
inline size_t lora_part_floats(int64_t M, int nsec, int r) { return (size_t)nsec * kLoraDownChunks * M * r; }
hipError_t lora_down(const LoraDown& a, hipStream_t s);

// out += scale * sum_t P[t, pcol0 + j] * Q[t, qoff + q] for j < r, q < nq.
//   transposed = false: out[j * nq + q]  (dA layout [r, in])
//   transposed = true:  out[q * r + j]   (dB layout [out, r])
struct LoraGradSec {
  const float* P = nullptr;
  int ldp = 0, pcol0 = 0;
  const uint16_t* Q = nullptr;
  int64_t ldq = 0;
  int qoff = 0, nq = 0;
  float* out = nullptr;
  bool transposed = false;
  float scale = 1.0f;
  bool overwrite = false;  // out = ... instead of out += ... (the first accumulation)
};
// Up to kLoraGradSecs sections in one launch.  part (part_floats floats of
// scratch, may be NULL) holds per-token-split partials when there are too few
// workgroups without splitting the tokens.
constexpr int kLoraGradSecs = 6;
hipError_t lora_grad(const LoraGradSec* secs, int nsec, int T, int r, float* part, size_t part_floats,
                     hipStream_t s);

// Elementwise / normalisation.
hipError_t rmsnorm_fwd(const uint16_t* x, const uint16_t* w, int T, int H, float eps, uint16_t* y, float* rstd,
                       hipStream_t s);
// dx = resid + rmsnorm'(x)^T dy   (resid may be NULL)
hipError_t rmsnorm_bwd(const uint16_t* dy, const uint16_t* x, const uint16_t* w, const float* rstd,
                       const uint16_t* resid, int T, int H, uint16_t* dx, hipStream_t s);
hipError_t rope_table(int seq, int d, float theta, float2* tab, hipStream_t s);
// In-place rotation of the q and k heads of a [T, ld] buffer; inverse = backward.
hipError_t rope_apply(uint16_t* qk, int64_t ld, int T, int seq, int n_heads_total, int d, const float2* tab,
                      bool inverse, hipStream_t s);
// x[t] = E[ids[t]]; an id outside [0, V) gives a zero row and sets *status = 1
// (status may be NULL).
hipError_t embed_gather(const int32_t* ids, const uint16_t* E, int T, int H, int V, uint16_t* x, int32_t* status,
                        hipStream_t s);
// CE over next-token labels; writes per-row loss terms, dlogits (bf16) and the mean loss.
hipError_t cross_entropy(const float* logits, const int32_t* ids, int batch, int seq, int V, float loss_scale,
                         uint16_t* dlogits, float* row_loss, float* loss, hipStream_t s);
// Per-sequence sums of next-token log-probabilities: lse [T], row_logp [T]
// (label log-probability, 0 on unlabelled rows) and lp [batch].
hipError_t seq_logprobs(const float* logits, const int32_t* ids, int batch, int seq, int V, float* lse,
                        float* row_logp, float* lp, hipStream_t s);
// DPO loss over batch/2 pairs (chosen sequences first) and, if dlogits is not
// NULL, its logits gradient times loss_scale; coef [batch] is scratch.
hipError_t dpo_head_grad(const float* logits, const int32_t* ids, const float* lse, const float* lp_pi,
                         const float* lp_ref, int batch, int seq, int V, float beta, float loss_scale, float* coef,
                         float* loss, uint16_t* dlogits, hipStream_t s);

// AdamW over n fp32 values (16-byte aligned arrays), moments m, v; t = step >= 1.
// Clips the gradient to max_grad_norm (> 0) by its global L2 norm first; writes
// that norm to grad_norm when it is not NULL.  ws: adamw_ws_bytes() of device memory.
size_t adamw_ws_bytes();
// The same update with 8-bit moment states: int8 codes qm, uint8 codes qv and
// one fp32 absmax per 2048 values for each (adamw8_blocks(n) entries).
size_t adamw8_ws_bytes();
int64_t adamw8_blocks(int64_t n);
hipError_t adamw8_update(float* p, const float* g, int8_t* qm, uint8_t* qv, float* am, float* av, int64_t n,
                         float lr, float beta1, float beta2, float eps, float weight_decay, float max_grad_norm,
                         int step, float* grad_norm, float* ws, hipStream_t s);
hipError_t adamw_update(float* p, const float* g, float* m, float* v, int64_t n, float lr, float beta1, float beta2,
                        float eps, float weight_decay, float max_grad_norm, int step, float* grad_norm, float* ws,
                        hipStream_t s);

// Attention (head_dim 128, causal, GQA).  qkv: [T, ldqkv] with q heads, then
// k heads, then v heads; o: [T, nq*128]; lse: [batch, nq, seq].
struct AttnArgs {
  int batch = 0, seq = 0, nq = 0, nkv = 0;
  const uint16_t* qkv = nullptr;
  int64_t ldqkv = 0;
  uint16_t* o = nullptr;
  float* lse = nullptr;
  // backward
  const uint16_t* dout = nullptr;
  float* Dsum = nullptr;   // [batch, nq, seq], then the dK / dV partials (see below)
  uint16_t* dqkv = nullptr;  // same layout as qkv
};
hipError_t attention_fwd(const AttnArgs& a, hipStream_t s);
// a.Dsum points at attention_dsum_floats(batch, nq, seq) + 2 * batch*seq * nq * 128
// floats of device scratch (16-byte aligned): Dsum, then the per-query-head dK
// and dV partials.
hipError_t attention_bwd(const AttnArgs& a, hipStream_t s);
inline int64_t attention_dsum_floats(int64_t batch, int64_t nq, int64_t seq) { return (batch * nq * seq + 63) / 64 * 64; }

hipError_t zero_f32(float* p, int64_t n, hipStream_t s);
// Fill bytes (a multiple of 16, 16-byte aligned) with the 32-bit pattern v.
hipError_t fill_pattern(void* p, int64_t bytes, uint32_t v, hipStream_t s);
// A kernel that only waits, for `iters` fixed-length sleeps.
hipError_t delay(int iters, hipStream_t s);

}  // namespace lsf
