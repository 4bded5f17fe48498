// Layer composition (host side, internal).
#pragma once
#include <hip/hip_runtime.h>

#include "../../include/lsf.h"
#include "kernels.h"

namespace lsf {

// Optional event probe around the big kernels (used by the streamer's timing).
struct Probe {
  virtual hipError_t begin(int kind, hipStream_t s) = 0;
  virtual hipError_t end(int kind, hipStream_t s) = 0;
  virtual ~Probe() = default;
};

// Scratch layout of one decoder layer's forward + recompute + backward.
struct LayerWs {
  uint16_t *h1, *qkv, *att, *x2, *h2, *g, *u, *a, *y;
  float *rstd1, *rstd2, *lse, *Uqkv, *Uo, *Ugu, *Ud;
  float2* rope;
  uint16_t *dgu, *dh, *dx2, *dob, *dqkv;
  float *dU, *attn_scratch, *part;
  size_t part_floats;
  float* lpart;  // LoRA down-projection partials (never the split-K partials' memory)
  size_t lpart_floats;
  Probe* probe = nullptr;
  bool grads_overwrite = false;  // the backward stores dA, dB instead of adding to them
  // The LoRA activations (Uqkv, Uo, Ugu, Ud) already hold this layer's values
  // for this input (kept from its forward): the forward does not recompute them.
  bool u_ready = false;
  // Order of the adapter-gradient accumulations when several workspaces run
  // on different streams: before its k-th gradient launch (k = 0..3: down,
  // gate|up, o, q|k|v) the backward makes its stream wait for grad_after[k],
  // and afterwards records grad_done[k] (each only when set).
  hipEvent_t grad_after[4] = {nullptr, nullptr, nullptr, nullptr};
  hipEvent_t grad_done[4] = {nullptr, nullptr, nullptr, nullptr};
  static size_t bytes(const lsf_layer_cfg& c);
  static LayerWs carve(const lsf_layer_cfg& c, void* base);
  // The tensors a forward with save = true leaves for the backward (h1, qkv,
  // att, lse, x2, h2, g, u, a, rstd1, rstd2 and the LoRA activations), laid
  // out from `base`: this workspace with those pointers moved there.
  static size_t saved_bytes(const lsf_layer_cfg& c);
  LayerWs with_saved(const lsf_layer_cfg& c, void* base) const;
  // Only the LoRA activations (Uqkv, Uo, Ud, Ugu), laid out from `base`.
  static size_t u_bytes(const lsf_layer_cfg& c);
  LayerWs with_u(const lsf_layer_cfg& c, void* base) const;
};

WeightRef weight_ref(const lsf_weight& w, int fmt, int64_t ld);

// x -> y.  save keeps every intermediate the backward needs; rope_ready skips
// rebuilding the RoPE table already in ws.rope.  y may be NULL when only the
// saved state is wanted (the recompute inside the backward).
hipError_t layer_forward(const lsf_layer_cfg& c, const lsf_layer_weights& w, const lsf_layer_lora* lora,
                         const uint16_t* x, uint16_t* y, const LayerWs& ws, bool save, bool rope_ready,
                         hipStream_t s);
// recompute = false: ws already holds what layer_forward(save = true) of the
// same x left (LayerWs::with_saved), and the forward is not run again.
hipError_t layer_backward(const lsf_layer_cfg& c, const lsf_layer_weights& w, const lsf_layer_lora* lora,
                          const uint16_t* x, const uint16_t* dy, uint16_t* dx, const LayerWs& ws, bool rope_ready,
                          hipStream_t s, bool recompute = true);

// Split count for a GEMM with `tiles` output tiles and contraction K.
int choose_splits(int tiles, int K);

// One GEMM with split-K and the final epilogue handled.
hipError_t run_gemm(bool nn, GemmArgs g, const EpiArgs& e, float* part, size_t part_floats, hipStream_t s);

}  // namespace lsf
