// C ABI of liblsf.so: argument validation, error reporting, NF4 and single
// linear entry points, layer entry points, the host-store layout and the
// two-buffer layer streamer with the stack step.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <algorithm>
#include <vector>

#include "../../include/lsf.h"
#include "kernels.h"
#include "layer.h"

using namespace lsf;

namespace {

thread_local std::string g_err;

lsf_status fail(lsf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

lsf_status ok() {
  g_err.clear();
  return LSF_OK;
}

#define HIPCK(x)                                                                                  \
  do {                                                                                            \
    hipError_t e_ = (x);                                                                          \
    if (e_ != hipSuccess) return fail(LSF_ERR_HIP, "%s: %s", #x, hipGetErrorString(e_));        \
  } while (0)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_rank(int r) { return r == 4 || r == 8 || r == 16 || r == 32 || r == 64; }

lsf_status check_cfg(const lsf_layer_cfg* c) {
  if (c == nullptr) return fail(LSF_ERR_INVALID_ARG, "cfg is NULL");
  if (c->batch < 1 || c->seq < 1) return fail(LSF_ERR_SHAPE, "batch and seq must be >= 1 (got %d, %d)", c->batch, c->seq);
  if (c->hidden <= 0 || c->hidden % 128) return fail(LSF_ERR_SHAPE, "hidden must be a positive multiple of 128");
  if (c->intermediate <= 0 || c->intermediate % 128)
    return fail(LSF_ERR_SHAPE, "intermediate must be a positive multiple of 128");
  if (c->head_dim != 128) return fail(LSF_ERR_SHAPE, "head_dim must be 128");
  if (c->n_heads <= 0 || c->n_kv_heads <= 0 || c->n_heads % c->n_kv_heads)
    return fail(LSF_ERR_SHAPE, "n_heads must be a positive multiple of n_kv_heads");
  if (!valid_rank(c->rank)) return fail(LSF_ERR_SHAPE, "rank must be one of 4, 8, 16, 32, 64");
  if ((int64_t)c->batch * c->seq > (1 << 20)) return fail(LSF_ERR_SHAPE, "too many tokens per call");
  return LSF_OK;
}

lsf_status check_weight(const lsf_weight& w, int fmt, const char* name) {
  if (w.data == nullptr || !aligned(w.data, 16)) return fail(LSF_ERR_ALIGN, "%s: data NULL or not 16-byte aligned", name);
  if (fmt == LSF_FMT_NF4 && (w.scale == nullptr || !aligned(w.scale, 4)))
    return fail(LSF_ERR_INVALID_ARG, "%s: NF4 absmax missing", name);
  if (fmt == LSF_FMT_NF4_DQ && (w.scale == nullptr || w.scale2 == nullptr || !aligned(w.scale2, 8)))
    return fail(LSF_ERR_INVALID_ARG, "%s: double-quantised scales missing", name);
  return LSF_OK;
}

lsf_status check_weights(const lsf_layer_weights* w) {
  if (w == nullptr) return fail(LSF_ERR_INVALID_ARG, "weights is NULL");
  if (w->format != LSF_FMT_NF4 && w->format != LSF_FMT_BF16 && w->format != LSF_FMT_NF4_DQ)
    return fail(LSF_ERR_INVALID_ARG, "unknown weight format %d", w->format);
  lsf_status s;
  if ((s = check_weight(w->qkv, w->format, "qkv")) != LSF_OK) return s;
  if ((s = check_weight(w->o, w->format, "o")) != LSF_OK) return s;
  if ((s = check_weight(w->gate_up, w->format, "gate_up")) != LSF_OK) return s;
  if ((s = check_weight(w->down, w->format, "down")) != LSF_OK) return s;
  if (w->norm1 == nullptr || w->norm2 == nullptr || !aligned(w->norm1, 16) || !aligned(w->norm2, 16))
    return fail(LSF_ERR_ALIGN, "norm weights NULL or not 16-byte aligned");
  return LSF_OK;
}

lsf_status check_lora(const lsf_layer_lora* l) {
  if (l == nullptr) return LSF_OK;
  const lsf_lora_proj* p = &l->q;
  for (int i = 0; i < 7; ++i) {
    if (p[i].A == nullptr) continue;
    if (p[i].B == nullptr) return fail(LSF_ERR_INVALID_ARG, "adapter %d has A but no B", i);
    if (!aligned(p[i].A, 16) || !aligned(p[i].B, 4)) return fail(LSF_ERR_ALIGN, "adapter %d not aligned", i);
  }
  return LSF_OK;
}

lsf_status check_dev(const void* p, const char* name) {
  if (p == nullptr) return fail(LSF_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(LSF_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return LSF_OK;
}

hipStream_t S(lsf_stream s) { return static_cast<hipStream_t>(s); }

// ------------------------------------------------------------ blob layout
struct Blob {
  uint64_t off[10];
  uint64_t bytes, stride;
};

uint64_t al256(uint64_t v) { return (v + 255) / 256 * 256; }

Blob blob_layout(const lsf_layer_cfg& c, int fmt) {
  const uint64_t H = c.hidden, I = c.intermediate, Dq = (uint64_t)c.n_heads * c.head_dim;
  const uint64_t Nqkv = (uint64_t)(c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const uint64_t n[4] = {Nqkv * H, H * Dq, 2 * I * H, H * I};
  Blob b{};
  uint64_t p = 0;
  for (int i = 0; i < 4; ++i) {
    b.off[i] = p;
    p += al256(fmt == LSF_FMT_BF16 ? n[i] * 2 : n[i] / 2);
  }
  for (int i = 0; i < 4; ++i) {
    b.off[4 + i] = p;
    if (fmt == LSF_FMT_NF4) p += al256(n[i] / 64 * 4);
    else if (fmt == LSF_FMT_NF4_DQ) p += al256(n[i] / 64) + al256((n[i] / 64 + 255) / 256 * 8);
    // BF16 has no scales: the section is empty
  }
  b.off[8] = p;
  p += al256(H * 2);
  b.off[9] = p;
  p += al256(H * 2);
  b.bytes = p;
  b.stride = (p + 4095) / 4096 * 4096;
  return b;
}

void weights_from_blob(const lsf_layer_cfg& c, int fmt, const void* blob, lsf_layer_weights* w) {
  const Blob b = blob_layout(c, fmt);
  const uint64_t H = c.hidden, I = c.intermediate, Dq = (uint64_t)c.n_heads * c.head_dim;
  const uint64_t Nqkv = (uint64_t)(c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const uint64_t n[4] = {Nqkv * H, H * Dq, 2 * I * H, H * I};
  const char* base = static_cast<const char*>(blob);
  lsf_weight* ws[4] = {&w->qkv, &w->o, &w->gate_up, &w->down};
  w->format = fmt;
  for (int i = 0; i < 4; ++i) {
    ws[i]->data = base + b.off[i];
    ws[i]->scale = (fmt == LSF_FMT_BF16) ? nullptr : base + b.off[4 + i];
    ws[i]->scale2 = (fmt == LSF_FMT_NF4_DQ)
                        ? reinterpret_cast<const float*>(base + b.off[4 + i] + al256(n[i] / 64))
                        : nullptr;
  }
  w->norm1 = reinterpret_cast<const uint16_t*>(base + b.off[8]);
  w->norm2 = reinterpret_cast<const uint16_t*>(base + b.off[9]);
}

// ---------------------------------------------- allocation-free scratch
// The scratch of linear_fwd_noalloc: a device array the code object carries,
// so the loader places one copy on every GPU the library runs on.  Its name is
// a host-side stand-in in host code; the device address of each GPU's copy
// comes from hipGetSymbolAddress with that GPU current, once, and is the only
// form host code passes on.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

lsf_status noalloc_scratch(void** out) {
  int dev = -1;
  HIPCK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(LSF_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(LSF_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LSF_OK;
}

}  // namespace

// ================================================================ C ABI ==
extern "C" {

const char* lsf_last_error(void) { return g_err.c_str(); }
const char* lsf_version(void) { return "lsf 0.1.0 (gfx950)"; }

lsf_status gemm_set_wide(int32_t enable) {
  if (enable != 0 && enable != 1 && enable != 256 && enable != 512)
    return fail(LSF_ERR_INVALID_ARG, "enable must be 0, 1, 256 or 512 (got %d)", (int)enable);
  set_gemm_wide(enable != 0);
  set_gemm_wide_tile(enable > 1 ? enable : 0);
  return ok();
}

int64_t gemm_wide_launch_count(void) { return gemm_wide_launches(); }

lsf_status nf4_quantize(const float* w, int64_t n, int32_t blocksize, uint8_t* packed, float* absmax,
                        lsf_stream stream) {
  if (blocksize != 64) return fail(LSF_ERR_SHAPE, "blocksize must be 64");
  if (n < 0 || n % 64) return fail(LSF_ERR_SHAPE, "n must be a non-negative multiple of 64 (got %lld)", (long long)n);
  if (n == 0) return ok();
  lsf_status s;
  if ((s = check_dev(w, "w")) || (s = check_dev(packed, "packed")) || (s = check_dev(absmax, "absmax"))) return s;
  HIPCK(nf4_quantize_launch(w, n, packed, absmax, S(stream)));
  return ok();
}

lsf_status nf4_dequantize(const uint8_t* packed, const float* absmax, int64_t n, int32_t blocksize, uint16_t* out,
                          lsf_stream stream) {
  if (blocksize != 64) return fail(LSF_ERR_SHAPE, "blocksize must be 64");
  if (n < 0 || n % 64) return fail(LSF_ERR_SHAPE, "n must be a non-negative multiple of 64 (got %lld)", (long long)n);
  if (n == 0) return ok();
  lsf_status s;
  if ((s = check_dev(packed, "packed")) || (s = check_dev(absmax, "absmax")) || (s = check_dev(out, "out"))) return s;
  HIPCK(nf4_dequantize_launch(packed, absmax, n, out, S(stream)));
  return ok();
}

lsf_status nf4dq_quantize(const float* w, int64_t n, int32_t blocksize, uint8_t* packed, float* absmax,
                          uint8_t* absq, float* scale2, lsf_stream stream) {
  if (blocksize != 64) return fail(LSF_ERR_SHAPE, "blocksize must be 64");
  if (n < 0 || n % 64) return fail(LSF_ERR_SHAPE, "n must be a non-negative multiple of 64 (got %lld)", (long long)n);
  if (n == 0) return ok();
  lsf_status s;
  if ((s = check_dev(w, "w")) || (s = check_dev(packed, "packed")) || (s = check_dev(absmax, "absmax"))) return s;
  if (absq == nullptr || scale2 == nullptr) return fail(LSF_ERR_INVALID_ARG, "absq or scale2 is NULL");
  if (!aligned(scale2, 8)) return fail(LSF_ERR_ALIGN, "scale2 must be 8-byte aligned");
  HIPCK(nf4_quantize_launch(w, n, packed, absmax, S(stream)));
  HIPCK(dq_encode_launch(absmax, n / 64, absq, scale2, S(stream)));
  return ok();
}

lsf_status nf4dq_dequantize(const uint8_t* packed, const uint8_t* absq, const float* scale2, int64_t n,
                            int32_t blocksize, uint16_t* out, lsf_stream stream) {
  if (blocksize != 64) return fail(LSF_ERR_SHAPE, "blocksize must be 64");
  if (n < 0 || n % 64) return fail(LSF_ERR_SHAPE, "n must be a non-negative multiple of 64 (got %lld)", (long long)n);
  if (n == 0) return ok();
  lsf_status s;
  if ((s = check_dev(packed, "packed")) || (s = check_dev(out, "out"))) return s;
  if (absq == nullptr || scale2 == nullptr) return fail(LSF_ERR_INVALID_ARG, "absq or scale2 is NULL");
  if (!aligned(scale2, 8)) return fail(LSF_ERR_ALIGN, "scale2 must be 8-byte aligned");
  HIPCK(nf4dq_dequantize_launch(packed, absq, scale2, n, out, S(stream)));
  return ok();
}

// ----------------------------------------------------------- single linear
// Largest tokens, n_out and n_in a single linear call accepts (keeps every
// size product far inside 64 bits).
constexpr int32_t kLinearMaxDim = 1 << 20;

size_t linear_workspace_bytes(int32_t tokens, int32_t n_out, int32_t n_in, int32_t rank) {
  if (tokens <= 0 || n_out <= 0 || n_in <= 0) return 0;
  if (tokens > kLinearMaxDim || n_out > kLinearMaxDim || n_in > kLinearMaxDim) return 0;
  const size_t T = tokens, r = rank > 0 ? rank : 1;
  const size_t N = n_out > n_in ? n_out : n_in;
  return 4 * 256 + (T * r * 4 + 255) / 256 * 256 * 2 + (size_t)8 * T * N * 4 +
         (lora_part_floats(tokens, 1, (int)r) * 4 + 255) / 256 * 256;
}

static lsf_status linear_common(const lsf_weight* w, int32_t format, int32_t n_out, int32_t n_in, const float* A,
                                const float* B, int32_t rank, int32_t tokens, void* ws, size_t ws_bytes,
                                bool check_ws = true) {
  if (w == nullptr) return fail(LSF_ERR_INVALID_ARG, "weight is NULL");
  if (format != LSF_FMT_NF4 && format != LSF_FMT_BF16 && format != LSF_FMT_NF4_DQ)
    return fail(LSF_ERR_INVALID_ARG, "unknown weight format %d", format);
  if (n_out <= 0 || n_out % 128) return fail(LSF_ERR_SHAPE, "n_out must be a positive multiple of 128");
  if (n_in <= 0 || n_in % 128) return fail(LSF_ERR_SHAPE, "n_in must be a positive multiple of 128");
  if (tokens < 1) return fail(LSF_ERR_SHAPE, "tokens must be >= 1");
  if (tokens > kLinearMaxDim || n_out > kLinearMaxDim || n_in > kLinearMaxDim)
    return fail(LSF_ERR_SHAPE, "tokens, n_out and n_in must be at most %d", (int)kLinearMaxDim);
  if (A != nullptr && (B == nullptr || !valid_rank(rank)))
    return fail(LSF_ERR_SHAPE, "adapter needs B and a rank in {4, 8, 16, 32, 64}");
  if (A != nullptr && !aligned(A, 16)) return fail(LSF_ERR_ALIGN, "A not 16-byte aligned");
  lsf_status s = check_weight(*w, format, "w");
  if (s) return s;
  if (check_ws && (ws == nullptr || ws_bytes < linear_workspace_bytes(tokens, n_out, n_in, rank)))
    return fail(LSF_ERR_WORKSPACE, "workspace too small (need %zu bytes)", linear_workspace_bytes(tokens, n_out, n_in, rank));
  return LSF_OK;
}

struct LinWs {
  float *U, *dU, *part, *lpart;
  size_t part_floats, lpart_floats;
};
static LinWs lin_ws(void* ws, int32_t tokens, int32_t n_out, int32_t n_in, int32_t rank) {
  uintptr_t p = ((uintptr_t)ws + 255) / 256 * 256;
  const size_t T = tokens, r = rank > 0 ? rank : 1;
  LinWs l;
  l.U = (float*)p;
  p += (T * r * 4 + 255) / 256 * 256;
  l.dU = (float*)p;
  p += (T * r * 4 + 255) / 256 * 256;
  l.part = (float*)p;
  l.part_floats = (size_t)8 * T * (n_out > n_in ? n_out : n_in);
  p += (l.part_floats * 4 + 255) / 256 * 256;
  l.lpart = (float*)p;
  l.lpart_floats = lora_part_floats(tokens, 1, (int)r);
  return l;
}

// The forward of one NF4 linear on workspace ws (validated by the caller).
static lsf_status linear_fwd_impl(const lsf_weight* w, int32_t format, int32_t n_out, int32_t n_in, const float* A,
                                  const float* B, int32_t rank, float scale, const uint16_t* x, int32_t tokens,
                                  uint16_t* y, void* ws, lsf_stream stream) {
  const LinWs l = lin_ws(ws, tokens, n_out, n_in, rank);
  GemmArgs g;
  g.M = tokens; g.N = n_out; g.K = n_in; g.A = x; g.lda = n_in; g.W = weight_ref(*w, format, n_in);
  if (A != nullptr) {
    LoraDown d;
    d.M = tokens; d.K = n_in; d.X = x; d.ldx = n_in; d.nsec = 1; d.r = rank; d.mat[0] = A; d.scale = 1.0f;
    d.U = l.U; d.ldu = rank; d.part = l.lpart; d.part_floats = l.lpart_floats;
    HIPCK(lora_down(d, S(stream)));
    g.ext.kx = rank; g.ext.u = l.U; g.ext.ldu = rank; g.ext.uscale = scale; g.ext.nsec = 1; g.ext.r = rank;
    g.ext.mat[0] = B; g.ext.row_off[1] = n_out;
  }
  EpiArgs e; e.kind = EPI_BF16; e.C = y; e.ldc = n_out;
  HIPCK(run_gemm(false, g, e, l.part, l.part_floats, S(stream)));
  return ok();
}

lsf_status linear_fwd(const lsf_weight* w, int32_t format, int32_t n_out, int32_t n_in, const float* A, const float* B,
                      int32_t rank, float scale, const uint16_t* x, int32_t tokens, uint16_t* y, void* ws,
                      size_t ws_bytes, lsf_stream stream) {
  lsf_status s = linear_common(w, format, n_out, n_in, A, B, rank, tokens, ws, ws_bytes);
  if (s) return s;
  if ((s = check_dev(x, "x")) || (s = check_dev(y, "y"))) return s;
  return linear_fwd_impl(w, format, n_out, n_in, A, B, rank, scale, x, tokens, y, ws, stream);
}

size_t linear_noalloc_max_bytes(void) { return kNoallocScratchBytes; }

lsf_status linear_fwd_noalloc(const lsf_weight* w, int32_t format, int32_t n_out, int32_t n_in, const float* A,
                              const float* B, int32_t rank, float scale, const uint16_t* x, int32_t tokens,
                              uint16_t* y, lsf_stream stream) {
  const size_t need = linear_workspace_bytes(tokens, n_out, n_in, rank);
  if (need > kNoallocScratchBytes)
    return fail(LSF_ERR_WORKSPACE,
                "linear_fwd_noalloc: %d tokens x %d x %d needs %zu bytes of scratch, more than the %zu the library "
                "holds; use linear_fwd with a workspace",
                (int)tokens, (int)n_out, (int)n_in, need, kNoallocScratchBytes);
  lsf_status s = linear_common(w, format, n_out, n_in, A, B, rank, tokens, nullptr, 0, /*check_ws=*/false);
  if (s) return s;
  if ((s = check_dev(x, "x")) || (s = check_dev(y, "y"))) return s;
  void* ws = nullptr;
  if ((s = noalloc_scratch(&ws))) return s;
  return linear_fwd_impl(w, format, n_out, n_in, A, B, rank, scale, x, tokens, y, ws, stream);
}

lsf_status linear_bwd(const lsf_weight* w, int32_t format, int32_t n_out, int32_t n_in, const float* A, const float* B,
                      int32_t rank, float scale, const uint16_t* x, const uint16_t* dy, int32_t tokens, uint16_t* dx,
                      float* dA, float* dB, void* ws, size_t ws_bytes, lsf_stream stream) {
  lsf_status s = linear_common(w, format, n_out, n_in, A, B, rank, tokens, ws, ws_bytes);
  if (s) return s;
  if ((s = check_dev(x, "x")) || (s = check_dev(dy, "dy")) || (s = check_dev(dx, "dx"))) return s;
  const LinWs l = lin_ws(ws, tokens, n_out, n_in, rank);
  GemmArgs g;
  g.M = tokens; g.N = n_in; g.K = n_out; g.A = dy; g.lda = n_out; g.W = weight_ref(*w, format, n_in);
  if (A != nullptr) {
    LoraDown d;
    d.M = tokens; d.K = n_in; d.X = x; d.ldx = n_in; d.nsec = 1; d.r = rank; d.mat[0] = A; d.scale = 1.0f;
    d.U = l.U; d.ldu = rank; d.part = l.lpart; d.part_floats = l.lpart_floats;
    HIPCK(lora_down(d, S(stream)));
    LoraDown b;
    b.M = tokens; b.K = n_out; b.X = dy; b.ldx = n_out; b.nsec = 1; b.r = rank; b.mat[0] = B; b.bside = true;
    b.ksec[0] = n_out; b.scale = scale; b.U = l.dU; b.ldu = rank; b.part = l.lpart; b.part_floats = l.lpart_floats;
    HIPCK(lora_down(b, S(stream)));
    g.ext.kx = rank; g.ext.u = l.dU; g.ext.ldu = rank; g.ext.nsec = 1; g.ext.r = rank; g.ext.mat[0] = A;
    g.ext.ldmat = n_in;
  }
  EpiArgs e; e.kind = EPI_BF16; e.C = dx; e.ldc = n_in;
  HIPCK(run_gemm(true, g, e, l.part, l.part_floats, S(stream)));
  if (A != nullptr) {
    LoraGradSec gs[2];
    int n = 0;
    if (dA) {
      LoraGradSec& ga = gs[n++];
      ga.P = l.dU; ga.ldp = rank; ga.Q = x; ga.ldq = n_in; ga.nq = n_in; ga.out = dA; ga.scale = 1.0f;
    }
    if (dB) {
      LoraGradSec& gb = gs[n++];
      gb.P = l.U; gb.ldp = rank; gb.Q = dy; gb.ldq = n_out; gb.nq = n_out; gb.out = dB; gb.transposed = true;
      gb.scale = scale;
    }
    HIPCK(lora_grad(gs, n, tokens, rank, l.part, l.part_floats, S(stream)));
  }
  return ok();
}

// ------------------------------------------------------------------ layer
size_t layer_workspace_bytes(const lsf_layer_cfg* cfg) {
  if (check_cfg(cfg) != LSF_OK) return 0;
  return LayerWs::bytes(*cfg);
}

lsf_status layer_fwd(const lsf_layer_cfg* cfg, const lsf_layer_weights* w, const lsf_layer_lora* lora,
                     const uint16_t* x, uint16_t* y, void* ws, size_t ws_bytes, lsf_stream stream) {
  lsf_status s;
  if ((s = check_cfg(cfg)) || (s = check_weights(w)) || (s = check_lora(lora))) return s;
  if ((s = check_dev(x, "x")) || (s = check_dev(y, "y"))) return s;
  if (ws == nullptr || ws_bytes < LayerWs::bytes(*cfg))
    return fail(LSF_ERR_WORKSPACE, "workspace too small (need %zu bytes)", LayerWs::bytes(*cfg));
  const LayerWs l = LayerWs::carve(*cfg, ws);
  HIPCK(layer_forward(*cfg, *w, lora, x, y, l, false, false, S(stream)));
  return ok();
}

lsf_status layer_bwd(const lsf_layer_cfg* cfg, const lsf_layer_weights* w, const lsf_layer_lora* lora,
                     const uint16_t* x, const uint16_t* dy, uint16_t* dx, void* ws, size_t ws_bytes,
                     lsf_stream stream) {
  lsf_status s;
  if ((s = check_cfg(cfg)) || (s = check_weights(w)) || (s = check_lora(lora))) return s;
  if ((s = check_dev(x, "x")) || (s = check_dev(dy, "dy")) || (s = check_dev(dx, "dx"))) return s;
  if (ws == nullptr || ws_bytes < LayerWs::bytes(*cfg))
    return fail(LSF_ERR_WORKSPACE, "workspace too small (need %zu bytes)", LayerWs::bytes(*cfg));
  const LayerWs l = LayerWs::carve(*cfg, ws);
  HIPCK(layer_backward(*cfg, *w, lora, x, dy, dx, l, false, S(stream)));
  return ok();
}

lsf_status layer_blob_layout(const lsf_layer_cfg* cfg, int32_t format, lsf_blob_layout* out) {
  lsf_status s;
  if ((s = check_cfg(cfg))) return s;
  if (out == nullptr) return fail(LSF_ERR_INVALID_ARG, "out is NULL");
  if (format != LSF_FMT_NF4 && format != LSF_FMT_BF16 && format != LSF_FMT_NF4_DQ)
    return fail(LSF_ERR_INVALID_ARG, "unknown weight format %d", format);
  const Blob b = blob_layout(*cfg, format);
  for (int i = 0; i < 10; ++i) out->off[i] = b.off[i];
  out->bytes = b.bytes;
  out->stride = b.stride;
  return ok();
}

lsf_status layer_weights_from_blob(const lsf_layer_cfg* cfg, int32_t format, const void* blob,
                                   lsf_layer_weights* out) {
  lsf_status s;
  if ((s = check_cfg(cfg))) return s;
  if (out == nullptr || blob == nullptr) return fail(LSF_ERR_INVALID_ARG, "blob or out is NULL");
  if (!aligned(blob, 256)) return fail(LSF_ERR_ALIGN, "blob must be 256-byte aligned");
  weights_from_blob(*cfg, format, blob, out);
  return ok();
}

}  // extern "C"

// ============================================================ the streamer
namespace {

// Timing events: created on demand, returned to a free list once harvested.
struct EventPool {
  std::vector<hipEvent_t> all, free;
  hipEvent_t get() {
    if (!free.empty()) {
      hipEvent_t e = free.back();
      free.pop_back();
      return e;
    }
    // Timing-only events: no system-scope fence (no cache writeback and
    // invalidate on record), so measuring does not slow the work measured.
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    all.push_back(e);
    return e;
  }
  void put(hipEvent_t e) { free.push_back(e); }
};

using EvPairs = std::vector<std::pair<hipEvent_t, hipEvent_t>>;

// Add the durations of the recorded pairs that have completed (all of them,
// waiting, when `wait`), recycle their events, keep the rest.  Pairs of one
// list complete in order (they sit on one stream).
hipError_t harvest(EventPool& pool, EvPairs& v, double& ms_sum, int64_t* count, bool wait) {
  size_t done = 0;
  for (; done < v.size(); ++done) {
    if (wait) {
      hipError_t e = hipEventSynchronize(v[done].second);
      if (e != hipSuccess) return e;
    } else if (hipEventQuery(v[done].second) != hipSuccess) {
      (void)hipGetLastError();  // clear the not-ready status
      break;
    }
    float ms = 0.0f;
    hipError_t e = hipEventElapsedTime(&ms, v[done].first, v[done].second);
    if (e != hipSuccess) return e;
    ms_sum += ms;
    if (count) ++*count;
    pool.put(v[done].first);
    pool.put(v[done].second);
  }
  v.erase(v.begin(), v.begin() + done);
  return hipSuccess;
}

// Brackets the big kernels of every layer call with events (LSF_STACK_TIMING).
struct KernelProbe : Probe {
  EventPool* pool = nullptr;
  uint32_t mask = 0;  // bit k: kernel class k is timed
  hipEvent_t open[LSF_K_COUNT] = {};
  EvPairs ev[LSF_K_COUNT];
  hipError_t begin(int kind, hipStream_t s) override {
    if (!((mask >> kind) & 1u)) return hipSuccess;
    open[kind] = pool->get();
    if (open[kind] == nullptr) return hipErrorOutOfMemory;
    return hipEventRecord(open[kind], s);
  }
  hipError_t end(int kind, hipStream_t s) override {
    if (!((mask >> kind) & 1u)) return hipSuccess;
    hipEvent_t e = pool->get();
    if (e == nullptr) return hipErrorOutOfMemory;
    hipError_t r = hipEventRecord(e, s);
    ev[kind].emplace_back(open[kind], e);
    return r;
  }
};

}  // namespace

struct lsf_stack {
  lsf_layer_cfg cfg;
  lsf_stack_desc d;
  Blob blob;
  hipEvent_t ready[2], freed[2];
  bool used[2];
  int slot_layer[2];
  // A second compute stream for accumulated steps: micro-batches alternate
  // between the caller's compute stream and this one within each layer visit
  // (fork and join events around the visit; gorder[m & 1][k] orders the k-th
  // gradient accumulation of micro-batch m before that of m + 1).
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // A second copy stream: each layer copy from a page-locked store goes out as
  // two halves, the second on this stream, forked from and joined back to the
  // caller's copy stream by events (unless LSF_STACK_ONE_COPY_STREAM).
  hipStream_t copy2 = nullptr;
  hipEvent_t cfork = nullptr, cjoin = nullptr;
  bool split_copies = false;
  // Without per-copy timing or a stress mode the two copy streams are not
  // linked: each waits for the buffer's release itself, and the second half's
  // arrival in buffer b is ready2[b], which the compute stream waits for too
  // (two_ready[b]: the last copy into buffer b went out that way).
  hipEvent_t ready2[2] = {};
  bool two_ready[2] = {};
  hipEvent_t gorder[2][4] = {};
  // timing (LSF_STACK_TIMING), accumulated until stack_reset_stats
  EventPool events;
  KernelProbe probe;
  EvPairs copy_ev, wait_ev;
  lsf_stack_stats stats;  // counters; the *_ms fields accumulate harvested durations
};

namespace {

hipEvent_t timing_event(lsf_stack* st) { return st->events.get(); }

hipError_t harvest_all(lsf_stack* st, bool wait) {
  hipError_t e;
  if ((e = harvest(st->events, st->copy_ev, st->stats.copy_ms, nullptr, wait)) != hipSuccess) return e;
  if ((e = harvest(st->events, st->wait_ev, st->stats.wait_ms, nullptr, wait)) != hipSuccess) return e;
  for (int k = 0; k < LSF_K_COUNT; ++k)
    if ((e = harvest(st->events, st->probe.ev[k], st->stats.kernel_ms[k], &st->stats.kernel_launches[k], wait)) !=
        hipSuccess)
      return e;
  return hipSuccess;
}

// Sleeps of the copy-delay stress mode (about 0.2 ms in all).
constexpr int kDebugDelayIters = 64;

// Make layer j resident in buffer b: copy unless the buffer already holds it.
lsf_status acquire(lsf_stack* st, int j, int b, bool allow_reuse) {
  if (allow_reuse && st->slot_layer[b] == j) return LSF_OK;
  hipStream_t cs = S(st->d.copy);
  if (st->used[b]) HIPCK(hipStreamWaitEvent(cs, st->freed[b], 0));
  // Stress modes: between the release and the copy the buffer holds NaN
  // bytes, and the copy starts late.
  if (st->d.flags & LSF_STACK_DEBUG_POISON) HIPCK(fill_pattern(st->d.dev_buf[b], (int64_t)st->blob.bytes, ~0u, cs));
  if (st->d.flags & LSF_STACK_DEBUG_COPY_DELAY) HIPCK(delay(kDebugDelayIters, cs));
  const bool timing = st->d.flags & LSF_STACK_TIMING;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (timing) {
    e0 = timing_event(st);
    e1 = timing_event(st);
    if (!e0 || !e1) return fail(LSF_ERR_HIP, "hipEventCreate failed");
    HIPCK(hipEventRecord(e0, cs));
  }
  const char* src = static_cast<const char*>(st->d.host_store) + (uint64_t)j * st->d.blob_stride;
  if (st->split_copies) {
    // Two halves on two copy streams, so two copy engines share the layer:
    // measured on MI355X, a single engine's layer copies settle for runs of
    // dozens of copies at one of a few slower rates (2.42, 3.06, 3.38 ms
    // instead of 2.17 per 8B-shaped layer) that two engines do not show
    // (streamed 512-token step 148.6 -> 138.1 ms, replayed outside the stack).
    // With per-copy timing or a stress mode the second stream starts after
    // everything before it on this one (the buffer's release, the stress
    // modes) and this one waits for it before the buffer is marked ready, so
    // one pair of timing events brackets the whole layer; otherwise both
    // streams wait for the release and the compute stream for both halves.
    const uint64_t half = st->blob.bytes / 2 / 4096 * 4096;
    char* dst = static_cast<char*>(st->d.dev_buf[b]);
    const bool linked = timing || (st->d.flags & (LSF_STACK_DEBUG_POISON | LSF_STACK_DEBUG_COPY_DELAY));
    if (linked) {
      HIPCK(hipEventRecord(st->cfork, cs));
      HIPCK(hipStreamWaitEvent(st->copy2, st->cfork, 0));
    } else if (st->used[b]) {
      // Each stream waits for the release on its own, so the wait that
      // separates one stream's copies overlaps the other stream's copy.
      HIPCK(hipStreamWaitEvent(st->copy2, st->freed[b], 0));
    }
    HIPCK(hipMemcpyAsync(dst, src, half, hipMemcpyHostToDevice, cs));
    HIPCK(hipMemcpyAsync(dst + half, src + half, st->blob.bytes - half, hipMemcpyHostToDevice, st->copy2));
    if (linked) {
      HIPCK(hipEventRecord(st->cjoin, st->copy2));
      HIPCK(hipStreamWaitEvent(cs, st->cjoin, 0));
    } else {
      HIPCK(hipEventRecord(st->ready2[b], st->copy2));
    }
    st->two_ready[b] = !linked;
  } else {
    HIPCK(hipMemcpyAsync(st->d.dev_buf[b], src, st->blob.bytes, hipMemcpyHostToDevice, cs));
  }
  if (timing) {
    HIPCK(hipEventRecord(e1, cs));
    st->copy_ev.emplace_back(e0, e1);
  }
  HIPCK(hipEventRecord(st->ready[b], cs));
  st->slot_layer[b] = j;
  st->stats.copies += 1;
  st->stats.bytes += (int64_t)st->blob.bytes;
  return LSF_OK;
}

// Order the compute stream after the copy into buffer b.
lsf_status wait_ready(lsf_stack* st, int b) {
  hipStream_t cs = S(st->d.compute);
  const bool timing = st->d.flags & LSF_STACK_TIMING;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (timing) {
    e0 = timing_event(st);
    e1 = timing_event(st);
    if (!e0 || !e1) return fail(LSF_ERR_HIP, "hipEventCreate failed");
    HIPCK(hipEventRecord(e0, cs));
  }
  HIPCK(hipStreamWaitEvent(cs, st->ready[b], 0));
  if (st->two_ready[b]) HIPCK(hipStreamWaitEvent(cs, st->ready2[b], 0));
  if (timing) {
    HIPCK(hipEventRecord(e1, cs));
    st->wait_ev.emplace_back(e0, e1);
  }
  return LSF_OK;
}

struct StackWs {
  LayerWs layer;
  LayerWs layer2;  // the second stream's layer workspace (accumulated steps)
  uint16_t *hN, *dhN, *dlog, *dx[2], *rx[2];
  float *rstdN, *row_loss, *part, *lse, *lp, *coef;
  size_t part_floats;
  uint16_t* dx_more;  // micro-batches 1.. of an accumulated step: two [T, H] each
  char* uarena;       // every layer's LoRA activations, per micro-batch (LayerWs::u_bytes each)
  int n_layers;
};

size_t head_part_floats(const lsf_layer_cfg& c) { return (size_t)8 * c.batch * c.seq * c.hidden; }

size_t stack_ws_bytes(const lsf_layer_cfg& c, int V) {
  const size_t T = (size_t)c.batch * c.seq, H = c.hidden;
  size_t b = LayerWs::bytes(c);
  b += al256(T * H * 2) * 6;  // hN, dhN, dx[0], dx[1], rx[0], rx[1]
  b += al256(T * (size_t)V * 2);
  b += al256(T * 4) * 3;      // rstdN, row_loss, lse
  b += al256((size_t)c.batch * 8) + al256((size_t)c.batch * 4);  // lp (policy, reference), coef
  b += al256(head_part_floats(c) * 4);
  return b + 512;
}

// With n micro-batches per walk, each keeps its own pair of gradient buffers
// between the head and the backward walk; and every layer keeps the LoRA
// activations U its forward computed, per micro-batch, for the recompute in
// the backward walk (which then reuses them instead of recomputing them).
size_t stack_accum_ws_bytes(const lsf_layer_cfg& c, int V, int L, int n) {
  const size_t T = (size_t)c.batch * c.seq, H = c.hidden;
  return stack_ws_bytes(c, V) + 256 + (size_t)(n - 1) * 2 * al256(T * H * 2) + 256 +
         (size_t)L * n * LayerWs::u_bytes(c) + (n > 1 ? 256 + al256(LayerWs::bytes(c)) : 0);
}

StackWs carve_stack(const lsf_layer_cfg& c, int V, int L, int n, void* base) {
  const size_t T = (size_t)c.batch * c.seq, H = c.hidden;
  StackWs w;
  w.layer = LayerWs::carve(c, base);
  uintptr_t p = ((uintptr_t)base + LayerWs::bytes(c) + 255) / 256 * 256;
  auto take = [&](size_t n) {
    void* r = (void*)p;
    p += al256(n);
    return r;
  };
  w.hN = (uint16_t*)take(T * H * 2);
  w.dhN = (uint16_t*)take(T * H * 2);
  w.dx[0] = (uint16_t*)take(T * H * 2);
  w.dx[1] = (uint16_t*)take(T * H * 2);
  w.rx[0] = (uint16_t*)take(T * H * 2);
  w.rx[1] = (uint16_t*)take(T * H * 2);
  w.dlog = (uint16_t*)take(T * (size_t)V * 2);
  w.rstdN = (float*)take(T * 4);
  w.row_loss = (float*)take(T * 4);
  w.lse = (float*)take(T * 4);
  w.lp = (float*)take((size_t)c.batch * 8);
  w.coef = (float*)take((size_t)c.batch * 4);
  w.part_floats = head_part_floats(c);
  w.part = (float*)take(w.part_floats * 4);
  w.dx_more = (uint16_t*)((p + 255) / 256 * 256);
  const uintptr_t ua = (uintptr_t)w.dx_more + (size_t)(n - 1) * 2 * al256(T * H * 2);
  w.uarena = (char*)((ua + 255) / 256 * 256);
  w.n_layers = L;
  w.layer2 = w.layer;
  if (n > 1) {
    const uintptr_t l2 = (uintptr_t)w.uarena + (size_t)L * n * LayerWs::u_bytes(c);
    w.layer2 = LayerWs::carve(c, (void*)((l2 + 255) / 256 * 256));
    w.layer2.rope = w.layer.rope;  // one RoPE table, built once per step, read by both
  }
  return w;
}

// Gradient buffer k (0, 1) of micro-batch m.
uint16_t* dx_buf(const StackWs& w, const lsf_layer_cfg& c, int m, int k) {
  if (m == 0) return w.dx[k];
  const size_t TH = al256((size_t)c.batch * c.seq * c.hidden * 2);
  return reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(w.dx_more) + ((size_t)(m - 1) * 2 + k) * TH);
}

// One walk over the stack: layers 0..L-1 (forward) or L-1..0.  Layer j
// computes from buffer j % 2; once it is done the buffer is released and the
// layer two further along is copied into it.  The first two layers of the walk
// are taken as the buffers hold them when allow_reuse is set (the frozen store
// never changes, so a buffer that holds layer j holds the right bytes).
template <class Fn>
lsf_status walk_layers(lsf_stack* st, bool resident, bool forward, bool allow_reuse, Fn&& fn) {
  const int L = st->d.n_layers;
  const int first = forward ? 0 : L - 1, dir = forward ? 1 : -1;
  hipStream_t cs = S(st->d.compute);
  lsf_status s;
  if (!resident) {
    if ((s = acquire(st, first, first & 1, allow_reuse))) return s;
    if (L > 1 && (s = acquire(st, first + dir, (first + dir) & 1, allow_reuse))) return s;
  }
  for (int n = 0; n < L; ++n) {
    const int j = first + n * dir, b = j & 1;
    if (!resident && (s = wait_ready(st, b))) return s;
    const void* blob = resident ? static_cast<const char*>(st->d.resident_store) + (uint64_t)j * st->d.blob_stride
                                : st->d.dev_buf[b];
    lsf_layer_weights lw;
    weights_from_blob(st->cfg, st->d.format, blob, &lw);
    HIPCK(fn(j, lw));
    if (!resident) {
      HIPCK(hipEventRecord(st->freed[b], cs));
      st->used[b] = true;
      const int nx = j + 2 * dir;
      if (nx >= 0 && nx < L && (s = acquire(st, nx, b, false))) return s;
    }
  }
  return LSF_OK;
}

// Final RMSNorm of x (into hN, rstdN) and the fp32 logits through lm_head.
hipError_t head_logits(lsf_stack* st, const lsf_stack_io* io, const StackWs& w, const uint16_t* x, bool timing) {
  const lsf_layer_cfg& c = st->cfg;
  const int T = c.batch * c.seq, H = c.hidden;
  hipStream_t cs = S(st->d.compute);
  hipError_t e;
  if ((e = rmsnorm_fwd(x, io->final_norm, T, H, c.rms_eps, w.hN, w.rstdN, cs)) != hipSuccess) return e;
  GemmArgs g;
  g.M = T; g.N = io->vocab; g.K = H; g.A = w.hN; g.lda = H;
  g.W.fmt = FMT_BF16; g.W.bf16 = io->lm_head; g.W.ld = H;
  EpiArgs ep; ep.kind = EPI_F32; ep.C = io->logits; ep.ldc = io->vocab;
  if (timing && (e = st->probe.begin(LSF_K_HEAD_FWD, cs)) != hipSuccess) return e;
  if ((e = gemm_nt(g, ep, cs)) != hipSuccess) return e;
  if (timing && (e = st->probe.end(LSF_K_HEAD_FWD, cs)) != hipSuccess) return e;
  return hipSuccess;
}

// dlogits (bf16, in w.dlog) back through lm_head and the final RMSNorm of x.
hipError_t head_backward(lsf_stack* st, const lsf_stack_io* io, const StackWs& w, const uint16_t* x, uint16_t* dx,
                         bool timing) {
  const lsf_layer_cfg& c = st->cfg;
  const int T = c.batch * c.seq, H = c.hidden;
  hipStream_t cs = S(st->d.compute);
  hipError_t e;
  GemmArgs g;
  g.M = T; g.N = H; g.K = io->vocab; g.A = w.dlog; g.lda = io->vocab;
  g.W.fmt = FMT_BF16; g.W.bf16 = io->lm_head; g.W.ld = H;
  EpiArgs ep; ep.kind = EPI_BF16; ep.C = w.dhN; ep.ldc = H;
  if (timing && (e = st->probe.begin(LSF_K_HEAD_BWD, cs)) != hipSuccess) return e;
  if ((e = run_gemm(true, g, ep, w.part, w.part_floats, cs)) != hipSuccess) return e;
  if (timing && (e = st->probe.end(LSF_K_HEAD_BWD, cs)) != hipSuccess) return e;
  return rmsnorm_bwd(w.dhN, x, io->final_norm, w.rstdN, nullptr, T, H, dx, cs);
}

// n micro-batches of SFT (dpo == NULL; io[0..n-1]) or one DPO micro-batch
// with the adapters-off reference (n == 1).  Every layer visit serves all n
// micro-batches in turn, so the stack is read once per direction however
// many micro-batches there are; each layer's gradients receive the
// micro-batches' contributions in the order 0, 1, ..., n-1.
lsf_status run_step(lsf_stack* st, const lsf_stack_io* io_all, int n_micro, const lsf_dpo_io* dpo) {
  if (st == nullptr || io_all == nullptr) return fail(LSF_ERR_INVALID_ARG, "stack or io is NULL");
  if (n_micro < 1) return fail(LSF_ERR_INVALID_ARG, "n_micro must be >= 1 (got %d)", n_micro);
  if (dpo != nullptr && n_micro != 1) return fail(LSF_ERR_INVALID_ARG, "DPO takes one micro-batch per call");
  const lsf_stack_io* io = io_all;  // the shared fields come from io[0]
  const lsf_layer_cfg& c = st->cfg;
  const int L = st->d.n_layers;
  const int V = io->vocab;
  const int T = c.batch * c.seq, H = c.hidden;
  lsf_status s;
  if (V < 128 || V % 128) return fail(LSF_ERR_SHAPE, "vocab must be a positive multiple of 128 (got %d)", V);
  if ((s = check_dev(io->embed, "embed")) || (s = check_dev(io->final_norm, "final_norm")) ||
      (s = check_dev(io->lm_head, "lm_head")))
    return s;
  for (int m = 0; m < n_micro; ++m) {
    if ((s = check_dev(io_all[m].ids, "ids")) || (s = check_dev(io_all[m].ckpt, "ckpt")) ||
        (s = check_dev(io_all[m].logits, "logits")) || (s = check_dev(io_all[m].loss, "loss")))
      return s;
    if (io_all[m].id_status != nullptr && !aligned(io_all[m].id_status, 4))
      return fail(LSF_ERR_ALIGN, "id_status is not 4-byte aligned");
  }
  if (io->lora == nullptr) return fail(LSF_ERR_INVALID_ARG, "lora array is NULL");
  for (int i = 0; i < L; ++i)
    if ((s = check_lora(&io->lora[i]))) return s;
  const bool resident = io->mode & LSF_MODE_RESIDENT;
  if (resident && st->d.resident_store == nullptr) return fail(LSF_ERR_INVALID_ARG, "RESIDENT mode needs a resident store");
  if (!resident && st->d.host_store == nullptr) return fail(LSF_ERR_INVALID_ARG, "STREAMED mode needs a host store");
  const size_t ws_need = stack_accum_ws_bytes(c, V, L, n_micro);
  if (io->ws == nullptr || io->ws_bytes < ws_need) return fail(LSF_ERR_WORKSPACE, "workspace too small (need %zu bytes)", ws_need);
  const bool keep = io->mode & LSF_MODE_KEEP_ACTIVATIONS;
  const size_t saved = LayerWs::saved_bytes(c);
  if (keep) {
    const size_t need = saved * L * (size_t)n_micro;
    if (io->act == nullptr || io->act_bytes < need)
      return fail(LSF_ERR_WORKSPACE, "activation arena too small (need %zu bytes)", need);
    if (!aligned(io->act, 256)) return fail(LSF_ERR_ALIGN, "activation arena must be 256-byte aligned");
  }
  if (dpo != nullptr) {
    if (c.batch < 2 || c.batch % 2)
      return fail(LSF_ERR_SHAPE, "DPO needs an even batch (chosen, then rejected sequences); got %d", c.batch);
    if (!(dpo->beta > 0.0f) || !std::isfinite(dpo->beta))
      return fail(LSF_ERR_INVALID_ARG, "DPO beta must be positive and finite");
    if (dpo->seq_logp != nullptr && !aligned(dpo->seq_logp, 4)) return fail(LSF_ERR_ALIGN, "seq_logp is not aligned");
  }

  hipStream_t cs = S(st->d.compute);
  StackWs w = carve_stack(c, V, L, n_micro, io->ws);
  const uint32_t all_classes = (1u << LSF_K_COUNT) - 1u;
  const uint32_t class_mask = (st->d.flags & (LSF_STACK_TIMING | LSF_STACK_KERNEL_TIMING))
                                  ? all_classes
                                  : (st->d.flags / LSF_STACK_TIME_KERNEL(0)) & all_classes;
  const bool timing = class_mask != 0;
  if (timing) {
    st->probe.mask = class_mask;
    st->probe.pool = &st->events;
    w.layer.probe = &st->probe;
    HIPCK(harvest_all(st, false));  // recycle the events of work that has finished
  }
  const size_t act = (size_t)T * H;
  st->stats.steps += n_micro;

  // Micro-batch m's descriptor: io[0] with m's own ids, checkpoints, logits,
  // loss and loss scale.
  auto io_of = [&](int m) {
    lsf_stack_io r = *io;
    r.ids = io_all[m].ids;
    r.ckpt = io_all[m].ckpt;
    r.logits = io_all[m].logits;
    r.loss = io_all[m].loss;
    r.loss_scale = io_all[m].loss_scale;
    return r;
  };

  // LSF_MODE_ZERO_GRADS: the backward of every enabled layer stores its dA, dB
  // (overwrite) instead of adding to them; only gradients no backward will
  // write (forward-only calls, disabled layers) are zeroed here.
  // Gradient arrays shared between layers (tied adapters) accumulate over
  // the step, so they take the zero-then-add path.  With several
  // micro-batches only the first one's backward overwrites.
  const bool zero_grads = (io->mode & LSF_MODE_ZERO_GRADS) != 0;
  bool overwrite = zero_grads && (io->mode & LSF_MODE_FWD_ONLY) == 0;
  if (overwrite) {
    std::vector<const float*> seen;
    for (int i = 0; i < L; ++i) {
      const lsf_layer_lora* li = &io->lora[i];
      const lsf_lora_proj* p = &li->q;
      for (int k = 0; k < 7; ++k) {
        if (p[k].A == nullptr) continue;
        if (p[k].dA) seen.push_back(p[k].dA);
        if (p[k].dB) seen.push_back(p[k].dB);
      }
    }
    std::sort(seen.begin(), seen.end());
    overwrite = std::adjacent_find(seen.begin(), seen.end()) == seen.end();
  }
  if (zero_grads) {
    const int64_t Dq = (int64_t)c.n_heads * c.head_dim, Dk = (int64_t)c.n_kv_heads * c.head_dim;
    const int64_t in[7] = {c.hidden, c.hidden, c.hidden, Dq, c.hidden, c.hidden, c.intermediate};
    const int64_t outd[7] = {Dq, Dk, Dk, c.hidden, c.intermediate, c.intermediate, c.hidden};
    for (int i = 0; i < L; ++i) {
      if (overwrite && io->lora[i].enabled) continue;
      const lsf_lora_proj* p = &io->lora[i].q;
      for (int k = 0; k < 7; ++k) {
        if (p[k].A == nullptr) continue;
        if (p[k].dA) HIPCK(zero_f32(p[k].dA, (int64_t)c.rank * in[k], cs));
        if (p[k].dB) HIPCK(zero_f32(p[k].dB, (int64_t)c.rank * outd[k], cs));
      }
    }
  }

  HIPCK(rope_table(c.seq, c.head_dim, c.rope_theta, w.layer.rope, cs));
  for (int m = 0; m < n_micro; ++m)
    HIPCK(embed_gather(io_all[m].ids, io->embed, T, H, V, io_all[m].ckpt, io_all[m].id_status, cs));

  // With several micro-batches, recomputing backward and no per-kernel timing
  // (whose events time each launch alone), the odd ones run on the second
  // stream with their own layer workspace, so that two micro-batches' kernels
  // overlap (measured at 4 x 2048 tokens: 4.6% more tokens/s; with kept
  // activations 0.9% fewer, so that mode keeps one stream): within each
  // layer visit the second stream waits for everything before the visit on
  // the compute stream (fork), and the compute stream waits for the second
  // stream's work before the visit ends (join), so the buffer-free event and
  // the head see both.  Gradient accumulations keep the order 0, 1, ..., n-1
  // through the gorder events, so the bits are those of one stream.
  const bool two = n_micro > 1 && !keep && !(st->d.flags & (LSF_STACK_TIMING | LSF_STACK_KERNEL_TIMING));
  w.layer2.probe = w.layer.probe;
  auto stream_of = [&](int m) { return (two && (m & 1)) ? st->side : cs; };
  const LayerWs& lbase0 = w.layer;
  auto lbase = [&](int m) -> const LayerWs& { return (two && (m & 1)) ? w.layer2 : lbase0; };
  auto fork_side = [&]() -> hipError_t {
    hipError_t e;
    if (!two) return hipSuccess;
    if ((e = hipEventRecord(st->fork, cs)) != hipSuccess) return e;
    return hipStreamWaitEvent(st->side, st->fork, 0);
  };
  auto join_side = [&]() -> hipError_t {
    hipError_t e;
    if (!two) return hipSuccess;
    if ((e = hipEventRecord(st->join, st->side)) != hipSuccess) return e;
    return hipStreamWaitEvent(cs, st->join, 0);
  };
  // Layer i's saved intermediates for micro-batch m (LSF_MODE_KEEP_ACTIVATIONS).
  auto kept = [&](int m, int i) {
    return lbase(m).with_saved(c, static_cast<char*>(io->act) + ((size_t)m * L + i) * saved);
  };
  // Otherwise the workspace with layer i's LoRA activations for micro-batch m
  // in their own slot, so that the backward walk's recompute finds them.
  const size_t ub = LayerWs::u_bytes(c);
  auto with_u = [&](int m, int i) { return lbase(m).with_u(c, w.uarena + ((size_t)m * L + i) * ub); };
  // Policy forward of layer i for micro-batch m: ckpt[i] -> ckpt[i+1] (kept for the backward).
  auto policy_fwd = [&](int m, int i, const lsf_layer_weights& lw) {
    uint16_t* ck = io_all[m].ckpt;
    return layer_forward(c, lw, &io->lora[i], ck + (size_t)i * act, ck + (size_t)(i + 1) * act,
                         keep ? kept(m, i) : with_u(m, i), keep, true, stream_of(m));
  };
  auto all_fwd = [&](int i, const lsf_layer_weights& lw) {
    hipError_t e;
    if ((e = fork_side()) != hipSuccess) return e;
    for (int m = 0; m < n_micro; ++m)
      if ((e = policy_fwd(m, i, lw)) != hipSuccess) return e;
    return join_side();
  };
  // Reference (adapters off) forward of layer i, through the rx ping-pong:
  // input rx[i % 2] (the embeddings for layer 0), output rx[(i + 1) % 2].
  auto reference_fwd = [&](int i, const lsf_layer_weights& lw) {
    const uint16_t* x = i == 0 ? io->ckpt : w.rx[i & 1];
    return layer_forward(c, lw, nullptr, x, w.rx[(i + 1) & 1], w.layer, false, true, cs);
  };
  float* lp_pi = w.lp;
  float* lp_ref = w.lp + c.batch;
  auto reference_head = [&]() -> hipError_t {
    hipError_t e;
    if ((e = head_logits(st, io, w, w.rx[L & 1], timing)) != hipSuccess) return e;
    return seq_logprobs(io->logits, io->ids, c.batch, c.seq, V, w.lse, w.row_loss, lp_ref, cs);
  };

  // ---- forward.  A full step ends with layers 1 and 0 in buffers 1 and 0,
  // which is what the next forward reads first: they are reused unless
  // LSF_STACK_NO_TURN_REUSE asks for every copy.
  const bool reuse = !(st->d.flags & LSF_STACK_NO_TURN_REUSE);
  if (dpo != nullptr && !dpo->fused_reference) {
    if ((s = walk_layers(st, resident, true, reuse, reference_fwd))) return s;
    HIPCK(reference_head());
  }
  if (dpo != nullptr && dpo->fused_reference) {
    auto both = [&](int i, const lsf_layer_weights& lw) {
      const hipError_t e = policy_fwd(0, i, lw);
      return e != hipSuccess ? e : reference_fwd(i, lw);
    };
    if ((s = walk_layers(st, resident, true, reuse, both))) return s;
    HIPCK(reference_head());
  } else if ((s = walk_layers(st, resident, true, reuse, all_fwd))) {
    return s;
  }

  // ---- heads: final norm, lm_head, loss and dlogits, lm_head input gradient
  const bool fwd_only = io->mode & LSF_MODE_FWD_ONLY;
  for (int m = 0; m < n_micro; ++m) {
    const lsf_stack_io iom = io_of(m);
    const uint16_t* xL = iom.ckpt + (size_t)L * act;
    HIPCK(head_logits(st, &iom, w, xL, timing));
    if (dpo == nullptr) {
      HIPCK(cross_entropy(iom.logits, iom.ids, c.batch, c.seq, V, iom.loss_scale, w.dlog, w.row_loss, iom.loss, cs));
    } else {
      HIPCK(seq_logprobs(iom.logits, iom.ids, c.batch, c.seq, V, w.lse, w.row_loss, lp_pi, cs));
      HIPCK(dpo_head_grad(iom.logits, iom.ids, w.lse, lp_pi, lp_ref, c.batch, c.seq, V, dpo->beta, iom.loss_scale,
                          w.coef, iom.loss, fwd_only ? nullptr : w.dlog, cs));
      if (dpo->seq_logp != nullptr)
        HIPCK(hipMemcpyAsync(dpo->seq_logp, w.lp, (size_t)c.batch * 8, hipMemcpyDeviceToDevice, cs));
    }
    if (!fwd_only) HIPCK(head_backward(st, &iom, w, xL, dx_buf(w, c, m, L & 1), timing));
  }
  if (fwd_only) return ok();

  // ---- backward: layers L-1 .. 0, each read again and recomputed
  auto all_bwd = [&](int j, const lsf_layer_weights& lw) {
    hipError_t e;
    if ((e = fork_side()) != hipSuccess) return e;
    for (int m = 0; m < n_micro; ++m) {
      LayerWs lws = keep ? kept(m, j) : with_u(m, j);
      lws.u_ready = !keep;  // the recompute reuses the forward's LoRA activations
      lws.grads_overwrite = overwrite && m == 0;
      if (two)
        for (int k = 0; k < 4; ++k) {
          lws.grad_after[k] = m > 0 ? st->gorder[(m - 1) & 1][k] : nullptr;
          lws.grad_done[k] = m + 1 < n_micro ? st->gorder[m & 1][k] : nullptr;
        }
      e = layer_backward(c, lw, &io->lora[j], io_all[m].ckpt + (size_t)j * act, dx_buf(w, c, m, (j + 1) & 1),
                         dx_buf(w, c, m, j & 1), lws, true, stream_of(m), !keep);
      if (e != hipSuccess) return e;
    }
    return join_side();
  };
  if ((s = walk_layers(st, resident, false, reuse, all_bwd))) return s;
  return ok();
}

}  // namespace

extern "C" {

lsf_status stack_create(const lsf_layer_cfg* cfg, const lsf_stack_desc* desc, lsf_stack** out) {
  lsf_status s;
  if ((s = check_cfg(cfg))) return s;
  if (desc == nullptr || out == nullptr) return fail(LSF_ERR_INVALID_ARG, "desc or out is NULL");
  *out = nullptr;
  if (desc->n_layers < 1) return fail(LSF_ERR_INVALID_ARG, "n_layers must be >= 1");
  {
    const uint32_t known = LSF_STACK_ALLOW_PAGEABLE | LSF_STACK_NO_TURN_REUSE | LSF_STACK_TIMING |
                           LSF_STACK_KERNEL_TIMING | LSF_STACK_SOURCE_DISK | LSF_STACK_DEBUG_POISON |
                           LSF_STACK_DEBUG_COPY_DELAY | LSF_STACK_ONE_COPY_STREAM |
                           LSF_STACK_TIME_KERNEL(0) * ((1u << LSF_K_COUNT) - 1u);
    if (desc->flags & ~known) return fail(LSF_ERR_INVALID_ARG, "unknown stack flags 0x%x", desc->flags & ~known);
    if (desc->flags & LSF_STACK_SOURCE_DISK)
      return fail(LSF_ERR_UNSUPPORTED, "a disk-backed store (the NVMe tier) is not built; load it into RAM");
  }
  if (desc->format != LSF_FMT_NF4 && desc->format != LSF_FMT_BF16 && desc->format != LSF_FMT_NF4_DQ)
    return fail(LSF_ERR_INVALID_ARG, "unknown weight format %d", desc->format);
  const Blob b = blob_layout(*cfg, desc->format);
  if (desc->blob_stride < b.bytes || desc->blob_stride % 256)
    return fail(LSF_ERR_SHAPE, "blob_stride %llu must be >= %llu and a multiple of 256",
                (unsigned long long)desc->blob_stride, (unsigned long long)b.bytes);
  if (desc->dev_buf[0] == nullptr || desc->dev_buf[1] == nullptr)
    return fail(LSF_ERR_INVALID_ARG, "two device buffers are required");
  if (!aligned(desc->dev_buf[0], 256) || !aligned(desc->dev_buf[1], 256))
    return fail(LSF_ERR_ALIGN, "device buffers must be 256-byte aligned");
  if (desc->resident_store != nullptr && !aligned(desc->resident_store, 256))
    return fail(LSF_ERR_ALIGN, "resident store must be 256-byte aligned");
  bool pinned = false;
  if (desc->host_store == nullptr) {
    if (desc->resident_store == nullptr) return fail(LSF_ERR_INVALID_ARG, "no host store and no resident store");
  } else {
    hipPointerAttribute_t attr;
    const hipError_t e = hipPointerGetAttributes(&attr, desc->host_store);
    pinned = (e == hipSuccess) && (attr.type == hipMemoryTypeHost);
    if (e != hipSuccess) (void)hipGetLastError();  // clear the sticky error of a pageable query
    if (!pinned && !(desc->flags & LSF_STACK_ALLOW_PAGEABLE))
      return fail(LSF_ERR_NOT_PINNED, "host store is not page-locked (pass LSF_STACK_ALLOW_PAGEABLE to accept it)");
  }
  lsf_stack* st = new (std::nothrow) lsf_stack();
  if (st == nullptr) return fail(LSF_ERR_INVALID_ARG, "out of host memory");
  st->cfg = *cfg;
  st->d = *desc;
  st->blob = b;
  for (int i = 0; i < 2; ++i) {
    st->used[i] = false;
    st->slot_layer[i] = -1;
    if (hipEventCreateWithFlags(&st->ready[i], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&st->freed[i], hipEventDisableTiming) != hipSuccess) {
      delete st;
      return fail(LSF_ERR_HIP, "hipEventCreateWithFlags failed");
    }
  }
  std::memset(&st->stats, 0, sizeof(st->stats));
  bool evs_ok = hipStreamCreateWithFlags(&st->side, hipStreamNonBlocking) == hipSuccess &&
                hipEventCreateWithFlags(&st->fork, hipEventDisableTiming) == hipSuccess &&
                hipEventCreateWithFlags(&st->join, hipEventDisableTiming) == hipSuccess;
  st->split_copies = pinned && !(desc->flags & LSF_STACK_ONE_COPY_STREAM);
  if (evs_ok && st->split_copies)
    evs_ok = hipStreamCreateWithFlags(&st->copy2, hipStreamNonBlocking) == hipSuccess &&
             hipEventCreateWithFlags(&st->cfork, hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&st->cjoin, hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&st->ready2[0], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&st->ready2[1], hipEventDisableTiming) == hipSuccess;
  for (int i = 0; i < 2 && evs_ok; ++i)
    for (int k = 0; k < 4 && evs_ok; ++k)
      evs_ok = hipEventCreateWithFlags(&st->gorder[i][k], hipEventDisableTiming) == hipSuccess;
  if (!evs_ok) {
    (void)stack_destroy(st);
    return fail(LSF_ERR_HIP, "creating the second compute or copy stream or their events failed");
  }
  *out = st;
  return ok();
}

lsf_status stack_destroy(lsf_stack* st) {
  if (st == nullptr) return ok();
  for (int i = 0; i < 2; ++i) {
    (void)hipEventDestroy(st->ready[i]);
    (void)hipEventDestroy(st->freed[i]);
  }
  (void)harvest_all(st, true);  // no event may be destroyed while still pending
  for (hipEvent_t e : st->events.all) (void)hipEventDestroy(e);
  if (st->side) (void)hipStreamSynchronize(st->side);
  if (st->copy2) (void)hipStreamSynchronize(st->copy2);
  if (st->fork) (void)hipEventDestroy(st->fork);
  if (st->join) (void)hipEventDestroy(st->join);
  if (st->cfork) (void)hipEventDestroy(st->cfork);
  if (st->cjoin) (void)hipEventDestroy(st->cjoin);
  for (int i = 0; i < 2; ++i)
    if (st->ready2[i]) (void)hipEventDestroy(st->ready2[i]);
  for (int i = 0; i < 2; ++i)
    for (int k = 0; k < 4; ++k)
      if (st->gorder[i][k]) (void)hipEventDestroy(st->gorder[i][k]);
  if (st->side) (void)hipStreamDestroy(st->side);
  if (st->copy2) (void)hipStreamDestroy(st->copy2);
  delete st;
  return ok();
}

size_t stack_activation_bytes(const lsf_layer_cfg* cfg, int32_t n_layers) {
  if (check_cfg(cfg) != LSF_OK || n_layers <= 0) return 0;
  return LayerWs::saved_bytes(*cfg) * (size_t)n_layers;
}

size_t stack_workspace_bytes(const lsf_layer_cfg* cfg, int32_t vocab, int32_t n_layers) {
  if (check_cfg(cfg) != LSF_OK || vocab <= 0 || n_layers < 1) return 0;
  return stack_accum_ws_bytes(*cfg, vocab, n_layers, 1);
}

size_t stack_accum_workspace_bytes(const lsf_layer_cfg* cfg, int32_t vocab, int32_t n_layers, int32_t n_micro) {
  if (check_cfg(cfg) != LSF_OK || vocab <= 0 || n_layers < 1 || n_micro < 1) return 0;
  return stack_accum_ws_bytes(*cfg, vocab, n_layers, n_micro);
}

lsf_status stream_stack_step(lsf_stack* st, const lsf_stack_io* io) {
  if (io == nullptr) return fail(LSF_ERR_INVALID_ARG, "stack or io is NULL");
  return run_step(st, io, 1, nullptr);
}

lsf_status stream_stack_accum_step(lsf_stack* st, const lsf_stack_io* io, int32_t n_micro) {
  if (io == nullptr) return fail(LSF_ERR_INVALID_ARG, "stack or io is NULL");
  return run_step(st, io, n_micro, nullptr);
}

lsf_status dpo_stack_step(lsf_stack* st, const lsf_dpo_io* io) {
  if (io == nullptr) return fail(LSF_ERR_INVALID_ARG, "stack or io is NULL");
  return run_step(st, &io->base, 1, io);
}

size_t adamw_workspace_bytes(void) { return adamw_ws_bytes(); }

namespace {
lsf_status check_adamw_cfg(const lsf_adamw_cfg* cfg, int64_t n) {
  if (cfg == nullptr) return fail(LSF_ERR_INVALID_ARG, "cfg is NULL");
  if (n < 0) return fail(LSF_ERR_INVALID_ARG, "n must be >= 0");
  const lsf_adamw_cfg& c = *cfg;
  if (!(c.lr >= 0.0f) || !std::isfinite(c.lr)) return fail(LSF_ERR_INVALID_ARG, "lr must be finite and >= 0");
  if (!(c.beta1 >= 0.0f && c.beta1 < 1.0f) || !(c.beta2 >= 0.0f && c.beta2 < 1.0f))
    return fail(LSF_ERR_INVALID_ARG, "beta1 and beta2 must lie in [0, 1)");
  if (!(c.eps > 0.0f) || !std::isfinite(c.eps)) return fail(LSF_ERR_INVALID_ARG, "eps must be positive");
  if (!(c.weight_decay >= 0.0f) || !std::isfinite(c.weight_decay))
    return fail(LSF_ERR_INVALID_ARG, "weight_decay must be finite and >= 0");
  if (!(c.max_grad_norm >= 0.0f) || !std::isfinite(c.max_grad_norm))
    return fail(LSF_ERR_INVALID_ARG, "max_grad_norm must be finite and >= 0");
  if (c.step < 1) return fail(LSF_ERR_INVALID_ARG, "step must be >= 1 (got %d)", c.step);
  return LSF_OK;
}
}  // namespace

lsf_status adamw_step(float* param, const float* grad, float* m, float* v, int64_t n, const lsf_adamw_cfg* cfg,
                      float* grad_norm, void* ws, size_t ws_bytes, lsf_stream stream) {
  lsf_status cs = check_adamw_cfg(cfg, n);
  if (cs != LSF_OK) return cs;
  const lsf_adamw_cfg& c = *cfg;
  if (n == 0) return ok();
  lsf_status s;
  if ((s = check_dev(param, "param")) || (s = check_dev(grad, "grad")) || (s = check_dev(m, "m")) ||
      (s = check_dev(v, "v")))
    return s;
  if (grad_norm != nullptr && !aligned(grad_norm, 4)) return fail(LSF_ERR_ALIGN, "grad_norm is not aligned");
  if (ws == nullptr || ws_bytes < adamw_ws_bytes() || !aligned(ws, 16))
    return fail(LSF_ERR_WORKSPACE, "workspace too small or unaligned (need %zu bytes)", adamw_ws_bytes());
  HIPCK(adamw_update(param, grad, m, v, n, c.lr, c.beta1, c.beta2, c.eps, c.weight_decay, c.max_grad_norm, c.step,
                     grad_norm, static_cast<float*>(ws), S(stream)));
  return ok();
}

int64_t adamw8_state_blocks(int64_t n) { return n > 0 ? adamw8_blocks(n) : 0; }
size_t adamw8_workspace_bytes(void) { return adamw8_ws_bytes(); }

lsf_status adamw8_step(float* param, const float* grad, int8_t* m_codes, uint8_t* v_codes, float* m_absmax,
                       float* v_absmax, int64_t n, const lsf_adamw_cfg* cfg, float* grad_norm, void* ws,
                       size_t ws_bytes, lsf_stream stream) {
  lsf_status cs = check_adamw_cfg(cfg, n);
  if (cs != LSF_OK) return cs;
  const lsf_adamw_cfg& c = *cfg;
  if (n == 0) return ok();
  lsf_status s;
  if ((s = check_dev(param, "param")) || (s = check_dev(grad, "grad"))) return s;
  if (m_codes == nullptr || v_codes == nullptr || m_absmax == nullptr || v_absmax == nullptr)
    return fail(LSF_ERR_INVALID_ARG, "state pointer is NULL");
  if (!aligned(m_codes, 8) || !aligned(v_codes, 8) || !aligned(m_absmax, 4) || !aligned(v_absmax, 4))
    return fail(LSF_ERR_ALIGN, "codes must be 8-byte and absmax 4-byte aligned");
  if (grad_norm != nullptr && !aligned(grad_norm, 4)) return fail(LSF_ERR_ALIGN, "grad_norm is not aligned");
  if (ws == nullptr || ws_bytes < adamw8_ws_bytes() || !aligned(ws, 16))
    return fail(LSF_ERR_WORKSPACE, "workspace too small or unaligned (need %zu bytes)", adamw8_ws_bytes());
  HIPCK(adamw8_update(param, grad, m_codes, v_codes, m_absmax, v_absmax, n, c.lr, c.beta1, c.beta2, c.eps,
                      c.weight_decay, c.max_grad_norm, c.step, grad_norm, static_cast<float*>(ws), S(stream)));
  return ok();
}

lsf_status stack_stats(lsf_stack* st, lsf_stack_stats* out) {
  if (st == nullptr || out == nullptr) return fail(LSF_ERR_INVALID_ARG, "stack or out is NULL");
  HIPCK(harvest_all(st, true));
  *out = st->stats;
  return ok();
}

lsf_status stack_reset_stats(lsf_stack* st) {
  if (st == nullptr) return fail(LSF_ERR_INVALID_ARG, "stack is NULL");
  HIPCK(harvest_all(st, true));  // pending events must finish before they are recycled
  std::memset(&st->stats, 0, sizeof(st->stats));
  return ok();
}

}  // extern "C"
