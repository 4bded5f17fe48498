/*
 * lsf.h - C ABI of the layer-streamed frozen-base NF4 + LoRA training library
 * (liblsf.so, built for AMD Instinct MI355X / gfx950).
 *
 * The method: LoRA adapters are trained over a frozen base whose decoder
 * layers stay in page-locked host memory, NF4-quantised, and reach the GPU one
 * layer at a time through two fixed device buffers; each layer is read twice
 * per micro-batch (forward, then a recomputed forward inside the backward
 * walk), and the input gradient still flows through the frozen weight.
 *
 * Pages cited below (by address and section title):
 *   [NEWS]     aizxs.com/ai-learning/13312.html - section "the principle:
 *              frozen layers streamed through the card".
 *   [README]   feinterview.poetries.top/ai-monitor/news/makazhanalpamys-soup -
 *              the project README: the layer-streaming paragraph, the soup.yaml
 *              block, the preference-loss paragraph, the preprint/v3 paragraph.
 *   [REVIEW]   repodaily.xyz/zh/projects/2026-08-17/soup/ - section
 *              "architecture: how layer streaming fits in 4 GB".
 *   [BLOG]     agentlenshq.com/zh-TW/blogs/2a477d3d-636b-4b92-baad-75af680d87d9
 *              - sections "layer streaming: implementation and memory
 *              efficiency" and "DPO support / reference model without memory".
 *   [TUTORIAL] alphalab.site/soup-layer-streaming - section "the four-stage
 *              data path" items 1 (NF4), 2 (pinned memory), 3 (forward +
 *              backward), 4 (RAM-first); section "step 2: one YAML".
 *
 * Conventions shared by every entry point
 *   - Every call returns lsf_status.  Nothing aborts, and no C++ exception
 *     crosses the ABI.  On failure lsf_last_error() returns a message (owned
 *     by the library, valid until the calling thread's next call).
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed validation enqueues nothing.
 *   - Pointers are borrowed, never freed or retained beyond the call, except
 *     for the stack handle, which keeps the pointers given to stack_create
 *     until stack_destroy.  Device pointers must come from device memory
 *     (hipMalloc / torch); "host" pointers are host memory.
 *   - No call allocates device memory: scratch space is a caller-provided
 *     workspace whose size a *_workspace_bytes() query gives, except for
 *     linear_fwd_noalloc, whose scratch is a fixed device array the library
 *     holds from load to process end.
 *   - Work is enqueued on the given HIP stream (lsf_stream is a hipStream_t;
 *     NULL is the null stream) and the call returns without waiting; faults
 *     surface at the caller's next synchronisation.
 *   - bf16 tensors are passed as uint16_t bit patterns; matrices are
 *     row-major.  Weights are [out, in] as in nn.Linear; LoRA A is [r, in]
 *     and B is [out, r], fp32.
 *   - Results are deterministic: no floating-point atomics, and the same
 *     inputs give the same bits wherever the weights live.
 */
#ifndef LSF_H
#define LSF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every function below is exported from liblsf.so; nothing else is. */
#if defined(__GNUC__)
#define LSF_API __attribute__((visibility("default")))
#else
#define LSF_API
#endif

typedef void* lsf_stream; /* hipStream_t */

typedef enum {
  LSF_OK = 0,
  LSF_ERR_INVALID_ARG = 1, /* NULL where a pointer is required, bad flag, bad count */
  LSF_ERR_SHAPE = 2,       /* a size the kernels do not support (see each call) */
  LSF_ERR_ALIGN = 3,       /* a pointer or stride below the required alignment */
  LSF_ERR_NOT_PINNED = 4,  /* host store is not page-locked (and pageable not allowed) */
  LSF_ERR_UNSUPPORTED = 5, /* a feature the pages describe that this library does not build */
  LSF_ERR_HIP = 6,         /* the HIP runtime reported an error (message has hipGetErrorString) */
  LSF_ERR_WORKSPACE = 7    /* workspace smaller than the matching *_workspace_bytes() */
} lsf_status;

/* Message of the calling thread's last failed call ("" if none). */
LSF_API const char* lsf_last_error(void);
/* Library version string. */
LSF_API const char* lsf_version(void);

/* Diagnostics: the kernel that runs wide forward NF4 GEMMs (fp32 absmax,
 * whole 256-column tiles, K >= 2048, at least 256 tokens, no split-K, and
 * either N >= 16384 or at least 192 tiles of 256 x 256: the gate|up
 * projection of an 8B-shaped layer, and q|k|v from 2048 tokens on, with the
 * bf16 or SwiGLU epilogue).  enable = 1 (the default) or 512: the ping-pong
 * kernel on 512 x 128 tiles; 256: the same kernel on 256 x 256 tiles; 0: the
 * general 128-column kernel.  All compute the same contraction in the same
 * order and give bitwise-identical results; the switch lets tests and
 * profiles compare them.  Process-wide; GEMMs already enqueued are not
 * affected.  Other values: LSF_ERR_INVALID_ARG. */
LSF_API lsf_status gemm_set_wide(int32_t enable);
/* Diagnostics: number of GEMMs launched on the wide kernel so far in this
 * process (lets a test confirm which kernel ran). */
LSF_API int64_t gemm_wide_launch_count(void);

/* ------------------------------------------------------------------ NF4 --
 * [TUTORIAL] item 1: the decoder's Linear weights are stored offline as QLoRA
 * NF4; compute runs in higher precision.  Blocks of `blocksize` (= 64)
 * consecutive elements of the flattened weight, one fp32 absmax each.
 * code = number of fp32 midpoints of the 16 NF4 levels strictly below
 * w / absmax (IEEE fp32 division); all-zero block -> absmax 0, codes 7.
 * Packing: byte j = code[2j] << 4 | code[2j+1].
 */

/* Quantise n fp32 values (device) into packed codes (device, n/2 bytes) and
 * absmax (device, n/blocksize floats).  n % 64 == 0 and blocksize == 64, else
 * LSF_ERR_SHAPE.  Pointers must be 16-byte aligned (LSF_ERR_ALIGN). */
LSF_API lsf_status nf4_quantize(const float* w, int64_t n, int32_t blocksize,
                        uint8_t* packed, float* absmax, lsf_stream stream);

/* Dequantise: out[i] = bf16_rne(level[code[i]] * absmax[i / blocksize]).
 * Same shape rules as nf4_quantize; out is device bf16 [n]. */
LSF_API lsf_status nf4_dequantize(const uint8_t* packed, const float* absmax, int64_t n,
                          int32_t blocksize, uint16_t* out, lsf_stream stream);

/* Double-quantised NF4 ([REVIEW]: the pages' 113 MB per 8B layer fits NF4
 * codes with an 8-bit absmax; the pages give no second-level code, so a plain
 * affine one is used).  Codes are chosen exactly as nf4_quantize (against the
 * fp32 absmax, also written to `absmax`, device fp32 [n/64]); then per group
 * of 256 consecutive blocks offset = min, scale = (max - min) / 255 and each
 * absmax becomes code = clamp(rint((a - offset) / scale), 0, 255) (ties to
 * even; 0 when scale is 0) in `absq` (device uint8 [n/64]); `scale2` (device
 * fp32 [2 * ceil(n/64/256)], 8-byte aligned) holds (scale, offset) pairs.
 * The absmax used to dequantise is fp32(fp32(code * scale) + offset). */
LSF_API lsf_status nf4dq_quantize(const float* w, int64_t n, int32_t blocksize, uint8_t* packed,
                                  float* absmax, uint8_t* absq, float* scale2, lsf_stream stream);
/* out[i] = bf16_rne(level[code[i]] * absmax'(block)), absmax' as above. */
LSF_API lsf_status nf4dq_dequantize(const uint8_t* packed, const uint8_t* absq, const float* scale2,
                                    int64_t n, int32_t blocksize, uint16_t* out, lsf_stream stream);

/* --------------------------------------------------------- layer config -- */

typedef struct {
  int32_t hidden;       /* H; multiple of 128 */
  int32_t intermediate; /* I; multiple of 128 */
  int32_t n_heads;      /* query heads */
  int32_t n_kv_heads;   /* key/value heads; n_heads % n_kv_heads == 0 */
  int32_t head_dim;     /* 128 (the attention kernels are built for it) */
  int32_t rank;         /* LoRA rank r of every adapter: 4, 8, 16, 32 or 64 (else LSF_ERR_SHAPE) */
  float lora_scale;     /* s = alpha / r */
  float rope_theta;     /* RoPE base, e.g. 500000 */
  float rms_eps;        /* RMSNorm epsilon, e.g. 1e-5 */
  int32_t batch;        /* sequences per micro-batch (>= 1) */
  int32_t seq;          /* tokens per sequence (>= 1); positions restart at 0;
                           batch * seq <= 2^20 (else LSF_ERR_SHAPE) */
} lsf_layer_cfg;

/* Weight storage formats of the frozen projections. */
#define LSF_FMT_NF4 0    /* data = packed codes [out*in/2], scale = fp32 absmax [out*in/64] */
#define LSF_FMT_BF16 1   /* data = bf16 [out*in], scale = NULL (unquantised streamed base) */
#define LSF_FMT_NF4_DQ 2 /* data = packed codes, scale = uint8 absmax codes [out*in/64],
                            scale2 = fp32 (scale, offset) pairs [ceil(out*in/64/256)]
                            (see nf4dq_quantize) */

typedef struct {
  const void* data;
  const void* scale;
  const float* scale2;
} lsf_weight;

/* The frozen weights of one decoder layer.  q|k|v and gate|up are row
 * concatenations: qkv is [(nq + 2 nkv) * d, H] with q rows first, gate_up is
 * [2 I, H] with gate rows first. */
typedef struct {
  int32_t format; /* LSF_FMT_* */
  lsf_weight qkv, o, gate_up, down;
  const uint16_t* norm1; /* bf16 [H], input RMSNorm weight */
  const uint16_t* norm2; /* bf16 [H], post-attention RMSNorm weight */
} lsf_layer_weights;

/* One projection's adapter.  A == NULL means no adapter on that projection
 * (the pages' narrow q/v-only setting, [TUTORIAL] "step 2").  dA/dB receive
 * gradients, accumulated (+=) in fp32; they may be NULL in forward-only use. */
typedef struct {
  const float* A; /* [r, in] */
  const float* B; /* [out, r] */
  float* dA;      /* [r, in] */
  float* dB;      /* [out, r] */
} lsf_lora_proj;

typedef struct {
  lsf_lora_proj q, k, v, o, gate, up, down;
  int32_t enabled; /* 0: adapters switched off for this call (the frozen base
                      alone, as the DPO reference pass of [README]/[BLOG]) */
} lsf_layer_lora;

/* -------------------------------------------------------- one NF4 linear --
 * y = x W^T + s (x A^T) B^T   (LoRA on a frozen NF4 weight; [NEWS], [TUTORIAL]
 * item 3).  x: device bf16 [tokens, n_in]; y: device bf16 [tokens, n_out].
 * n_out % 128 == 0, n_in % 128 == 0, 1 <= tokens; tokens, n_out and n_in at
 * most 2^20 (larger sizes: LSF_ERR_SHAPE, and a size query of 0); with an adapter, rank is one
 * of 4, 8, 16, 32, 64 (else LSF_ERR_SHAPE).  A/B may be NULL (no adapter).
 * ws: device workspace of at least linear_workspace_bytes() bytes. */
LSF_API size_t linear_workspace_bytes(int32_t tokens, int32_t n_out, int32_t n_in, int32_t rank);
LSF_API lsf_status linear_fwd(const lsf_weight* w, int32_t format, int32_t n_out, int32_t n_in,
                      const float* A, const float* B, int32_t rank, float scale,
                      const uint16_t* x, int32_t tokens, uint16_t* y,
                      void* ws, size_t ws_bytes, lsf_stream stream);
/* linear_fwd for callers that cannot allocate device memory or hand over a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels, launch shapes and bits as linear_fwd,
 * with the scratch in a library-owned device array of
 * linear_noalloc_max_bytes() bytes (32 MiB) on each GPU, kept until the
 * process ends.  Sizes whose linear_workspace_bytes() exceed that give
 * LSF_ERR_WORKSPACE and enqueue nothing.  The call allocates nothing.  All
 * calls on one GPU share its array: calls that overlap in time on one GPU
 * (on different streams, or from different threads) race and must be ordered
 * by the caller.  Other arguments and errors as linear_fwd. */
LSF_API size_t linear_noalloc_max_bytes(void);
LSF_API lsf_status linear_fwd_noalloc(const lsf_weight* w, int32_t format, int32_t n_out, int32_t n_in,
                                      const float* A, const float* B, int32_t rank, float scale,
                                      const uint16_t* x, int32_t tokens, uint16_t* y, lsf_stream stream);
/* Backward of linear_fwd: dx = dy W + s (dy B) A (the input gradient through the
 * frozen weight, [TUTORIAL] item 3); dA += s (dy B)^T x; dB += s dy^T (x A^T).
 * dx: device bf16 [tokens, n_in]. dA/dB accumulate. */
LSF_API lsf_status linear_bwd(const lsf_weight* w, int32_t format, int32_t n_out, int32_t n_in,
                      const float* A, const float* B, int32_t rank, float scale,
                      const uint16_t* x, const uint16_t* dy, int32_t tokens, uint16_t* dx,
                      float* dA, float* dB, void* ws, size_t ws_bytes, lsf_stream stream);

/* ------------------------------------------------------ one decoder layer --
 * Llama-style layer: h1 = rmsnorm(x); q,k,v = LoRA-linear(h1) with rotate-half
 * RoPE on q,k; causal GQA attention; x2 = x + LoRA-linear_o(attn);
 * h2 = rmsnorm(x2); a = silu(gate(h2)) * up(h2); y = x2 + down(a).
 * x, y: device bf16 [batch*seq, H].  Requires hidden, intermediate and
 * (nq + 2 nkv) * d to be multiples of 128 and head_dim == 128. */
LSF_API size_t layer_workspace_bytes(const lsf_layer_cfg* cfg);
LSF_API lsf_status layer_fwd(const lsf_layer_cfg* cfg, const lsf_layer_weights* w,
                     const lsf_layer_lora* lora, const uint16_t* x, uint16_t* y,
                     void* ws, size_t ws_bytes, lsf_stream stream);
/* Recomputes the forward from the checkpoint x (the layer input), then walks
 * it backward ([TUTORIAL] item 3: each layer is read a second time and
 * dL/dx = W^T dL/dy still needs the frozen weight).  dy, dx: device bf16
 * [batch*seq, H]; dA/dB of every adapted projection accumulate (+=). */
LSF_API lsf_status layer_bwd(const lsf_layer_cfg* cfg, const lsf_layer_weights* w,
                     const lsf_layer_lora* lora, const uint16_t* x, const uint16_t* dy,
                     uint16_t* dx, void* ws, size_t ws_bytes, lsf_stream stream);

/* ------------------------------------------------------------ host store --
 * One contiguous blob per layer ([REVIEW]: the frozen store is pinned in RAM
 * and cut into per-layer slices).  NF4 blob, in order, each section 256-byte
 * aligned: packed qkv, packed o, packed gate_up, packed down, absmax qkv,
 * absmax o, absmax gate_up, absmax down, norm1 (bf16), norm2 (bf16).
 * layer_blob_layout fills the byte offsets of those ten sections and the blob
 * size; the stride between blobs in a store is the size rounded up to 4096. */
typedef struct {
  uint64_t off[10];
  uint64_t bytes;  /* size of one blob */
  uint64_t stride; /* bytes rounded up to 4096 */
} lsf_blob_layout;
LSF_API lsf_status layer_blob_layout(const lsf_layer_cfg* cfg, int32_t format, lsf_blob_layout* out);
/* Point a lsf_layer_weights at a blob (host or device address). */
LSF_API lsf_status layer_weights_from_blob(const lsf_layer_cfg* cfg, int32_t format, const void* blob,
                                   lsf_layer_weights* out);

/* --------------------------------------------------- the streamed stack --
 * [REVIEW], [BLOG], [TUTORIAL] item 2: two fixed device buffers; while layer i
 * computes from one, a dedicated copy stream loads layer i+1 into the other
 * from page-locked host memory with asynchronous host-to-device copies (two
 * halves on two copy streams, see LSF_STACK_ONE_COPY_STREAM).
 * Order of one micro-batch: forward layers 0..L-1, head and loss, backward
 * layers L-1..0 (each re-read and recomputed; [TUTORIAL] item 3).  The two
 * layers still resident at the turn are reused, and so are layers 0 and 1,
 * which a full step leaves in the buffers for the next step's forward, unless
 * LSF_STACK_NO_TURN_REUSE is given: 2L-2 copies for the first micro-batch,
 * 2L-4 for each later one, instead of 2L.  Reuse assumes what the frozen base
 * is: the host store does not change while the stack exists.
 */
typedef struct lsf_stack lsf_stack;

#define LSF_STACK_ALLOW_PAGEABLE 0x1u /* accept a pageable host store (slow fallback, [TUTORIAL] item 2) */
#define LSF_STACK_NO_TURN_REUSE 0x2u  /* copy every layer twice per micro-batch */
#define LSF_STACK_TIMING 0x4u         /* record copy, compute-wait and kernel events for stack_stats */
#define LSF_STACK_KERNEL_TIMING 0x8u  /* record only the kernel events (leaves the copy stream untouched) */
/* The host store is a file on disk ([TUTORIAL] item 4: the NVMe tier used when
 * RAM is short).  Not built: stack_create returns LSF_ERR_UNSUPPORTED. */
#define LSF_STACK_SOURCE_DISK 0x10u
/* Event-ordering stress modes ([BLOG] "correctness and bit-exactness": the
 * streamed result must not depend on timing).  Both act on the copy stream
 * only, between its wait for a buffer's release and the copy into it, and
 * change no result of a correctly ordered stack:
 *   DEBUG_POISON: fill the released buffer with 0xFF bytes (NaN as bf16 and
 *   fp32) before the copy, so compute that read the buffer outside its
 *   ready/freed window would see NaN;
 *   DEBUG_COPY_DELAY: run a fixed-length delay kernel (a bounded number of
 *   s_sleep iterations, about 0.2 ms) before the copy, so a compute stream
 *   that did not wait for the copy would read the previous contents. */
#define LSF_STACK_DEBUG_POISON 0x20u
#define LSF_STACK_DEBUG_COPY_DELAY 0x40u
/* Copy each layer from a page-locked store as one transfer on the copy stream.
 * By default it goes out as two halves, the second on a copy stream the stack
 * owns, so that two copy engines share it; the bytes are the same either way.
 * Each copy stream waits for the buffer's release and the compute stream for
 * both halves; with LSF_STACK_TIMING or a stress mode the second stream is
 * instead forked from the first after the release (and the stress work) and
 * joined back before the layer is marked ready, so that one pair of events
 * times the whole layer copy. */
#define LSF_STACK_ONE_COPY_STREAM 0x80u
/* Record only kernel class k (an LSF_K_* value; several may be or-ed), for a
 * measurement that must disturb the step as little as possible. */
#define LSF_STACK_TIME_KERNEL(k) (0x100u << (k))

typedef struct {
  int32_t n_layers;
  int32_t format;           /* LSF_FMT_* of every blob */
  uint64_t blob_stride;     /* bytes between blobs; >= layout.bytes, multiple of 256 */
  const void* host_store;   /* host memory holding n_layers blobs (page-locked) */
  void* dev_buf[2];         /* two device buffers of >= layout.bytes each, 256-B aligned */
  const void* resident_store; /* optional: device copy of the whole store (RESIDENT mode) */
  lsf_stream compute;       /* stream the layer kernels run on */
  lsf_stream copy;          /* dedicated stream for host-to-device layer copies */
  uint32_t flags;           /* LSF_STACK_* */
} lsf_stack_desc;
/* HIP runs a process's streams on a few hardware queues (GPU_MAX_HW_QUEUES,
 * four by default) and lets later streams share them.  Work queued on a
 * hardware queue runs in order, so a copy stream (the caller's, or the
 * stack's second one) that shares the compute stream's queue makes the layer
 * kernels wait for the copies: the step then takes the copies' time plus the
 * compute's instead of the larger of the two.  A stack uses the compute and
 * copy streams given here plus up to two of its own (the second copy stream,
 * and a second compute stream for several micro-batches); keep the process's
 * streams in use within the queue count, e.g. by giving every stack the same
 * copy stream. */

LSF_API lsf_status stack_create(const lsf_layer_cfg* cfg, const lsf_stack_desc* desc, lsf_stack** out);
LSF_API lsf_status stack_destroy(lsf_stack* st);

#define LSF_MODE_STREAMED 0x0u   /* weights come through the two buffers */
#define LSF_MODE_RESIDENT 0x1u   /* weights read in place from resident_store */
#define LSF_MODE_FWD_ONLY 0x2u   /* stop after the loss (no backward) */
#define LSF_MODE_ZERO_GRADS 0x4u /* zero every dA/dB before accumulating (the first write of each stores) */
/* Keep every layer's forward intermediates in io->act and skip the recompute
 * in the backward walk.  Each layer is still read twice (the input gradient
 * needs the frozen weight); the recompute is traded for
 * stack_activation_bytes() of device memory.  Same bits as the default. */
#define LSF_MODE_KEEP_ACTIVATIONS 0x8u

typedef struct {
  const int32_t* ids;          /* device [batch, seq] token ids in [0, vocab) */
  const uint16_t* embed;       /* device bf16 [vocab, H] (resident, frozen) */
  const uint16_t* final_norm;  /* device bf16 [H] */
  const uint16_t* lm_head;     /* device bf16 [vocab, H] (resident, frozen, untied) */
  int32_t vocab;               /* positive multiple of 128 */
  const lsf_layer_lora* lora;  /* host array [n_layers] of adapter descriptors */
  uint16_t* ckpt;              /* device bf16 [n_layers + 1, batch*seq, H]: layer inputs */
  float* logits;               /* device fp32 [batch*seq, vocab] */
  float* loss;                 /* device fp32 [1]: mean CE over batch*(seq-1) positions */
  void* ws;                    /* device workspace */
  size_t ws_bytes;             /* >= stack_workspace_bytes(cfg, vocab, n_layers) */
  float loss_scale;            /* multiplies dL/dlogits (e.g. 1/accumulation) */
  uint32_t mode;               /* LSF_MODE_* */
  void* act;                   /* LSF_MODE_KEEP_ACTIVATIONS: device, 256-B aligned; else ignored */
  size_t act_bytes;            /* >= stack_activation_bytes(cfg, n_layers) */
  /* Optional device int32 [1] (4-byte aligned) or NULL.  Token ids live on the
   * device, so they cannot be checked before the step is enqueued; instead the
   * step sets *id_status = 1 when any id of this micro-batch lies outside
   * [0, vocab), and never writes it otherwise (the caller zeroes it and reads
   * it after synchronising).  A bad id's embedding row is zero and a bad
   * next-token label leaves its position unlabelled (no loss term, zero
   * gradient row), so no memory outside the tables is read. */
  int32_t* id_status;
} lsf_stack_io;

/* Device workspace of one micro-batch's step over n_layers layers (it holds,
 * besides the layer and head scratch, every layer's LoRA activations from the
 * forward walk, which the backward walk's recompute reuses). */
LSF_API size_t stack_workspace_bytes(const lsf_layer_cfg* cfg, int32_t vocab, int32_t n_layers);
/* Device bytes LSF_MODE_KEEP_ACTIVATIONS needs for n_layers layers. */
LSF_API size_t stack_activation_bytes(const lsf_layer_cfg* cfg, int32_t n_layers);
/* One SFT micro-batch: embedding gather, streamed forward, final RMSNorm,
 * lm_head, cross-entropy over next-token labels, lm_head input gradient,
 * streamed recompute + backward, LoRA gradients accumulated. */
LSF_API lsf_status stream_stack_step(lsf_stack* st, const lsf_stack_io* io);

/* Gradient accumulation over n_micro SFT micro-batches ([TUTORIAL] "step 2"
 * configuration: accumulation 4) in one walk over the stack per direction:
 * every layer copied in serves the forward (then the backward) of micro-batch
 * 0, 1, ..., n_micro-1 before the next layer is read, so the stack is streamed
 * twice per optimizer step instead of twice per micro-batch.  io points to
 * n_micro descriptors; io[m] supplies micro-batch m's ids, ckpt, logits, loss
 * loss_scale and id_status (logits, loss and id_status may be shared), io[0] everything else
 * (embed, vocab, final_norm, lm_head, lora, ws, act, mode).  All n_micro
 * checkpoint arrays are live at once.  The result is that of n_micro
 * stream_stack_step calls on io[0], io[1], ... in turn with
 * LSF_MODE_ZERO_GRADS (if set) on the first only, bit for bit: each layer's
 * gradients receive the micro-batches' contributions in the same order.
 * With n_micro > 1 (recomputing backward, no per-kernel timing flag) the odd micro-batches run
 * on a second stream the stack owns, overlapping with the even ones within
 * each layer visit; every visit starts after the work already on the compute
 * stream and ends with the compute stream waiting for it, so to the caller the
 * step is ordered on the compute stream as before, with the same bits.
 * ws: at least stack_accum_workspace_bytes(cfg, vocab, n_layers, n_micro); act
 * (LSF_MODE_KEEP_ACTIVATIONS): n_micro * stack_activation_bytes(cfg, n_layers).
 * Errors: LSF_ERR_INVALID_ARG for n_micro < 1, plus those of stream_stack_step. */
LSF_API size_t stack_accum_workspace_bytes(const lsf_layer_cfg* cfg, int32_t vocab, int32_t n_layers,
                                           int32_t n_micro);
LSF_API lsf_status stream_stack_accum_step(lsf_stack* st, const lsf_stack_io* io, int32_t n_micro);

/* One DPO micro-batch ([README] paragraph on preference losses with layer
 * streaming; [BLOG] section on DPO support): the reference model is the same
 * frozen base with every adapter switched off, so it needs no second copy of
 * the weights.  The batch holds P = batch/2 chosen sequences, then the P
 * rejected ones (pair p = sequences p and P+p).  With l(s) the sum of the
 * next-token log-probabilities of sequence s,
 *   h_p = (l_pi(p) - l_ref(p)) - (l_pi(P+p) - l_ref(P+p)),
 *   loss = mean_p softplus(-beta h_p)   (written to base.loss, unscaled),
 * and only the adapters (policy) receive gradients, times base.loss_scale.
 * fused_reference = 1 runs the reference forward of layer i in the same visit
 * as the policy forward of layer i, so each layer is read once per forward
 * (2L copies per step, as for SFT); 0 runs a separate reference pass over the
 * stack first (3L copies).  Both give the same bits.  base.logits ends with the
 * policy logits; base.ckpt holds the policy's layer inputs.  seq_logp (may be
 * NULL): device fp32 [2, batch], policy log-probabilities then reference.
 * Errors: LSF_ERR_SHAPE for an odd batch, LSF_ERR_INVALID_ARG for beta <= 0
 * or non-finite, plus every error of stream_stack_step.  Workspace: the same
 * stack_workspace_bytes(cfg, vocab, n_layers). */
typedef struct {
  lsf_stack_io base;
  float beta;               /* DPO temperature, e.g. 0.1 */
  int32_t fused_reference;  /* 1: reference forward in the policy's layer visit */
  float* seq_logp;          /* optional device fp32 [2, batch] */
} lsf_dpo_io;

LSF_API lsf_status dpo_stack_step(lsf_stack* st, const lsf_dpo_io* io);

/* ------------------------------------------------------------ optimizer --
 * [TUTORIAL] "step 2: one YAML" trains the adapters with an Adam-family
 * optimizer with decoupled weight decay at lr 2e-4; [NEWS] keeps the adapters,
 * their gradients and the optimizer state on the GPU.  AdamW (fp32 state here;
 * adamw8_step below keeps the moments in 8 bits) over ONE flat fp32 array of n values:
 * a caller that lays every adapter A and B of the stack end to end (and their
 * gradients likewise) updates all of them with one call.  For step t >= 1:
 *   g <- g * min(1, max_grad_norm / (||g||_2 + 1e-6))   when max_grad_norm > 0
 *   p <- p - lr*weight_decay*p
 *   m <- beta1 m + (1 - beta1) g;   v <- beta2 v + (1 - beta2) g^2
 *   p <- p - lr/(1 - beta1^t) * m / (sqrt(v)/sqrt(1 - beta2^t) + eps)
 * The norm is summed in a fixed order (deterministic).  grad is not modified. */
typedef struct {
  float lr;             /* learning rate, >= 0 */
  float beta1, beta2;   /* in [0, 1), e.g. 0.9, 0.999 */
  float eps;            /* > 0, e.g. 1e-8 */
  float weight_decay;   /* decoupled decay, >= 0 (0 = none) */
  float max_grad_norm;  /* > 0: clip by the global L2 norm first; 0 = no clipping */
  int32_t step;         /* t >= 1: updates made so far, this one included */
} lsf_adamw_cfg;

/* Device workspace adamw_step needs (a few KiB, independent of n). */
LSF_API size_t adamw_workspace_bytes(void);
/* param, m, v: device fp32 [n], updated in place; grad: device fp32 [n].  All
 * four 16-byte aligned (LSF_ERR_ALIGN).  grad_norm (optional, device fp32 [1])
 * receives ||grad||_2 before clipping.  n >= 0 (0 enqueues nothing).  Bad
 * hyper-parameters give LSF_ERR_INVALID_ARG. */
LSF_API lsf_status adamw_step(float* param, const float* grad, float* m, float* v, int64_t n,
                              const lsf_adamw_cfg* cfg, float* grad_norm, void* ws, size_t ws_bytes,
                              lsf_stream stream);

/* [TUTORIAL] "step 2: one YAML" names the optimizer paged_adamw_8bit.  The
 * same AdamW update with the two moments stored between steps in 8 bits, as in
 * the published block-wise 8-bit optimizer method: blocks of 2048 consecutive
 * values, one fp32 absmax per block and moment, and each value stored as the
 * nearest entry (a tie to the smaller) of a fixed code after division by the
 * absmax.  Code values: 0 and +-(0.1 + 0.9 (j + 1) / 2^F) / 10^E, where E is
 * the number of zero bits after the sign, then an indicator bit, then F
 * fraction bits holding j; m uses 7 magnitude bits (F = 6 - E, 255 values,
 * stored as int8: the entry's position relative to 0 in the sorted code), v
 * uses 8 (F = 7 - E, 256 values, stored as uint8: the position in the sorted
 * code).  Each step dequantises, updates in fp32 exactly as adamw_step
 * (every operation rounded, no fused multiply-add; beta^t by repeated
 * multiplication), then re-quantises with the new block maxima.  Zeroed codes
 * and absmax are the zero state.  "Paged" (spilling state to host memory under
 * memory pressure) has no counterpart: the state is resident.
 * param, grad: device fp32 [n], 16-byte aligned; m_codes, v_codes: device [n],
 * 8-byte aligned; m_absmax, v_absmax: device fp32 [adamw8_state_blocks(n)];
 * all updated in place except grad.  grad_norm, cfg, ws and errors as
 * adamw_step (ws: adamw8_workspace_bytes()). */
LSF_API int64_t adamw8_state_blocks(int64_t n);
LSF_API size_t adamw8_workspace_bytes(void);
LSF_API lsf_status adamw8_step(float* param, const float* grad, int8_t* m_codes, uint8_t* v_codes,
                               float* m_absmax, float* v_absmax, int64_t n, const lsf_adamw_cfg* cfg,
                               float* grad_norm, void* ws, size_t ws_bytes, lsf_stream stream);

/* Kernel classes timed with HIP events under LSF_STACK_TIMING or
 * LSF_STACK_KERNEL_TIMING (index into
 * lsf_stack_stats.kernel_ms / kernel_launches).  A GEMM's time includes its
 * split-K reduction when it has one. */
enum {
  LSF_K_QKV_FWD = 0, LSF_K_O_FWD, LSF_K_GATEUP_FWD, LSF_K_DOWN_FWD, /* fused NF4 GEMMs, forward */
  LSF_K_QKV_BWD, LSF_K_O_BWD, LSF_K_GATEUP_BWD, LSF_K_DOWN_BWD,     /* fused NF4 GEMMs, input gradient */
  LSF_K_ATTN_FWD, LSF_K_ATTN_BWD, LSF_K_HEAD_FWD, LSF_K_HEAD_BWD,
  LSF_K_COUNT
};

typedef struct {
  int64_t steps;       /* micro-batches since create / reset (n_micro per stream_stack_accum_step) */
  int64_t copies;      /* host-to-device layer copies enqueued */
  int64_t bytes;       /* bytes those copies moved */
  double copy_ms;      /* summed copy durations (LSF_STACK_TIMING only) */
  double wait_ms;      /* summed compute-stream stalls on copies (LSF_STACK_TIMING only) */
  double kernel_ms[16];        /* summed durations per LSF_K_* class (either timing flag) */
  int64_t kernel_launches[16]; /* launches per class (either timing flag) */
} lsf_stack_stats;
/* Counters and event timings since the last reset (or create).  Waits for the
 * recorded events, so it synchronises with the work they bracket. */
LSF_API lsf_status stack_stats(lsf_stack* st, lsf_stack_stats* out);
/* Zero the counters and drop the recorded events. */
LSF_API lsf_status stack_reset_stats(lsf_stack* st);

#ifdef __cplusplus
}
#endif
#endif /* LSF_H */
