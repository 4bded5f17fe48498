"""ctypes binding of liblsf.so.

Argument marshalling only: every computation of the path runs in the HIP
library.  Tensors are torch tensors (PyTorch supplies device memory, pinned
host memory and streams); their data pointers are handed to the C ABI.
Non-OK statuses raise ``LsfError`` carrying ``lsf_last_error()``.

The library must have been built (``layer_streamed_frozen_amd.build``); if it
is missing, importing this module still works but every call raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# LSF_LIB names another build of the same library (the host-sanitizer build).
LIB_PATH = os.environ.get("LSF_LIB") or os.path.join(HERE, "liblsf.so")

LSF_OK, LSF_ERR_INVALID_ARG, LSF_ERR_SHAPE, LSF_ERR_ALIGN, LSF_ERR_NOT_PINNED, LSF_ERR_UNSUPPORTED, \
    LSF_ERR_HIP, LSF_ERR_WORKSPACE = range(8)
STATUS_NAMES = ["LSF_OK", "LSF_ERR_INVALID_ARG", "LSF_ERR_SHAPE", "LSF_ERR_ALIGN", "LSF_ERR_NOT_PINNED",
                "LSF_ERR_UNSUPPORTED", "LSF_ERR_HIP", "LSF_ERR_WORKSPACE"]

FMT_NF4, FMT_BF16, FMT_NF4_DQ = 0, 1, 2

STACK_ALLOW_PAGEABLE, STACK_NO_TURN_REUSE, STACK_TIMING, STACK_KERNEL_TIMING, STACK_SOURCE_DISK = 0x1, 0x2, 0x4, 0x8, 0x10
STACK_DEBUG_POISON, STACK_DEBUG_COPY_DELAY, STACK_ONE_COPY_STREAM = 0x20, 0x40, 0x80


def STACK_TIME_KERNEL(k):
    """Flag that times only kernel class k (an index into KERNELS)."""
    return 0x100 << k
MODE_STREAMED, MODE_RESIDENT, MODE_FWD_ONLY, MODE_ZERO_GRADS, MODE_KEEP_ACTIVATIONS = 0x0, 0x1, 0x2, 0x4, 0x8

c_void_p, c_int32, c_int64, c_uint32, c_uint64, c_float, c_size_t = (
    ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float,
    ctypes.c_size_t)


class LsfError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{name}: {message}")


class LayerCfg(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("intermediate", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("rank", c_int32), ("lora_scale", c_float), ("rope_theta", c_float),
                ("rms_eps", c_float), ("batch", c_int32), ("seq", c_int32)]


class Weight(ctypes.Structure):
    _fields_ = [("data", c_void_p), ("scale", c_void_p), ("scale2", c_void_p)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("format", c_int32), ("qkv", Weight), ("o", Weight), ("gate_up", Weight), ("down", Weight),
                ("norm1", c_void_p), ("norm2", c_void_p)]


class LoraProj(ctypes.Structure):
    _fields_ = [("A", c_void_p), ("B", c_void_p), ("dA", c_void_p), ("dB", c_void_p)]


class LayerLora(ctypes.Structure):
    _fields_ = [("q", LoraProj), ("k", LoraProj), ("v", LoraProj), ("o", LoraProj), ("gate", LoraProj),
                ("up", LoraProj), ("down", LoraProj), ("enabled", c_int32)]


class BlobLayout(ctypes.Structure):
    _fields_ = [("off", c_uint64 * 10), ("bytes", c_uint64), ("stride", c_uint64)]


class StackDesc(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("format", c_int32), ("blob_stride", c_uint64), ("host_store", c_void_p),
                ("dev_buf", c_void_p * 2), ("resident_store", c_void_p), ("compute", c_void_p),
                ("copy", c_void_p), ("flags", c_uint32)]


class StackIO(ctypes.Structure):
    _fields_ = [("ids", c_void_p), ("embed", c_void_p), ("final_norm", c_void_p), ("lm_head", c_void_p),
                ("vocab", c_int32), ("lora", ctypes.POINTER(LayerLora)), ("ckpt", c_void_p), ("logits", c_void_p),
                ("loss", c_void_p), ("ws", c_void_p), ("ws_bytes", c_size_t), ("loss_scale", c_float),
                ("mode", c_uint32), ("act", c_void_p), ("act_bytes", c_size_t), ("id_status", c_void_p)]


class DpoIO(ctypes.Structure):
    _fields_ = [("base", StackIO), ("beta", c_float), ("fused_reference", c_int32), ("seq_logp", c_void_p)]


class AdamwCfg(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("weight_decay", c_float), ("max_grad_norm", c_float), ("step", c_int32)]


class StackStats(ctypes.Structure):
    _fields_ = [("steps", c_int64), ("copies", c_int64), ("bytes", c_int64), ("copy_ms", ctypes.c_double),
                ("wait_ms", ctypes.c_double), ("kernel_ms", ctypes.c_double * 16),
                ("kernel_launches", c_int64 * 16)]


KERNELS = ["qkv_fwd", "o_fwd", "gate_up_fwd", "down_fwd", "qkv_bwd", "o_bwd", "gate_up_bwd", "down_bwd",
           "attn_fwd", "attn_bwd", "head_fwd", "head_bwd"]


_PROTOS = {
    "lsf_last_error": (ctypes.c_char_p, []),
    "lsf_version": (ctypes.c_char_p, []),
    "gemm_set_wide": (ctypes.c_int, [ctypes.c_int32]),
    "gemm_wide_launch_count": (ctypes.c_int64, []),
    "nf4_quantize": (c_int32, [c_void_p, c_int64, c_int32, c_void_p, c_void_p, c_void_p]),
    "nf4_dequantize": (c_int32, [c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_void_p]),
    "nf4dq_quantize": (c_int32, [c_void_p, c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "nf4dq_dequantize": (c_int32, [c_void_p, c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_void_p]),
    "linear_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "linear_fwd": (c_int32, [ctypes.POINTER(Weight), c_int32, c_int32, c_int32, c_void_p, c_void_p, c_int32,
                             c_float, c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "linear_noalloc_max_bytes": (c_size_t, []),
    "linear_fwd_noalloc": (c_int32, [ctypes.POINTER(Weight), c_int32, c_int32, c_int32, c_void_p, c_void_p, c_int32,
                                     c_float, c_void_p, c_int32, c_void_p, c_void_p]),
    "linear_bwd": (c_int32, [ctypes.POINTER(Weight), c_int32, c_int32, c_int32, c_void_p, c_void_p, c_int32,
                             c_float, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_size_t, c_void_p]),
    "layer_workspace_bytes": (c_size_t, [ctypes.POINTER(LayerCfg)]),
    "layer_fwd": (c_int32, [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerLora),
                            c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "layer_bwd": (c_int32, [ctypes.POINTER(LayerCfg), ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerLora),
                            c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "layer_blob_layout": (c_int32, [ctypes.POINTER(LayerCfg), c_int32, ctypes.POINTER(BlobLayout)]),
    "layer_weights_from_blob": (c_int32, [ctypes.POINTER(LayerCfg), c_int32, c_void_p,
                                          ctypes.POINTER(LayerWeights)]),
    "stack_create": (c_int32, [ctypes.POINTER(LayerCfg), ctypes.POINTER(StackDesc), ctypes.POINTER(c_void_p)]),
    "stack_destroy": (c_int32, [c_void_p]),
    "stack_workspace_bytes": (c_size_t, [ctypes.POINTER(LayerCfg), c_int32, c_int32]),
    "stream_stack_step": (c_int32, [c_void_p, ctypes.POINTER(StackIO)]),
    "stack_accum_workspace_bytes": (c_size_t, [ctypes.POINTER(LayerCfg), c_int32, c_int32, c_int32]),
    "stream_stack_accum_step": (c_int32, [c_void_p, ctypes.POINTER(StackIO), c_int32]),
    "dpo_stack_step": (c_int32, [c_void_p, ctypes.POINTER(DpoIO)]),
    "stack_stats": (c_int32, [c_void_p, ctypes.POINTER(StackStats)]),
    "stack_reset_stats": (c_int32, [c_void_p]),
    "stack_activation_bytes": (c_size_t, [c_void_p, c_int32]),
    "adamw_workspace_bytes": (c_size_t, []),
    "adamw_step": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, ctypes.POINTER(AdamwCfg), c_void_p,
                             c_void_p, c_size_t, c_void_p]),
    "adamw8_state_blocks": (c_int64, [c_int64]),
    "adamw8_workspace_bytes": (c_size_t, []),
    "adamw8_step": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64,
                              ctypes.POINTER(AdamwCfg), c_void_p, c_void_p, c_size_t, c_void_p]),
}

_LIB = None


def lib():
    """The loaded liblsf.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m layer_streamed_frozen_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def check(status):
    if status != LSF_OK:
        raise LsfError(status, lib().lsf_last_error().decode())


def ptr(t):
    """Data pointer of a tensor (None -> NULL)."""
    return None if t is None else t.data_ptr()


def stream_ptr(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def layer_cfg(hidden, intermediate, n_heads, n_kv_heads, head_dim, rank, lora_scale, rope_theta, rms_eps, batch,
              seq):
    return LayerCfg(hidden, intermediate, n_heads, n_kv_heads, head_dim, rank, lora_scale, rope_theta, rms_eps,
                    batch, seq)


# ----------------------------------------------------------------- calls

def gemm_set_wide(enable):
    """Select the kernel of the wide forward NF4 GEMMs (True or 512: the
    ping-pong kernel on 512 x 128 tiles, the default; 256: on 256 x 256
    tiles; False: the general kernel).  Results are bitwise identical
    whichever runs."""
    v = enable if enable in (256, 512) else (1 if enable else 0)
    check(lib().gemm_set_wide(v))


def gemm_wide_launch_count():
    """GEMMs launched on the wide kernel so far in this process."""
    return int(lib().gemm_wide_launch_count())


def nf4_quantize(w, packed=None, absmax=None, stream=None):
    """w: fp32 device tensor (numel % 64 == 0) -> (packed uint8 [n/2], absmax fp32 [n/64])."""
    n = w.numel()
    if packed is None:
        packed = torch.empty(n // 2, dtype=torch.uint8, device=w.device)
    if absmax is None:
        absmax = torch.empty(n // 64, dtype=torch.float32, device=w.device)
    check(lib().nf4_quantize(ptr(w), n, 64, ptr(packed), ptr(absmax), stream_ptr(stream)))
    return packed, absmax


def nf4_dequantize(packed, absmax, n, out=None, stream=None):
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=packed.device)
    check(lib().nf4_dequantize(ptr(packed), ptr(absmax), n, 64, ptr(out), stream_ptr(stream)))
    return out


def nf4dq_quantize(w, packed=None, absmax=None, absq=None, scale2=None, stream=None):
    """Double-quantised NF4: -> (packed uint8 [n/2], absmax fp32 [n/64], absq uint8 [n/64],
    scale2 fp32 [ceil(n/64/256), 2])."""
    n = w.numel()
    nb = n // 64
    dev = w.device
    packed = torch.empty(n // 2, dtype=torch.uint8, device=dev) if packed is None else packed
    absmax = torch.empty(nb, dtype=torch.float32, device=dev) if absmax is None else absmax
    absq = torch.empty(nb, dtype=torch.uint8, device=dev) if absq is None else absq
    scale2 = torch.empty(((nb + 255) // 256, 2), dtype=torch.float32, device=dev) if scale2 is None else scale2
    check(lib().nf4dq_quantize(ptr(w), n, 64, ptr(packed), ptr(absmax), ptr(absq), ptr(scale2),
                               stream_ptr(stream)))
    return packed, absmax, absq, scale2


def nf4dq_dequantize(packed, absq, scale2, n, out=None, stream=None):
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=packed.device)
    check(lib().nf4dq_dequantize(ptr(packed), ptr(absq), ptr(scale2), n, 64, ptr(out), stream_ptr(stream)))
    return out


def weight(data, scale=None, scale2=None):
    return Weight(ptr(data), ptr(scale), ptr(scale2))


def linear_workspace_bytes(tokens, n_out, n_in, rank):
    return lib().linear_workspace_bytes(tokens, n_out, n_in, rank)


def linear_fwd(w, fmt, n_out, n_in, A, B, rank, scale, x, y, ws, stream=None):
    check(lib().linear_fwd(ctypes.byref(w), fmt, n_out, n_in, ptr(A), ptr(B), rank, scale, ptr(x), x.shape[0],
                           ptr(y), ptr(ws), ws.numel() * ws.element_size(), stream_ptr(stream)))


def linear_noalloc_max_bytes():
    return int(lib().linear_noalloc_max_bytes())


def linear_fwd_noalloc(w, fmt, n_out, n_in, A, B, rank, scale, x, y, stream=None):
    """linear_fwd with the library's own device scratch (no workspace)."""
    check(lib().linear_fwd_noalloc(ctypes.byref(w), fmt, n_out, n_in, ptr(A), ptr(B), rank, scale, ptr(x),
                                   x.shape[0], ptr(y), stream_ptr(stream)))


def linear_bwd(w, fmt, n_out, n_in, A, B, rank, scale, x, dy, dx, dA, dB, ws, stream=None):
    check(lib().linear_bwd(ctypes.byref(w), fmt, n_out, n_in, ptr(A), ptr(B), rank, scale, ptr(x), ptr(dy),
                           x.shape[0], ptr(dx), ptr(dA), ptr(dB), ptr(ws), ws.numel() * ws.element_size(),
                           stream_ptr(stream)))


def layer_workspace_bytes(cfg):
    return lib().layer_workspace_bytes(ctypes.byref(cfg))


def layer_fwd(cfg, weights, lora, x, y, ws, stream=None):
    check(lib().layer_fwd(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(lora) if lora else None, ptr(x),
                          ptr(y), ptr(ws), ws.numel() * ws.element_size(), stream_ptr(stream)))


def layer_bwd(cfg, weights, lora, x, dy, dx, ws, stream=None):
    check(lib().layer_bwd(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(lora) if lora else None, ptr(x),
                          ptr(dy), ptr(dx), ptr(ws), ws.numel() * ws.element_size(), stream_ptr(stream)))


def layer_blob_layout(cfg, fmt=FMT_NF4):
    out = BlobLayout()
    check(lib().layer_blob_layout(ctypes.byref(cfg), fmt, ctypes.byref(out)))
    return out


def layer_weights_from_blob(cfg, fmt, blob_ptr):
    out = LayerWeights()
    check(lib().layer_weights_from_blob(ctypes.byref(cfg), fmt, blob_ptr, ctypes.byref(out)))
    return out


def stack_create(cfg, desc):
    h = c_void_p()
    check(lib().stack_create(ctypes.byref(cfg), ctypes.byref(desc), ctypes.byref(h)))
    return h


def stack_destroy(h):
    check(lib().stack_destroy(h))


def stack_workspace_bytes(cfg, vocab, n_layers):
    return lib().stack_workspace_bytes(ctypes.byref(cfg), vocab, n_layers)


def stream_stack_step(h, io):
    check(lib().stream_stack_step(h, ctypes.byref(io)))


def stack_accum_workspace_bytes(cfg, vocab, n_layers, n_micro):
    return lib().stack_accum_workspace_bytes(ctypes.byref(cfg), vocab, n_layers, n_micro)


def stream_stack_accum_step(h, ios):
    """ios: a sequence of StackIO, one per micro-batch."""
    arr = (StackIO * len(ios))(*ios)
    check(lib().stream_stack_accum_step(h, arr, len(ios)))


def dpo_stack_step(h, io):
    check(lib().dpo_stack_step(h, ctypes.byref(io)))


def stack_stats(h):
    out = StackStats()
    check(lib().stack_stats(h, ctypes.byref(out)))
    return out


def stack_reset_stats(h):
    check(lib().stack_reset_stats(h))


def adamw_workspace_bytes():
    return lib().adamw_workspace_bytes()


def adamw_step(param, grad, m, v, cfg, grad_norm, ws, n=None, stream=None):
    """AdamW over flat fp32 device tensors (n defaults to param.numel())."""
    n = param.numel() if n is None else n
    check(lib().adamw_step(ptr(param), ptr(grad), ptr(m), ptr(v), n, ctypes.byref(cfg),
                           ptr(grad_norm) if grad_norm is not None else None, ptr(ws),
                           ws.numel() * ws.element_size(), stream_ptr(stream)))


def adamw8_state_blocks(n):
    return int(lib().adamw8_state_blocks(n))


def adamw8_workspace_bytes():
    return lib().adamw8_workspace_bytes()


def adamw8_step(param, grad, m_codes, v_codes, m_absmax, v_absmax, cfg, grad_norm, ws, n=None, stream=None):
    """AdamW with 8-bit moment states over flat device tensors: param, grad
    fp32 [n]; m_codes int8 [n]; v_codes uint8 [n]; m_absmax, v_absmax fp32
    [adamw8_state_blocks(n)]."""
    n = param.numel() if n is None else n
    check(lib().adamw8_step(ptr(param), ptr(grad), ptr(m_codes), ptr(v_codes), ptr(m_absmax), ptr(v_absmax), n,
                            ctypes.byref(cfg), ptr(grad_norm) if grad_norm is not None else None, ptr(ws),
                            ws.numel() * ws.element_size(), stream_ptr(stream)))


def stack_activation_bytes(cfg, n_layers):
    return lib().stack_activation_bytes(ctypes.byref(cfg), n_layers)
