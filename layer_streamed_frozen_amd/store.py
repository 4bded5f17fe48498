"""Host-side plumbing: layer shapes, frozen-weight stores and adapter sets.

PyTorch provides the memory (device tensors, page-locked host tensors); every
quantisation and every byte of the layer blobs is produced by the HIP library
(``nf4_quantize``) or copied verbatim.  Seeded inputs come from ``synth``.
"""
import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import binding as B
from . import synth

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass
class LayerShape:
    hidden: int = 4096
    intermediate: int = 14336
    n_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    rank: int = 16
    alpha: float = 16.0
    rope_theta: float = 500000.0
    rms_eps: float = 1e-5

    @property
    def lora_scale(self):
        return self.alpha / self.rank

    def proj_shapes(self):
        H, I = self.hidden, self.intermediate
        q, kv = self.n_heads * self.head_dim, self.n_kv_heads * self.head_dim
        return {"q": (q, H), "k": (kv, H), "v": (kv, H), "o": (H, q), "gate": (I, H), "up": (I, H), "down": (H, I)}

    def cfg(self, batch, seq):
        return B.layer_cfg(self.hidden, self.intermediate, self.n_heads, self.n_kv_heads, self.head_dim, self.rank,
                           self.lora_scale, self.rope_theta, self.rms_eps, batch, seq)


# The decoder layer of a Llama-3.1-8B-shaped model (LoRA rank 16, alpha 16).
LLAMA8B = LayerShape()


def layer_weights_fp32(prefix, shape, std=0.02):
    """Seeded frozen weights of one layer (host fp32, N(0, std)); norms 1.0."""
    W = {n: synth.normal(f"{prefix}.{n}.W", s, std) for n, s in shape.proj_shapes().items()}
    one = np.full(shape.hidden, 0x3F80, dtype=np.uint16)  # bf16 1.0
    W["norm1"] = one.copy()
    W["norm2"] = one.copy()
    return W


def random_norms(prefix, shape):
    """Non-trivial bf16 norm weights for tests (1 + N(0, 0.1), bf16-exact)."""
    out = {}
    for k in ("norm1", "norm2"):
        _, bits = synth.bf16_exact(1.0 + synth.normal(f"{prefix}.{k}", (shape.hidden,), 0.1))
        out[k] = bits
    return out


def _sections(W):
    return [np.concatenate([W["q"], W["k"], W["v"]], axis=0), W["o"],
            np.concatenate([W["gate"], W["up"]], axis=0), W["down"]]


def build_layer_blob(shape, W, fmt=B.FMT_NF4, device="cuda", out=None):
    """Assemble one layer blob on the device.

    NF4: every section is quantised by the library's nf4_quantize.  BF16: the
    fp32 weights must already be bfloat16-exact; their bits are copied.
    Returns a uint8 device tensor of ``stride`` bytes (or fills ``out``).
    """
    cfg = shape.cfg(1, 1)
    lay = B.layer_blob_layout(cfg, fmt)
    blob = out if out is not None else torch.zeros(lay.stride, dtype=torch.uint8, device=device)
    for i, w in enumerate(_sections(W)):
        n = w.size
        wd = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(device)
        if fmt == B.FMT_NF4:
            packed = blob[lay.off[i]: lay.off[i] + n // 2]
            absmax = blob[lay.off[4 + i]: lay.off[4 + i] + n // 16].view(torch.float32)
            B.nf4_quantize(wd.reshape(-1), packed, absmax)
        elif fmt == B.FMT_BF16:
            bits = (wd.reshape(-1).view(torch.int32) >> 16).to(torch.int16)
            blob[lay.off[i]: lay.off[i] + 2 * n].view(torch.int16).copy_(bits)
        elif fmt == B.FMT_NF4_DQ:
            nb = n // 64
            packed = blob[lay.off[i]: lay.off[i] + n // 2]
            absq = blob[lay.off[4 + i]: lay.off[4 + i] + nb]
            s2o = lay.off[4 + i] + (nb + 255) // 256 * 256
            ng = (nb + 255) // 256
            scale2 = blob[s2o: s2o + 8 * ng].view(torch.float32).view(ng, 2)
            B.nf4dq_quantize(wd.reshape(-1), packed, None, absq, scale2)
        else:
            raise ValueError(f"unknown weight format {fmt}")
        del wd
    for k, sec in (("norm1", 8), ("norm2", 9)):
        nb = torch.from_numpy(np.ascontiguousarray(W[k]).view(np.int16)).to(device)
        blob[lay.off[sec]: lay.off[sec] + 2 * shape.hidden].view(torch.int16).copy_(nb)
    return blob


class Store:
    """The frozen decoder stack: one blob per layer, in pinned host memory
    (streamed mode) and optionally also resident on the device."""

    def __init__(self, shape, n_layers, fmt=B.FMT_NF4, device="cuda", resident=False, pinned=True,
                 weights_fn=None, prefix="layer"):
        self.shape, self.n_layers, self.fmt = shape, n_layers, fmt
        cfg = shape.cfg(1, 1)
        self.layout = B.layer_blob_layout(cfg, fmt)
        self.stride = self.layout.stride
        total = self.stride * n_layers
        self.host = torch.empty(total, dtype=torch.uint8, pin_memory=pinned)
        self.dev = torch.empty(total, dtype=torch.uint8, device=device) if resident else None
        tmp = torch.zeros(self.stride, dtype=torch.uint8, device=device)
        for i in range(n_layers):
            W = weights_fn(i) if weights_fn is not None else layer_weights_fp32(f"{prefix}{i}", shape)
            tmp.zero_()
            build_layer_blob(shape, W, fmt, device, out=tmp)
            if self.dev is not None:
                self.dev[i * self.stride:(i + 1) * self.stride].copy_(tmp)
            self.host[i * self.stride:(i + 1) * self.stride].copy_(tmp.cpu())
        torch.cuda.synchronize()

    def blob_bytes(self):
        return self.layout.bytes


class LoraSet:
    """Trainable adapters of a stack: fp32 A [r, in], B [out, r] and their
    gradients, per layer and projection (``targets`` picks the projections).

    Every A and B lives in one flat fp32 arena (``params``), and every dA, dB
    at the same offsets in a second one (``grads``), each tensor starting on a
    256-byte boundary with zero padding between, so one optimizer call updates
    the whole set."""

    ALIGN = 64  # elements (256 bytes)

    def __init__(self, shape, n_layers, targets=PROJ, device="cuda", prefix="lora", b_zero=False):
        self.shape, self.n_layers, self.targets = shape, n_layers, tuple(targets)
        self.A, self.B, self.dA, self.dB = [], [], [], []
        r = shape.rank
        slots, total = [], 0
        for i in range(n_layers):
            for n, (o, inn) in shape.proj_shapes().items():
                if n not in self.targets:
                    continue
                for which, shp in (("A", (r, inn)), ("B", (o, r))):
                    slots.append((i, n, which, shp, total))
                    total += -(-shp[0] * shp[1] // self.ALIGN) * self.ALIGN
        self.params = torch.zeros(max(total, self.ALIGN), dtype=torch.float32, device=device)
        self.grads = torch.zeros_like(self.params)
        for i in range(n_layers):
            for lst in (self.A, self.B, self.dA, self.dB):
                lst.append({})
        for i, n, which, shp, off in slots:
            cnt = shp[0] * shp[1]
            if which == "A":
                lim = 1.0 / np.sqrt(shp[1])
                vals = synth.uniform(f"{prefix}{i}.{n}.A", shp, -lim, lim)
            else:
                vals = synth.normal(f"{prefix}{i}.{n}.B", shp, 0.01)
                if b_zero:
                    vals = np.zeros_like(vals)
            view = self.params[off:off + cnt].view(shp)
            view.copy_(torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)))
            (self.A if which == "A" else self.B)[i][n] = view
            (self.dA if which == "A" else self.dB)[i][n] = self.grads[off:off + cnt].view(shp)
        self._arr = None

    def struct(self, i, enabled=True, grads=True):
        L = B.LayerLora()
        for n in PROJ:
            p = getattr(L, n)
            if n in self.targets:
                p.A, p.B = B.ptr(self.A[i][n]), B.ptr(self.B[i][n])
                if grads:
                    p.dA, p.dB = B.ptr(self.dA[i][n]), B.ptr(self.dB[i][n])
        L.enabled = 1 if enabled else 0
        return L

    def array(self, enabled=True, grads=True):
        arr = (B.LayerLora * self.n_layers)()
        for i in range(self.n_layers):
            arr[i] = self.struct(i, enabled, grads)
        self._arr = arr
        return arr

    def zero_grads(self):
        self.grads.zero_()

    def numpy(self, i, enabled=True):
        """LoRA dict in the oracle's form (fp64 numpy), None where absent."""
        if not enabled:
            return None
        return {n: ((self.A[i][n].double().cpu().numpy(), self.B[i][n].double().cpu().numpy())
                    if n in self.targets else None) for n in PROJ}

    def grads_numpy(self, i):
        return {n: (self.dA[i][n].double().cpu().numpy(), self.dB[i][n].double().cpu().numpy())
                for n in self.targets}


class AdamW:
    """AdamW (fp32 moments) over a LoraSet's flat parameter arena, one launch
    per update."""

    def __init__(self, lora, lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, max_grad_norm=0.0):
        self.lora = lora
        self.cfg = B.AdamwCfg(lr=lr, beta1=betas[0], beta2=betas[1], eps=eps, weight_decay=weight_decay,
                              max_grad_norm=max_grad_norm, step=0)
        self.m = torch.zeros_like(lora.params)
        self.v = torch.zeros_like(lora.params)
        self.ws = torch.empty(B.adamw_workspace_bytes(), dtype=torch.uint8, device=lora.params.device)
        self.grad_norm = torch.zeros(1, dtype=torch.float32, device=lora.params.device)

    def step(self, stream=None):
        self.cfg.step += 1
        B.adamw_step(self.lora.params, self.lora.grads, self.m, self.v, self.cfg, self.grad_norm, self.ws,
                     stream=stream)


class AdamW8:
    """AdamW with 8-bit block-wise quantised moments (the pages'
    paged_adamw_8bit, resident) over a LoraSet's flat parameter arena."""

    def __init__(self, lora, lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, max_grad_norm=0.0):
        self.lora = lora
        self.cfg = B.AdamwCfg(lr=lr, beta1=betas[0], beta2=betas[1], eps=eps, weight_decay=weight_decay,
                              max_grad_norm=max_grad_norm, step=0)
        n = lora.params.numel()
        dev = lora.params.device
        nb = B.adamw8_state_blocks(n)
        self.m_codes = torch.zeros(n, dtype=torch.int8, device=dev)
        self.v_codes = torch.zeros(n, dtype=torch.uint8, device=dev)
        self.m_absmax = torch.zeros(nb, dtype=torch.float32, device=dev)
        self.v_absmax = torch.zeros(nb, dtype=torch.float32, device=dev)
        self.ws = torch.empty(B.adamw8_workspace_bytes(), dtype=torch.uint8, device=dev)
        self.grad_norm = torch.zeros(1, dtype=torch.float32, device=dev)

    def step(self, stream=None):
        self.cfg.step += 1
        B.adamw8_step(self.lora.params, self.lora.grads, self.m_codes, self.v_codes, self.m_absmax, self.v_absmax,
                      self.cfg, self.grad_norm, self.ws, stream=stream)


_COPY_STREAMS = {}


def copy_stream(torch_device=None):
    """One host-to-device copy stream per device for the whole process.

    HIP runs a process's streams on a few hardware queues (four unless
    GPU_MAX_HW_QUEUES says otherwise) and makes later streams share them.  A
    copy stream that lands on the compute stream's queue makes every kernel
    queued behind a copy wait for that copy, and torch never releases a
    stream it hands out, so a new stream per stack would, after a few stacks,
    put one there.  Every stack therefore reuses this one."""
    dev = torch.device("cuda") if torch_device is None else torch.device(torch_device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if idx not in _COPY_STREAMS:
        _COPY_STREAMS[idx] = torch.cuda.Stream(device=idx)
    return _COPY_STREAMS[idx]


class Stack:
    """A streamed stack: store + two device buffers + streams + handle."""

    def __init__(self, shape, store, batch, seq, vocab, flags=0, device="cuda", keep_activations=False, n_micro=1):
        self.shape, self.store, self.batch, self.seq, self.vocab = shape, store, batch, seq, vocab
        self.cfg = shape.cfg(batch, seq)
        nbytes = store.layout.bytes
        self.bufs = [torch.empty(nbytes, dtype=torch.uint8, device=device) for _ in range(2)]
        self.compute = torch.cuda.current_stream()
        self.copy = copy_stream(device)
        d = B.StackDesc()
        d.n_layers = store.n_layers
        d.format = store.fmt
        d.blob_stride = store.stride
        d.host_store = store.host.data_ptr()
        d.dev_buf[0] = self.bufs[0].data_ptr()
        d.dev_buf[1] = self.bufs[1].data_ptr()
        d.resident_store = store.dev.data_ptr() if store.dev is not None else None
        d.compute = self.compute.cuda_stream
        d.copy = self.copy.cuda_stream
        d.flags = flags
        self.handle = B.stack_create(self.cfg, d)
        T = batch * seq
        H = shape.hidden
        # n_micro > 1: accum_step keeps that many micro-batches' checkpoints
        self.n_micro = n_micro
        self.ws = torch.empty(B.stack_accum_workspace_bytes(self.cfg, vocab, store.n_layers, n_micro), dtype=torch.uint8,
                              device=device)
        self.ckpts = [torch.empty((store.n_layers + 1, T, H), dtype=torch.bfloat16, device=device)
                      for _ in range(n_micro)]
        self.ckpt = self.ckpts[0]
        self.logits = torch.empty((T, vocab), dtype=torch.float32, device=device)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self.seq_logp = torch.zeros((2, batch), dtype=torch.float32, device=device)  # DPO: policy, reference
        # set to 1 by a step that meets a token id outside [0, vocab); zeroed only here and by clear_id_status
        self.id_status = torch.zeros(1, dtype=torch.int32, device=device)
        # every layer's forward intermediates, when the backward skips the recompute
        self.act = None
        if keep_activations:
            self.act = torch.empty(B.stack_activation_bytes(self.cfg, store.n_layers) * n_micro, dtype=torch.uint8,
                                   device=device)

    def _io(self, ids, embed, final_norm, lm_head, lora_arr, mode, loss_scale):
        io = B.StackIO()
        io.ids = ids.data_ptr()
        io.embed = embed.data_ptr()
        io.final_norm = final_norm.data_ptr()
        io.lm_head = lm_head.data_ptr()
        io.vocab = self.vocab
        io.lora = ctypes.cast(lora_arr, ctypes.POINTER(B.LayerLora))
        io.ckpt = self.ckpt.data_ptr()
        io.logits = self.logits.data_ptr()
        io.loss = self.loss.data_ptr()
        io.ws = self.ws.data_ptr()
        io.ws_bytes = self.ws.numel()
        io.loss_scale = loss_scale
        io.mode = mode
        io.id_status = self.id_status.data_ptr()
        if self.act is not None:
            io.mode |= B.MODE_KEEP_ACTIVATIONS
            io.act = self.act.data_ptr()
            io.act_bytes = self.act.numel()
        return io

    def step(self, ids, embed, final_norm, lm_head, lora_arr, mode=B.MODE_STREAMED, loss_scale=1.0):
        """One SFT micro-batch (cross-entropy on next tokens)."""
        B.stream_stack_step(self.handle, self._io(ids, embed, final_norm, lm_head, lora_arr, mode, loss_scale))

    def accum_step(self, ids_list, embed, final_norm, lm_head, lora_arr, mode=B.MODE_STREAMED, loss_scale=None):
        """len(ids_list) SFT micro-batches in one walk over the stack per
        direction (gradient accumulation); loss_scale defaults to 1/n.  The
        loss of the last micro-batch ends in self.loss."""
        n = len(ids_list)
        if n > self.n_micro:
            raise ValueError(f"this Stack holds checkpoints for {self.n_micro} micro-batches, not {n}")
        scale = 1.0 / n if loss_scale is None else loss_scale
        ios = []
        for m, ids in enumerate(ids_list):
            io = self._io(ids, embed, final_norm, lm_head, lora_arr, mode, scale)
            io.ckpt = self.ckpts[m].data_ptr()
            ios.append(io)
        B.stream_stack_accum_step(self.handle, ios)

    def dpo_step(self, ids, embed, final_norm, lm_head, lora_arr, beta=0.1, fused=True, mode=B.MODE_STREAMED,
                 loss_scale=1.0):
        """One DPO micro-batch: ids holds the chosen sequences, then the
        rejected ones.  Fills self.seq_logp [2, batch] (policy, reference)."""
        io = B.DpoIO()
        io.base = self._io(ids, embed, final_norm, lm_head, lora_arr, mode, loss_scale)
        io.beta = beta
        io.fused_reference = 1 if fused else 0
        io.seq_logp = self.seq_logp.data_ptr()
        B.dpo_stack_step(self.handle, io)

    def stats(self):
        return B.stack_stats(self.handle)

    def ids_were_valid(self):
        """False if a step since the last clear_id_status met a token id
        outside [0, vocab) (synchronises with the device)."""
        return int(self.id_status.item()) == 0

    def clear_id_status(self):
        self.id_status.zero_()

    def close(self):
        if self.handle is not None:
            B.stack_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
