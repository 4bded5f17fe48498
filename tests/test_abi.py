"""The C ABI without a GPU: the library loads, exports every function the
header declares, and its host-side calls (layouts, workspace sizes, argument
validation, error reporting) behave as documented.  No kernel is launched."""
import ctypes
import os
import re
import subprocess

import pytest

from layer_streamed_frozen_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsf.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from layer_streamed_frozen_amd import build
        build.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^LSF_API\s+[\w\s\*]*?(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_core_calls():
    names = declared_functions()
    for core in ("nf4_quantize", "layer_fwd", "layer_bwd", "stream_stack_step"):
        assert core in names
    assert len(names) >= 18


def test_every_declared_function_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)


def test_blob_layout_of_8b_layer(lib):
    from layer_streamed_frozen_amd.store import LLAMA8B
    lay = B.layer_blob_layout(LLAMA8B.cfg(1, 512), B.FMT_NF4)
    # packed q|k|v, o, gate|up, down, then their fp32 absmax, then two bf16 norms
    sizes = [6144 * 4096 // 2, 4096 * 4096 // 2, 28672 * 4096 // 2, 4096 * 14336 // 2,
             6144 * 4096 // 16, 4096 * 4096 // 16, 28672 * 4096 // 16, 4096 * 14336 // 16, 8192, 8192]
    assert list(lay.off) == [sum(sizes[:i]) for i in range(10)]
    assert lay.bytes == sum(sizes) == 122699776
    assert lay.stride == 122699776
    bf = B.layer_blob_layout(LLAMA8B.cfg(1, 512), B.FMT_BF16)
    assert bf.bytes == 2 * 218103808 + 2 * 8192


def test_workspace_sizes(lib):
    from layer_streamed_frozen_amd.store import LLAMA8B
    w1 = B.layer_workspace_bytes(LLAMA8B.cfg(1, 512))
    w4 = B.layer_workspace_bytes(LLAMA8B.cfg(4, 512))
    assert 0 < w1 < w4 < 8 * w1
    assert B.stack_workspace_bytes(LLAMA8B.cfg(1, 512), 128256, 32) > B.stack_workspace_bytes(LLAMA8B.cfg(1, 512),
                                                                                              128256, 1) > w1
    assert B.stack_workspace_bytes(LLAMA8B.cfg(1, 512), 128256, 0) == 0
    assert B.linear_workspace_bytes(64, 256, 256, 8) > 0
    assert B.linear_workspace_bytes(0, 256, 256, 8) == 0
    # at most 2^20 tokens per call: one more and the size query reports 0
    assert B.layer_workspace_bytes(LLAMA8B.cfg(2048, 512)) > 0
    assert B.layer_workspace_bytes(LLAMA8B.cfg(2049, 512)) == 0


def _status(fn, *args):
    return fn(*args)


def test_invalid_arguments_are_rejected_before_any_launch(lib):
    L = lib
    st = L.nf4_quantize(None, 100, 64, None, None, None)
    assert st == B.LSF_ERR_SHAPE and b"multiple of 64" in L.lsf_last_error()
    assert L.nf4_quantize(None, 128, 32, None, None, None) == B.LSF_ERR_SHAPE
    assert L.nf4_quantize(None, 128, 64, None, None, None) == B.LSF_ERR_INVALID_ARG
    assert L.nf4_quantize(None, 0, 64, None, None, None) == B.LSF_OK
    assert L.nf4_dequantize(8, 8, 128, 64, 8, None) == B.LSF_ERR_ALIGN  # misaligned pointers
    assert L.layer_fwd(None, None, None, None, None, None, 0, None) == B.LSF_ERR_INVALID_ARG
    from layer_streamed_frozen_amd.store import LLAMA8B
    cfg = LLAMA8B.cfg(1, 512)
    cfg.head_dim = 64
    assert L.layer_fwd(ctypes.byref(cfg), None, None, None, None, None, 0, None) == B.LSF_ERR_SHAPE
    cfg = LLAMA8B.cfg(1, 512)
    cfg.rank = 12
    assert L.layer_fwd(ctypes.byref(cfg), None, None, None, None, None, 0, None) == B.LSF_ERR_SHAPE
    cfg = LLAMA8B.cfg(0, 512)
    assert L.layer_bwd(ctypes.byref(cfg), None, None, None, None, None, None, 0, None) == B.LSF_ERR_SHAPE
    cfg = LLAMA8B.cfg(2049, 512)
    assert L.layer_fwd(ctypes.byref(cfg), None, None, None, None, None, 0, None) == B.LSF_ERR_SHAPE
    assert b"too many tokens" in L.lsf_last_error()
    cfg = LLAMA8B.cfg(1, 512)
    cfg.n_kv_heads = 5
    assert L.layer_workspace_bytes(ctypes.byref(cfg)) == 0
    w = B.LayerWeights()
    assert L.layer_fwd(ctypes.byref(LLAMA8B.cfg(1, 512)), ctypes.byref(w), None, None, None, None, 0,
                       None) == B.LSF_ERR_ALIGN
    # stack descriptor checks that need no device
    d = B.StackDesc()
    d.n_layers = 0
    h = ctypes.c_void_p()
    assert L.stack_create(ctypes.byref(LLAMA8B.cfg(1, 512)), ctypes.byref(d), ctypes.byref(h)) == \
        B.LSF_ERR_INVALID_ARG
    d.n_layers = 2
    d.flags = 1 << 31  # unknown flag
    assert L.stack_create(ctypes.byref(LLAMA8B.cfg(1, 512)), ctypes.byref(d), ctypes.byref(h)) == \
        B.LSF_ERR_INVALID_ARG
    d.flags = B.STACK_SOURCE_DISK  # the disk tier is not built
    assert L.stack_create(ctypes.byref(LLAMA8B.cfg(1, 512)), ctypes.byref(d), ctypes.byref(h)) == \
        B.LSF_ERR_UNSUPPORTED
    d.flags = 0
    d.format = B.FMT_NF4
    d.blob_stride = 1000
    assert L.stack_create(ctypes.byref(LLAMA8B.cfg(1, 512)), ctypes.byref(d), ctypes.byref(h)) == B.LSF_ERR_SHAPE
    d.blob_stride = 122699776
    assert L.stack_create(ctypes.byref(LLAMA8B.cfg(1, 512)), ctypes.byref(d), ctypes.byref(h)) == \
        B.LSF_ERR_INVALID_ARG  # no device buffers
    assert L.stream_stack_step(None, None) == B.LSF_ERR_INVALID_ARG
    assert L.stack_destroy(None) == B.LSF_OK


def test_binding_raises_with_message(lib):
    with pytest.raises(B.LsfError) as e:
        B.check(lib.nf4_quantize(None, 100, 64, None, None, None))
    assert e.value.status == B.LSF_ERR_SHAPE
    assert "LSF_ERR_SHAPE" in str(e.value)


def test_gemm_schedule_switch_validates(lib):
    B.gemm_set_wide(False)
    B.gemm_set_wide(True)
    assert lib.gemm_set_wide(128) == B.LSF_ERR_INVALID_ARG
    assert lib.gemm_set_wide(2) == B.LSF_ERR_INVALID_ARG
    assert "enable" in lib.lsf_last_error().decode()
    B.gemm_set_wide(512)
    B.gemm_set_wide(256)
    B.gemm_set_wide(True)
    assert B.gemm_wide_launch_count() >= 0


def test_optimizer_arguments_are_rejected_before_any_launch(lib):
    L = lib
    good = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, max_grad_norm=0.0, step=1)
    for fn, extra in ((L.adamw_step, (None, None)), (L.adamw8_step, (None, None, None, None))):
        def call(cfg, n=16, ws=None, ws_bytes=0):
            args = (None, None) + extra + (n, ctypes.byref(cfg) if cfg is not None else None, None, ws, ws_bytes,
                                           None)
            return fn(*args)
        assert call(None) == B.LSF_ERR_INVALID_ARG
        for field, bad in (("lr", -1.0), ("beta1", 1.0), ("beta2", -0.1), ("eps", 0.0), ("weight_decay", -1.0),
                           ("max_grad_norm", float("inf")), ("step", 0)):
            cfg = B.AdamwCfg(**dict(good, **{field: bad}))
            assert call(cfg) == B.LSF_ERR_INVALID_ARG, field
        assert call(B.AdamwCfg(**good), n=-1) == B.LSF_ERR_INVALID_ARG
        assert call(B.AdamwCfg(**good), n=0) == B.LSF_OK  # nothing to do
        assert call(B.AdamwCfg(**good)) == B.LSF_ERR_INVALID_ARG  # NULL tensors
    # 8-bit states: misaligned codes, and a workspace that is too small
    st = L.adamw8_step(16, 16, 3, 16, 16, 16, 16, ctypes.byref(B.AdamwCfg(**good)), None, 16, 64, None)
    assert st == B.LSF_ERR_ALIGN
    st = L.adamw8_step(16, 16, 16, 16, 16, 16, 16, ctypes.byref(B.AdamwCfg(**good)), None, 16, 64, None)
    assert st == B.LSF_ERR_WORKSPACE
    assert B.adamw8_state_blocks(4097) == 3 and B.adamw8_workspace_bytes() > B.adamw_workspace_bytes()


def test_noalloc_linear_limits_without_a_device(lib):
    L = lib
    assert L.linear_noalloc_max_bytes() == 32 << 20
    # more scratch than the library holds: refused before anything is enqueued
    w = B.Weight(16, 16, None)
    st = L.linear_fwd_noalloc(ctypes.byref(w), B.FMT_NF4, 4096, 4096, None, None, 0, 1.0, 16, 512, 16, None)
    assert st == B.LSF_ERR_WORKSPACE and b"scratch" in L.lsf_last_error()
    # ordinary argument errors as linear_fwd
    st = L.linear_fwd_noalloc(ctypes.byref(w), B.FMT_NF4, 100, 256, None, None, 0, 1.0, 16, 8, 16, None)
    assert st == B.LSF_ERR_SHAPE
    st = L.linear_fwd_noalloc(None, B.FMT_NF4, 256, 256, None, None, 0, 1.0, 16, 8, 16, None)
    assert st == B.LSF_ERR_INVALID_ARG


def test_linear_sizes_are_bounded(lib):
    L = lib
    big = 1 << 21
    assert B.linear_workspace_bytes(big, 256, 256, 8) == 0
    assert B.linear_workspace_bytes(64, big * 64, 256, 8) == 0
    w = B.Weight(16, 16, None)
    st = L.linear_fwd(ctypes.byref(w), B.FMT_NF4, 256, 256, None, None, 0, 1.0, 16, big, 16, 16, 1 << 40, None)
    assert st == B.LSF_ERR_SHAPE and b"at most" in L.lsf_last_error()


def test_stack_io_layout_matches_the_header(lib):
    # the binding's StackIO must end with id_status, as lsf_stack_io does
    names = [f[0] for f in B.StackIO._fields_]
    assert names[-1] == "id_status"
    text = open(HEADER).read()
    body = text[text.index("typedef struct {\n  const int32_t* ids;"):text.index("} lsf_stack_io;")]
    fields = re.findall(r"^\s+[\w\s\*]+?[\s\*](\w+);", re.sub(r"/\*.*?\*/", "", body, flags=re.S), flags=re.M)
    assert fields == names, (fields, names)
