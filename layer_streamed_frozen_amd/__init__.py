"""Layer-streamed NF4 + LoRA training on AMD Instinct MI355X (gfx950).

The compute path lives in the HIP library liblsf.so (C ABI in include/lsf.h);
``binding`` marshals torch tensors into it, ``store`` builds the frozen-weight
stores and adapter sets, ``synth`` draws the seeded synthetic inputs.
"""
__version__ = "0.1.0"
