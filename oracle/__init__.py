"""CPU oracle for layer-streamed NF4 + LoRA training.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (``layer_streamed_frozen_amd`` and its HIP library) never
imports, calls or links anything here, and nothing here imports the product.

What it computes is the plain definition of the method, written out slowly and
obviously in NumPy:

* ``nf4``    - blockwise NormalFloat-4 quantise / pack / dequantise, in fp32,
               because the codes are integers decided by fp32 comparisons.
* ``model``  - a LoRA-augmented linear layer, a Llama-style decoder layer
               (RMSNorm, RoPE, GQA causal attention, SwiGLU) and a stack with
               an embedding, final norm, untied head and cross-entropy loss;
               forward and hand-derived backward, fp64 by default.
* ``dpo``    - the preference loss whose reference model is the same frozen
               base with the adapters switched off.
* ``optim``  - the AdamW update of the trainable LoRA tensors (fp32 state).
* ``optim8`` - the same update with 8-bit block-wise quantised moment states.

Streaming and per-layer recomputation change where the frozen weights live,
never what is computed (news article "aizxs.com/ai-learning/13312.html",
section on exact layer streaming; tutorial "alphalab.site/soup-layer-streaming",
section "four-stage data path", item 3).  So the oracle is an ordinary,
un-streamed, un-checkpointed forward and backward over the dequantised base.

Parity status of each function is listed in its module header.
"""
