"""Event-ordering stress modes of the streamer (the pages' blog, section on
correctness and bit-exactness: a streamed result must not depend on timing).

Under LSF_STACK_DEBUG_POISON every released buffer is filled with NaN bytes
before the next copy lands in it, and under LSF_STACK_DEBUG_COPY_DELAY every
copy starts late; a compute stream that read a buffer outside the window its
ready/freed events give it would produce NaN or stale-weight results.  The
streamed runs must still give the resident run's bits: SFT, the accumulated
walk and DPO (fused and separate reference pass)."""
import pytest
import torch

from layer_streamed_frozen_amd import binding as B
from layer_streamed_frozen_amd import store as S
from layer_streamed_frozen_amd import synth
from tests.test_gpu_dpo import DpoSetup
from tests.test_gpu_dpo import same as dpo_same
from tests.test_gpu_layer import SMALL
from tests.test_gpu_stack import Setup, same

pytestmark = pytest.mark.gpu

MODES = {"poison": B.STACK_DEBUG_POISON, "delay": B.STACK_DEBUG_COPY_DELAY,
         "poison+delay": B.STACK_DEBUG_POISON | B.STACK_DEBUG_COPY_DELAY}


@pytest.mark.parametrize("mode", list(MODES))
def test_sft_stream_equals_resident_under_stress(mode):
    s = Setup(SMALL, 4, 512, 2, 64, f"stress.sft.{mode}", flags=MODES[mode])
    s.step(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    ref = s.snapshot()
    for _ in range(2):  # the second step also reuses layers 0 and 1 from the first
        s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
        assert same(ref, s.snapshot())
    s.step(mode=B.MODE_STREAMED | B.MODE_FWD_ONLY)
    assert torch.equal(ref[0], s.stack.logits) and torch.equal(ref[1], s.stack.loss)
    st = s.stack.stats()
    assert st.copies == (2 * 4 - 2) + (2 * 4 - 4) + (4 - 2)
    s.stack.close()


@pytest.mark.parametrize("mode", list(MODES))
def test_accumulated_walk_under_stress(mode):
    n = 3
    s = Setup(SMALL, 4, 512, 2, 48, f"stress.acc.{mode}")
    ids = [torch.from_numpy(synth.token_ids(f"stress.acc.ids{m}", (2, 48), 512)).cuda() for m in range(n)]
    arr = s.lora.array()
    out = []
    for m_flags, m_mode in ((0, B.MODE_RESIDENT), (MODES[mode], B.MODE_STREAMED)):
        acc = S.Stack(SMALL, s.store, 2, 48, 512, n_micro=n, flags=m_flags)
        acc.accum_step(ids, s.emb, s.fnorm, s.head, arr, mode=m_mode | B.MODE_ZERO_GRADS)
        torch.cuda.synchronize()
        g = [{k: (s.lora.dA[i][k].clone(), s.lora.dB[i][k].clone()) for k in s.lora.targets} for i in range(s.L)]
        out.append((acc.logits.clone(), acc.loss.clone(), g))
        acc.close()
    assert same(out[0], out[1])


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("fused", [True, False])
def test_dpo_under_stress(mode, fused):
    s = DpoSetup(SMALL, 3, 512, 2, 64, f"stress.dpo.{mode}", flags=MODES[mode])
    s.dpo(fused=fused, mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    ref = s.snapshot()
    s.dpo(fused=fused, mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    assert dpo_same(ref, s.snapshot())
    s.stack.close()


def test_stress_flags_at_8b_shapes():
    # Four Llama-3.1-8B-shaped layers (123 MB per copy, so each copy takes
    # about 2 ms) under both stress modes at once.
    s = Setup(S.LLAMA8B, 4, 1024, 1, 512, "stress.8b", random_norms=False,
              flags=B.STACK_DEBUG_POISON | B.STACK_DEBUG_COPY_DELAY)
    s.step(mode=B.MODE_RESIDENT | B.MODE_ZERO_GRADS)
    ref = s.snapshot()
    s.step(mode=B.MODE_STREAMED | B.MODE_ZERO_GRADS)
    assert same(ref, s.snapshot())
    s.stack.close()
