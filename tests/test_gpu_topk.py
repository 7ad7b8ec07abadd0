"""GPU parity: fdllm_unmask_topk (fixed-step rule) against the fp64 oracle
(decisions bit-exact except oracle-flagged near ties at the k-th / (k+1)-th
confidence boundary, confidences within 1e-6)."""
import numpy as np
import pytest

import block_wise_kv_amd as fd
from gpu_util import compare_unmask, require_gpu, run_unmask, say
from oracle import tokens_per_step, unmask_topk_ref
from workloads import (make_decode_state, make_logits, n_masked_c5, shape_c1, shape_c2, shape_c3,
                       shape_c4, shape_c5, shape_custom)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _ref(s, logits, tokens, mask, k, advance=False):
    return unmask_topk_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, k,
                           advance=advance)


@pytest.mark.parametrize("k", [1, 3, 20, 40])
def test_c1_tiny_f32(k):
    s = shape_c1()
    logits = make_logits(s, "spike")
    tokens, mask = make_decode_state(s, 20)
    say(f"c1 topk k={k}")
    g, reps = run_unmask(s, logits, tokens, mask, None, reps=2, topk=k)
    compare_unmask(g, _ref(s, logits, tokens, mask, k), s, label=f"c1 k={k}")
    for key in ("tokens", "mask", "n_decoded", "decoded_pos"):
        assert np.array_equal(reps[0][key], reps[1][key])


@pytest.mark.parametrize("recipe", ["peak", "calibrated"])
@pytest.mark.parametrize("k", [1, 2, 8, 32])
def test_c2_llada(recipe, k):
    s = shape_c2(3)
    logits = make_logits(s, recipe)
    tokens, mask = make_decode_state(s)
    say(f"c2 topk {recipe} k={k}")
    g, _ = run_unmask(s, logits, tokens, mask, None, topk=k)
    ref = _ref(s, logits, tokens, mask, k)
    compare_unmask(g, ref, s, label=f"c2 {recipe} k={k}")
    if not ref.tie_step[0]:
        assert g["n_decoded"][0] == min(k, 32)


@pytest.mark.parametrize("k", [1, 4])
def test_c3_dream(k):
    s = shape_c3(5)
    logits = make_logits(s, "calibrated")
    tokens, mask = make_decode_state(s)
    say(f"c3 topk k={k}")
    g, _ = run_unmask(s, logits, tokens, mask, None, topk=k)
    compare_unmask(g, _ref(s, logits, tokens, mask, k), s, label=f"c3 k={k}")


@pytest.mark.parametrize("B,k", [(16, 4), (64, 7), (128, 1), (128, 16), (128, 128)])
def test_c4_blocks(B, k):
    # B = 128 takes the workgroup finalisation, B <= 64 the one-wave one
    s = shape_c4(B, block_idx=1, batch=8)
    logits = make_logits(s, "calibrated")
    tokens, mask = make_decode_state(s)
    say(f"c4 topk B={B} k={k}")
    g, _ = run_unmask(s, logits, tokens, mask, None, topk=k)
    compare_unmask(g, _ref(s, logits, tokens, mask, k), s, label=f"c4 B={B} k={k}")


def test_fixed_step_loop_forced_state():
    # the pages' schedule (steps split evenly over the blocks): a 512-token
    # generation in 16-row blocks with 128 steps takes 4 steps per block of
    # 4 tokens each; every step starts both sides from the oracle's state
    s = shape_c4(16, block_idx=2, batch=8)
    k = tokens_per_step(s.gen_len, 16, 128)
    tokens, mask = make_decode_state(s)
    per_step = []
    for step in range(16):
        logits = make_logits(s, "calibrated" if step % 2 == 0 else "peak", step=step)
        ref = _ref(s, logits, tokens, mask, k)
        g, _ = run_unmask(s, logits, tokens, mask, None, topk=k)
        compare_unmask(g, ref, s, label=f"topk loop step={step}")
        per_step.append(int(ref.n_decoded.sum()))
        tokens, mask = ref.tokens, ref.mask
        if ref.done.all():
            break
    say(f"  fixed-step loop k={k}: steps={len(per_step)} tokens/step={per_step}")
    assert ref.done.all() and len(per_step) == -(-16 // k)


def test_c5_ragged_advance_done_list():
    # 64 sequences (above the 48 of the one-wave finished-sequence list)
    s = shape_c5()
    logits = make_logits(s, "calibrated")
    tokens, mask = make_decode_state(s, n_masked_c5(s))
    say("c5 topk ragged + advance")
    g, reps = run_unmask(s, logits, tokens, mask, None, ragged=True, flags=1, reps=2, topk=3)
    ref = _ref(s, logits, tokens, mask, 3, advance=True)
    compare_unmask(g, ref, s, label="c5 topk")
    if not ref.tie_step.any():
        assert g["n_done"] == ref.n_done and np.array_equal(g["done_seqs"], ref.done_seqs)
        assert np.array_equal(g["block_idxs"], ref.block_idxs)
    assert ref.n_done > 0
    assert np.array_equal(reps[0]["done_seqs"], reps[1]["done_seqs"])


def test_equal_confidences_take_lower_offset():
    # identical rows tie exactly on the GPU too: the lower offsets win
    s = shape_custom("ties", "bf16", 2, 1, 1, 8, [3, 9], 16, 8, [1, 0], 3000, cfg_id=62)
    logits = make_logits(s, "calibrated")
    logits[:, 5] = logits[:, 1]
    logits[:, 6] = logits[:, 1]
    logits[:, 1, 7] = logits[:, 1].max() + 4.0          # make the tied rows the most confident
    logits[:, 5] = logits[:, 1]
    logits[:, 6] = logits[:, 1]
    tokens, mask = make_decode_state(s, [8, 8])
    g, _ = run_unmask(s, logits, tokens, mask, None, ragged=True, topk=2)
    ref = _ref(s, logits, tokens, mask, 2)
    compare_unmask(g, ref, s, label="ties")
    assert list(g["decoded_pos"][0, :2]) == [1, 5] == list(ref.decoded_pos[0, :2])


def test_rejects_k_below_one():
    s = shape_custom("bad", "bf16", 1, 1, 1, 8, [3], 16, 8, [1], 300, cfg_id=63)
    logits = make_logits(s, "peak")
    tokens, mask = make_decode_state(s, [4])
    with pytest.raises(fd.FdllmError):
        run_unmask(s, logits, tokens, mask, None, topk=0)
