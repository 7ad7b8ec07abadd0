"""GPU parity: fdllm_unmask_threshold against the fp64 oracle (decisions
bit-exact except oracle-flagged near ties, confidences within 1e-6)."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, compare_unmask, require_gpu, run_unmask, say, to_dev
from oracle import unmask_ref
from workloads import (make_decode_state, make_logits, n_masked_c5, shape_c1, shape_c2, shape_c3,
                       shape_c4, shape_c5, shape_custom)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _ref(s, logits, tokens, mask, tau, advance=False):
    return unmask_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, tau,
                      advance=advance)


@pytest.mark.parametrize("recipe,tau", [("spike", 0.9), ("calibrated", 0.5), ("calibrated", 0.8),
                                        ("spike", 1.0), ("spike", 0.0)])
def test_c1_tiny_f32(recipe, tau):
    s = shape_c1()
    logits = make_logits(s, recipe)
    tokens, mask = make_decode_state(s, 20)
    say(f"c1 unmask {recipe} tau={tau}")
    g, reps = run_unmask(s, logits, tokens, mask, tau, reps=2)
    compare_unmask(g, _ref(s, logits, tokens, mask, tau), s, label=f"c1 {recipe} {tau}")
    for key in ("tokens", "mask", "n_decoded", "decoded_pos"):
        assert np.array_equal(reps[0][key], reps[1][key])


@pytest.mark.parametrize("recipe", ["peak", "calibrated"])
@pytest.mark.parametrize("tau", [0.7, 0.9, 1.0])
def test_c2_llada(recipe, tau):
    s = shape_c2(3)
    logits = make_logits(s, recipe)
    tokens, mask = make_decode_state(s)
    say(f"c2 unmask {recipe} tau={tau}")
    g, _ = run_unmask(s, logits, tokens, mask, tau)
    ref = _ref(s, logits, tokens, mask, tau)
    compare_unmask(g, ref, s, label=f"c2 {recipe} {tau}")
    if tau >= 1.0:
        assert g["n_decoded"][0] == 1


@pytest.mark.parametrize("recipe", ["peak", "calibrated"])
def test_c3_dream(recipe):
    s = shape_c3(5)
    logits = make_logits(s, recipe)
    tokens, mask = make_decode_state(s)
    say(f"c3 unmask {recipe}")
    g, _ = run_unmask(s, logits, tokens, mask, 0.9)
    compare_unmask(g, _ref(s, logits, tokens, mask, 0.9), s, label=f"c3 {recipe}")


@pytest.mark.parametrize("B", [4, 8, 16, 32, 64, 128])
def test_c4_block_sweep_first_step(B):
    s = shape_c4(B, block_idx=1)
    logits = make_logits(s, "calibrated")
    tokens, mask = make_decode_state(s)
    say(f"c4 unmask B={B}")
    g, _ = run_unmask(s, logits, tokens, mask, 0.8)
    compare_unmask(g, _ref(s, logits, tokens, mask, 0.8), s, label=f"c4 B={B}")


@pytest.mark.parametrize("tau", [0.5, 0.6, 0.7, 0.8, 0.9, 1.0])
def test_c4_decode_loop_forced_state(tau):
    # In-block loop, logits regenerated per step; both sides start each step
    # from the oracle's tokens and mask, so one flagged tie cannot cascade.
    s = shape_c4(16, block_idx=3, batch=8)
    tokens, mask = make_decode_state(s)
    per_step = []
    excluded = 0
    for step in range(64):
        logits = make_logits(s, "calibrated" if step % 2 == 0 else "peak", step=step)
        ref = _ref(s, logits, tokens, mask, tau)
        g, _ = run_unmask(s, logits, tokens, mask, tau)
        excluded += compare_unmask(g, ref, s, label=f"c4 loop tau={tau} step={step}")
        per_step.append(int(ref.n_decoded.sum()))
        tokens, mask = ref.tokens, ref.mask
        if ref.done.all():
            break
    say(f"  c4 loop tau={tau}: steps={len(per_step)} tokens/step={per_step} excluded={excluded}")
    assert ref.done.all()
    if tau >= 1.0:
        assert all(n == s.batch for n in per_step)


def test_c5_ragged_advance_done_list():
    s = shape_c5()
    logits = make_logits(s, "calibrated")
    tokens, mask = make_decode_state(s, n_masked_c5(s))
    say("c5 unmask ragged + advance")
    g, reps = run_unmask(s, logits, tokens, mask, 0.6, ragged=True, flags=1, reps=2)
    ref = _ref(s, logits, tokens, mask, 0.6, advance=True)
    compare_unmask(g, ref, s, label="c5")
    if not ref.tie_step.any() and not ref.tie_tau.any():
        assert g["n_done"] == ref.n_done and np.array_equal(g["done_seqs"], ref.done_seqs)
        assert np.array_equal(g["block_idxs"], ref.block_idxs)
    assert ref.n_done > 0
    assert np.array_equal(reps[0]["done_seqs"], reps[1]["done_seqs"])


EDGE = [
    # name, dtype, V, b, B, P, G, k, n_masked, tau
    ("vocab_tail", "bf16", 1000, 2, 8, [3, 5], 16, [1, 0], [8, 3], 0.3),
    ("vocab_7", "bf16", 7, 2, 4, [1, 2], 8, [0, 1], [4, 2], 0.4),
    ("f32_odd", "f32", 4099, 3, 8, [9, 2, 0], 16, [0, 1, 1], [5, 8, 1], 0.2),
    ("tau_one", "bf16", 5000, 2, 16, [4, 8], 32, [1, 0], [16, 9], 1.0),
    ("tau_neg", "bf16", 5000, 2, 16, [4, 8], 32, [1, 0], [16, 9], -1.0),
    ("block1", "bf16", 3000, 4, 1, [1, 2, 3, 4], 4, [0, 1, 2, 3], [1, 1, 0, 1], 0.9),
    ("nothing_masked", "bf16", 3000, 2, 8, [5, 5], 16, [0, 1], [0, 4], 0.9),
    ("big_vocab_f32", "f32", 152064, 2, 32, [64, 0], 64, [1, 0], [32, 17], 0.5),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: c[0])
def test_edge_cases(case):
    name, dt, V, b, B, P, G, k, nm, tau = case
    s = shape_custom(name, dt, b, 1, 1, 8, P, G, B, k, V, cfg_id=60)
    logits = make_logits(s, "calibrated" if V > 100 else "peak")
    tokens, mask = make_decode_state(s, nm)
    # logits of rows that are not masked are never read: poison them
    lg = logits.copy()
    for i in range(b):
        st = int(s.prompt_lens[i]) + int(s.block_idxs[i]) * B
        for t in range(B):
            if not mask[i, st + t]:
                lg[i, t] = np.nan
    say(f"edge {name}")
    g, _ = run_unmask(s, lg, tokens, mask, tau, ragged=not s.uniform)
    compare_unmask(g, _ref(s, logits, tokens, mask, tau), s, label=name)


def test_unaligned_rows_scalar_path():
    # logits rows at an odd element offset and stride force the scalar loads
    s = shape_custom("unal", "bf16", 2, 1, 1, 8, [3, 7], 32, 16, [0, 1], 2049, cfg_id=61)
    logits = make_logits(s, "calibrated")
    tokens, mask = make_decode_state(s, [16, 11])
    big = torch.zeros((2, 16, 2051), dtype=torch.bfloat16, device=DEV)
    big[:, :, 1:2050] = to_dev(logits, "bf16")
    view = big[:, :, 1:2050]
    say("edge unaligned")
    g, _ = run_unmask(s, None, tokens, mask, 0.7, ragged=True, logits_dev=view)
    compare_unmask(g, _ref(s, logits, tokens, mask, 0.7), s, label="unaligned")


def _vpos(it, u, thread, e):
    # vocab id of element e of the 16-byte vector that thread `thread` loads
    # in slot u of iteration it of a row read whole (bf16: 8 logits per
    # vector, 256 threads x 8 slots per iteration)
    return 8 * (it * 2048 + u * 256 + thread) + e


# (first, second) planted positions of an equal row maximum; the committed
# token must be the lower one (the oracle's argmax)
TIE_POSITIONS = [
    (_vpos(0, 0, 5, 2), _vpos(0, 0, 5, 6)),      # one vector
    (_vpos(0, 3, 7, 1), _vpos(4, 3, 7, 0)),      # one thread and slot, iterations 0 and 4
    (_vpos(8, 1, 100, 5), _vpos(9, 0, 10, 4)),   # the last two iterations, thread 100 then 10
    (_vpos(0, 0, 0, 7), _vpos(9, 2, 3, 0)),      # the first and the last iteration
    (_vpos(2, 0, 8, 6), _vpos(2, 0, 9, 3)),      # neighbouring threads
    (_vpos(1, 2, 11, 4), _vpos(1, 5, 11, 4)),    # one thread, slots 2 and 5
    (152064 - 9, 152064 - 1),                    # the row's last vector
    (_vpos(9, 1, 50, 3), None),                  # a single maximum in the last iteration
]


@pytest.mark.parametrize("chunks", [0, 4])
def test_tied_maxima_take_the_lowest_index(chunks):
    # Dream-7B vocabulary, 96 rows (read whole by default, or in 4 chunks):
    # every row's maximum 64.0 (exact in bf16) is planted at positions that
    # put the tie inside one thread's vector, across its iterations and
    # slots, in the last two iterations and across threads.
    s = shape_custom("ties", "bf16", 3, 1, 1, 8, [16, 40, 5], 64, 32, [0, 1, 0], 152064, cfg_id=62)
    logits = make_logits(s, "peak")
    for i in range(s.batch):
        for t in range(s.block_size):
            p1, p2 = TIE_POSITIONS[(i * s.block_size + t) % len(TIE_POSITIONS)]
            logits[i, t, p1] = 64.0
            if p2 is not None:
                logits[i, t, p2] = 64.0
    tokens, mask = make_decode_state(s, 32)
    fd_tuning = __import__("block_wise_kv_amd").set_tuning
    fd_tuning(unmask_wgs=4 * s.batch * s.block_size if chunks else 0)
    try:
        say(f"ties chunks={chunks or 1}")
        g, _ = run_unmask(s, logits, tokens, mask, 0.3, ragged=True)
    finally:
        fd_tuning()
    ref = _ref(s, logits, tokens, mask, 0.3)
    compare_unmask(g, ref, s, label=f"ties {chunks}")
    for i in range(s.batch):
        start = int(s.prompt_lens[i]) + int(s.block_idxs[i]) * s.block_size
        for t in range(s.block_size):
            p1, _ = TIE_POSITIONS[(i * s.block_size + t) % len(TIE_POSITIONS)]
            assert g["tokens"][i, start + t] == p1, (i, t)
