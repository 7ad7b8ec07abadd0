"""Pins for the oracle's LM-head step: logits from the final hidden states,
and the unmasking rules applied to them (CPU only)."""
import math

import numpy as np
import pytest

from oracle import lmhead_logits_ref, lmhead_unmask_ref, unmask_ref, unmask_topk_ref
from workloads import make_decode_state, make_lmhead_inputs, shape_custom


def _shape(b=2, B=8, V=50, cfg=81):
    return shape_custom("lm", "bf16", b, 1, 1, 8, [6, 9][:b], 32, B, [1, 2][:b], V, cfg_id=cfg)


def check_brute_force(lf):
    # every logit is the plain dot product of a hidden row with a weight row:
    # exact with integers, fsum-accurate with floats (H != V, so a transposed
    # operand cannot pass by shape)
    g = np.random.default_rng(11)
    xi = g.integers(-5, 6, size=(2, 3, 5))
    wi = g.integers(-5, 6, size=(7, 5))
    got = lf(xi.astype(np.float64), wi.astype(np.float64))
    assert got.shape == (2, 3, 7)
    for i in range(2):
        for t in range(3):
            for v in range(7):
                assert got[i, t, v] == sum(int(xi[i, t, k]) * int(wi[v, k]) for k in range(5))
    xf = g.standard_normal((2, 4, 9))
    wf = g.standard_normal((6, 9))
    got = lf(xf, wf)
    for i in range(2):
        for t in range(4):
            for v in range(6):
                ref = math.fsum(float(xf[i, t, k]) * float(wf[v, k]) for k in range(9))
                assert abs(got[i, t, v] - ref) <= 1e-12 * (1 + abs(ref))


def check_one_hot(lf):
    # w[v] = a * e_pi(v) picks hidden coordinate pi(v); all-zero rows give 0
    g = np.random.default_rng(12)
    H = 6
    pi = g.permutation(H)
    w = np.zeros((H + 2, H))
    for v in range(H):
        w[v, pi[v]] = 2.5
    x = g.standard_normal((1, 4, H))
    got = lf(x, w)
    for v in range(H):
        assert np.array_equal(got[..., v], 2.5 * x[..., pi[v]])
    assert np.all(got[..., H:] == 0.0)


def check_zero_hidden(lf):
    # no bias: a zero hidden state has all-zero logits
    w = np.random.default_rng(13).standard_normal((9, 4))
    assert np.all(lf(np.zeros((2, 3, 4)), w) == 0.0)


def check_grid_exact(lf):
    # grid inputs: logit * 2^e_r is the exact integer dot product of the codes
    s = _shape(V=61)
    inp = make_lmhead_inputs(s, 48)
    got = lf(inp.x, inp.weight())
    scale = np.exp2(inp.row_exp.astype(np.float64))[:, :, None]
    cx = np.rint(inp.x.astype(np.float64) * scale).astype(np.int64)
    assert np.array_equal(cx.astype(np.float64), inp.x * scale)  # the codes are integers
    exact = cx @ inp.w_codes.astype(np.int64).T
    assert np.array_equal(got * scale, exact.astype(np.float64))


def check_planted_argmax(lf):
    # rows of a Hadamard matrix are orthogonal: hidden state = weight row v*
    # gives logit H at v* and 0 elsewhere
    H = 8
    had = np.array([[1.0]])
    while had.shape[0] < H:
        had = np.block([[had, had], [had, -had]])
    x = had[[5, 2, 7]][None]
    got = lf(x, had)
    assert list(np.argmax(got[0], axis=-1)) == [5, 2, 7]
    for r, v in enumerate([5, 2, 7]):
        assert got[0, r, v] == H and np.count_nonzero(got[0, r]) == 1


LOGIT_CHECKS = [check_brute_force, check_one_hot, check_zero_hidden, check_grid_exact,
                check_planted_argmax]


@pytest.mark.parametrize("check", LOGIT_CHECKS, ids=lambda c: c.__name__)
def test_logits_pin(check):
    check(lmhead_logits_ref)


def _brute_logits(x, w):
    b, B, H = x.shape
    out = np.empty((b, B, w.shape[0]))
    for i in range(b):
        for t in range(B):
            for v in range(w.shape[0]):
                out[i, t, v] = math.fsum(float(x[i, t, k]) * float(w[v, k]) for k in range(H))
    return out


@pytest.mark.parametrize("rule", ["threshold", "topk"])
def test_unmask_on_brute_force_logits(rule):
    # the composed step equals the pinned unmasking rules on brute-force logits
    s = _shape()
    inp = make_lmhead_inputs(s, 24)
    tokens, mask = make_decode_state(s, [8, 5])
    w = inp.weight()
    logits = _brute_logits(inp.x, w)
    args = (tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs)
    if rule == "threshold":
        got = lmhead_unmask_ref(inp.x, w, *args, threshold=0.6)
        ref = unmask_ref(logits, *args, 0.6)
    else:
        got = lmhead_unmask_ref(inp.x, w, *args, k=3)
        ref = unmask_topk_ref(logits, *args, 3)
    for f in ("tokens", "mask", "n_decoded", "decoded_pos", "done"):
        assert np.array_equal(getattr(got, f), getattr(ref, f)), f
    np.testing.assert_allclose(got.conf, ref.conf, rtol=1e-12, atol=0)
    assert int(got.n_decoded.sum()) > 0
    with pytest.raises(ValueError):
        lmhead_unmask_ref(inp.x, w, *args)
    with pytest.raises(ValueError):
        lmhead_unmask_ref(inp.x, w, *args, threshold=0.5, k=2)


def test_grid_recipe_spans_confidences():
    # the grid recipe gives unsure and confident rows at a real vocabulary
    # size (so a threshold sweep decodes varying numbers of tokens)
    s = shape_custom("lm", "bf16", 1, 1, 1, 8, [4], 32, 32, [0], 20000, cfg_id=82)
    inp = make_lmhead_inputs(s, 256)
    logits = lmhead_logits_ref(inp.x, inp.weight())
    m = logits.max(-1, keepdims=True)
    conf = 1.0 / np.exp(logits - m).sum(-1)
    assert conf.min() < 0.2 and conf.max() > 0.8


# ---------------------------------------------------------------------------
# mutation tests: a planted mistake in a copy of the logits step fails a pin
# ---------------------------------------------------------------------------

def _mutant(kind):
    def lf(x, w):
        x = np.asarray(x, np.float64)
        w = np.asarray(w, np.float64)
        if kind == "transposed":
            return x @ w.reshape(w.shape[1], w.shape[0])
        if kind == "drop_last_dim":
            return x[..., :-1] @ w[:, :-1].T
        if kind == "bias":
            return x @ w.T + 0.25
        if kind == "scaled":
            return (x @ w.T) / np.sqrt(x.shape[-1])
        if kind == "row_shift":
            return np.roll(x, 1, axis=-2) @ w.T
        if kind == "vocab_shift":
            return np.roll(x @ w.T, 1, axis=-1)
        return x @ w.T
    return lf


@pytest.mark.parametrize("kind", ["transposed", "drop_last_dim", "bias", "scaled", "row_shift",
                                  "vocab_shift"])
def test_pins_catch_planted_mistake(kind):
    lf = _mutant(kind)
    failures = 0
    for check in LOGIT_CHECKS:
        try:
            check(lf)
        except (AssertionError, ValueError):
            failures += 1
    assert failures > 0, f"no pin caught the planted mistake {kind!r}"


def test_unmutated_copy_passes_all_pins():
    lf = _mutant("none")
    for check in LOGIT_CHECKS:
        check(lf)
