"""Pins for the oracle's confidence-threshold unmasking (CPU only)."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import NEAR_TIE, decode_block_ref, row_confidence, unmask_ref
from workloads import (calibrated_targets, make_decode_state, make_logits, shape_c1,
                       shape_custom)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _shape(b=2, B=8, V=8, P=(3, 5), G=16, k=(1, 0), dtype="f32", cfg=77):
    return shape_custom("u", dtype, b, 1, 1, 8, list(P)[:b], G, B, list(k)[:b], V, cfg_id=cfg)


# ---------------------------------------------------------------------------
# confidence of one row
# ---------------------------------------------------------------------------

def check_conf_library(rc):
    # conf = the largest softmax probability (scipy) and tok = the first argmax
    g = np.random.default_rng(3)
    for V in (2, 7, 1024, 126464):
        row = (g.standard_normal(V) * 3).astype(np.float32)
        c, tok, m, Z = rc(row)
        p = scipy.special.softmax(row.astype(np.float64))
        assert abs(c - p.max()) <= 1e-14
        assert tok == int(np.argmax(row))


def check_conf_sigmoid(rc):
    # a second formula: conf = sigmoid(l* - logsumexp of the other logits)
    g = np.random.default_rng(4)
    for _ in range(20):
        row = g.standard_normal(500) * 2
        c, tok, _, _ = rc(row)
        others = np.delete(row, tok)
        want = scipy.special.expit(row[tok] - scipy.special.logsumexp(others))
        assert abs(c - want) <= 1e-14


def check_conf_calibrated(rc):
    # the calibrated recipe sets the seeded token's probability to u exactly
    # before quantisation (fp32 here, so only float32 rounding remains)
    s = _shape(b=3, B=8, V=4096, cfg=78)
    x = make_logits(s, "calibrated")
    u = calibrated_targets(s)
    for i in range(3):
        for t in range(8):
            c, _, _, _ = rc(x[i, t])
            assert abs(c - u[i, t]) <= 2e-5


def check_conf_golden(rc):
    with open(os.path.join(GOLDEN, "unmask_hand.json")) as f:
        g = json.load(f)
    env = {"exp": math.exp, "e": math.e}
    for t, (row, expr, tok) in enumerate(zip(g["logits"], g["conf_expr"], g["tok"])):
        if expr is None:
            continue
        c, tk, _, _ = rc(np.array(row, float))
        assert abs(c - eval(expr, {"__builtins__": {}}, env)) <= 1e-14
        assert tk == tok


def check_conf_bounds(rc):
    g = np.random.default_rng(5)
    for V in (2, 3, 64):
        for _ in range(50):
            row = np.round(g.standard_normal(V) * 4)  # integer logits -> frequent ties
            c, tok, m, _ = rc(row)
            assert 1.0 / V - 1e-15 <= c <= 1.0 + 1e-15
            assert row[tok] == m and np.all(row[:tok] < m)
            if c > 0.5:
                assert np.sum(row == m) == 1


CONF_CHECKS = [check_conf_library, check_conf_sigmoid, check_conf_calibrated, check_conf_golden,
               check_conf_bounds]


@pytest.mark.parametrize("check", CONF_CHECKS, ids=lambda c: c.__name__)
def test_conf_pin(check):
    check(row_confidence)


# ---------------------------------------------------------------------------
# the unmask step
# ---------------------------------------------------------------------------

def _golden_case():
    with open(os.path.join(GOLDEN, "unmask_hand.json")) as f:
        g = json.load(f)
    P, G, B, k, V = g["P"], g["G"], g["B"], g["k"], g["V"]
    Lcap = P + G
    tokens = np.full((1, Lcap), 5, np.int32)
    mask = np.zeros((1, Lcap), np.uint8)
    start = P + k * B
    mask[0, start:start + B] = g["mask_block"]
    mask[0, start + B:] = 1
    tokens[mask == 1] = V
    logits = np.array([[[float(x) for x in row] for row in g["logits"]]])
    return g, tokens, mask, logits, start


def check_unmask_golden(um):
    g, tokens, mask, logits, start = _golden_case()
    for case in g["cases"]:
        r = um(logits, tokens, mask, [g["P"]], g["G"], g["B"], [g["k"]], case["tau"])
        dec = case["decoded"]
        assert list(r.decoded_pos[0, :len(dec)]) == dec and np.all(r.decoded_pos[0, len(dec):] == -1)
        assert r.n_decoded[0] == len(dec)
        for t, tok in case["tokens"].items():
            assert r.tokens[0, start + int(t)] == tok and r.mask[0, start + int(t)] == 0
        untouched = [t for t in range(g["B"]) if t not in dec]
        for t in untouched:
            assert r.tokens[0, start + t] == tokens[0, start + t]
            assert r.mask[0, start + t] == mask[0, start + t]
        assert bool(r.fallback[0]) == case["fallback"]
        assert bool(r.done[0]) == case["done"]
        # nothing outside the block changes
        outside = np.ones(tokens.shape[1], bool)
        outside[start:start + g["B"]] = False
        assert np.array_equal(r.tokens[0, outside], tokens[0, outside])
        assert np.array_equal(r.mask[0, outside], mask[0, outside])


def _random_case(seed, b=3, B=8, V=8, scale=2.0):
    s = _shape(b=b, B=B, V=V, P=(3, 5, 4, 2)[:b], k=(1, 0, 1, 0)[:b], cfg=seed)
    g = np.random.default_rng(seed)
    logits = g.standard_normal((b, B, V)) * scale
    nm = g.integers(1, B + 1, size=b)
    tokens, mask = make_decode_state(s, nm)
    return s, logits, tokens, mask


def check_tau_one_single_token(um):
    # A threshold of 1 or more can never be exceeded, so every step takes the
    # fallback and decodes exactly one token: the most confident masked row.
    # Rows with conf == 1.0 exactly (huge logit gaps) make '>=' detectable.
    for seed in range(6):
        s, logits, tokens, mask = _random_case(seed)
        logits[:, 1, :] = 0.0
        logits[:, 1, 2] = 900.0
        logits[:, 3, :] = 0.0
        logits[:, 3, 5] = 900.0
        for tau in (1.0, 1.5):
            r = um(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, tau)
            for i in range(s.batch):
                start = int(s.prompt_lens[i]) + int(s.block_idxs[i]) * s.block_size
                masked = [t for t in range(s.block_size) if mask[i, start + t]]
                assert r.n_decoded[i] == 1
                confs = [row_confidence(logits[i, t])[0] for t in masked]
                best = masked[int(np.argmax(confs))]
                assert r.decoded_pos[i, 0] == best
                assert r.tokens[i, start + best] == int(np.argmax(logits[i, best]))


def check_tau_low_whole_block(um):
    # If every masked confidence exceeds the threshold, the whole block is
    # decoded in one step (and the block is done).
    for seed in range(6):
        s, logits, tokens, mask = _random_case(seed)
        for tau in (0.0, -1.0, 1.0 / 8 - 1e-3):
            r = um(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, tau)
            for i in range(s.batch):
                start = int(s.prompt_lens[i]) + int(s.block_idxs[i]) * s.block_size
                masked = [t for t in range(s.block_size) if mask[i, start + t]]
                assert list(r.decoded_pos[i, :len(masked)]) == masked
                assert r.done[i] and not r.fallback[i]
                for t in masked:
                    assert r.tokens[i, start + t] == int(np.argmax(logits[i, t]))


def check_monotone(um):
    # Raising the threshold can only shrink the decoded set (no fallback).
    for seed in range(6):
        s, logits, tokens, mask = _random_case(seed, B=8, V=6, scale=3.0)
        prev = None
        for tau in np.linspace(0.1, 0.95, 12):
            r = um(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, tau)
            sets = [set(r.decoded_pos[i][r.decoded_pos[i] >= 0]) if not r.fallback[i] else None
                    for i in range(s.batch)]
            if prev is not None:
                for a, b_ in zip(prev, sets):
                    if a is not None and b_ is not None:
                        assert b_ <= a
            prev = sets


def _brute(logits_row_list, masked, tau):
    """Sort-based restatement: probabilities sorted descending per row."""
    conf, tok = {}, {}
    for t in masked:
        row = np.asarray(logits_row_list[t], float)
        order = sorted(range(len(row)), key=lambda v: (-row[v], v))
        p = np.exp(row - row[order[0]])
        conf[t] = p[order[0]] / p.sum()
        tok[t] = order[0]
    passing = [t for t in masked if conf[t] > tau]
    if not passing and masked:
        passing = [sorted(masked, key=lambda t: (-conf[t], t))[0]]
    return sorted(passing), tok


def check_brute_force(um):
    # every mask pattern of a 6-position block, vocabulary <= 8
    g = np.random.default_rng(9)
    B, V = 6, 5
    s = _shape(b=1, B=B, V=V, P=(2,), G=12, k=(1,))
    start = 2 + B
    for tau in (0.3, 0.5, 0.7):
        logits = np.round(g.standard_normal((1, B, V)) * 3) / 2  # ties happen
        for bits in itertools.product([0, 1], repeat=B):
            tokens = np.full((1, 2 + 12), 1, np.int32)
            mask = np.zeros((1, 14), np.uint8)
            mask[0, start:start + B] = bits
            r = um(logits, tokens, mask, s.prompt_lens, s.gen_len, B, s.block_idxs, tau)
            masked = [t for t in range(B) if bits[t]]
            want, tok = _brute(logits[0], masked, tau)
            got = list(r.decoded_pos[0][r.decoded_pos[0] >= 0])
            assert got == want, (bits, tau, got, want)
            for t in want:
                assert r.tokens[0, start + t] == tok[t]


def check_unread_rows(um):
    # logits rows of unmasked positions are never read
    for seed in range(3):
        s, logits, tokens, mask = _random_case(seed)
        r1 = um(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, 0.4)
        lg = logits.copy()
        for i in range(s.batch):
            start = int(s.prompt_lens[i]) + int(s.block_idxs[i]) * s.block_size
            for t in range(s.block_size):
                if not mask[i, start + t]:
                    lg[i, t] = np.nan
        r2 = um(lg, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, 0.4)
        assert np.array_equal(r1.tokens, r2.tokens) and np.array_equal(r1.mask, r2.mask)


def check_advance_and_done(um):
    s, logits, tokens, mask = _random_case(1)
    r = um(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, -1.0,
           advance=True)
    assert r.done.all() and list(r.done_seqs) == list(range(s.batch))
    nb = s.gen_len // s.block_size
    assert np.array_equal(r.block_idxs, np.where(s.block_idxs + 1 < nb, s.block_idxs + 1,
                                                 s.block_idxs))
    # the last block is never advanced past the end
    last = s.block_idxs.copy()
    last[:] = s.gen_len // s.block_size - 1
    tk, mk = tokens.copy(), mask.copy()
    for i in range(s.batch):
        mk[i, :] = 0
        st = int(s.prompt_lens[i]) + int(last[i]) * s.block_size
        mk[i, st] = 1
    r = um(logits, tk, mk, s.prompt_lens, s.gen_len, s.block_size, last, 0.99, advance=True)
    assert r.done.all() and np.array_equal(r.block_idxs, last)


UNMASK_CHECKS = [check_unmask_golden, check_tau_one_single_token, check_tau_low_whole_block,
                 check_monotone, check_brute_force, check_unread_rows, check_advance_and_done]


@pytest.mark.parametrize("check", UNMASK_CHECKS, ids=lambda c: c.__name__)
def test_unmask_pin(check):
    check(unmask_ref)


def test_decode_block_step_counts():
    # the in-block loop ends in 1..m steps for m masked rows, every step
    # decodes at least one token, and tau >= 1 takes exactly m steps
    s = shape_c1()
    tokens, mask = make_decode_state(s, 20)
    for tau, exact in ((0.9, None), (1.0, 20), (0.0, 1)):
        steps = decode_block_ref(lambda st: make_logits(s, step=st), tokens, mask, s.prompt_lens,
                                 s.gen_len, s.block_size, s.block_idxs, tau)
        assert 1 <= len(steps) <= 20
        assert all(int(n[0]) >= 1 for n in steps)
        assert sum(int(n[0]) for n in steps) == 20
        if exact is not None:
            assert len(steps) == exact


def test_near_tie_flags():
    s = _shape(b=1, B=4, V=4, P=(2,), G=8, k=(1,))
    tokens, mask = make_decode_state(s, 4)
    logits = np.zeros((1, 4, 4))
    logits[0, 0] = [0.0, 0.0, 0.0, 0.0]          # conf 0.25, exact top-2 tie
    logits[0, 1] = [math.log(3 * 0.9 / 0.1), 0, 0, 0]  # conf 0.9 -> at tau
    logits[0, 2] = [2.0, 0, 0, 0]
    logits[0, 3] = [2.0, 0, 0, 0]                # same conf as row 2
    r = unmask_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, 4, s.block_idxs, 0.9)
    assert r.tie_top2[0, 0] and not r.tie_top2[0, 2]
    assert r.tie_tau[0, 1]
    assert r.tie_step[0]            # the decision hinges on row 1 vs tau
    r = unmask_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, 4, s.block_idxs, 0.95)
    assert r.fallback[0] and r.decoded_pos[0, 0] == 1 and not r.tie_step[0]


# ---------------------------------------------------------------------------
# mutation tests
# ---------------------------------------------------------------------------

def _mutant(kind):
    from oracle import fdllm_oracle as fo

    def rc(row):
        l = np.asarray(row, np.float64)
        m = l.max()
        tok = int(np.flatnonzero(l == m)[-1 if kind == "last_argmax" else 0])
        if kind == "no_max_shift":
            Z = float(np.exp(l).sum()) / math.exp(m) if m < 700 else float("inf")
        else:
            Z = float(np.exp(l - m).sum())
        if kind == "conf_is_z":
            return Z, tok, float(m), Z
        if kind == "drop_term":
            Z = Z - float(np.exp(l[-1] - m)) + 1e-300 if l.size > 1 else Z
        return 1.0 / Z, tok, float(m), Z

    def um(logits, tokens, mask, prompt_lens, gen_len, block_size, block_idxs, threshold,
           advance=False):
        tokens = np.array(tokens, np.int32, copy=True)
        mask = np.array(mask, np.uint8, copy=True)
        bidx = np.array(block_idxs, np.int32, copy=True).reshape(-1)
        b, B = tokens.shape[0], block_size
        tau = float(np.float32(threshold))
        n_dec = np.zeros(b, np.int32); dpos = np.full((b, B), -1, np.int32)
        done = np.zeros(b, bool); fb = np.zeros(b, bool)
        for i in range(b):
            start = int(prompt_lens[i]) + int(bidx[i]) * B
            if kind == "off_by_block":
                start += B if bidx[i] == 0 else 0
            masked = [t for t in range(B) if mask[i, start + t] == 1]
            conf, tok = {}, {}
            for t in masked:
                conf[t], tok[t], _, _ = rc(logits[i][t])
            if kind == "ge":
                chosen = [t for t in masked if conf[t] >= tau]
            else:
                chosen = [t for t in masked if conf[t] > tau]
            if not chosen and masked and kind != "no_fallback":
                key = (lambda t: (conf[t], t)) if kind == "last_best" else (lambda t: (conf[t], -t))
                chosen = [max(masked, key=key)]
                fb[i] = True
            for t in chosen:
                tokens[i, start + t] = tok[t]
                mask[i, start + t] = 0
            chosen.sort()
            n_dec[i] = len(chosen); dpos[i, :len(chosen)] = chosen
            done[i] = not any(mask[i, start + t] == 1 for t in range(B))
            if advance and done[i] and bidx[i] + 1 < gen_len // B:
                bidx[i] += 1
        z = np.zeros((b, B), bool)
        return fo.UnmaskResult(tokens, mask, n_dec, dpos, np.full((b, B), np.nan), done,
                               np.flatnonzero(done).astype(np.int32), bidx, fb, z, z,
                               np.zeros(b, bool))
    return rc, um


@pytest.mark.parametrize("kind", ["last_argmax", "no_max_shift", "conf_is_z", "drop_term", "ge",
                                  "no_fallback", "last_best", "off_by_block"])
def test_pins_catch_planted_mistake(kind):
    rc, um = _mutant(kind)
    failures = 0
    for check in CONF_CHECKS:
        try:
            check(rc)
        except (AssertionError, OverflowError, FloatingPointError):
            failures += 1
    for check in UNMASK_CHECKS:
        try:
            check(um)
        except (AssertionError, IndexError):
            failures += 1
    assert failures > 0, f"no pin caught the planted mistake {kind!r}"


def test_unmutated_copy_passes_all_pins():
    rc, um = _mutant("none")
    for check in CONF_CHECKS:
        check(rc)
    for check in UNMASK_CHECKS:
        check(um)
