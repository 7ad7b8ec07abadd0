"""Pins for the oracle's attention (CPU only).

Each check is written as a function of the attention routine so that the
mutation tests at the bottom can plant a mistake in a copy of the oracle and
show that some pin fails.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attn_ref, fresh_range
from workloads import make_attn_inputs, shape_c1, shape_custom

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _small_shape(mode, hq=4, hkv=2, d=16, P=(5, 9), G=12, B=4, k=(1, 2)):
    return shape_custom("t", "f32", len(P), hq, hkv, d, list(P), G, B, list(k), 16)


# ---------------------------------------------------------------------------
# checks (each takes the attention routine under test)
# ---------------------------------------------------------------------------

def check_fresh_range(fr):
    # Hand-worked: prompt 64, gen 128, block 32, block index 1 -> the block is
    # positions 96..127; 96 cached prefix rows and 64 cached suffix rows.
    assert fr(64, 128, 32, 1, "dual") == (96, 128)
    assert fr(64, 128, 32, 1, "prefix") == (96, 192)
    assert fr(64, 128, 32, 1, "none") == (0, 192)
    assert fr(512, 256, 32, 7, "dual") == (736, 768)
    assert fr(512, 256, 32, 0, "prefix") == (512, 768)


def check_golden(attn):
    with open(os.path.join(GOLDEN, "attn_hand.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], float)[None, :, None, :]
    kn = np.array(g["k_new"], float)[None, :, None, :]
    vn = np.array(g["v_new"], float)[None, :, None, :]
    kc = np.array(g["k_cache"], float)[None, None]
    vc = np.array(g["v_cache"], float)[None, None]
    out = attn(q, kn, vn, kc, vc, [g["P"]], g["G"], g["B"], [g["k"]], g["mode"])
    env = {"exp": math.exp, "e": math.e}
    want = np.array([eval(s, {"__builtins__": {}}, env) for s in g["expected_expr"]])
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=0, atol=1e-14)


def _sdpa_rows(q, K, V, g_):
    """CPU float64 torch SDPA for one sequence: q [nq][Hq][d], K/V [L][Hkv][d]."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, enable_gqa=(g_ > 1))
    return o[0].numpy().transpose(1, 0, 2)


def check_none_vs_sdpa(attn):
    # No-cache mode: every key row is fresh, so the result is plain
    # bidirectional softmax attention over [0, L); torch's SDPA (no mask,
    # default 1/sqrt(d) scale, query head h -> kv head h // g) is the pin.
    s = _small_shape("none")
    a = make_attn_inputs(s, "none")
    q, kn, vn = (x.astype(np.float64) for x in (a.q, a.k_new, a.v_new))
    out = attn(q, kn, vn, None, None, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, "none")
    g_ = s.n_q_heads // s.n_kv_heads
    for i in range(s.batch):
        L = int(s.prompt_lens[i]) + s.gen_len
        want = _sdpa_rows(q[i, :L], kn[i, :L], vn[i, :L], g_)
        np.testing.assert_allclose(out[i, :L], want, rtol=0, atol=1e-12)
        assert np.isnan(out[i, L:]).all()


def _truth(s, seed):
    """Full-forward K/V, token-major [b][Lcap][Hkv][d], and queries per position."""
    K = _rand((s.batch, s.max_seq_len, s.n_kv_heads, s.head_dim), seed)
    V = _rand((s.batch, s.max_seq_len, s.n_kv_heads, s.head_dim), seed + 1)
    Q = _rand((s.batch, s.max_seq_len, s.n_q_heads, s.head_dim), seed + 2)
    return Q, K, V


def _mode_inputs(s, mode, Q, K, V, kc, vc):
    """Fresh rows of `mode` taken from the truth; caches given (head-major)."""
    cap = s.fresh_capacity(mode)
    q = np.full((s.batch, cap, s.n_q_heads, s.head_dim), 7.0)
    kn = np.full((s.batch, cap, s.n_kv_heads, s.head_dim), 7.0)
    vn = np.full((s.batch, cap, s.n_kv_heads, s.head_dim), 7.0)
    for i in range(s.batch):
        P, k = int(s.prompt_lens[i]), int(s.block_idxs[i])
        if mode == "dual":
            a0, a1 = P + k * s.block_size, P + (k + 1) * s.block_size
        elif mode == "prefix":
            a0, a1 = P + k * s.block_size, P + s.gen_len
        else:
            a0, a1 = 0, P + s.gen_len
        q[i, :a1 - a0] = Q[i, a0:a1]
        kn[i, :a1 - a0] = K[i, a0:a1]
        vn[i, :a1 - a0] = V[i, a0:a1]
    return q, kn, vn, kc, vc


def _block_rows(s, out, mode):
    """Output rows of the current block, [b][B][Hq][d]."""
    res = []
    for i in range(s.batch):
        P, k = int(s.prompt_lens[i]), int(s.block_idxs[i])
        off = {"dual": 0, "prefix": 0, "none": P + k * s.block_size}[mode]
        res.append(out[i, off:off + s.block_size])
    return np.stack(res)


def check_post_refresh_identity(attn):
    # Right after a refresh the cache holds exactly the full forward's K/V, so
    # dual and prefix caching reproduce the full recompute on the block rows.
    s = _small_shape("dual")
    Q, K, V = _truth(s, 11)
    kc = K.transpose(0, 2, 1, 3).copy()
    vc = V.transpose(0, 2, 1, 3).copy()
    outs = {}
    for mode in ("none", "prefix", "dual"):
        args = _mode_inputs(s, mode, Q, K, V, kc, vc)
        outs[mode] = _block_rows(s, attn(*args, s.prompt_lens, s.gen_len, s.block_size,
                                         s.block_idxs, mode), mode)
    np.testing.assert_allclose(outs["dual"], outs["none"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(outs["prefix"], outs["none"], rtol=0, atol=1e-12)


def check_nested_modes(attn):
    # Inject staleness into one cache region at a time.  The recomputed sets
    # nest (none > prefix > dual), so: a stale suffix or stale block rows in
    # the cache leave prefix == none while dual differs (suffix) or stays
    # equal (block rows are always recomputed); a stale prefix makes
    # prefix == dual != none.
    s = _small_shape("dual")
    Q, K, V = _truth(s, 21)
    base_k = K.transpose(0, 2, 1, 3).copy()
    base_v = V.transpose(0, 2, 1, 3).copy()
    for region in ("prefix", "block", "suffix"):
        kc, vc = base_k.copy(), base_v.copy()
        for i in range(s.batch):
            P, k = int(s.prompt_lens[i]), int(s.block_idxs[i])
            a0, a1, L = P + k * s.block_size, P + (k + 1) * s.block_size, P + s.gen_len
            lo, hi = {"prefix": (0, a0), "block": (a0, a1), "suffix": (a1, L)}[region]
            kc[i, :, lo:hi] += 0.5 * _rand(kc[i, :, lo:hi].shape, 99 + i)
            vc[i, :, lo:hi] += 0.5 * _rand(vc[i, :, lo:hi].shape, 199 + i)
        outs = {}
        for mode in ("none", "prefix", "dual"):
            args = _mode_inputs(s, mode, Q, K, V, kc, vc)
            outs[mode] = _block_rows(s, attn(*args, s.prompt_lens, s.gen_len, s.block_size,
                                             s.block_idxs, mode), mode)
        eq = lambda a, b: np.allclose(a, b, rtol=0, atol=1e-12)
        if region == "prefix":
            assert eq(outs["prefix"], outs["dual"]) and not eq(outs["prefix"], outs["none"])
        elif region == "block":
            assert eq(outs["dual"], outs["none"]) and eq(outs["prefix"], outs["none"])
        else:
            assert eq(outs["prefix"], outs["none"]) and not eq(outs["dual"], outs["none"])


def check_closed_forms(attn):
    s = _small_shape("dual", P=(6,), k=(1,))
    a = make_attn_inputs(s, "dual")
    q, kn, vn, kc, vc = (x.astype(np.float64) for x in (a.q, a.k_new, a.v_new, a.k_cache, a.v_cache))
    args = (s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, "dual")
    L = int(s.prompt_lens[0]) + s.gen_len
    nq = s.block_size
    # every value row equal to c -> output c
    c = np.arange(s.head_dim, dtype=float) * 0.25 - 1.0
    out = attn(q, kn, np.broadcast_to(c, vn.shape).copy(), kc, np.broadcast_to(c, vc.shape).copy(), *args)
    np.testing.assert_allclose(out[0, :nq], np.broadcast_to(c, out[0, :nq].shape), atol=1e-13)
    # q = 0 -> uniform weights -> mean of the L value rows the step reads
    out = attn(np.zeros_like(q), kn, vn, kc, vc, *args)
    a0 = int(s.prompt_lens[0]) + int(s.block_idxs[0]) * s.block_size
    for hq in range(s.n_q_heads):
        hk = hq // (s.n_q_heads // s.n_kv_heads)
        rows = np.concatenate([vc[0, hk, :a0], vn[0, :nq, hk], vc[0, hk, a0 + nq:L]])
        np.testing.assert_allclose(out[0, :nq, hq], np.broadcast_to(rows.mean(0), (nq, s.head_dim)),
                                   atol=1e-13)
    # one key aligned with a huge query dominates -> output ~ that key's value
    q2 = np.zeros_like(q)
    kc2 = kc.copy()
    kc2[0, :, 2] = 0.0
    kc2[0, :, 2, 0] = 1.0
    q2[0, :, :, 0] = 4000.0
    kn2 = kn.copy()
    kn2[..., 0] = np.minimum(kn2[..., 0], 0.5)
    kc2[..., 0] = np.where(np.arange(s.max_seq_len)[None, None, :] == 2, 1.0,
                           np.minimum(kc2[..., 0], 0.5))
    out = attn(q2, kn2, vn, kc2, vc, *args)
    for hq in range(s.n_q_heads):
        hk = hq // (s.n_q_heads // s.n_kv_heads)
        np.testing.assert_allclose(out[0, :nq, hq], np.broadcast_to(vc[0, hk, 2], (nq, s.head_dim)),
                                   atol=1e-9)


def check_gqa_and_permutation(attn):
    s = _small_shape("dual", hq=6, hkv=2, P=(5, 9, 7), k=(1, 2, 0))
    a = make_attn_inputs(s, "dual")
    q, kn, vn, kc, vc = (x.astype(np.float64) for x in (a.q, a.k_new, a.v_new, a.k_cache, a.v_cache))
    args = (s.gen_len, s.block_size)
    out = attn(q, kn, vn, kc, vc, s.prompt_lens, *args, s.block_idxs, "dual")
    g_ = 3
    # GQA == MHA with each kv head repeated for its g consecutive query heads
    rep = lambda x, ax: np.repeat(x, g_, axis=ax)
    out_mha = attn(q, rep(kn, 2), rep(vn, 2), rep(kc, 1), rep(vc, 1), s.prompt_lens, *args,
                   s.block_idxs, "dual")
    np.testing.assert_allclose(out, out_mha, rtol=0, atol=1e-13, equal_nan=True)
    # a ragged batch == each sequence alone; permuting the batch permutes outputs
    perm = np.array([2, 0, 1])
    out_p = attn(q[perm], kn[perm], vn[perm], kc[perm], vc[perm], s.prompt_lens[perm], *args,
                 s.block_idxs[perm], "dual")
    np.testing.assert_allclose(out_p, out[perm], rtol=0, atol=1e-13, equal_nan=True)
    for i in range(s.batch):
        sl = slice(i, i + 1)
        o1 = attn(q[sl], kn[sl], vn[sl], kc[sl], vc[sl], s.prompt_lens[sl], *args,
                  s.block_idxs[sl], "dual")
        np.testing.assert_allclose(o1[0], out[i], rtol=0, atol=1e-13, equal_nan=True)


def check_dual_vs_sdpa(attn):
    # Dual mode against SDPA over K/V assembled in this test from the
    # definition: cache rows outside the block, fresh rows inside it.
    s = _small_shape("dual", hq=4, hkv=1, P=(7, 3), k=(2, 0))
    a = make_attn_inputs(s, "dual")
    q, kn, vn, kc, vc = (x.astype(np.float64) for x in (a.q, a.k_new, a.v_new, a.k_cache, a.v_cache))
    out = attn(q, kn, vn, kc, vc, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, "dual")
    for i in range(s.batch):
        P, k = int(s.prompt_lens[i]), int(s.block_idxs[i])
        L, a0, B = P + s.gen_len, P + k * s.block_size, s.block_size
        K = kc[i].transpose(1, 0, 2)[:L].copy()
        V = vc[i].transpose(1, 0, 2)[:L].copy()
        K[a0:a0 + B] = kn[i, :B]
        V[a0:a0 + B] = vn[i, :B]
        want = _sdpa_rows(q[i, :B], K, V, s.n_q_heads)
        np.testing.assert_allclose(out[i, :B], want, rtol=0, atol=1e-12)


CHECKS = [check_golden, check_none_vs_sdpa, check_post_refresh_identity, check_nested_modes,
          check_closed_forms, check_gqa_and_permutation, check_dual_vs_sdpa]


def test_fresh_range():
    check_fresh_range(fresh_range)


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_attn_pin(check):
    check(attn_ref)


def test_c1_shape_is_finite_and_untouched_rows_nan():
    s = shape_c1()
    a = make_attn_inputs(s, "dual")
    out = attn_ref(a.q, a.k_new, a.v_new, a.k_cache, a.v_cache, s.prompt_lens, s.gen_len,
                   s.block_size, s.block_idxs, "dual")
    assert out.shape == (1, 32, 4, 64) and np.isfinite(out).all()


# ---------------------------------------------------------------------------
# mutation tests: a plausible mistake planted in a copy of the oracle must
# fail at least one pin
# ---------------------------------------------------------------------------

def _mutant(kind):
    def attn(q, k_new, v_new, k_cache, v_cache, prompt_lens, gen_len, block_size, block_idxs,
             mode, scale=None):
        q = np.asarray(q, np.float64)
        k_new = np.asarray(k_new, np.float64)
        v_new = np.asarray(v_new, np.float64)
        b, cap, Hq, d = q.shape
        Hkv = k_new.shape[2]
        g = Hq // Hkv
        sc = 1.0 / np.sqrt(d) if kind != "no_scale" else 1.0
        out = np.full((b, cap, Hq, d), np.nan)
        for i in range(b):
            P, k = int(prompt_lens[i]), int(block_idxs[i])
            L = P + gen_len
            a0, a1 = fresh_range(P, gen_len, block_size, k, mode)
            nq = a1 - a0
            if kind == "drop_suffix" and mode == "dual":
                L = a1
            for hk in range(Hkv):
                K = np.empty((L, d)); Vv = np.empty((L, d))
                for j in range(L):
                    fresh = a0 <= j < a1 and (j - a0) < k_new.shape[1]
                    if kind == "cache_only" and mode != "none":
                        fresh = False
                    if fresh:
                        jj = j if kind == "no_offset" else j - a0
                        jj = min(jj, k_new.shape[1] - 1)
                        K[j] = k_new[i, jj, hk]; Vv[j] = v_new[i, jj, hk]
                    else:
                        K[j] = k_cache[i, hk, j]; Vv[j] = v_cache[i, hk, j]
                heads = range(hk * g, (hk + 1) * g)
                if kind == "gqa_modulo":
                    heads = [h for h in range(Hq) if h % Hkv == hk]
                for h in heads:
                    S = (q[i, :nq, h] @ K.T) * sc
                    if kind == "causal":
                        pos = np.arange(a0, a0 + nq)[:, None]
                        S = np.where(np.arange(L)[None, :] <= pos, S, -np.inf)
                    S = S - S.max(axis=1, keepdims=True)
                    W = np.exp(S)
                    W = W / (W.sum(axis=0, keepdims=True) if kind == "wrong_axis"
                             else W.sum(axis=1, keepdims=True))
                    out[i, :nq, h] = W @ Vv
        return out
    return attn


@pytest.mark.parametrize("kind", ["no_scale", "cache_only", "no_offset", "gqa_modulo", "causal",
                                  "wrong_axis", "drop_suffix"])
def test_pins_catch_planted_mistake(kind):
    bad = _mutant(kind)
    failures = 0
    for check in CHECKS:
        try:
            check(bad)
        except (AssertionError, IndexError, ValueError):
            failures += 1
    assert failures > 0, f"no pin caught the planted mistake {kind!r}"


def test_unmutated_copy_passes_all_pins():
    good = _mutant("none")
    for check in CHECKS:
        check(good)
