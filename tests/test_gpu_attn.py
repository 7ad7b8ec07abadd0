"""GPU parity: fdllm_block_attn against the fp64 oracle."""
import numpy as np
import pytest

from gpu_util import (check_attn, nq_of, oracle_attn_subset, require_gpu, run_attn, say)
from oracle import attn_ref
from workloads import (make_attn_inputs, shape_c1, shape_c2, shape_c3, shape_c4, shape_c5,
                       shape_custom)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _full(inp):
    s = inp.shape
    return attn_ref(inp.q, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache, s.prompt_lens, s.gen_len,
                    s.block_size, s.block_idxs, inp.mode)


@pytest.mark.parametrize("mode", ["dual", "prefix", "none"])
def test_c1_tiny_f32(mode):
    s = shape_c1()
    inp = make_attn_inputs(s, mode)
    say(f"c1 f32 {mode}")
    out, _, _ = run_attn(inp)
    check_attn(out, _full(inp), inp, label=f"c1 {mode}")


@pytest.mark.parametrize("k", range(8))
def test_c2_llada_dual(k):
    s = shape_c2(k)
    inp = make_attn_inputs(s, "dual", variant=k)
    say(f"c2 dual k={k}")
    out, outs, _ = run_attn(inp, reps=2)
    check_attn(out, _full(inp), inp, label=f"c2 k={k}")
    assert np.array_equal(outs[0], outs[1], equal_nan=True), "second run differs bitwise"


SMALL = [
    # name, dtype, b, Hq, Hkv, d, P, G, B, k, mode
    ("mha_aligned", "bf16", 2, 4, 4, 128, [64, 64], 64, 32, [1, 1], "dual"),
    ("gqa7_ragged", "bf16", 3, 14, 2, 128, [37, 100, 5], 96, 32, [0, 2, 1], "dual"),
    ("block4", "bf16", 2, 8, 2, 128, [13, 40], 16, 4, [3, 0], "dual"),
    ("block8_prefix", "bf16", 2, 8, 4, 128, [29, 3], 48, 8, [1, 5], "prefix"),
    ("prefix_long", "bf16", 1, 4, 1, 128, [300], 200, 40, [2], "prefix"),
    ("none_gqa", "bf16", 2, 6, 3, 128, [17, 70], 32, 16, [0, 1], "none"),
    ("none_tail", "bf16", 1, 2, 2, 128, [1], 4, 4, [0], "none"),
    ("one_key_block", "bf16", 1, 2, 1, 128, [0], 1, 1, [0], "dual"),
    ("bf16_d64_gqa", "bf16", 2, 8, 2, 64, [33, 9], 64, 16, [1, 3], "dual"),
    ("bf16_d64_prefix", "bf16", 2, 4, 4, 64, [10, 21], 32, 8, [2, 0], "prefix"),
    ("f32_d128_gqa", "f32", 2, 4, 2, 128, [33, 9], 64, 16, [1, 3], "dual"),
    ("f32_d64_prefix", "f32", 2, 4, 4, 64, [10, 21], 32, 8, [2, 0], "prefix"),
    ("f32_none", "f32", 1, 3, 1, 64, [7], 9, 3, [1], "none"),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_small_cases(case):
    name, dt, b, hq, hkv, d, P, G, B, k, mode = case
    s = shape_custom(name, dt, b, hq, hkv, d, P, G, B, k, 64, cfg_id=50)
    inp = make_attn_inputs(s, mode)
    ragged = not s.uniform
    say(f"small {name} ragged={ragged}")
    out, outs, _ = run_attn(inp, ragged=ragged, reps=2)
    check_attn(out, _full(inp), inp, label=name)
    assert np.array_equal(outs[0], outs[1], equal_nan=True)
    if not ragged:
        # the same batch through the per-sequence (device array) path
        out2, _, _ = run_attn(inp, ragged=True)
        assert np.array_equal(out, out2, equal_nan=True)


@pytest.mark.parametrize("mode,k", [("dual", 0), ("dual", 17), ("dual", 31), ("prefix", 0), ("prefix", 30)])
def test_c3_dream_gqa(mode, k):
    s = shape_c3(k)
    inp = make_attn_inputs(s, mode, variant=k)
    say(f"c3 {mode} k={k}")
    out, outs, _ = run_attn(inp, reps=2)
    check_attn(out, _full(inp), inp, label=f"c3 {mode} k={k}")
    assert np.array_equal(outs[0], outs[1], equal_nan=True)


@pytest.mark.parametrize("B", [4, 8, 16, 32, 64, 128])
def test_c4_large_batch(B):
    # full-size launch (all 32 sequences x 32 heads, 2560 keys), every
    # sequence compared with the oracle
    s = shape_c4(B, block_idx=(512 // B) // 2)
    inp = make_attn_inputs(s, "dual")
    say(f"c4 B={B}")
    out, _, _ = run_attn(inp)
    check_attn(out, _full(inp), inp, label=f"c4 B={B}")


@pytest.mark.parametrize("qt", [0, 8, 16])
def test_c5_ragged(qt):
    # all 64 ragged sequences (prompts 256..4096, block index 0..15), with
    # the planner's kernel and the two 8-wave rings
    import block_wise_kv_amd as fd
    s = shape_c5()
    inp = make_attn_inputs(s, "dual")
    say(f"c5 ragged qt={qt}")
    fd.set_tuning(attn_qt=qt)
    try:
        out, outs, _ = run_attn(inp, ragged=True, reps=2)
    finally:
        fd.set_tuning()
    check_attn(out, _full(inp), inp, label=f"c5 qt={qt}")
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("qt", [0, 1, 2, 4, 8, 16])
def test_prefix_workspace_reused_over_block_indices(qt):
    # One workspace, zeroed once, serves a whole prefix-mode decode loop on
    # the LLaDA-8B shape: the query rows shrink from 256 to 32 as the block
    # index grows, the keys are split over workgroups at every block index,
    # and the merge counters must stay where the previous call left them
    # (at zero), never under that call's partials.  Block indices run up and
    # back down so the per-call plan both shrinks and grows.
    import block_wise_kv_amd as fd
    s0 = shape_c2(0)
    ad = fd.attn_desc(32, 32, 128, fd.BF16)
    fd.set_tuning(attn_qt=qt)
    try:
        seq0 = fd.seq_desc(1, s0.max_seq_len, s0.gen_len, 32, 512, 0)
        ws = fd.new_workspace(fd.block_attn_workspace(seq0, ad, "prefix", s0.gen_len))
        assert ws is not None
        for k in list(range(8)) + list(range(7, -1, -1)):
            s = shape_c2(k)
            inp = make_attn_inputs(s, "prefix", variant=k)
            say(f"prefix workspace reuse qt={qt} k={k}")
            out, _, _ = run_attn(inp, ws=ws)
            check_attn(out, _full(inp), inp, label=f"reuse qt={qt} k={k}")
    finally:
        fd.set_tuning()


def _dominant_key_case(mode):
    """Inputs where every query row has one dominant key.

    In each (sequence, KV head) slot the positions to probe are every
    32-key boundary (32 t - 1 and 32 t: the tile and key-chunk edges of
    every kernel variant), 0, L - 1 and both edges of the fresh range
    [a0, a1).  Probe t gets a seeded unit direction w_t; its key row holds
    K = 8 w_t in the source the step must read it from (the fresh rows when
    a0 <= j < a1, the cache otherwise) while the other source keeps an
    ordinary N(0, 1) key there.  Query row r of every head of the slot is
    3 sqrt(d) w_t plus N(0, 0.5^2) noise, t = (32 hk + r) mod (number of
    probes), so the KV heads of a sequence together probe every position.
    The row's score for its own probe is about 24 above the others' (random
    keys: standard deviation 3; other probes: 24 w_t.w_u, about 2), so that
    key's softmax weight is above 1 - 1e-5 and the output row equals its
    V_j to well within the bf16 tolerance.  A kernel that reads row j from
    the wrong source, drops it (a tile or chunk edge off by one) or pairs
    K_j with another row's V lands O(1) away.  Returns the inputs and, per
    slot, the expected output of each query row."""
    from workloads import AttnInputs, bf16_round, normal, rng_for
    b, hq, hkv, d, G, B = 8, 8, 4, 128, 256, 32
    P = np.array([512, 500, 517, 480, 530, 512, 499, 505], np.int32)
    kidx = np.array([3, 0, 7, 5, 1, 6, 2, 4], np.int32)
    s = shape_custom("domkey", "bf16", b, hq, hkv, d, P, G, B, kidx, 64, cfg_id=54)
    cap = s.fresh_capacity(mode)
    ids = (54, {"dual": 2, "prefix": 1, "none": 0}[mode])
    q = normal((b, cap, hq, d), 0.5, "f32", *ids, 1)
    kn = normal((b, cap, hkv, d), 1.0, "bf16", *ids, 2)
    vn = normal((b, cap, hkv, d), 1.0, "bf16", *ids, 3)
    kc = normal((b, hkv, s.max_seq_len, d), 1.0, "bf16", *ids, 4)
    vc = normal((b, hkv, s.max_seq_len, d), 1.0, "bf16", *ids, 5)
    g = hq // hkv
    expect = {}
    for i in range(b):
        L = int(P[i]) + G
        a0 = int(P[i]) + int(kidx[i]) * B if mode != "none" else 0
        a1 = a0 + B if mode == "dual" else L
        pos = sorted({0, L - 1, a0 - 1, a0, a1 - 1, a1} | {p for t in range(1, L // 32 + 1)
                                                          for p in (32 * t - 1, 32 * t)})
        pos = [p for p in pos if 0 <= p < L]
        n = len(pos)
        nq = a1 - a0
        for hk in range(hkv):
            dirs = rng_for(54, i, hk, 9).standard_normal((n, d))
            dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
            vrows = np.empty((nq, d))
            for t, j in enumerate(pos):
                kd = bf16_round((8.0 * dirs[t]).astype(np.float32))
                if a0 <= j < a1:
                    kn[i, j - a0, hk] = kd
                else:
                    kc[i, hk, j] = kd
            for r in range(nq):
                t = (32 * hk + r) % n
                j = pos[t]
                q[i, r, hk * g:(hk + 1) * g] += (3.0 * np.sqrt(d) * dirs[t]).astype(np.float32)
                vrows[r] = vn[i, j - a0, hk] if a0 <= j < a1 else vc[i, hk, j]
            expect[(i, hk)] = vrows
    q = bf16_round(q)
    inp = AttnInputs(s, mode, q, kn, vn, None if mode == "none" else kc, None if mode == "none" else vc)
    return inp, expect


@pytest.mark.parametrize("mode", ["dual", "prefix", "none"])
@pytest.mark.parametrize("wgs", [0, 16, 4096])
@pytest.mark.parametrize("qt", [1, 2, 4, 8, 16])
def test_dominant_key_at_boundaries(qt, wgs, mode):
    # every kernel variant and key split: each query row must return the V
    # row of its planted key, at every tile / chunk edge and fresh-range edge
    import block_wise_kv_amd as fd
    inp, expect = _dominant_key_case(mode)
    fd.set_tuning(attn_qt=qt, attn_wgs=wgs)
    try:
        say(f"dominant key qt={qt} wgs={wgs} {mode}")
        out, _, _ = run_attn(inp, ragged=True)
    finally:
        fd.set_tuning()
    s = inp.shape
    g = s.n_q_heads // s.n_kv_heads
    worst = 0.0
    for (i, hk), vrows in expect.items():
        nq = nq_of(s, mode, i)
        got = out[i, :nq, hk * g:(hk + 1) * g]
        assert np.isfinite(got).all()
        err = np.max(np.abs(got - vrows[:, None, :]), axis=(1, 2))
        bad = np.nonzero(err > 2e-2)[0]
        assert bad.size == 0, f"seq {i} kv head {hk}: rows {bad[:8].tolist()} do not return their planted V"
        worst = max(worst, float(err.max()))
    # the planted construction itself, checked by the oracle on two sequences
    seqs = [1, 3]
    ref = oracle_attn_subset(inp, seqs)
    for n_, i in enumerate(seqs):
        for hk in range(s.n_kv_heads):
            nq = nq_of(s, mode, i)
            assert np.max(np.abs(ref[n_, :nq, hk * g:(hk + 1) * g] - expect[(i, hk)][:, None, :])) <= 1e-2
    check_attn(out, ref, inp, seqs=seqs, label=f"domkey qt={qt} wgs={wgs} {mode}")
    say(f"  every row returns its planted V: max|err| = {worst:.3e}")


def test_post_refresh_identity_on_gpu():
    # right after a refresh, DUAL and PREFIX block outputs equal the full
    # no-cache recompute (within bf16 output rounding)
    s = shape_custom("pri", "bf16", 2, 8, 2, 128, [70, 70], 128, 32, [2, 2], 64, cfg_id=51)
    rng = np.random.default_rng(5)
    from workloads import bf16_round
    L = 70 + 128
    K = bf16_round(rng.standard_normal((2, L, 2, 128)).astype(np.float32))
    V = bf16_round(rng.standard_normal((2, L, 2, 128)).astype(np.float32))
    Q = bf16_round(rng.standard_normal((2, L, 8, 128)).astype(np.float32))
    kc = np.ascontiguousarray(K.transpose(0, 2, 1, 3))
    vc = np.ascontiguousarray(V.transpose(0, 2, 1, 3))
    from workloads import AttnInputs
    a0 = 70 + 2 * 32
    outs = {}
    for mode, lo, hi in (("dual", a0, a0 + 32), ("prefix", a0, L), ("none", 0, L)):
        inp = AttnInputs(s, mode, np.ascontiguousarray(Q[:, lo:hi]), np.ascontiguousarray(K[:, lo:hi]),
                         np.ascontiguousarray(V[:, lo:hi]), kc, vc)
        out, _, _ = run_attn(inp)
        outs[mode] = out[:, (a0 - lo):(a0 - lo) + 32]
    assert np.max(np.abs(outs["dual"] - outs["none"])) <= 1e-2
    assert np.max(np.abs(outs["prefix"] - outs["none"])) <= 1e-2


VARIANTS = [
    # name, dtype, b, Hq, Hkv, d, P, G, B, k, mode
    ("c3like_dual", "bf16", 2, 28, 4, 128, [1024, 1024], 1024, 32, [5, 5], "dual"),
    ("c3like_prefix", "bf16", 2, 28, 4, 128, [1024, 1024], 1024, 32, [20, 20], "prefix"),
    ("gqa7_ragged", "bf16", 3, 14, 2, 128, [37, 100, 5], 96, 32, [0, 2, 1], "dual"),
    ("gqa8_ragged", "bf16", 3, 16, 2, 128, [37, 100, 5], 96, 32, [0, 2, 1], "dual"),
    ("block4_gqa", "bf16", 2, 8, 2, 128, [13, 40], 16, 4, [3, 0], "dual"),
    ("none_gqa", "bf16", 2, 6, 3, 128, [17, 70], 32, 16, [0, 1], "none"),
    ("mha_prefix", "bf16", 2, 4, 4, 128, [130, 64], 160, 32, [1, 2], "prefix"),
]


@pytest.mark.parametrize("wgs", [0, 16, 4096])
@pytest.mark.parametrize("qt", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("case", VARIANTS, ids=lambda c: c[0])
def test_kernel_variants(case, qt, wgs):
    # every attention kernel (split-key, LDS ring with 2 or 4 query tiles per
    # workgroup, 8-wave LDS ring with one per wave, the 8-wave ring over the
    # batch's tile stream, with a loader wave when g < 8) and key split on
    # the same inputs
    import block_wise_kv_amd as fd
    name, dt, b, hq, hkv, d, P, G, B, k, mode = case
    s = shape_custom(name, dt, b, hq, hkv, d, P, G, B, k, 64, cfg_id=52)
    inp = make_attn_inputs(s, mode)
    ragged = not s.uniform
    say(f"variant {name} qt={qt} wgs={wgs}")
    fd.set_tuning(attn_qt=qt, attn_wgs=wgs)
    try:
        out, outs, _ = run_attn(inp, ragged=ragged, reps=2)
    finally:
        fd.set_tuning()
    check_attn(out, _full(inp), inp, label=f"{name} qt={qt} wgs={wgs}")
    assert np.array_equal(outs[0], outs[1], equal_nan=True)


@pytest.mark.parametrize("qt", [1, 2, 4, 8, 16])
def test_output_scales_exactly_with_v(qt):
    # Attention is linear in V, and scaling V by 2^e scales every product,
    # sum and stored partial by 2^e exactly (the 8-wave ring stores its split
    # partials in fp16 with a power-of-two scale per row), so the output must
    # scale bit-exactly: at 2^40 an unscaled fp16 partial would overflow, at
    # 2^-40 it would flush to zero.
    import block_wise_kv_amd as fd
    from dataclasses import replace
    s = shape_custom("scale", "bf16", 3, 14, 2, 128, [37, 100, 5], 96, 32, [0, 2, 1], 64, cfg_id=53)
    inp = make_attn_inputs(s, "dual")
    fd.set_tuning(attn_qt=qt, attn_wgs=4096)
    try:
        base, _, _ = run_attn(inp, ragged=True)
        for e in (40, -40):
            f = 2.0 ** e
            sc = replace(inp, v_new=inp.v_new * f, v_cache=inp.v_cache * f)
            got, _, _ = run_attn(sc, ragged=True)
            live = ~np.isnan(base)
            assert np.array_equal(np.isnan(got), ~live)
            assert np.array_equal(got[live], base[live] * f), f"qt={qt}: output at V * 2^{e} is not 2^{e} times the output"
    finally:
        fd.set_tuning()
    check_attn(base, _full(inp), inp, label=f"scale qt={qt}")
    say(f"  qt={qt}: outputs at V * 2^40 and V * 2^-40 equal the scaled output bit for bit")
