"""GPU parity: fdllm_block_attn against the fp64 oracle."""
import numpy as np
import pytest

from gpu_util import (check_attn, oracle_attn_subset, require_gpu, run_attn, say)
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
def test_c4_large_batch_sampled(B):
    # full-size launch; the oracle checks three sampled sequences exactly
    s = shape_c4(B, block_idx=(512 // B) // 2)
    inp = make_attn_inputs(s, "dual")
    say(f"c4 B={B}")
    out, _, _ = run_attn(inp)
    seqs = [0, 13, 31]
    ref = oracle_attn_subset(inp, seqs)
    check_attn(out, ref, inp, seqs=seqs, label=f"c4 B={B}")
    assert np.isfinite(out[:, :B]).all()


def test_c5_ragged_sampled():
    s = shape_c5()
    inp = make_attn_inputs(s, "dual")
    say("c5 ragged")
    out, outs, _ = run_attn(inp, ragged=True, reps=2)
    order = np.argsort(s.prompt_lens)
    seqs = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), 7})
    ref = oracle_attn_subset(inp, seqs)
    check_attn(out, ref, inp, seqs=seqs, label="c5")
    assert np.isfinite(out).all()
    assert np.array_equal(outs[0], outs[1])


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
    ("block4_gqa", "bf16", 2, 8, 2, 128, [13, 40], 16, 4, [3, 0], "dual"),
    ("none_gqa", "bf16", 2, 6, 3, 128, [17, 70], 32, 16, [0, 1], "none"),
    ("mha_prefix", "bf16", 2, 4, 4, 128, [130, 64], 160, 32, [1, 2], "prefix"),
]


@pytest.mark.parametrize("wgs", [0, 16, 4096])
@pytest.mark.parametrize("qt", [1, 2, 4, 8])
@pytest.mark.parametrize("case", VARIANTS, ids=lambda c: c[0])
def test_kernel_variants(case, qt, wgs):
    # every attention kernel (split-key, LDS ring with 2 or 4 query tiles per
    # workgroup, 8-wave LDS ring with one per wave) and key split on the same inputs
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


@pytest.mark.parametrize("qt", [1, 2, 4, 8])
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
