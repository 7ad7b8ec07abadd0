"""Pins for the oracle's cache refresh (CPU only), plus the input generators."""
import numpy as np
import pytest
import torch

from oracle import refresh_ref
from workloads import (bf16_round, make_decode_state, make_logits, make_refresh_src, shape_c1,
                       shape_c5, shape_custom)


def _shape():
    return shape_custom("r", "f32", 3, 4, 2, 8, [5, 9, 7], 12, 4, [1, 2, 0], 16)


def _sentinel_caches(s):
    shp = (s.batch, s.n_kv_heads, s.max_seq_len, s.head_dim)
    return np.full(shp, -123.0, np.float32), np.full(shp, 456.0, np.float32)


def _rows(s, i, mode):
    P, k = int(s.prompt_lens[i]), int(s.block_idxs[i])
    return {"dual": P + s.gen_len, "prefix": P + k * s.block_size, "none": 0}[mode]


def check_copy(rf):
    s = _shape()
    ks, vs = make_refresh_src(s)
    for mode in ("dual", "prefix", "none"):
        kc0, vc0 = _sentinel_caches(s)
        kc, vc = rf(ks, vs, kc0, vc0, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, mode)
        # the expected cache, built from the definition with a transpose
        for i in range(s.batch):
            hi = _rows(s, i, mode)
            assert np.array_equal(kc[i, :, :hi], ks[i, :hi].transpose(1, 0, 2))
            assert np.array_equal(vc[i, :, :hi], vs[i, :hi].transpose(1, 0, 2))
            assert np.all(kc[i, :, hi:] == -123.0) and np.all(vc[i, :, hi:] == 456.0)
        # inputs untouched, idempotent
        assert np.all(kc0 == -123.0)
        kc2, vc2 = rf(ks, vs, kc, vc, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, mode)
        assert np.array_equal(kc2, kc) and np.array_equal(vc2, vc)


def check_subset(rf):
    s = _shape()
    ks, vs = make_refresh_src(s)
    kc0, vc0 = _sentinel_caches(s)
    kc, vc = rf(ks, vs, kc0, vc0, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, "dual",
                seq_ids=[2, 0])
    assert np.all(kc[1] == -123.0) and np.all(vc[1] == 456.0)
    for i in (0, 2):
        hi = _rows(s, i, "dual")
        assert np.array_equal(kc[i, :, :hi], ks[i, :hi].transpose(1, 0, 2))


@pytest.mark.parametrize("check", [check_copy, check_subset], ids=lambda c: c.__name__)
def test_refresh_pin(check):
    check(refresh_ref)


def test_planted_mistakes_fail():
    def wrong_range(ks, vs, kc, vc, pl, G, B, bi, mode, seq_ids=None):
        kc = kc.copy(); vc = vc.copy()
        for i in range(kc.shape[0]):
            hi = int(pl[i]) + (int(bi[i]) + 1) * B if mode == "prefix" else (
                int(pl[i]) + G if mode == "dual" else 0)
            kc[i, :, :hi] = ks[i, :hi].transpose(1, 0, 2)
            vc[i, :, :hi] = vs[i, :hi].transpose(1, 0, 2)
        return kc, vc

    def no_transpose(ks, vs, kc, vc, pl, G, B, bi, mode, seq_ids=None):
        kc = kc.copy(); vc = vc.copy()
        for i in range(kc.shape[0]):
            hi = _rows(_shape(), i, mode)
            kc[i].reshape(-1)[:ks[i, :hi].size] = ks[i, :hi].reshape(-1)
            vc[i].reshape(-1)[:vs[i, :hi].size] = vs[i, :hi].reshape(-1)
        return kc, vc

    for bad in (wrong_range, no_transpose):
        with pytest.raises(AssertionError):
            check_copy(bad)


def test_bf16_round_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 7,
                        np.array([1.00390625, 1.01171875, -1.00390625, 65504.0, 1e-30], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_round(x), want)


def test_generators_are_seeded_and_shaped():
    s = shape_c1()
    a = make_logits(s)
    b = make_logits(s)
    assert a.shape == (1, 32, 1024) and np.array_equal(a, b)
    t, m = make_decode_state(s, 20)
    start = 64 + 32
    assert m[0, start:start + 32].sum() == 20 and m[0, start + 32:192].all() and not m[0, :start].any()
    s5 = shape_c5()
    assert s5.prompt_lens.min() >= 256 and s5.prompt_lens.max() <= 4096
    assert s5.block_idxs.max() < 16
