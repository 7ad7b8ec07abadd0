"""Pins for the oracle's fixed-step (top-k) unmasking (CPU only)."""
import itertools

import numpy as np
import pytest

from oracle import (decode_block_topk_ref, row_confidence, tokens_per_step, unmask_ref,
                    unmask_topk_ref)
from workloads import make_decode_state, make_logits, shape_c1, shape_custom


def _shape(b=3, B=8, V=8, P=(3, 5, 4), G=16, k=(1, 0, 1), cfg=78):
    return shape_custom("k", "f32", b, 1, 1, 8, list(P)[:b], G, B, list(k)[:b], V, cfg_id=cfg)


def _random_case(seed, b=3, B=8, V=8, scale=2.0):
    s = _shape(b=b, B=B, V=V, cfg=seed)
    g = np.random.default_rng(seed)
    logits = g.standard_normal((b, B, V)) * scale
    nm = g.integers(1, B + 1, size=b)
    tokens, mask = make_decode_state(s, nm)
    return s, logits, tokens, mask


def _start(s, i):
    return int(s.prompt_lens[i]) + int(s.block_idxs[i]) * s.block_size


def check_k_covers_block(tk):
    # k >= m decodes every masked row of the block in one step
    for seed in range(5):
        s, logits, tokens, mask = _random_case(seed)
        for k in (s.block_size, s.block_size + 3):
            r = tk(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, k)
            for i in range(s.batch):
                st = _start(s, i)
                masked = [t for t in range(s.block_size) if mask[i, st + t]]
                assert list(r.decoded_pos[i, :len(masked)]) == masked
                assert np.all(r.decoded_pos[i, len(masked):] == -1)
                assert r.done[i]
                for t in masked:
                    assert r.tokens[i, st + t] == int(np.argmax(logits[i, t]))


def check_k1_is_single_best(tk):
    # k = 1 decodes what the threshold rule's fallback decodes (tau = 1 can
    # never be exceeded): the single most confident masked row
    for seed in range(6):
        s, logits, tokens, mask = _random_case(seed, scale=1.0)
        logits[:, 2] = logits[:, 5]  # equal confidences: the lower offset wins
        r1 = tk(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, 1)
        rt = unmask_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size,
                        s.block_idxs, 1.0)
        assert np.array_equal(r1.tokens, rt.tokens) and np.array_equal(r1.mask, rt.mask)
        assert np.array_equal(r1.decoded_pos, rt.decoded_pos)
        assert np.array_equal(r1.n_decoded, np.minimum(1, r1.n_decoded + 1))


def check_ties_lower_offset(tk):
    # equal confidences are taken in block order: three identical most
    # confident rows, k = 1 and k = 2 take the lowest offsets among them
    s = _shape(b=1, B=8, V=6, P=(3,), G=16, k=(1,))
    tokens, mask = make_decode_state(s, np.array([8]))
    g = np.random.default_rng(5)
    logits = g.standard_normal((1, 8, 6)) * 0.1  # other rows: confidence about 1/6
    peak = np.array([0.5, 5.0, 0.0, 5.0, 0.2, 0.1])  # two equal maxima: token 1, the lower id
    for t in (6, 2, 4):
        logits[0, t] = peak                   # identical rows: identical confidence
    st = _start(s, 0)
    r = tk(logits, tokens, mask, s.prompt_lens, s.gen_len, 8, s.block_idxs, 1)
    assert list(r.decoded_pos[0, :1]) == [2]
    r = tk(logits, tokens, mask, s.prompt_lens, s.gen_len, 8, s.block_idxs, 2)
    assert list(r.decoded_pos[0, :2]) == [2, 4]
    assert r.tokens[0, st + 2] == 1 and r.tokens[0, st + 4] == 1


def check_matches_threshold_between(tk):
    # For a threshold strictly between the k-th and (k+1)-th largest
    # confidences the threshold rule decodes exactly the top k: two
    # independently written selection rules agree.
    for seed in range(8):
        s, logits, tokens, mask = _random_case(seed, B=8, V=6, scale=3.0)
        for i in range(s.batch):
            st = _start(s, i)
            masked = [t for t in range(s.block_size) if mask[i, st + t]]
            confs = sorted((row_confidence(logits[i, t])[0] for t in masked), reverse=True)
            for k in range(1, len(masked)):
                hi, lo = confs[k - 1], confs[k]
                if hi - lo < 1e-9:
                    continue
                tau = float(np.float32((hi + lo) / 2))
                if not lo < tau < hi:
                    continue
                r = tk(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, k)
                rt = unmask_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size,
                                s.block_idxs, tau)
                assert np.array_equal(r.decoded_pos[i], rt.decoded_pos[i]), (seed, i, k)
                assert np.array_equal(r.tokens[i], rt.tokens[i])
                assert not rt.fallback[i]


def check_brute_force_order(tk):
    # every mask pattern of a 6-position block: the chosen set has min(k, m)
    # rows and every chosen row outranks every unchosen masked row (higher
    # confidence, or equal confidence and a lower offset); confidences from a
    # sort-based restatement
    g = np.random.default_rng(11)
    B, V = 6, 5
    s = _shape(b=1, B=B, V=V, P=(2,), G=12, k=(1,))
    start = 2 + B
    for k in (1, 2, 4):
        logits = np.round(g.standard_normal((1, B, V)) * 3) / 2  # ties happen
        conf = {}
        for t in range(B):
            row = logits[0, t]
            top = sorted(range(V), key=lambda v: (-row[v], v))[0]
            p = np.exp(row - row[top])
            conf[t] = p[top] / p.sum()
        for bits in itertools.product([0, 1], repeat=B):
            tokens = np.full((1, 14), 1, np.int32)
            mask = np.zeros((1, 14), np.uint8)
            mask[0, start:start + B] = bits
            r = tk(logits, tokens, mask, s.prompt_lens, s.gen_len, B, s.block_idxs, k)
            masked = [t for t in range(B) if bits[t]]
            got = [int(t) for t in r.decoded_pos[0] if t >= 0]
            assert len(got) == min(k, len(masked))
            assert got == sorted(got)
            for a in got:
                for u in masked:
                    if u in got:
                        continue
                    assert conf[a] > conf[u] + 1e-12 or (abs(conf[a] - conf[u]) <= 1e-12 and a < u), \
                        (bits, k, got)


def check_unread_rows(tk):
    # logits rows of unmasked positions are never read
    for seed in range(3):
        s, logits, tokens, mask = _random_case(seed)
        r1 = tk(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, 2)
        lg = logits.copy()
        for i in range(s.batch):
            st = _start(s, i)
            for t in range(s.block_size):
                if not mask[i, st + t]:
                    lg[i, t] = np.nan
        r2 = tk(lg, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, 2)
        assert np.array_equal(r1.tokens, r2.tokens) and np.array_equal(r1.mask, r2.mask)


TOPK_CHECKS = [check_k_covers_block, check_k1_is_single_best, check_ties_lower_offset,
               check_matches_threshold_between, check_brute_force_order, check_unread_rows]


@pytest.mark.parametrize("check", TOPK_CHECKS, ids=lambda c: c.__name__)
def test_topk_pin(check):
    check(unmask_topk_ref)


def test_tokens_per_step_pages_settings():
    # the pages' flag settings: gen 128 / steps 128 and gen 64 / steps 64 with
    # blocks of 32 commit one token per step
    assert tokens_per_step(128, 32, 128) == 1
    assert tokens_per_step(64, 32, 64) == 1
    assert tokens_per_step(256, 32, 64) == 4
    assert tokens_per_step(256, 32, 8) == 32
    for bad in ((128, 32, 6), (128, 32, 96), (100, 32, 4)):
        with pytest.raises(ValueError):
            tokens_per_step(*bad)


def test_fixed_step_loop_counts():
    # m masked rows take ceil(m / k) steps of k tokens (the last may be short)
    s = shape_c1()
    tokens, mask = make_decode_state(s, 20)
    for k in (1, 3, 4, 20, 32):
        steps = decode_block_topk_ref(lambda st: make_logits(s, step=st), tokens, mask,
                                      s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, k)
        assert len(steps) == -(-20 // k)
        assert [int(n[0]) for n in steps] == [k] * (20 // k) + ([20 % k] if 20 % k else [])


def test_near_tie_step_flag():
    s = _shape(b=1, B=4, V=4, P=(2,), G=8, k=(1,))
    tokens, mask = make_decode_state(s, 4)
    logits = np.zeros((1, 4, 4))
    logits[0, 0] = [3.0, 0, 0, 0]
    logits[0, 1] = [2.0, 0, 0, 0]
    logits[0, 2] = [2.0, 0, 0, 0]            # ties row 1: the 2nd/3rd boundary
    logits[0, 3] = [0.5, 0, 0, 0]
    r = unmask_topk_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, 4, s.block_idxs, 2)
    assert r.tie_step[0] and list(r.decoded_pos[0, :2]) == [0, 1]
    r = unmask_topk_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, 4, s.block_idxs, 1)
    assert not r.tie_step[0] and r.decoded_pos[0, 0] == 0
    with pytest.raises(ValueError):
        unmask_topk_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, 4, s.block_idxs, 0)


# ---------------------------------------------------------------------------
# mutation tests: a planted mistake in a copy of the rule fails some pin
# ---------------------------------------------------------------------------

def _mutant(kind):
    from oracle import fdllm_oracle as fo

    def tk(logits, tokens, mask, prompt_lens, gen_len, block_size, block_idxs, k, advance=False):
        tokens = np.array(tokens, np.int32, copy=True)
        mask = np.array(mask, np.uint8, copy=True)
        bidx = np.array(block_idxs, np.int32, copy=True).reshape(-1)
        b, B = tokens.shape[0], block_size
        n_dec = np.zeros(b, np.int32)
        dpos = np.full((b, B), -1, np.int32)
        done = np.zeros(b, bool)
        for i in range(b):
            start = int(prompt_lens[i]) + int(bidx[i]) * B
            masked = [t for t in range(B) if mask[i, start + t] == 1]
            conf, tok = {}, {}
            for t in masked:
                conf[t], tok[t], _, _ = fo.row_confidence(logits[i][t])
                if kind == "last_argmax":
                    l = np.asarray(logits[i][t], np.float64)
                    tok[t] = int(np.flatnonzero(l == l.max())[-1])
            if kind == "ascending":
                order = sorted(masked, key=lambda t: (conf[t], t))
            elif kind == "tie_high_offset":
                order = sorted(masked, key=lambda t: (-conf[t], -t))
            else:
                order = sorted(masked, key=lambda t: (-conf[t], t))
            kk = k + 1 if kind == "k_plus_one" else k
            chosen = order[:kk]
            if kind == "unmasked_too" and len(masked) < B:
                extra = [t for t in range(B) if t not in masked][:1]
                for t in extra:
                    tok[t] = int(np.argmax(logits[i][t]))
                chosen = chosen + extra
            for t in chosen:
                tokens[i, start + t] = tok[t]
                mask[i, start + t] = 0
            chosen.sort()
            n_dec[i] = len(chosen)
            dpos[i, :len(chosen)] = chosen
            done[i] = not any(mask[i, start + t] == 1 for t in range(B))
        z = np.zeros((b, B), bool)
        return fo.UnmaskResult(tokens, mask, n_dec, dpos, np.full((b, B), np.nan), done,
                               np.flatnonzero(done).astype(np.int32), bidx, np.zeros(b, bool), z, z,
                               np.zeros(b, bool))
    return tk


@pytest.mark.parametrize("kind", ["ascending", "tie_high_offset", "k_plus_one", "unmasked_too",
                                  "last_argmax"])
def test_pins_catch_planted_mistake(kind):
    tk = _mutant(kind)
    failures = 0
    for check in TOPK_CHECKS:
        try:
            check(tk)
        except (AssertionError, IndexError, ValueError):
            failures += 1
    assert failures > 0, f"no pin caught the planted mistake {kind!r}"


def test_unmutated_copy_passes_all_pins():
    tk = _mutant("none")
    for check in TOPK_CHECKS:
        check(tk)
