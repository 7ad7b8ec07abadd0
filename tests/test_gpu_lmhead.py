"""GPU parity of the vocabulary projection fused with the confidence pass
(fdllm_lmhead_pack, fdllm_lmhead_unmask_threshold / _topk) against the fp64
oracle.

Inputs use the exact-grid recipe (small integers times powers of two), on
which every fp32 sum of the products is exact: the kernel's logits equal
the oracle's, so tokens, masks and decoded positions must match bit for
bit (near ties of the threshold as flagged by the oracle aside) and conf
within CONF_TOL.  One case uses continuous inputs, where the fp32
accumulation rounds; there the bound gamma_H * sum_k |x_k w_k| (gamma_H =
H u / (1 - H u), u = 2^-24, valid for any summation order) decides which
tokens and confidences are acceptable.
"""
import numpy as np
import pytest
import torch

import block_wise_kv_amd as fd
from gpu_util import (CONF_TOL, DEV, compare_unmask, lmhead_weight_dev, require_gpu, run_lmhead, say, to_dev)
from oracle import lmhead_logits_ref, lmhead_unmask_ref, unmask_ref, unmask_topk_ref
from workloads import make_decode_state, make_lmhead_inputs, shape_c2, shape_c3, shape_custom

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _ref(s, inp, tokens, mask, tau=None, k=None, advance=False):
    return lmhead_unmask_ref(inp.x, inp.weight(), tokens, mask, s.prompt_lens, s.gen_len, s.block_size,
                             s.block_idxs, threshold=tau, k=k, advance=advance)


# (name, batch, block, hidden, vocab, prompt_lens, block_idxs, n_masked, cfg)
CASES = [
    ("b1_rt1", 1, 32, 512, 3000, [64], [1], [20], 90),          # one row tile, ragged last vocabulary tile
    ("b2_rt2_h200", 2, 32, 200, 1000, [40, 70], [0, 2], [32, 9], 91),  # hidden padded 200 -> 512
    ("b3_rt4", 3, 32, 1024, 5000, [100], [3], [17], 92),         # 96 rows: 4 row tiles, the last one empty
    ("b5_rt8", 5, 32, 512, 2300, [100], [3], [17], 89),          # 160 rows: 8 row tiles, 3 of them empty
    ("b9_rt8x2", 9, 32, 256, 1200, [20], [0], [30], 88),         # 288 rows: two row groups of 256
    ("B64", 1, 64, 256, 2000, [30], [1], [50], 93),              # 64-row block, one-wave finalisation
    ("B128", 2, 128, 256, 700, [10, 20], [0, 1], [128, 40], 94),  # 128-row block, workgroup finalisation
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
@pytest.mark.parametrize("rule", ["tau0.5", "tau0.9", "k1", "k4"])
def test_lmhead_matches_oracle(case, rule):
    name, b, B, H, V, plen, bidx, nm, cfg = case
    s = shape_custom(name, "bf16", b, 1, 1, 8, plen, 4 * B, B, bidx, V, cfg_id=cfg)
    inp = make_lmhead_inputs(s, H)
    tokens, mask = make_decode_state(s, nm * b if len(nm) == 1 else nm)
    say(f"lmhead {name} {rule}: b={b} B={B} H={H} V={V}")
    tau = float(rule[3:]) if rule.startswith("tau") else None
    k = int(rule[1:]) if rule.startswith("k") else None
    ragged = len(set(s.prompt_lens.tolist())) > 1 or len(set(s.block_idxs.tolist())) > 1
    g = run_lmhead(s, inp, tokens, mask, tau=tau, topk=k, ragged=ragged)
    ref = _ref(s, inp, tokens, mask, tau=tau, k=k)
    compare_unmask(g, ref, s, label=f"lmhead {name} {rule}")
    if not ref.tie_step.any() and not ref.tie_tau.any():
        assert np.array_equal(g["n_decoded"], ref.n_decoded)


@pytest.mark.parametrize("vt", [1, 2])
def test_lmhead_tiles_per_wave(vt):
    # both vocabulary-tile counts per wave give the same (exact) result
    s = shape_custom("vt", "bf16", 1, 1, 1, 8, [64], 128, 32, [1], 4100, cfg_id=95)
    inp = make_lmhead_inputs(s, 768)
    tokens, mask = make_decode_state(s, 32)
    try:
        fd.set_lmhead_tuning(vt)
        g = run_lmhead(s, inp, tokens, mask, tau=0.7)
    finally:
        fd.set_lmhead_tuning(0)
    ref = _ref(s, inp, tokens, mask, tau=0.7)
    compare_unmask(g, ref, s, label=f"lmhead vt={vt}")


def test_lmhead_ragged_advance_done_list():
    # device prompt lengths and block indices, block advance, finished list
    s = shape_custom("rag", "bf16", 3, 1, 1, 8, [33, 70, 5], 96, 32, [0, 2, 1], 1500, cfg_id=96)
    inp = make_lmhead_inputs(s, 512)
    tokens, mask = make_decode_state(s, [1, 32, 12])
    g = run_lmhead(s, inp, tokens, mask, tau=0.6, ragged=True, flags=fd.UNMASK_ADVANCE_BLOCK)
    ref = _ref(s, inp, tokens, mask, tau=0.6, advance=True)
    compare_unmask(g, ref, s, label="lmhead ragged")
    assert not ref.tie_step.any()
    assert list(g["done_seqs"]) == list(ref.done_seqs) and g["n_done"] == ref.n_done
    assert np.array_equal(g["block_idxs"], ref.block_idxs)
    assert ref.n_done >= 1


def test_lmhead_strided_rows():
    # hidden states as a view with padded rows and sequences
    s = shape_custom("str", "bf16", 2, 1, 1, 8, [50], 64, 32, [1], 900, cfg_id=97)
    inp = make_lmhead_inputs(s, 256)
    tokens, mask = make_decode_state(s, 32)
    big = torch.zeros((2, 35, 256 + 24), dtype=torch.bfloat16, device=DEV)
    big[:, :32, :256] = to_dev(inp.x, "bf16")
    x = big[:, :32, :256]
    assert x.stride(1) == 280 and x.stride(0) == 35 * 280
    g = run_lmhead(s, inp, tokens, mask, tau=0.8, x_dev=x)
    compare_unmask(g, _ref(s, inp, tokens, mask, tau=0.8), s, label="lmhead strided")


def test_lmhead_vocab_of_one_and_one_tile():
    # vocab 1: every masked row has confidence 1 and token 0; vocab 33: two
    # tiles, the second with one live row
    for V in (1, 33):
        s = shape_custom(f"v{V}", "bf16", 1, 1, 1, 8, [8], 64, 32, [0], V, cfg_id=98)
        inp = make_lmhead_inputs(s, 64)
        tokens, mask = make_decode_state(s, 32)
        g = run_lmhead(s, inp, tokens, mask, tau=0.5)
        ref = _ref(s, inp, tokens, mask, tau=0.5)
        compare_unmask(g, ref, s, label=f"lmhead vocab {V}")
        if V == 1:
            assert np.all(g["conf"] == 1.0) and int(g["n_decoded"][0]) == 32


def test_pack_layout_bit_exact():
    # fragment (tile, step), lane l holds w[32 tile + l % 32][16 step + 8 (l / 32) + 0..7], zero padded
    V, H = 100, 200
    g = np.random.default_rng(5)
    wbits = g.integers(0, 1 << 16, size=(V, H), dtype=np.uint16)
    wbits[(wbits & 0x7f80) == 0x7f80] &= 0x3fff  # no NaN / inf patterns
    w = torch.from_numpy(wbits.view(np.int16)).to(DEV).view(torch.bfloat16)
    wp = fd.lmhead_pack(w)
    torch.cuda.synchronize()
    got = wp.cpu().numpy().view(np.uint16)
    Hp = 512
    nvt = (V + 31) // 32
    pad = np.zeros((nvt * 32, Hp), np.uint16)
    pad[:V, :H] = wbits
    # [tile][32 rows][steps][2 halves][8] -> [tile][steps][halves][rows][8]
    exp = pad.reshape(nvt, 32, Hp // 16, 2, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert got.size == exp.size and np.array_equal(got, exp)
    say(f"  pack: {got.size * 2} bytes bit-exact")


def test_continuous_inputs_within_rounding_bound():
    # x ~ N(0, 1), w ~ N(0, 3 / sqrt(H)) in bf16: fp32 accumulation rounds;
    # the kernel's token must be within 2 E of the row maximum and its conf
    # within exp(2 E) - 1 relative (E = the row's largest bound)
    s = shape_custom("cont", "bf16", 2, 1, 1, 8, [20], 64, 32, [1], 2500, cfg_id=99)
    inp = make_lmhead_inputs(s, 1024, recipe="normal")
    tokens, mask = make_decode_state(s, 32)
    g = run_lmhead(s, inp, tokens, mask, tau=2.0)  # tau >= 1: one token per sequence, conf of every row
    w = inp.weight()
    logits = lmhead_logits_ref(inp.x, w)
    H = inp.hidden
    u = 2.0 ** -24
    gam = H * u / (1 - H * u)
    E = gam * (np.abs(inp.x.astype(np.float64)) @ np.abs(w).T).max(-1)  # [b][B]
    m = logits.max(-1)
    conf = 1.0 / np.exp(logits - m[..., None]).sum(-1)
    worst = 0.0
    for i in range(2):
        for t in range(32):
            tol = conf[i, t] * np.expm1(2 * E[i, t]) + CONF_TOL
            err = abs(g["conf"][i, t] - conf[i, t])
            worst = max(worst, err / tol)
            assert err <= tol, (i, t, g["conf"][i, t], conf[i, t], tol)
        start = int(s.prompt_lens[i]) + int(s.block_idxs[i]) * 32
        sel = g["decoded_pos"][i, 0]
        tok = g["tokens"][i, start + sel]
        assert logits[i, sel, tok] >= m[i, sel] - 2 * E[i, sel]
        # the selected row is the most confident one up to the bound
        assert conf[i, sel] >= conf[i].max() * np.exp(-4 * E[i].max()) - CONF_TOL
    say(f"  continuous: worst conf error / bound = {worst:.3f}; E max = {E.max():.2e}")


def _big_case(shape, H, tau=None, k=None, label="", seqs=None):
    inp = make_lmhead_inputs(shape, H)
    s = shape
    tokens, mask = make_decode_state(s, None)
    wdev = lmhead_weight_dev(inp)
    wp = fd.lmhead_pack(wdev)
    del wdev
    g = run_lmhead(s, inp, tokens, mask, tau=tau, topk=k, w_packed=wp)
    del wp
    torch.cuda.empty_cache()
    # oracle logits by vocabulary chunks (the same definition per chunk), for
    # the sampled sequences (a sequence's step depends on its own rows only)
    sel = list(range(s.batch)) if seqs is None else list(seqs)
    x = inp.x[sel]
    chunks = []
    step = 16384
    for v0 in range(0, s.vocab, step):
        chunks.append(lmhead_logits_ref(x, inp.weight(v0, v0 + step)))
    logits = np.concatenate(chunks, axis=-1)
    sub = shape_custom(s.name, s.dtype, len(sel), s.n_q_heads, s.n_kv_heads, s.head_dim, s.prompt_lens[sel],
                       s.gen_len, s.block_size, s.block_idxs[sel], s.vocab, s.max_seq_len, cfg_id=s.cfg_id)
    args = (tokens[sel], mask[sel], sub.prompt_lens, sub.gen_len, sub.block_size, sub.block_idxs)
    ref = unmask_ref(logits, *args, tau) if k is None else unmask_topk_ref(logits, *args, k)
    gs = {key: (v[sel] if isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == s.batch else v)
          for key, v in g.items()}
    compare_unmask(gs, ref, sub, label=label)


def test_llada8b_full_size():
    # LLaDA-8B: hidden 4096, vocabulary 126464, one sequence, block of 32
    say("lmhead full size: LLaDA-8B b1")
    _big_case(shape_c2(), 4096, tau=0.9, label="lmhead llada8b b1 tau0.9")


def test_dream7b_full_size_topk():
    # Dream-7B: hidden 3584, vocabulary 152064, 8 sequences (256 rows: two row groups)
    say("lmhead full size: Dream-7B b8")
    _big_case(shape_c3(), 3584, k=2, label="lmhead dream7b b8 k2")


def test_llada8b_b32_full_size_sampled():
    # LLaDA-8B at batch 32 (1024 rows: four row groups of 256), the shape
    # bench.py --lmhead --workload c4 times; sequences 0, 13 and 31 checked
    # against the oracle (each sequence's step depends only on its own rows)
    from workloads import shape_c4
    say("lmhead full size: LLaDA-8B b32 (sampled sequences)")
    _big_case(shape_c4(), 4096, tau=0.7, label="lmhead llada8b b32 tau0.7", seqs=[0, 13, 31])


@pytest.mark.parametrize("rule", ["threshold", "topk"])
def test_block_decode_loop_in_one_graph(rule):
    # the in-block loop on the device: every step of a block (fused LM head +
    # unmask, updating tokens and mask in place) captured in one HIP graph;
    # each step's n_decoded equals the oracle's loop step by step and the
    # final tokens and mask match (exact-grid logits, fixed across steps)
    s = shape_custom("loop", "bf16", 2, 1, 1, 8, [10, 40], 96, 32, [1, 2], 3000, cfg_id=85)
    inp = make_lmhead_inputs(s, 256)
    tokens, mask = make_decode_state(s, [32, 17])
    k = 3
    n_steps = -(-32 // k) if rule == "topk" else 32
    keep = []
    from gpu_util import seq_for
    seq = seq_for(s, True, keep)
    x = to_dev(inp.x, "bf16")
    wp = fd.lmhead_pack(lmhead_weight_dev(inp))
    ws = fd.new_workspace(fd.lmhead_unmask_workspace(seq, s.vocab, 256))
    tk = torch.from_numpy(tokens).to(DEV)
    mk = torch.from_numpy(mask).to(DEV)
    nd = torch.full((n_steps, 2), -7, dtype=torch.int32, device=DEV)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for st in range(n_steps):
                if rule == "topk":
                    fd.lmhead_unmask_topk(seq, x, wp, s.vocab, k, tk, mk, nd[st], workspace=ws)
                else:
                    fd.lmhead_unmask_threshold(seq, x, wp, s.vocab, 0.6, tk, mk, nd[st], workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    tk.copy_(torch.from_numpy(tokens))
    mk.copy_(torch.from_numpy(mask))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    # the oracle's loop on the same logits
    w = inp.weight()
    t_ref, m_ref = tokens, mask
    per_step = []
    for st in range(n_steps):
        if rule == "topk":
            r = lmhead_unmask_ref(inp.x, w, t_ref, m_ref, s.prompt_lens, s.gen_len, 32, s.block_idxs, k=k)
        else:
            r = lmhead_unmask_ref(inp.x, w, t_ref, m_ref, s.prompt_lens, s.gen_len, 32, s.block_idxs, threshold=0.6)
        assert not r.tie_step.any() and not r.tie_tau.any(), f"near tie at step {st}"
        t_ref, m_ref = r.tokens, r.mask
        per_step.append(r.n_decoded)
    got = nd.cpu().numpy()
    assert np.array_equal(got, np.array(per_step)), (got.tolist(), np.array(per_step).tolist())
    assert np.array_equal(tk.cpu().numpy(), t_ref) and np.array_equal(mk.cpu().numpy(), m_ref)
    assert int(got.sum()) == 32 + 17
    say(f"  in-graph {rule} loop: tokens per step {got[:, 0].tolist()} / {got[:, 1].tolist()}")
