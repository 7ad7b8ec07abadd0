"""GPU parity: fdllm_kv_refresh and fdllm_kv_refresh_layers against the
oracle (bit-exact), and the full ragged step (28 x attention, one unmask,
one refresh of the finished sequences' 28 layer caches)."""
import numpy as np
import pytest
import torch

import block_wise_kv_amd as fd
from gpu_util import (DEV, check_attn, compare_unmask, oracle_attn_subset, require_gpu, run_attn, say,
                      seq_for, to_dev)
from oracle import attn_ref, refresh_ref, unmask_ref
from workloads import (AttnInputs, make_attn_inputs, make_decode_state, make_logits, make_refresh_src,
                       n_masked_c5, shape_c1, shape_c2, shape_c3, shape_c5, shape_custom)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _sentinel(s, dt):
    shp = (s.batch, s.n_kv_heads, s.max_seq_len, s.head_dim)
    return np.full(shp, -3.0, np.float32), np.full(shp, 5.0, np.float32)


def _run_refresh(s, mode, ks, vs, kc0, vc0, ragged, seq_ids=None):
    keep = []
    seq = seq_for(s, ragged, keep)
    k_src, v_src = to_dev(ks, s.dtype), to_dev(vs, s.dtype)
    kc, vc = to_dev(kc0, s.dtype), to_dev(vc0, s.dtype)
    ids = n = None
    if seq_ids is not None:
        ids = torch.tensor(list(seq_ids) + [0] * (s.batch - len(seq_ids)), dtype=torch.int32, device=DEV)
        n = torch.tensor([len(seq_ids)], dtype=torch.int32, device=DEV)
    fd.kv_refresh(seq, mode, k_src, v_src, kc, vc, ids, n)
    torch.cuda.synchronize()
    return kc.float().cpu().numpy(), vc.float().cpu().numpy()


CASES = [
    ("c1", shape_c1(), False),
    ("ragged_bf16", shape_custom("rr", "bf16", 3, 4, 2, 128, [37, 100, 5], 96, 32, [0, 2, 1], 64, cfg_id=70), True),
    ("f32_d64", shape_custom("rf", "f32", 2, 4, 3, 64, [12, 4], 32, 8, [1, 3], 64, cfg_id=71), True),
    # one LLaDA-8B sequence: the launch with 6 vectors per thread (one
    # workgroup per CU); the cases above take 3, the Dream-7B tests 4
    ("c2_llada", shape_c2(), False),
]


@pytest.mark.parametrize("mode", ["dual", "prefix", "none"])
@pytest.mark.parametrize("name,s,ragged", CASES, ids=[c[0] for c in CASES])
def test_refresh_modes(name, s, ragged, mode):
    ks, vs = make_refresh_src(s)
    kc0, vc0 = _sentinel(s, s.dtype)
    say(f"refresh {name} {mode}")
    kc, vc = _run_refresh(s, mode, ks, vs, kc0, vc0, ragged)
    rk, rv = refresh_ref(ks, vs, kc0, vc0, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, mode)
    assert np.array_equal(kc, rk) and np.array_equal(vc, rv)


@pytest.mark.parametrize("subset", [False, True])
@pytest.mark.parametrize("mode", ["dual", "prefix", "none"])
@pytest.mark.parametrize("name,s,ragged", CASES, ids=[c[0] for c in CASES])
def test_refresh_layers(name, s, ragged, mode, subset):
    """fdllm_kv_refresh_layers: three layers in one launch, each layer with
    its own sources and caches, equal to the oracle's per-layer refresh bit
    for bit (rows it does not refresh keep their sentinels)."""
    n_layers = 3
    keep = []
    seq = seq_for(s, ragged, keep)
    ids_host = [s.batch - 1, 0][:s.batch] if subset else None
    ids = n = None
    if subset:
        ids = torch.tensor(ids_host + [0] * (s.batch - len(ids_host)), dtype=torch.int32, device=DEV)
        n = torch.tensor([len(ids_host)], dtype=torch.int32, device=DEV)
    srcs = [make_refresh_src(s, variant=l) for l in range(n_layers)]
    kc0, vc0 = _sentinel(s, s.dtype)
    k_src = [to_dev(x[0], s.dtype) for x in srcs]
    v_src = [to_dev(x[1], s.dtype) for x in srcs]
    kcs = [to_dev(kc0 * (l + 1), s.dtype) for l in range(n_layers)]
    vcs = [to_dev(vc0 * (l + 1), s.dtype) for l in range(n_layers)]
    say(f"refresh layers {name} {mode} subset={subset}")
    fd.kv_refresh_layers(seq, mode, k_src, v_src, kcs, vcs, ids, n)
    torch.cuda.synchronize()
    for l in range(n_layers):
        rk, rv = refresh_ref(srcs[l][0], srcs[l][1], kc0 * (l + 1), vc0 * (l + 1), s.prompt_lens, s.gen_len,
                             s.block_size, s.block_idxs, mode, seq_ids=ids_host)
        assert np.array_equal(kcs[l].float().cpu().numpy(), rk), f"layer {l} K"
        assert np.array_equal(vcs[l].float().cpu().numpy(), rv), f"layer {l} V"


def test_refresh_subset_from_device_list():
    s = shape_custom("rs", "bf16", 5, 4, 2, 128, [10, 20, 30, 40, 50], 64, 16, [0, 1, 2, 3, 0], 64, cfg_id=72)
    ks, vs = make_refresh_src(s)
    kc0, vc0 = _sentinel(s, s.dtype)
    say("refresh subset")
    kc, vc = _run_refresh(s, "dual", ks, vs, kc0, vc0, True, seq_ids=[4, 1])
    rk, rv = refresh_ref(ks, vs, kc0, vc0, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, "dual",
                         seq_ids=[4, 1])
    assert np.array_equal(kc, rk) and np.array_equal(vc, rv)


def test_c3_refresh_every_block_boundary():
    # Dream-7B shape: prefix-mode refresh at each of the 32 block boundaries
    # (rows [0, P + kB)) and the DualCache refresh (rows [0, L)).
    base = shape_c3(0)
    ks, vs = make_refresh_src(base)
    k_src, v_src = to_dev(ks, "bf16"), to_dev(vs, "bf16")
    kc0, vc0 = _sentinel(base, "bf16")
    kc, vc = to_dev(kc0, "bf16"), to_dev(vc0, "bf16")
    ks_t = torch.from_numpy(ks).to(DEV).to(torch.bfloat16)
    for k in range(32):
        s = shape_c3(k)
        say(f"c3 refresh prefix k={k}")
        fd.kv_refresh(seq_for(s), "prefix", k_src, v_src, kc, vc)
        torch.cuda.synchronize()
        hi = 1024 + 32 * k
        # rows below hi equal the source, the rest keep the sentinel (checked on the device)
        assert torch.equal(kc[:, :, :hi], ks_t[:, :hi].transpose(1, 2))
        assert bool((kc[:, :, hi:] == -3.0).all())
    # exact check against the oracle for the final state
    rk, rv = refresh_ref(ks, vs, kc0, vc0, base.prompt_lens, base.gen_len, base.block_size,
                         np.full(8, 31, np.int32), "prefix")
    assert np.array_equal(kc.float().cpu().numpy(), rk) and np.array_equal(vc.float().cpu().numpy(), rv)
    fd.kv_refresh(seq_for(base), "dual", k_src, v_src, kc, vc)
    torch.cuda.synchronize()
    rk, rv = refresh_ref(ks, vs, kc0, vc0, base.prompt_lens, base.gen_len, base.block_size, base.block_idxs,
                         "dual")
    assert np.array_equal(kc.float().cpu().numpy(), rk) and np.array_equal(vc.float().cpu().numpy(), rv)


def test_c5_full_step_28_layers():
    """Ragged Dream-7B batch: 28 x block attention (one cache per layer), one
    unmask with block advance, then refresh of every finished sequence's 28
    layer caches from the device-side done list."""
    s = shape_c5()
    n_layers = 28
    keep = []
    bidx = torch.from_numpy(s.block_idxs.astype(np.int32)).to(DEV)
    seq = seq_for(s, True, keep, bidx)
    inp = make_attn_inputs(s, "dual")
    q, kn, vn = to_dev(inp.q, "bf16"), to_dev(inp.k_new, "bf16"), to_dev(inp.v_new, "bf16")
    kc0, vc0 = to_dev(inp.k_cache, "bf16"), to_dev(inp.v_cache, "bf16")
    # each layer owns its cache; layer l holds the same values scaled by a
    # power of two (exact in bf16), so every layer's output is distinct
    kcs = [kc0 * (2.0 ** -(l % 3)) for l in range(n_layers)]
    vcs = [vc0.clone() for _ in range(n_layers)]
    ad = fd.attn_desc(28, 4, 128, fd.BF16)
    ws = fd.new_workspace(fd.block_attn_workspace(seq, ad, "dual", q.shape[1]))
    outs = [torch.empty_like(q) for _ in range(n_layers)]
    logits = make_logits(s, "calibrated")
    tokens, mask = make_decode_state(s, n_masked_c5(s))
    lg = to_dev(logits, "bf16")
    tk = torch.from_numpy(tokens).to(DEV)
    mk = torch.from_numpy(mask).to(DEV)
    nd = torch.zeros(s.batch, dtype=torch.int32, device=DEV)
    dp = torch.zeros((s.batch, 32), dtype=torch.int32, device=DEV)
    ds = torch.zeros(s.batch, dtype=torch.int32, device=DEV)
    nn = torch.zeros(1, dtype=torch.int32, device=DEV)
    uws = fd.new_workspace(fd.unmask_workspace(seq, s.vocab, fd.BF16))
    srcs = make_refresh_src(s)
    k_src, v_src = to_dev(srcs[0], "bf16"), to_dev(srcs[1], "bf16")
    say("c5 full step: 28 x attn + unmask + one refresh of the done list's 28 layers")
    for l in range(n_layers):
        fd.block_attn(seq, "dual", q, kn, vn, kcs[l], vcs[l], outs[l], ws)
    fd.unmask_threshold(seq, lg, 0.7, tk, mk, nd, dp, None, ds, nn, uws, flags=fd.UNMASK_ADVANCE_BLOCK)
    # every layer's caches from the same full-forward sources (shared)
    fd.kv_refresh_layers(seq, "dual", [k_src] * n_layers, [v_src] * n_layers, kcs, vcs, ds, nn)
    torch.cuda.synchronize()
    # attention of every sequence on layers 0-2 (the three distinct cache
    # scalings); layers 3..27 repeat them and must equal them bit for bit
    for l in (0, 1, 2):
        li = AttnInputs(s, "dual", inp.q, inp.k_new, inp.v_new, inp.k_cache * (2.0 ** -(l % 3)), inp.v_cache)
        ref = attn_ref(li.q, li.k_new, li.v_new, li.k_cache, li.v_cache, s.prompt_lens, s.gen_len, s.block_size,
                       s.block_idxs, "dual")
        out = outs[l].float().cpu().numpy().astype(np.float64)
        check_attn(out, ref, li, label=f"c5 step layer {l}")
    for l in range(3, n_layers):
        assert torch.equal(outs[l], outs[l % 3]), f"layer {l} differs from layer {l % 3} on identical inputs"
    # unmask decisions
    ref = unmask_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, 0.7,
                     advance=True)
    # the conf output was not requested in this step: compare decisions only
    g = dict(tokens=tk.cpu().numpy(), mask=mk.cpu().numpy(), n_decoded=nd.cpu().numpy(),
             decoded_pos=dp.cpu().numpy(), conf=ref.conf.copy())
    compare_unmask(g, ref, s, label="c5 step")
    done = sorted(int(x) for x in ds.cpu().numpy()[:int(nn.item())])
    if not ref.tie_step.any() and not ref.tie_tau.any():
        assert done == list(ref.done_seqs)
    # refreshed sequences' caches equal the source on every layer; others untouched
    ks_t, vs_t = k_src.transpose(1, 2), v_src.transpose(1, 2)
    for l in range(n_layers):
        for i in range(s.batch):
            L = int(s.prompt_lens[i]) + s.gen_len
            if i in done:
                assert torch.equal(kcs[l][i, :, :L], ks_t[i, :, :L]) and torch.equal(vcs[l][i, :, :L], vs_t[i, :, :L])
                assert torch.equal(kcs[l][i, :, L:], (kc0[i] * (2.0 ** -(l % 3)))[:, L:])
            else:
                assert torch.equal(kcs[l][i], kc0[i] * (2.0 ** -(l % 3))) and torch.equal(vcs[l][i], vc0[i])
    say(f"  c5 step: {len(done)} sequences finished their block and were refreshed")
