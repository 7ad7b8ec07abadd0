"""Debug mode (fdllm_set_debug): device-resident per-sequence arrays are
checked on the device before a call's kernels.  Valid arrays give the same
results as the trusted path; an invalid entry makes the call return
FDLLM_ERR_INVALID_ARG naming it, with nothing launched (outputs keep their
sentinels).  Invalid arrays are only ever passed with debug mode on, so no
compute kernel sees them."""
import numpy as np
import pytest
import torch

import block_wise_kv_amd as fd
from gpu_util import DEV, require_gpu, say, seq_for, to_dev
from workloads import make_attn_inputs, make_decode_state, make_lmhead_inputs, make_logits, make_refresh_src, \
    shape_custom

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    fd.set_debug(True)
    yield
    fd.set_debug(False)


def _shape():
    return shape_custom("dbg", "bf16", 3, 4, 2, 128, [40, 75, 20], 96, 32, [0, 2, 1], 900, cfg_id=86)


def _dev(a):
    return torch.tensor(np.asarray(a, np.int32), device=DEV)


def _seq(s, plens=None, bidx=None, max_p=None):
    pl = _dev(s.prompt_lens if plens is None else plens)
    bi = _dev(s.block_idxs if bidx is None else bidx)
    mp = int(s.prompt_lens.max()) if max_p is None else max_p
    return fd.seq_desc(s.batch, s.max_seq_len, s.gen_len, s.block_size, prompt_lens=pl, block_idxs=bi,
                       max_prompt_len=mp), (pl, bi)


def _attn(s, seq):
    inp = make_attn_inputs(s, "dual")
    q, kn, vn, kc, vc = (to_dev(x, "bf16") for x in (inp.q, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache))
    out = torch.full_like(q, 7.0)
    ws = fd.new_workspace(fd.block_attn_workspace(seq, fd.attn_desc(4, 2, 128, fd.BF16), "dual", q.shape[1]))
    fd.block_attn(seq, "dual", q, kn, vn, kc, vc, out, ws)
    torch.cuda.synchronize()
    return out


def test_valid_arrays_match_trusted_path():
    s = _shape()
    seq, keep = _seq(s)
    got = _attn(s, seq)
    fd.set_debug(False)
    ref = _attn(s, seq)
    fd.set_debug(True)
    assert torch.equal(got, ref)
    # unmask, LM head and refresh with valid arrays also run
    tokens, mask = make_decode_state(s, [5, 32, 9])
    lg = to_dev(make_logits(s, "calibrated"), "bf16")
    tk, mk = torch.from_numpy(tokens).to(DEV), torch.from_numpy(mask).to(DEV)
    nd = torch.zeros(3, dtype=torch.int32, device=DEV)
    fd.unmask_threshold(seq, lg, 0.7, tk, mk, nd, workspace=fd.new_workspace(fd.unmask_workspace(seq, 900, fd.BF16)))
    lm = make_lmhead_inputs(s, 256)
    wp = fd.lmhead_pack(torch.from_numpy(lm.w_codes).to(DEV).to(torch.bfloat16))
    fd.lmhead_unmask_threshold(seq, to_dev(lm.x, "bf16"), wp, 900, 0.7, tk, mk, nd,
                               workspace=fd.new_workspace(fd.lmhead_unmask_workspace(seq, 900, 256)))
    ks, vs = make_refresh_src(s)
    kc = torch.zeros((3, 2, s.max_seq_len, 128), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    fd.kv_refresh(seq, "dual", to_dev(ks, "bf16"), to_dev(vs, "bf16"), kc, vc, _dev([2, 0]), _dev([2]))
    torch.cuda.synchronize()
    say("  debug mode: valid arrays pass, attention identical to the trusted path")


@pytest.mark.parametrize("case, kw, msg", [
    ("block index = G/B", {"bidx": [0, 3, 1]}, "block_idxs[1] outside [0, 3)"),
    ("negative block index", {"bidx": [-1, 2, 1]}, "block_idxs[0] outside"),
    ("prompt above its bound", {"plens": [40, 76, 20], "max_p": 75}, "prompt_lens[1] outside [0, max_prompt_len 75]"),
    ("negative prompt", {"plens": [40, 75, -3]}, "prompt_lens[2] outside"),
])
def test_bad_sequence_arrays_rejected(case, kw, msg):
    s = _shape()
    seq, keep = _seq(s, **kw)
    inp = make_attn_inputs(s, "dual")
    q, kn, vn, kc, vc = (to_dev(x, "bf16") for x in (inp.q, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache))
    out = torch.full_like(q, 7.0)
    ws = fd.new_workspace(fd.block_attn_workspace(seq, fd.attn_desc(4, 2, 128, fd.BF16), "dual", q.shape[1]))
    with pytest.raises(fd.FdllmError) as ei:
        fd.block_attn(seq, "dual", q, kn, vn, kc, vc, out, ws)
    assert ei.value.status == 1 and msg in str(ei.value), str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a kernel ran despite the rejection"
    # the unmask rejects the same arrays, tokens untouched
    tokens, mask = make_decode_state(s, 32)
    tk, mk = torch.from_numpy(tokens).to(DEV), torch.from_numpy(mask).to(DEV)
    nd = torch.full((3,), -7, dtype=torch.int32, device=DEV)
    with pytest.raises(fd.FdllmError):
        fd.unmask_threshold(seq, to_dev(make_logits(s, "calibrated"), "bf16"), 0.5, tk, mk, nd,
                            workspace=fd.new_workspace(fd.unmask_workspace(seq, 900, fd.BF16)))
    torch.cuda.synchronize()
    assert np.array_equal(tk.cpu().numpy(), tokens) and bool((nd == -7).all())
    say(f"  {case}: rejected ({ei.value})")


@pytest.mark.parametrize("ids, n, msg", [
    ([0, 3], [2], "seq_ids[1] outside [0, batch 3)"),
    ([0, 1], [4], "n_seq outside [0, batch 3]"),
    ([-1], [1], "seq_ids[0] outside"),
])
def test_bad_refresh_list_rejected(ids, n, msg):
    s = _shape()
    seq, keep = _seq(s)
    ks, vs = make_refresh_src(s)
    kc = torch.full((3, 2, s.max_seq_len, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, 7.0)
    with pytest.raises(fd.FdllmError) as ei:
        fd.kv_refresh(seq, "dual", to_dev(ks, "bf16"), to_dev(vs, "bf16"), kc, vc, _dev(ids), _dev(n))
    assert ei.value.status == 1 and msg in str(ei.value), str(ei.value)
    torch.cuda.synchronize()
    assert bool((kc == 7.0).all()) and bool((vc == 7.0).all())
