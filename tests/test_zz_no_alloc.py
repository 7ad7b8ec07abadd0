"""GPU: the allocation-free threshold unmask (fdllm_unmask_threshold_static,
scratch in a static device array) decides exactly like
fdllm_unmask_threshold with a caller workspace, on two calls in a row, the
second with a smaller batch, block and vocabulary; it calls no allocator."""
import numpy as np
import pytest
import torch

import block_wise_kv_amd as fd
from gpu_util import DEV, require_gpu, say, seq_for, to_dev
from workloads import make_decode_state, make_logits, n_masked_c5, shape_c3, shape_custom

pytestmark = pytest.mark.gpu


def _both(s, logits, tokens, mask, tau, flags):
    """The same step through both entry points; returns their outputs."""
    lg = to_dev(logits, s.dtype)
    outs = []
    for static in (False, True):
        keep = []
        bidx = torch.from_numpy(s.block_idxs.astype(np.int32)).to(DEV)
        seq = seq_for(s, True, keep, bidx)
        tk = torch.from_numpy(tokens.astype(np.int32)).to(DEV)
        mk = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
        nd = torch.full((s.batch,), -7, dtype=torch.int32, device=DEV)
        dp = torch.full((s.batch, s.block_size), -7, dtype=torch.int32, device=DEV)
        cf = torch.full((s.batch, s.block_size), -7.0, dtype=torch.float64, device=DEV)
        ds = torch.full((s.batch,), -7, dtype=torch.int32, device=DEV)
        nn = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        if static:
            before = torch.cuda.memory_allocated()
            fd.unmask_threshold_static(seq, lg, tau, tk, mk, nd, dp, cf, ds, nn, flags=flags)
            assert torch.cuda.memory_allocated() == before
        else:
            ws = fd.new_workspace(fd.unmask_workspace(seq, s.vocab, fd.BF16 if s.dtype == "bf16" else fd.F32))
            fd.unmask_threshold(seq, lg, tau, tk, mk, nd, dp, cf, ds, nn, ws, flags=flags)
        torch.cuda.synchronize()
        outs.append(dict(tokens=tk.cpu().numpy(), mask=mk.cpu().numpy(), n_decoded=nd.cpu().numpy(),
                         decoded_pos=dp.cpu().numpy(), conf=cf.cpu().numpy(), n_done=int(nn.item()),
                         done_seqs=ds.cpu().numpy(), block_idxs=bidx.cpu().numpy()))
    return outs


def _same(a, b, label):
    for key in a:
        if key == "conf":
            assert np.array_equal(a[key].view(np.uint64), b[key].view(np.uint64)), f"{label}: conf differs"
        else:
            assert np.array_equal(a[key], b[key]), f"{label}: {key} differs"


def test_static_scratch_matches_workspace_entry_point():
    require_gpu()
    # call 1: the Dream-7B batch (8 x 32 rows of 152064 logits, 16 vocabulary
    # chunks per row), calibrated confidences, block advance, done list
    s = shape_c3(5)
    logits = make_logits(s, "calibrated")
    tokens, mask = make_decode_state(s, np.array([32, 1, 5, 32, 2, 17, 1, 9]))
    say("static scratch: Dream-7B batch, tau 0.8, block advance")
    ws_out, st_out = _both(s, logits, tokens, mask, 0.8, fd.UNMASK_ADVANCE_BLOCK)
    _same(ws_out, st_out, "call 1")
    assert st_out["n_done"] >= 1 and int(st_out["n_decoded"].sum()) > 8
    # call 2: smaller in every dimension (3 sequences, block 16, vocabulary
    # 1000, fp32 logits), so every counter and partial lands where call 1
    # left other values
    s2 = shape_custom("static_small", "f32", 3, 1, 1, 8, [40, 7, 90], 64, 16, [1, 3, 0], 1000, cfg_id=88)
    logits2 = make_logits(s2, "calibrated")
    tokens2, mask2 = make_decode_state(s2, np.array([16, 3, 1]))
    say("static scratch: 3 sequences, block 16, vocabulary 1000, fp32, tau 0.6")
    ws2, st2 = _both(s2, logits2, tokens2, mask2, 0.6, fd.UNMASK_ADVANCE_BLOCK)
    _same(ws2, st2, "call 2")
    say(f"  both calls bit-identical to the workspace entry point; call 1 decoded "
        f"{int(st_out['n_decoded'].sum())} tokens, call 2 {int(st2['n_decoded'].sum())}")


def test_static_scratch_rejects_oversized_batches():
    require_gpu()
    s = shape_custom("static_big", "bf16", 4097, 1, 1, 8, [4], 32, 32, [0], 64, cfg_id=89)
    seq = fd.seq_desc(s.batch, s.max_seq_len, s.gen_len, s.block_size, 4, 0)
    lg = torch.zeros((s.batch, 32, 64), dtype=torch.bfloat16, device=DEV)
    tk = torch.zeros((s.batch, s.max_seq_len), dtype=torch.int32, device=DEV)
    mk = torch.zeros((s.batch, s.max_seq_len), dtype=torch.uint8, device=DEV)
    nd = torch.zeros(s.batch, dtype=torch.int32, device=DEV)
    with pytest.raises(fd.FdllmError) as e:
        fd.unmask_threshold_static(seq, lg, 0.9, tk, mk, nd)
    assert e.value.status == 2 and "static scratch" in str(e.value)
