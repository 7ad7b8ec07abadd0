"""Helpers for the GPU parity tests: upload seeded inputs, run libfdllm
through its C ABI binding, and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import block_wise_kv_amd as fd
from oracle import attn_ref, unmask_ref

DEV = "cuda"

ATTN_TOL = {"bf16": 2e-2, "f32": 1e-5}
CONF_TOL = 1e-6


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fd.lib()  # fails loudly when libfdllm.so is missing


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def tdtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(x: np.ndarray, dtype: str):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV).to(tdtype(dtype))


def seq_for(shape, ragged: bool = False, keep: list = None, block_idxs_dev=None):
    """SeqDesc for a workloads.Shape; device arrays are appended to `keep`."""
    s = shape
    if not ragged:
        return fd.seq_desc(s.batch, s.max_seq_len, s.gen_len, s.block_size,
                           prompt_len=int(s.prompt_lens[0]), block_idx=int(s.block_idxs[0]))
    pl = torch.from_numpy(s.prompt_lens.astype(np.int32)).to(DEV)
    bi = block_idxs_dev if block_idxs_dev is not None else torch.from_numpy(
        s.block_idxs.astype(np.int32)).to(DEV)
    if keep is not None:
        keep += [pl, bi]
    return fd.seq_desc(s.batch, s.max_seq_len, s.gen_len, s.block_size, prompt_lens=pl, block_idxs=bi,
                       max_prompt_len=int(s.prompt_lens.max()))


def nq_of(shape, mode, i):
    P, k, B, G = int(shape.prompt_lens[i]), int(shape.block_idxs[i]), shape.block_size, shape.gen_len
    return {"dual": B, "prefix": G - k * B, "none": P + G}[mode]


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def run_attn(inp, ragged: bool = False, reps: int = 1, ws=None):
    """Run fdllm_block_attn on AttnInputs; returns (out float64 [b][cap][Hq][d], raw list,
    workspace).  `ws` reuses a caller's workspace instead of a fresh zeroed one."""
    s, mode = inp.shape, inp.mode
    keep = []
    seq = seq_for(s, ragged, keep)
    q = to_dev(inp.q, s.dtype)
    kn = to_dev(inp.k_new, s.dtype)
    vn = to_dev(inp.v_new, s.dtype)
    kc = to_dev(inp.k_cache, s.dtype) if inp.k_cache is not None else None
    vc = to_dev(inp.v_cache, s.dtype) if inp.v_cache is not None else None
    ad = fd.attn_desc(s.n_q_heads, s.n_kv_heads, s.head_dim, fd.BF16 if s.dtype == "bf16" else fd.F32)
    if ws is None:
        ws = fd.new_workspace(fd.block_attn_workspace(seq, ad, mode, q.shape[1]))
    outs = []
    for _ in range(reps):
        out = torch.full(q.shape, float("nan"), dtype=q.dtype, device=DEV)
        fd.block_attn(seq, mode, q, kn, vn, kc, vc, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    res = [o.float().cpu().numpy().astype(np.float64) for o in outs]
    return res[0], res, ws


def check_attn(out, ref, inp, seqs=None, label=""):
    """Max |err| over live rows within the dtype tolerance; rows past nq untouched (NaN)."""
    s, mode = inp.shape, inp.mode
    tol = ATTN_TOL[s.dtype]
    worst = 0.0
    for i in (range(s.batch) if seqs is None else seqs):
        nq = nq_of(s, mode, i)
        live_g = out[i, :nq]
        live_r = ref[i, :nq] if ref.shape[0] == s.batch else ref[list(seqs).index(i), :nq]
        assert np.isfinite(live_g).all(), f"{label}: non-finite output in sequence {i}"
        err = float(np.max(np.abs(live_g - live_r)))
        worst = max(worst, err)
        assert np.isnan(out[i, nq:]).all(), f"{label}: rows past nq written in sequence {i}"
    say(f"  {label}: max|err| = {worst:.3e} (tol {tol:g})")
    assert worst <= tol, f"{label}: max|err| {worst} > {tol}"
    return worst


def oracle_attn_subset(inp, seqs):
    s = inp.shape
    idx = list(seqs)
    kc = inp.k_cache[idx] if inp.k_cache is not None else None
    vc = inp.v_cache[idx] if inp.v_cache is not None else None
    return attn_ref(inp.q[idx], inp.k_new[idx], inp.v_new[idx], kc, vc, s.prompt_lens[idx], s.gen_len,
                    s.block_size, s.block_idxs[idx], inp.mode)


# ---------------------------------------------------------------------------
# unmask
# ---------------------------------------------------------------------------

def run_unmask(shape, logits_np, tokens, mask, tau, ragged=False, flags=0, logits_dev=None, reps=1,
               dtype=None, topk=None):
    """Run fdllm_unmask_threshold (or fdllm_unmask_topk with k = topk);
    returns dict of numpy outputs (of the first rep)."""
    s = shape
    dt = dtype or s.dtype
    keep = []
    bidx = torch.from_numpy(s.block_idxs.astype(np.int32)).to(DEV) if (ragged or flags) else None
    seq = seq_for(s, ragged or bool(flags), keep, bidx)
    lg = logits_dev if logits_dev is not None else to_dev(logits_np, dt)
    ws = fd.new_workspace(fd.unmask_workspace(seq, lg.shape[2], fd.BF16 if lg.dtype == torch.bfloat16 else fd.F32))
    results = []
    for _ in range(reps):
        tk = torch.from_numpy(tokens.astype(np.int32)).to(DEV)
        mk = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
        if bidx is not None:
            bidx.copy_(torch.from_numpy(s.block_idxs.astype(np.int32)))
        nd = torch.full((s.batch,), -7, dtype=torch.int32, device=DEV)
        dp = torch.full((s.batch, s.block_size), -7, dtype=torch.int32, device=DEV)
        cf = torch.full((s.batch, s.block_size), -7.0, dtype=torch.float64, device=DEV)
        ds = torch.full((s.batch,), -7, dtype=torch.int32, device=DEV)
        nn = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        if topk is None:
            fd.unmask_threshold(seq, lg, tau, tk, mk, nd, dp, cf, ds, nn, ws, flags=flags)
        else:
            fd.unmask_topk(seq, lg, topk, tk, mk, nd, dp, cf, ds, nn, ws, flags=flags)
        torch.cuda.synchronize()
        r = dict(tokens=tk.cpu().numpy(), mask=mk.cpu().numpy(), n_decoded=nd.cpu().numpy(),
                 decoded_pos=dp.cpu().numpy(), conf=cf.cpu().numpy(), n_done=int(nn.item()),
                 done_seqs=ds.cpu().numpy()[:max(0, int(nn.item()))],
                 block_idxs=bidx.cpu().numpy() if bidx is not None else None)
        results.append(r)
    return results[0], results


def compare_unmask(g, ref, shape, label="", tau=None):
    """Bit-exact decisions except oracle-flagged near ties; returns excluded row count."""
    s = shape
    B = s.block_size
    excluded = 0
    top2 = 0
    for i in range(s.batch):
        start = int(s.prompt_lens[i]) + int(s.block_idxs[i]) * B
        if ref.tie_step[i]:
            excluded += int(np.sum(~np.isnan(ref.conf[i])))
            continue
        t1 = ref.tie_tau[i]
        excluded += int(t1.sum())
        for t in range(B):
            masked = not np.isnan(ref.conf[i, t])
            if masked:
                assert abs(g["conf"][i, t] - ref.conf[i, t]) <= CONF_TOL, \
                    f"{label}: conf seq {i} row {t}: {g['conf'][i, t]} vs {ref.conf[i, t]}"
                if ref.tie_top2[i, t]:
                    top2 += 1
            else:
                assert np.isnan(g["conf"][i, t]), f"{label}: conf written for unmasked row {i},{t}"
            if t1[t]:
                continue
            p = start + t
            assert g["mask"][i, p] == ref.mask[i, p], f"{label}: mask seq {i} row {t}"
            assert g["tokens"][i, p] == ref.tokens[i, p], \
                f"{label}: token seq {i} row {t}: {g['tokens'][i, p]} vs {ref.tokens[i, p]}"
        if not t1.any():
            assert g["n_decoded"][i] == ref.n_decoded[i], f"{label}: n_decoded seq {i}"
            assert np.array_equal(g["decoded_pos"][i], ref.decoded_pos[i]), f"{label}: decoded_pos seq {i}"
        # nothing outside the block changes
        outside = np.ones(s.max_seq_len, bool)
        outside[start:start + B] = False
        assert np.array_equal(g["tokens"][i, outside], ref.tokens[i, outside])
        assert np.array_equal(g["mask"][i, outside], ref.mask[i, outside])
    say(f"  {label}: decisions bit-exact; near-tie rows excluded = {excluded}; top-2 ties compared = {top2}; "
        f"tokens decoded = {int(ref.n_decoded.sum())}")
    return excluded


def lmhead_weight_dev(inp):
    """The projection weight of a workloads.LmheadInputs as a bf16 device tensor."""
    if inp.w_codes is not None:
        return torch.from_numpy(inp.w_codes).to(DEV).to(torch.bfloat16)  # small integers: exact
    return to_dev(inp.w, "bf16")


def run_lmhead(shape, inp, tokens, mask, tau=None, topk=None, ragged=False, flags=0, x_dev=None, w_packed=None):
    """Run fdllm_lmhead_unmask_threshold (or _topk with k = topk) on the hidden
    states of `inp`; returns a dict of numpy outputs like run_unmask."""
    s = shape
    keep = []
    bidx = torch.from_numpy(s.block_idxs.astype(np.int32)).to(DEV) if (ragged or flags) else None
    seq = seq_for(s, ragged or bool(flags), keep, bidx)
    x = x_dev if x_dev is not None else to_dev(inp.x, "bf16")
    wp = w_packed if w_packed is not None else fd.lmhead_pack(lmhead_weight_dev(inp))
    ws = fd.new_workspace(fd.lmhead_unmask_workspace(seq, s.vocab, inp.hidden))
    tk = torch.from_numpy(tokens.astype(np.int32)).to(DEV)
    mk = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    nd = torch.full((s.batch,), -7, dtype=torch.int32, device=DEV)
    dp = torch.full((s.batch, s.block_size), -7, dtype=torch.int32, device=DEV)
    cf = torch.full((s.batch, s.block_size), -7.0, dtype=torch.float64, device=DEV)
    ds = torch.full((s.batch,), -7, dtype=torch.int32, device=DEV)
    nn = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    if topk is None:
        fd.lmhead_unmask_threshold(seq, x, wp, s.vocab, tau, tk, mk, nd, dp, cf, ds, nn, ws, flags=flags)
    else:
        fd.lmhead_unmask_topk(seq, x, wp, s.vocab, topk, tk, mk, nd, dp, cf, ds, nn, ws, flags=flags)
    torch.cuda.synchronize()
    return dict(tokens=tk.cpu().numpy(), mask=mk.cpu().numpy(), n_decoded=nd.cpu().numpy(),
                decoded_pos=dp.cpu().numpy(), conf=cf.cpu().numpy(), n_done=int(nn.item()),
                done_seqs=ds.cpu().numpy()[:max(0, int(nn.item()))],
                block_idxs=bidx.cpu().numpy() if bidx is not None else None)
