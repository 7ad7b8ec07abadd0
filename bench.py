#!/usr/bin/env python3
"""Benchmark of the Fast-dLLM block-decoding hot path on one MI355X.

Default workload: the ragged Dream-7B batch -- 64 sequences, 28 query / 4
KV heads x 128, prompt lengths U(256, 4096) per sequence, gen 512, block 32,
block index U{0..15} per sequence, U{1..32} masked block rows per sequence,
DualCache, vocabulary 152064, threshold 0.7 on calibrated confidences (each
masked row's top probability u ~ U(0.5, 1), so a step decodes several
tokens per sequence and some blocks finish, as in real decoding; the
literal peak recipe falls back to one token per row and, at this seed,
finishes no block).  One step is one full decoding
step of the 28-layer model's hot path: the block attention of every layer
(fdllm_block_attn over that layer's own cache), one threshold unmask over
the batch with block advance (fdllm_unmask_threshold), then the cache
refresh of every sequence whose block is finished, in every layer, in one
launch (fdllm_kv_refresh_layers from the device-side done list).  Inputs are seeded
synthetic tensors already resident in HBM (34 GB: each layer owns its
caches, refresh sources and fresh rows, so nothing is served from the
256 MB Infinity Cache); every step starts from the same decoding state (its
own copies of tokens, mask and block indices).

value = layer block-steps per second = 28 x steps / elapsed: each layer's
block attention counts as one block-step, with the step's single unmask and
its refresh amortised over the 28 layers (the reading of "block-steps/s per
layer (attn + unmask)" for a whole model step).  Beside it:
attn_unmask_block_steps_per_s = 1 / (t_attn + t_unmask) per call, the
sequence rates (times the batch) and the refresh reported on its own.

The K timed steps are captured once in a HIP graph and replayed between two
device synchronisations.  Per-kernel durations come from a second pass over
the same K steps in which every call is launched with its own start/stop
HIP events (libfdllm's timing hook, hipExtLaunchKernel), on the stream it
runs on.  The fp64 oracle is timed on the host's cores (all of them, then
one thread) on one layer of the same step, scaled to the full step.

--workload selects other shapes for measuring the kernels (c2: LLaDA-8B b1
DualCache swept over block index 0..7, c3 / c3p: Dream-7B b8 DualCache /
prefix cache, c4: LLaDA-8B b32).  --sweep-block-size times attention and
unmask of the large-batch LLaDA-8B layer at block sizes 4..128;
--sweep-tau decodes its blocks at thresholds 0.5..1.0 and counts the tokens
decoded per step.  Prints one JSON line.  --gpus N > 1 is refused: this path
runs on one GPU.

--lmhead measures the step before the unmask instead: the vocabulary
projection fused with the confidence pass (fdllm_lmhead_unmask_threshold,
the logits never written) on the workload's rows (c2: 32 rows, hidden 4096,
vocabulary 126464; c3: 256 rows, hidden 3584, vocabulary 152064; c4: 1024
rows, hidden 4096), K calls replayed from a HIP graph, then per-call events;
beside it the unfused path (torch's linear layer writing bf16 logits, then
fdllm_unmask_threshold reading them) for comparison.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-steps/s per layer (attn+unmask) and achieved HBM GB/s as % of peak, 1 GPU"
PEAK_HBM_BPS = 8.0e12
N_BLOCKS = 8                 # block indices of the LLaDA-8B workload (CPU baseline)
TAUS = (0.7, 0.9, 1.0)

# Workloads.  The default (c5, the largest single-GPU configuration) is
# measured by c5_main; the others exist for measuring the kernels at the
# other shapes.
WORKLOADS = {
    "c5": dict(desc="Ragged Dream-7B batch: 64 sequences, 28 q / 4 kv heads x 128, prompt U(256, 4096) per sequence, "
                    "gen 512, block 32, block index U{0..15} and U{1..32} masked rows per sequence, DualCache, "
                    "vocab 152064, calibrated confidences, tau 0.7; one step = 28 x block attention (one cache per layer) + 1 x threshold "
                    "unmask with block advance + refresh of the finished sequences' 28 layer caches (one launch)",
               steps=50, warmup=40, layers=28, logit_sets=2),
    "c2": dict(desc="LLaDA-8B-shaped layer: batch 1, 32 heads x 128 (MHA), prompt 512 + gen 256, block 32, "
                    "DualCache, block index 0..7 swept, tau in {0.7, 0.9, 1.0}, vocab 126464; "
                    "one block-step = refresh + attention + unmask",
               shape="c2", mode="dual", blocks=list(range(8)), layers=32, logit_sets=48, taus=(0.7, 0.9, 1.0),
               steps=200, warmup=20),
    "c3": dict(desc="Dream-7B-shaped GQA layer: batch 8, 28 q / 4 kv heads x 128, prompt 1024 + gen 1024, block 32, "
                    "DualCache, block index 0..31 swept, tau 0.9, vocab 152064",
               shape="c3", mode="dual", blocks=list(range(32)), layers=28, logit_sets=8, taus=(0.9,),
               steps=10, warmup=2),
    "c3p": dict(desc="Dream-7B-shaped GQA layer, prefix cache: batch 8, 28 q / 4 kv heads x 128, prompt 1024 + "
                     "gen 1024, block 32, block index 0, 8, 16, 24, 31, tau 0.9",
                shape="c3", mode="prefix", blocks=[0, 8, 16, 24, 31], layers=8, logit_sets=8, taus=(0.9,),
                steps=4, warmup=1),
    "c4": dict(desc="Large-batch LLaDA-8B-shaped layer: batch 32, 32 heads x 128, prompt 2048 + gen 512, block 32, "
                    "DualCache, block index 0..15 swept, tau 0.5..1.0",
               shape="c4", mode="dual", blocks=list(range(16)), layers=4, logit_sets=4,
               taus=(0.5, 0.6, 0.7, 0.8, 0.9, 1.0), steps=4, warmup=1),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOADS))
    ap.add_argument("--sweep-block-size", action="store_true",
                    help="large-batch LLaDA-8B layer: attention + unmask per call at block sizes 4..128")
    ap.add_argument("--sweep-tau", action="store_true",
                    help="large-batch LLaDA-8B layer: decode blocks at thresholds 0.5..1.0, tokens per step")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the all-core oracle baseline (0: the CPUs this process may use)")
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--layers", type=int, default=None, help="rotating cache/source sets")
    ap.add_argument("--logit-sets", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--rule", default="threshold", choices=("threshold", "topk"),
                    help="unmask rule: confidence threshold (default) or fixed-step top-k")
    ap.add_argument("--k", type=int, default=1, help="tokens per step of the fixed-step rule")
    ap.add_argument("--lmhead", action="store_true",
                    help="measure the fused vocabulary projection + unmask (c2, c3 or c4 rows)")
    ap.add_argument("--decode-block", action="store_true",
                    help="decode one LLaDA-8B block on the device: a graph of steps, each = attention of every "
                         "layer + fused LM head + unmask, tokens per step recorded")
    ap.add_argument("--tau", type=float, default=0.9, help="threshold of --decode-block")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB between two device buffers 3 times (counter calibration) and exit")
    args = ap.parse_args()
    w = WORKLOADS[args.workload]
    for key in ("steps", "warmup", "layers", "logit_sets"):
        if getattr(args, key) is None and not ((args.lmhead or args.decode_block or args.sweep_block_size
                                                 or args.sweep_tau) and key in ("steps", "warmup")):
            setattr(args, key, w[key])
    return args


def make_shape(name, k):
    from workloads import shape_c2, shape_c3, shape_c4
    return {"c2": shape_c2, "c3": shape_c3, "c4": lambda kk: shape_c4(32, kk)}[name](k)


class Bench:
    def __init__(self, args):
        import numpy as np
        import torch

        import block_wise_kv_amd as fd
        from workloads import make_attn_inputs, make_decode_state, make_logits, make_refresh_src

        self.fd, self.torch, self.np = fd, torch, np
        fd.lib()
        dev = "cuda"
        self.args = args
        self.unmask_name = "unmask_topk" if args.rule == "topk" else "unmask_threshold"
        w = WORKLOADS[args.workload]
        self.w = w
        self.blocks = w["blocks"]
        self.nb = len(self.blocks)
        self.mode = w["mode"]
        s0 = make_shape(w["shape"], self.blocks[0])
        self.shape = s0
        b, Hq, Hkv, d, B, V = s0.batch, s0.n_q_heads, s0.n_kv_heads, s0.head_dim, s0.block_size, s0.vocab
        bf = torch.bfloat16

        def up(x):
            return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(bf)

        # per-block-index fresh rows, per-layer caches and refresh sources
        self.seqs, self.fresh, self.out = [], [], []
        for n, k in enumerate(self.blocks):
            s = make_shape(w["shape"], k)
            self.seqs.append(fd.seq_desc(b, s.max_seq_len, s.gen_len, B, int(s.prompt_lens[0]), k))
            a = make_attn_inputs(s, self.mode, variant=k, caches=(n == 0))
            nq = {"dual": B, "prefix": s.gen_len - k * B}[self.mode]
            self.fresh.append(tuple(up(x[:, :nq]) for x in (a.q, a.k_new, a.v_new)))
            self.out.append(torch.empty_like(self.fresh[-1][0]))
            if n == 0:
                kc, vc = up(a.k_cache), up(a.v_cache)
            del a
        ks, vs = make_refresh_src(s0)
        ks, vs = up(ks), up(vs)
        L = args.layers
        self.kc = [kc.clone() for _ in range(L)]
        self.vc = [vc.clone() for _ in range(L)]
        self.ks = [ks.clone() for _ in range(L)]
        self.vs = [vs.clone() for _ in range(L)]
        del kc, vc, ks, vs
        lg = up(make_logits(s0, "peak"))
        self.logits = [lg.clone() for _ in range(args.logit_sets)]
        del lg
        # pristine decode state per block index: every block row masked
        tok0, mask0 = [], []
        for k in self.blocks:
            t, m = make_decode_state(make_shape(w["shape"], k))
            tok0.append(torch.from_numpy(t).to(dev))
            mask0.append(torch.from_numpy(m).to(dev))
        n_calls = (args.warmup + args.steps) * self.nb
        self.tok_pristine = torch.stack([tok0[c % self.nb] for c in range(n_calls)])
        self.mask_pristine = torch.stack([mask0[c % self.nb] for c in range(n_calls)])
        self.tok = torch.empty_like(self.tok_pristine)
        self.mask = torch.empty_like(self.mask_pristine)
        self.n_dec = torch.zeros(b, dtype=torch.int32, device=dev)
        self.dpos = torch.zeros((b, B), dtype=torch.int32, device=dev)
        self.done = torch.zeros(b, dtype=torch.int32, device=dev)
        self.n_done = torch.zeros(1, dtype=torch.int32, device=dev)
        ad = fd.attn_desc(Hq, Hkv, d, fd.BF16)
        self.ws_attn = [fd.new_workspace(fd.block_attn_workspace(sq, ad, self.mode, f[0].shape[1]))
                        for sq, f in zip(self.seqs, self.fresh)]
        self.ws_unmask = fd.new_workspace(fd.unmask_workspace(self.seqs[0], V, fd.BF16))
        self.reset_state()
        torch.cuda.synchronize()
        # algorithmic bytes per call, per block index
        L_full = int(s0.prompt_lens[0]) + s0.gen_len
        kv = 2 * b * Hkv * L_full * d * 2
        self.bytes = []
        self.flops = []
        for f in self.fresh:
            nq = f[0].shape[1]
            kv_read = kv if self.mode == "dual" else 2 * b * Hkv * (L_full - nq) * d * 2 + 2 * b * Hkv * nq * d * 2
            q_out = 2 * b * nq * Hq * d * 2
            self.bytes.append({"block_attn": kv_read + q_out,
                               self.unmask_name: b * B * V * 2,
                               "kv_refresh": 2 * kv if self.mode == "dual" else 0})
            self.flops.append(4 * b * Hq * nq * L_full * d)

    def reset_state(self):
        self.tok.copy_(self.tok_pristine)
        self.mask.copy_(self.mask_pristine)

    def launches(self, call):
        """The three kernels of block-step number `call` (in launch order)."""
        fd = self.fd
        n = call % self.nb
        L = self.args.layers
        la, lr = call % L, (call + L // 2) % L
        lg = self.logits[call % len(self.logits)]
        seq = self.seqs[n]
        q, kn, vn = self.fresh[n]
        taus = self.w["taus"]
        ops = []
        if self.mode == "dual":
            ops.append(("kv_refresh", lambda: fd.kv_refresh(seq, self.mode, self.ks[lr], self.vs[lr], self.kc[lr],
                                                            self.vc[lr])))
        ops.append(("block_attn", lambda: fd.block_attn(seq, self.mode, q, kn, vn, self.kc[la], self.vc[la],
                                                        self.out[n], self.ws_attn[n])))
        if self.args.rule == "topk":
            ops.append(("unmask_topk", lambda: fd.unmask_topk(
                seq, lg, self.args.k, self.tok[call], self.mask[call], self.n_dec, self.dpos, None,
                self.done, self.n_done, self.ws_unmask)))
        else:
            ops.append(("unmask_threshold", lambda: fd.unmask_threshold(
                seq, lg, taus[call % len(taus)], self.tok[call], self.mask[call], self.n_dec, self.dpos, None,
                self.done, self.n_done, self.ws_unmask)))
        return ops

    def run_steps(self, first_step, n_steps, events=None):
        """Launch the block-steps; with `events`, every kernel records its own
        start/stop HIP events (kernel n uses events 2n and 2n+1)."""
        names = []
        for st in range(first_step, first_step + n_steps):
            for n in range(self.nb):
                for name, fn in self.launches(st * self.nb + n):
                    if events is not None:
                        m = len(names)
                        self.fd.set_timing_events(events.ev[2 * m], events.ev[2 * m + 1])
                    fn()
                    names.append((name, n))
        return names


class HipEvents:
    """Timing events from the HIP runtime torch loaded (shared soname)."""

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e.value)

    def elapsed_s(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[a], self.ev[b])
        assert rc == 0, f"hipEventElapsedTime failed ({rc})"
        return ms.value * 1e-3

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def cpu_baseline(seconds: float):
    """The fp64 oracle on the host: C2 block-steps (refresh + attention +
    unmask) for block index 0..7 until the time budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attn_ref, refresh_ref, unmask_ref
    from workloads import make_attn_inputs, make_decode_state, make_logits, make_refresh_src, shape_c2

    s0 = shape_c2(0)
    ks, vs = make_refresh_src(s0)
    logits = make_logits(s0, "peak")
    inputs = []
    for k in range(N_BLOCKS):
        s = shape_c2(k)
        inputs.append((s, make_attn_inputs(s, "dual", variant=k), make_decode_state(s)))
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            s, a, (tok, msk) = inputs[done % N_BLOCKS]
            kc, vc = refresh_ref(ks, vs, a.k_cache, a.v_cache, s.prompt_lens, s.gen_len, s.block_size,
                                 s.block_idxs, "dual")
            attn_ref(a.q, a.k_new, a.v_new, kc, vc, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, "dual")
            unmask_ref(logits, tok, msk, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs,
                       TAUS[done % 3])
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": done / el, "unit": "block-steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} C2 block-steps (refresh + attention + unmask, block index 0..7 in turn) "
                      f"in {el:.1f} s, fp64 NumPy oracle, BLAS limited to 1 thread"}


# The sources each reported kernel is built from (besides the shared device
# and internal headers): counters taken on them stay valid until one changes.
KERNEL_SOURCES = {
    "block_attn": ["block_attn.hip"],
    "unmask_threshold": ["unmask.hip"],
    "kv_refresh": ["kv_refresh.hip"],
    "lmhead_unmask": ["lmhead.hip", "unmask.hip"],
}
SHARED_SOURCES = ["fdllm_device.h", "fdllm_internal.h"]


def kernel_source_sha256(kernel: str) -> str:
    """Digest of the HIP sources `kernel` is built from."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_wise_kv_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[kernel] + SHARED_SOURCES):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by what they read for a plain
    copy of known size); None when there is no summary for this workload or
    the kernel's sources have changed since the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "hbm_traffic.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    try:
        data = json.loads(text[start + 7:end])
    except ValueError:
        return None
    shas = data.get("source_sha256")
    if kernel not in KERNEL_SOURCES or not isinstance(shas, dict) or shas.get(kernel) != kernel_source_sha256(kernel):
        return None
    k = data.get("workloads", {}).get(workload, {}).get(kernel)
    if not k:
        return None
    return int(round(k["fetch_kib"] * 1024 * data["fetch_scale"] + k["write_kib"] * 1024 * data["write_scale"]))


def large_copy_rate() -> float:
    """Bytes/s (read + write) of a plain 1 GiB device-to-device copy, the
    measured reference beside the 8 TB/s peak."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / 5
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * n * 4 / t


def copy_probe(mib: int):
    """A plain device copy of known size, for scaling the HBM byte counters
    (FETCH_SIZE / WRITE_SIZE) of the profiler: each copy reads and writes
    exactly `mib` MiB."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "copies": 3}), flush=True)


# LM-head workloads: the rows of one decoding step of the same configs.
LMHEAD = {
    "c2": dict(desc="LLaDA-8B LM head fused with the threshold unmask: batch 1 x block 32 = 32 rows, hidden 4096, "
                    "vocab 126464, tau 0.9", shape="c2", hidden=4096, steps=50, warmup=5),
    "c3": dict(desc="Dream-7B LM head fused with the threshold unmask: batch 8 x block 32 = 256 rows, hidden 3584, "
                    "vocab 152064, tau 0.9", shape="c3", hidden=3584, steps=20, warmup=3),
    "c4": dict(desc="LLaDA-8B LM head fused with the threshold unmask: batch 32 x block 32 = 1024 rows, hidden 4096, "
                    "vocab 126464, tau 0.9", shape="c4", hidden=4096, steps=8, warmup=2),
}
PEAK_BF16_FLOPS = 2.5e15


def lmhead_cpu_baseline(inp, s, tokens, mask, tau, seconds):
    """The fp64 oracle's LM-head step (projection + threshold unmask) on the
    host, one thread, whole calls until the time budget is spent."""
    from threadpoolctl import threadpool_limits

    from oracle import lmhead_unmask_ref
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            lmhead_unmask_ref(inp.x, inp.weight(), tokens, mask, s.prompt_lens, s.gen_len, s.block_size,
                              s.block_idxs, threshold=tau)
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": done / el, "unit": "calls/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} whole LM-head + unmask calls of this workload in {el:.1f} s (fp64 NumPy oracle, "
                      "weight converted to fp64 inside each call, BLAS limited to 1 thread)"}


def lmhead_main(args):
    import numpy as np
    import torch

    import block_wise_kv_amd as fd
    from workloads import make_decode_state, make_lmhead_inputs, shape_c2, shape_c3, shape_c4

    if args.workload not in LMHEAD:
        print(f"--lmhead supports workloads {sorted(LMHEAD)}", file=sys.stderr)
        sys.exit(2)
    cfg = LMHEAD[args.workload]
    s = {"c2": shape_c2, "c3": shape_c3, "c4": shape_c4}[cfg["shape"]]()
    H, V, M = cfg["hidden"], s.vocab, s.batch * s.block_size
    K = args.steps or cfg["steps"]
    W = args.warmup if args.warmup is not None else cfg["warmup"]
    tau = 0.9
    inp = make_lmhead_inputs(s, H)
    dev = "cuda"
    x = torch.from_numpy(inp.x).to(dev).to(torch.bfloat16)
    w = torch.from_numpy(inp.w_codes).to(dev).to(torch.bfloat16)
    wp = fd.lmhead_pack(w)
    seq = fd.seq_desc(s.batch, s.max_seq_len, s.gen_len, s.block_size, int(s.prompt_lens[0]), int(s.block_idxs[0]))
    tokens, mask = make_decode_state(s, None)
    tk0 = torch.from_numpy(tokens).to(dev)
    mk0 = torch.from_numpy(mask).to(dev)
    n = W + K
    tks = [tk0.clone() for _ in range(n)]
    mks = [mk0.clone() for _ in range(n)]
    nd = torch.zeros(s.batch, dtype=torch.int32, device=dev)
    ws = fd.new_workspace(fd.lmhead_unmask_workspace(seq, V, H))

    def reset():
        for t in tks:
            t.copy_(tk0)
        for m in mks:
            m.copy_(mk0)

    def call(j):
        fd.lmhead_unmask_threshold(seq, x, wp, V, tau, tks[j], mks[j], nd, workspace=ws)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g_warm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_warm, stream=stream):
            for j in range(W):
                call(j)
        g_timed = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_timed, stream=stream):
            for j in range(W, n):
                call(j)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_timed.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-call events (both kernels of a call), eager on the default stream
    reset()
    torch.cuda.synchronize()
    events = HipEvents(2 * K)
    for m, j in enumerate(range(W, n)):
        fd.set_timing_events(events.ev[2 * m], events.ev[2 * m + 1])
        call(j)
    torch.cuda.synchronize()
    t_call = sum(events.elapsed_s(2 * m, 2 * m + 1) for m in range(K)) / K
    events.close()

    # the unfused path: torch's linear layer writes bf16 logits, the unmask reads them
    x2 = x.view(M, H)
    logits = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
    uws = fd.new_workspace(fd.unmask_workspace(seq, V, fd.BF16))
    reset()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t_gemm = t_unm = 0.0
    for j in range(n):
        e[0].record()
        torch.mm(x2, w.t(), out=logits)  # 2-D product (not batched): logits = x w^T
        e[1].record()
        fd.unmask_threshold(seq, logits.view(s.batch, s.block_size, V), tau, tks[j], mks[j], nd, workspace=uws)
        e[2].record()
        torch.cuda.synchronize()
        if j >= W:
            t_gemm += e[0].elapsed_time(e[1]) * 1e-3
            t_unm += e[1].elapsed_time(e[2]) * 1e-3
    t_gemm /= K
    t_unm /= K

    wbytes = V * H * 2
    alg_bytes = wbytes + M * H * 2
    flops = 2.0 * M * V * H
    hbm = flops / alg_bytes < PEAK_BF16_FLOPS / PEAK_HBM_BPS
    if hbm:
        roof = {"bound": "hbm", "kernel": "lmhead_unmask", "achieved": round(alg_bytes / t_call / 1e9, 1),
                "peak": 8000.0, "unit": "GB/s", "frac": round(alg_bytes / t_call / PEAK_HBM_BPS, 4)}
    else:
        roof = {"bound": "mfma", "kernel": "lmhead_unmask", "achieved": round(flops / t_call / 1e12, 1),
                "peak": 2500.0, "unit": "TFLOP/s", "frac": round(flops / t_call / PEAK_BF16_FLOPS, 4)}
    roof["traffic"] = measured_traffic("lm_" + args.workload, "lmhead_unmask")
    roof["algorithmic_bytes"] = alg_bytes
    roof["flops"] = flops
    result = {
        "metric": "fused LM-head projection + threshold unmask calls/s (logits never written), 1 GPU",
        "value": round(K / elapsed, 2),
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["desc"], "name": "lm_" + args.workload, "rows": M, "hidden": H, "vocab": V,
                   "graph": True},
        "roofline": roof,
        "kernels": {"lmhead_unmask": {"avg_us": round(t_call * 1e6, 3), "launches": K, "bytes": alg_bytes,
                                      "GB_per_s": round(alg_bytes / t_call / 1e9, 1),
                                      "TFLOP_per_s": round(flops / t_call / 1e12, 2)}},
        "unfused": {"linear_us": round(t_gemm * 1e6, 2), "unmask_us": round(t_unm * 1e6, 2),
                    "total_us": round((t_gemm + t_unm) * 1e6, 2),
                    "speedup_of_fused": round((t_gemm + t_unm) / t_call, 3)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = lmhead_cpu_baseline(inp, s, tokens, mask, tau, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def decode_block_main(args):
    """One block of the LLaDA-8B workload decoded on the device.

    A HIP graph holds every step of the block: per step, the DualCache block
    attention of each of the model's 32 layers (each layer its own cache),
    then the vocabulary projection fused with the unmask rule
    (fdllm_lmhead_unmask_threshold, or _topk with --rule topk), which updates
    the tokens and mask in place.  Each step writes its n_decoded and n_done
    into its own slots (tokens-per-step telemetry); steps after the block is
    done decode nothing.  The hidden states and the attention inputs are the
    same synthetic tensors every step (no model in between), so the
    telemetry shows the rule at work on fixed confidences, and the time is
    that of the hot path alone (no MLP or projections).
    """
    import numpy as np
    import torch

    import block_wise_kv_amd as fd
    from workloads import make_attn_inputs, make_decode_state, make_lmhead_inputs, shape_c2

    n_layers = 32
    s = shape_c2(3)
    H, V, B = 4096, s.vocab, s.block_size
    K = args.steps or 3
    W = args.warmup if args.warmup is not None else 1
    topk = args.rule == "topk"
    n_steps = -(-B // args.k) if topk else B
    dev = "cuda"
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(torch.bfloat16)
    a = make_attn_inputs(s, "dual")
    q, kn, vn = up(a.q), up(a.k_new), up(a.v_new)
    kc0, vc0 = up(a.k_cache), up(a.v_cache)
    kcs = [kc0.clone() for _ in range(n_layers)]
    vcs = [vc0.clone() for _ in range(n_layers)]
    del kc0, vc0
    out = torch.empty_like(q)
    seq = fd.seq_desc(1, s.max_seq_len, s.gen_len, B, int(s.prompt_lens[0]), int(s.block_idxs[0]))
    ad = fd.attn_desc(32, 32, 128, fd.BF16)
    ws_attn = fd.new_workspace(fd.block_attn_workspace(seq, ad, "dual", B))
    lm = make_lmhead_inputs(s, H)
    x = up(lm.x)
    wp = fd.lmhead_pack(torch.from_numpy(lm.w_codes).to(dev).to(torch.bfloat16))
    ws_lm = fd.new_workspace(fd.lmhead_unmask_workspace(seq, V, H))
    tokens, mask = make_decode_state(s, None)
    tk0, mk0 = torch.from_numpy(tokens).to(dev), torch.from_numpy(mask).to(dev)
    tk, mk = tk0.clone(), mk0.clone()
    nd = torch.zeros((n_steps, 1), dtype=torch.int32, device=dev)
    nn = torch.zeros((n_steps, 1), dtype=torch.int32, device=dev)
    done = torch.zeros((n_steps, 1), dtype=torch.int32, device=dev)
    tau = args.tau

    def block():
        for st in range(n_steps):
            for layer in range(n_layers):
                fd.block_attn(seq, "dual", q, kn, vn, kcs[layer], vcs[layer], out, ws_attn)
            if topk:
                fd.lmhead_unmask_topk(seq, x, wp, V, args.k, tk, mk, nd[st], None, None, done[st], nn[st], ws_lm)
            else:
                fd.lmhead_unmask_threshold(seq, x, wp, V, tau, tk, mk, nd[st], None, None, done[st], nn[st], ws_lm)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            block()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    times = []
    for r in range(W + K):
        tk.copy_(tk0)
        mk.copy_(mk0)
        torch.cuda.synchronize()
        ev[0].record()
        g.replay()
        ev[1].record()
        torch.cuda.synchronize()
        if r >= W:
            times.append(ev[0].elapsed_time(ev[1]) * 1e-3)
    t_block = sorted(times)[len(times) // 2]
    per_step = nd[:, 0].cpu().numpy().tolist()
    n_done = nn[:, 0].cpu().numpy().tolist()
    steps_to_done = next((i + 1 for i, v in enumerate(n_done) if v >= 1), None)
    rule = f"topk k={args.k}" if topk else f"threshold {tau}"
    result = {
        "metric": "LLaDA-8B blocks decoded per second on the device (in-block loop in one HIP graph), 1 GPU",
        "value": round(1.0 / t_block, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(t_block * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "LLaDA-8B block decode: batch 1, block 32 of gen 256 (block index 3), 32 layers of "
                               "DualCache attention per step, LM head (hidden 4096, vocab 126464) fused with the "
                               "unmask", "name": "decode_block_c2", "rule": rule, "graph_steps": n_steps,
                   "layers": n_layers},
        "telemetry": {"tokens_per_step": per_step, "steps_to_done": steps_to_done,
                      "tokens_decoded": int(sum(per_step)),
                      "us_per_step": round(t_block / n_steps * 1e6, 2),
                      "us_per_decoding_step": round(t_block / max(steps_to_done or n_steps, 1) * 1e6, 2)},
    }
    print(json.dumps(result), flush=True)


C5_LAYERS = 28
C5_TAU = 0.7


def cpu_threads(requested: int = 0) -> int:
    """Threads for the all-core oracle baseline: the CPUs this process may
    run on, capped by OMP_NUM_THREADS when the environment sets it."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return requested if requested > 0 else n


def c5_cpu_baseline(s, inp, logits, tokens, mask, srcs, done, threads: int):
    """The fp64 oracle on the host for the ragged Dream-7B step, BLAS limited
    to `threads`: one layer's block attention over all 64 sequences, the
    step's threshold unmask, and one layer's refresh of the finished
    sequences, each timed once; the full step is 28 x attention + unmask +
    28 x refresh, so the rate is 28 / that time (layer block-steps/s, the
    unit of `value`)."""
    from threadpoolctl import threadpool_limits

    from oracle import attn_ref, refresh_ref, unmask_ref
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        attn_ref(inp.q, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache, s.prompt_lens, s.gen_len, s.block_size,
                 s.block_idxs, "dual")
        t1 = time.perf_counter()
        unmask_ref(logits, tokens, mask, s.prompt_lens, s.gen_len, s.block_size, s.block_idxs, C5_TAU,
                   advance=True)
        t2 = time.perf_counter()
        if done:
            refresh_ref(srcs[0], srcs[1], inp.k_cache, inp.v_cache, s.prompt_lens, s.gen_len, s.block_size,
                        s.block_idxs, "dual", seq_ids=done)
        t3 = time.perf_counter()
    t_attn, t_unm, t_ref = t1 - t0, t2 - t1, t3 - t2
    t_step = C5_LAYERS * (t_attn + t_ref) + t_unm
    return {"value": round(C5_LAYERS / t_step, 4), "unit": "block-steps/s", "cores": threads, "kind": "oracle",
            "sample": f"one layer of the ragged Dream-7B step on the host (fp64 NumPy oracle, BLAS threads = "
                      f"{threads}): attention of all 64 sequences {t_attn:.2f} s, threshold unmask of the batch "
                      f"{t_unm:.2f} s, refresh of the {len(done)} finished sequences {t_ref:.2f} s; full step "
                      f"= 28 x (attention + refresh) + unmask = {t_step:.1f} s",
            "attn_s": round(t_attn, 3), "unmask_s": round(t_unm, 3), "refresh_s": round(t_ref, 3)}


def c5_main(args):
    """The ragged Dream-7B 28-layer step (the default workload)."""
    import numpy as np
    import torch

    import block_wise_kv_amd as fd
    from workloads import make_attn_inputs, make_decode_state, make_logits, make_refresh_src, n_masked_c5, shape_c5

    def note(msg):
        print(f"[bench c5] {msg}", file=sys.stderr, flush=True)

    fd.lib()
    dev = "cuda"
    s = shape_c5()
    b, Hq, Hkv, d, B, V, G, Lcap = (s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.block_size, s.vocab,
                                    s.gen_len, s.max_seq_len)
    nL = args.layers
    K, W = args.steps, args.warmup
    n_steps = W + K
    bf = torch.bfloat16

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(bf)

    note(f"generating inputs: 64 sequences, L = {int(s.prompt_lens.min()) + G}..{int(s.prompt_lens.max()) + G}")
    inp = make_attn_inputs(s, "dual")
    srcs = make_refresh_src(s)
    logits = make_logits(s, "calibrated")
    n_masked = n_masked_c5(s)
    tokens, mask = make_decode_state(s, n_masked)
    # per layer: caches, refresh sources, fresh rows and output of its own
    kc0, vc0, ks0, vs0 = up(inp.k_cache), up(inp.v_cache), up(srcs[0]), up(srcs[1])
    q0, kn0, vn0 = up(inp.q), up(inp.k_new), up(inp.v_new)
    kc = [kc0.clone() for _ in range(nL)]
    vc = [vc0.clone() for _ in range(nL)]
    ks = [ks0.clone() for _ in range(nL)]
    vs = [vs0.clone() for _ in range(nL)]
    qs = [q0.clone() for _ in range(nL)]
    kns = [kn0.clone() for _ in range(nL)]
    vns = [vn0.clone() for _ in range(nL)]
    outs = [torch.empty_like(q0) for _ in range(nL)]
    del kc0, vc0, ks0, vs0, q0, kn0, vn0
    lg0 = up(logits)
    lgs = [lg0.clone() for _ in range(args.logit_sets)]
    del lg0
    note(f"device inputs resident: {torch.cuda.memory_allocated() / 2**30:.1f} GiB")
    # every step starts from the same state: its own tokens, mask and block indices
    pl = torch.from_numpy(s.prompt_lens.astype(np.int32)).to(dev)
    tok0 = torch.from_numpy(tokens).to(dev)
    mask0 = torch.from_numpy(mask).to(dev)
    bidx0 = torch.from_numpy(s.block_idxs.astype(np.int32)).to(dev)
    tok = torch.stack([tok0] * n_steps)
    msk = torch.stack([mask0] * n_steps)
    bidx = torch.stack([bidx0] * n_steps)
    maxP = int(s.prompt_lens.max())
    seqs = [fd.seq_desc(b, Lcap, G, B, prompt_lens=pl, block_idxs=bidx[st], max_prompt_len=maxP)
            for st in range(n_steps)]
    nd = torch.zeros(b, dtype=torch.int32, device=dev)
    dpos = torch.zeros((b, B), dtype=torch.int32, device=dev)
    done = torch.zeros(b, dtype=torch.int32, device=dev)
    n_done = torch.zeros(1, dtype=torch.int32, device=dev)
    ad = fd.attn_desc(Hq, Hkv, d, fd.BF16)
    ws_attn = fd.new_workspace(fd.block_attn_workspace(seqs[0], ad, "dual", B))
    ws_unm = fd.new_workspace(fd.unmask_workspace(seqs[0], V, fd.BF16))

    def reset_state():
        tok.copy_(tok0.expand_as(tok))
        msk.copy_(mask0.expand_as(msk))
        bidx.copy_(bidx0.expand_as(bidx))

    def step(st, events=None, names=None):
        sq = seqs[st]
        calls = []
        for l in range(nL):
            calls.append(("block_attn", lambda l=l: fd.block_attn(sq, "dual", qs[l], kns[l], vns[l], kc[l], vc[l],
                                                                  outs[l], ws_attn)))
        calls.append(("unmask_threshold", lambda: fd.unmask_threshold(
            sq, lgs[st % len(lgs)], C5_TAU, tok[st], msk[st], nd, dpos, None, done, n_done, ws_unm,
            flags=fd.UNMASK_ADVANCE_BLOCK)))
        # every layer's refresh of the finished sequences in one launch
        calls.append(("kv_refresh", lambda: fd.kv_refresh_layers(sq, "dual", ks, vs, kc, vc, done, n_done)))
        for name, fn in calls:
            if events is not None:
                m = len(names)
                fd.set_timing_events(events.ev[2 * m], events.ev[2 * m + 1])
                names.append(name)
            fn()

    reset_state()
    torch.cuda.synchronize()
    note(f"capturing {W} warm-up and {K} timed steps ({nL + 2} calls each) in HIP graphs")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        g_warm = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_warm, stream=stream):
            for st in range(W):
                step(st)
        g_timed = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_timed, stream=stream):
            for st in range(W, n_steps):
                step(st)
    torch.cuda.synchronize()
    g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_timed.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    note(f"timed region: {K} steps in {elapsed * 1e3:.2f} ms")
    # what the step decoded and which sequences it refreshed (every step
    # starts from the same state, so every step's lists are the same)
    n_dec_step = int(nd.sum().item())
    done_list = sorted(int(x) for x in done.cpu().numpy()[:int(n_done.item())])

    # the same K steps again, every call bracketed by its own events
    reset_state()
    torch.cuda.synchronize()
    events = HipEvents(2 * K * (nL + 2))
    names = []
    for st in range(W, n_steps):
        step(st, events, names)
    torch.cuda.synchronize()
    L = s.prompt_lens.astype(np.int64) + G
    attn_bytes = 2 * Hkv * d * 2 * int(L.sum()) + 2 * b * B * Hq * d * 2  # K/V rows once + Q read + out written
    unm_bytes = int(n_masked.sum()) * V * 2
    ref_bytes = nL * sum(2 * 2 * int(L[i]) * Hkv * d * 2 for i in done_list)  # one launch, every layer
    per = {}
    for m, name in enumerate(names):
        e = per.setdefault(name, [])
        e.append(events.elapsed_s(2 * m, 2 * m + 1))
    events.close()
    copy_bps = large_copy_rate()
    flops_attn = 4 * Hq * B * int(L.sum()) * d  # S and P V: 2 B L d each per query head, L summed over the batch
    nbytes = {"block_attn": attn_bytes, "unmask_threshold": unm_bytes, "kv_refresh": ref_bytes}
    kernels = {}
    for name, ts in per.items():
        avg = sum(ts) / len(ts)
        gbs = nbytes[name] / avg / 1e9
        kernels[name] = {"avg_us": round(avg * 1e6, 3), "launches": len(ts), "bytes": nbytes[name],
                         "GB_per_s": round(gbs, 1), "frac_of_8TBps": round(gbs * 1e9 / PEAK_HBM_BPS, 4),
                         "frac_of_copy": round(gbs * 1e9 / copy_bps, 4)}
    kernels["block_attn"]["TFLOP_per_s"] = round(flops_attn / (sum(per["block_attn"]) / len(per["block_attn"]))
                                                 / 1e12, 2)
    total = {n: sum(ts) for n, ts in per.items()}
    dom = max(total, key=total.get)
    dk = kernels[dom]
    t_au = (kernels["block_attn"]["avg_us"] + kernels["unmask_threshold"]["avg_us"]) * 1e-6
    value = nL * K / elapsed
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "block-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS["c5"]["desc"], "name": "c5", "layers": nL,
                   "block_steps_per_step": nL, "sum_seq_len": int(L.sum()), "masked_rows": int(n_masked.sum()),
                   "logits": "calibrated", "tau": C5_TAU, "graph": True},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dk["GB_per_s"], 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(dk["GB_per_s"] / 8000.0, 4),
                     "traffic": measured_traffic("c5", dom), "algorithmic_bytes": dk["bytes"]},
        "kernels": kernels,
        "large_copy_GB_per_s": round(copy_bps / 1e9, 1),
        "model_steps_per_s": round(K / elapsed, 2),
        "sequence_block_steps_per_s": round(value * b, 1),
        "attn_unmask_block_steps_per_s": round(1.0 / t_au, 1),
        "attn_unmask_sequence_block_steps_per_s": round(b / t_au, 1),
        "step_telemetry": {"tokens_decoded": n_dec_step, "sequences_refreshed": len(done_list),
                           "refresh_us_per_step": round(kernels["kv_refresh"]["avg_us"], 2),
                           "refresh_us_per_layer_block_step": round(kernels["kv_refresh"]["avg_us"] / nL, 3)},
    }
    if not args.no_cpu_baseline:
        note("timing the fp64 oracle on the host")
        del kc, vc, ks, vs, lgs
        n_all = cpu_threads(args.cpu_threads)
        base = c5_cpu_baseline(s, inp, logits, tokens, mask, srcs, done_list, n_all)
        one = c5_cpu_baseline(s, inp, logits, tokens, mask, srcs, done_list, 1) if n_all > 1 else base
        base["one_thread"] = {"value": one["value"], "cores": 1, "sample": one["sample"]}
        result["cpu_baseline"] = base
    print(json.dumps(result), flush=True)


SWEEP_BLOCKS = (4, 8, 16, 32, 64, 128)
SWEEP_TAUS = (0.5, 0.6, 0.7, 0.8, 0.9, 1.0)


def _c4_common(max_block):
    """Caches, refresh-free attention inputs and peak logits of the
    large-batch LLaDA-8B layer for block sizes up to `max_block`.  The
    caches do not depend on the block size (same seeds); the logits of
    block size B are the first B rows of the `max_block`-row draw."""
    import numpy as np
    import torch
    from workloads import make_attn_inputs, make_logits, shape_c4
    dev = "cuda"
    bf = torch.bfloat16
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(bf)
    s_max = shape_c4(max_block, 0)
    a = make_attn_inputs(s_max, "dual")
    kc, vc = up(a.k_cache), up(a.v_cache)
    del a
    lg = up(make_logits(s_max, "peak"))
    return kc, vc, lg


def sweep_block_size_main(args):
    """Attention + threshold unmask of the large-batch LLaDA-8B layer
    (batch 32, 32 heads x 128, prompt 2048 + gen 512, DualCache) at each
    block size: per-call HIP events over K calls each (eager)."""
    import numpy as np
    import torch

    import block_wise_kv_amd as fd
    from workloads import make_attn_inputs, make_decode_state, shape_c4
    fd.lib()
    dev = "cuda"
    K = args.steps or 20
    W = args.warmup if args.warmup is not None else 3
    kc, vc, lg_all = _c4_common(max(SWEEP_BLOCKS))
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(torch.bfloat16)
    rows = []
    ev = HipEvents(4 * (W + K))
    for B in SWEEP_BLOCKS:
        k = (512 // B) // 2
        s = shape_c4(B, k)
        a = make_attn_inputs(s, "dual", caches=False)
        q, kn, vn = up(a.q), up(a.k_new), up(a.v_new)
        out = torch.empty_like(q)
        seq = fd.seq_desc(s.batch, s.max_seq_len, s.gen_len, B, 2048, k)
        ad = fd.attn_desc(32, 32, 128, fd.BF16)
        ws = fd.new_workspace(fd.block_attn_workspace(seq, ad, "dual", B))
        lg = lg_all[:, :B]
        tok0, msk0 = make_decode_state(s)
        tok0, msk0 = torch.from_numpy(tok0).to(dev), torch.from_numpy(msk0).to(dev)
        tk, mk = tok0.clone(), msk0.clone()
        nd = torch.zeros(s.batch, dtype=torch.int32, device=dev)
        uws = fd.new_workspace(fd.unmask_workspace(seq, s.vocab, fd.BF16))
        torch.cuda.synchronize()
        # the GPU idles while the next block size's inputs are drawn on the
        # host, and its clocks take longer to come back than a few calls
        # last: keep it busy with these calls for a quarter of a second first
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.25:
            for _ in range(8):
                fd.block_attn(seq, "dual", q, kn, vn, kc, vc, out, ws)
                fd.unmask_threshold(seq, lg, 0.9, tk, mk, nd, workspace=uws)
            torch.cuda.synchronize()
        for r in range(W + K):
            tk.copy_(tok0)
            mk.copy_(msk0)
            fd.set_timing_events(ev.ev[4 * r], ev.ev[4 * r + 1])
            fd.block_attn(seq, "dual", q, kn, vn, kc, vc, out, ws)
            fd.set_timing_events(ev.ev[4 * r + 2], ev.ev[4 * r + 3])
            fd.unmask_threshold(seq, lg, 0.9, tk, mk, nd, workspace=uws)
        torch.cuda.synchronize()
        t_a = sum(ev.elapsed_s(4 * r, 4 * r + 1) for r in range(W, W + K)) / K
        t_u = sum(ev.elapsed_s(4 * r + 2, 4 * r + 3) for r in range(W, W + K)) / K
        L = 2048 + 512
        ab = 2 * s.batch * 32 * L * 128 * 2 + 2 * s.batch * B * 32 * 128 * 2
        ub = s.batch * B * s.vocab * 2
        rows.append({"block_size": B, "block_idx": k, "attn_us": round(t_a * 1e6, 2), "unmask_us": round(t_u * 1e6, 2),
                     "attn_bytes": ab, "unmask_bytes": ub,
                     "attn_frac_of_8TBps": round(ab / t_a / PEAK_HBM_BPS, 4),
                     "unmask_frac_of_8TBps": round(ub / t_u / PEAK_HBM_BPS, 4),
                     "attn_TFLOP_per_s": round(4 * s.batch * 32 * B * L * 128 / t_a / 1e12, 1),
                     "block_steps_per_s": round(1.0 / (t_a + t_u), 1),
                     "sequence_block_steps_per_s": round(s.batch / (t_a + t_u), 1)})
        print(f"[sweep] B={B}: attention {t_a * 1e6:.1f} us, unmask {t_u * 1e6:.1f} us", file=sys.stderr, flush=True)
        del q, kn, vn, out, ws, uws
    ev.close()
    print(json.dumps({"metric": "block-steps/s per layer (attn+unmask) and HBM fraction across block sizes, 1 GPU",
                      "config": {"workload": WORKLOADS["c4"]["desc"].replace("block 32", "block size swept"),
                                 "name": "c4_block_size_sweep", "tau": 0.9, "logits": "peak", "calls": K},
                      "sweep": rows}), flush=True)


def sweep_tau_main(args):
    """Decode the large-batch LLaDA-8B layer's current block (batch 32,
    block 32, every block row masked at the first step) at each threshold:
    per step, the block attention and one threshold unmask whose logits come
    from a fresh seeded draw of the calibrated recipe (confidence u ~ U(0.5,
    1) per row; four draws rotate over the steps), until every sequence's
    block is done; records the tokens decoded per step and times each
    step's two calls with HIP events."""
    import numpy as np
    import torch

    import block_wise_kv_amd as fd
    from workloads import make_attn_inputs, make_decode_state, make_logits, shape_c4
    fd.lib()
    dev = "cuda"
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(torch.bfloat16)
    s = shape_c4(32, 8)
    a = make_attn_inputs(s, "dual")
    q, kn, vn, kc, vc = (up(x) for x in (a.q, a.k_new, a.v_new, a.k_cache, a.v_cache))
    del a
    out = torch.empty_like(q)
    lgs = [up(make_logits(s, "calibrated", step=st)) for st in range(4)]
    seq = fd.seq_desc(s.batch, s.max_seq_len, s.gen_len, 32, 2048, 8)
    ad = fd.attn_desc(32, 32, 128, fd.BF16)
    ws = fd.new_workspace(fd.block_attn_workspace(seq, ad, "dual", 32))
    uws = fd.new_workspace(fd.unmask_workspace(seq, s.vocab, fd.BF16))
    tok0, msk0 = make_decode_state(s)
    tok0, msk0 = torch.from_numpy(tok0).to(dev), torch.from_numpy(msk0).to(dev)
    nd = torch.zeros(s.batch, dtype=torch.int32, device=dev)
    done = torch.zeros(s.batch, dtype=torch.int32, device=dev)
    n_done = torch.zeros(1, dtype=torch.int32, device=dev)
    ev = HipEvents(4 * 32)
    rows = []
    # a quarter of a second of the same calls first (clocks up after the
    # host-side input generation)
    tk, mk = tok0.clone(), msk0.clone()
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.25:
        for _ in range(8):
            fd.block_attn(seq, "dual", q, kn, vn, kc, vc, out, ws)
            fd.unmask_threshold(seq, lgs[0], 1.0, tk, mk, nd, None, None, done, n_done, uws)
        torch.cuda.synchronize()
    for tau in SWEEP_TAUS:
        tk, mk = tok0.clone(), msk0.clone()
        per_step = []
        t_a = t_u = 0.0
        for st in range(32):
            fd.set_timing_events(ev.ev[4 * st], ev.ev[4 * st + 1])
            fd.block_attn(seq, "dual", q, kn, vn, kc, vc, out, ws)
            fd.set_timing_events(ev.ev[4 * st + 2], ev.ev[4 * st + 3])
            fd.unmask_threshold(seq, lgs[st % 4], tau, tk, mk, nd, None, None, done, n_done, uws)
            torch.cuda.synchronize()
            t_a += ev.elapsed_s(4 * st, 4 * st + 1)
            t_u += ev.elapsed_s(4 * st + 2, 4 * st + 3)
            per_step.append(int(nd.sum().item()))
            if int(n_done.item()) == s.batch:
                break
        n = len(per_step)
        rows.append({"tau": tau, "steps_to_finish_block": n, "tokens_per_step": per_step,
                     "mean_tokens_per_step_per_sequence": round(sum(per_step) / n / s.batch, 3),
                     "attn_us_per_step": round(t_a / n * 1e6, 2), "unmask_us_per_step": round(t_u / n * 1e6, 2),
                     "layer_us_per_block": round((t_a + t_u) * 1e6, 1)})
        print(f"[sweep] tau={tau}: {n} steps, {sum(per_step)} tokens", file=sys.stderr, flush=True)
    ev.close()
    print(json.dumps({"metric": "tokens decoded per step and steps per block across thresholds, 1 GPU",
                      "config": {"workload": "Large-batch LLaDA-8B-shaped layer: batch 32, 32 heads x 128, prompt "
                                             "2048 + gen 512, block 32 (block index 8), DualCache, calibrated "
                                             "confidences u ~ U(0.5, 1), four logits draws rotating over the steps",
                                 "name": "c4_tau_sweep"},
                      "sweep": rows}), flush=True)


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decoding hot path is "
              "measured on a single MI355X and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    if args.lmhead:
        lmhead_main(args)
        return
    if args.decode_block:
        decode_block_main(args)
        return
    if args.sweep_block_size:
        sweep_block_size_main(args)
        return
    if args.sweep_tau:
        sweep_tau_main(args)
        return
    if args.workload == "c5":
        c5_main(args)
        return
    import torch

    b = Bench(args)
    K, W = args.steps, args.warmup
    use_graph = not args.no_graph
    n_k = K * b.nb * 3
    events = HipEvents(2 * n_k)

    # timed region: K steps replayed from one HIP graph (or launched eagerly)
    if use_graph:
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            g_warm = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_warm, stream=stream):
                b.run_steps(0, W)
            g_timed = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_timed, stream=stream):
                b.run_steps(W, K)
        torch.cuda.synchronize()
        b.reset_state()
        torch.cuda.synchronize()
        g_warm.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g_timed.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    else:
        b.run_steps(0, W)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        b.run_steps(W, K)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    # the same K steps again, launched on the default stream with every
    # call bracketed by its own start/stop events
    b.reset_state()
    torch.cuda.synchronize()
    names = b.run_steps(W, K, events)
    torch.cuda.synchronize()

    elapsed = t1 - t0
    copy_bps = large_copy_rate()
    per = {}
    for m, (name, n) in enumerate(names):
        t = events.elapsed_s(2 * m, 2 * m + 1)
        e = per.setdefault(name, {"t": 0.0, "n": 0, "bytes": 0, "flops": 0})
        e["t"] += t
        e["n"] += 1
        e["bytes"] += b.bytes[n][name]
        e["flops"] += b.flops[n] if name == "block_attn" else 0
    events.close()
    kernels = {}
    for name, e in per.items():
        avg = e["t"] / e["n"]
        gbs = e["bytes"] / e["t"] / 1e9
        kernels[name] = {"avg_us": round(avg * 1e6, 3), "launches": e["n"], "bytes": e["bytes"] // e["n"],
                         "GB_per_s": round(gbs, 1), "frac_of_8TBps": round(gbs * 1e9 / PEAK_HBM_BPS, 4),
                         "frac_of_copy": round(gbs * 1e9 / copy_bps, 4)}
        if name == "block_attn":
            kernels[name]["TFLOP_per_s"] = round(e["flops"] / e["t"] / 1e12, 2)
    dom = max(kernels, key=lambda n: kernels[n]["avg_us"])
    dk = kernels[dom]
    block_steps = K * b.nb
    t_au = (kernels["block_attn"]["avg_us"] + kernels[b.unmask_name]["avg_us"]) * 1e-6
    result = {
        "metric": METRIC,
        "value": round(block_steps / elapsed, 1),
        "unit": "block-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": b.w["desc"], "name": args.workload, "block_steps_per_step": b.nb,
                   "unmask_rule": args.rule if args.rule == "threshold" else f"topk k={args.k}",
                   "graph": use_graph, "rotating_sets": {"layers": args.layers, "logits": args.logit_sets}},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dk["GB_per_s"], 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(dk["GB_per_s"] / 8000.0, 4),
                     "traffic": measured_traffic(args.workload, dom), "algorithmic_bytes": dk["bytes"]},
        "kernels": kernels,
        "large_copy_GB_per_s": round(copy_bps / 1e9, 1),
        "attn_unmask_block_steps_per_s": round(1.0 / t_au, 1),
        "attn_unmask_sequence_block_steps_per_s": round(b.shape.batch / t_au, 1),
    }
    if not args.no_cpu_baseline and args.workload == "c2":
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
