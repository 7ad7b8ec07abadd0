#!/usr/bin/env python3
"""Benchmark of the Fast-dLLM block-decoding hot path on one MI355X.

Workload: one LLaDA-8B-shaped layer, batch 1, 32 heads x 128 (MHA), prompt
512 + gen 256, block size 32, DualCache, block index swept 0..7, thresholds
cycled over {0.7, 0.9, 1.0}.  One step = for each of the 8 block indices:
the block-boundary cache refresh (fdllm_kv_refresh), the block attention
(fdllm_block_attn) and the threshold unmask over the 126464-wide vocabulary
(fdllm_unmask_threshold) -- every part of the hot path once per block-step.
Inputs are seeded synthetic tensors already resident in HBM.

To measure HBM and not the 256 MB Infinity Cache, buffers rotate over 32
layer sets (caches and refresh sources, 806 MB) and 48 logits sets (389 MB);
the refresh of a block-step writes the layer set 16 positions away from the
one its attention reads.  Each unmask call gets its own pristine token/mask
pair, so every step sees the first step after a refresh (all 32 block
positions masked).

The K timed steps are captured once in a HIP graph and replayed between two
device synchronisations.  Per-kernel durations come from a second pass over
the same K steps in which every kernel is launched with its own start/stop
HIP events (libfdllm's timing hook, hipExtLaunchKernel), on the stream it
runs on.

Prints one JSON line.  --gpus N > 1 is refused: this path runs on one GPU.
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
N_BLOCKS = 8
TAUS = (0.7, 0.9, 1.0)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=32, help="rotating cache/source sets")
    ap.add_argument("--logit-sets", type=int, default=48)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    return ap.parse_args()


class Bench:
    def __init__(self, args):
        import numpy as np
        import torch

        import block_wise_kv_amd as fd
        from workloads import make_attn_inputs, make_decode_state, make_logits, make_refresh_src, shape_c2

        self.fd, self.torch, self.np = fd, torch, np
        fd.lib()
        dev = "cuda"
        self.args = args
        s0 = shape_c2(0)
        self.shape = s0
        bf = torch.bfloat16

        def up(x):
            return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(bf)

        # per-block-index fresh rows and per-layer caches / refresh sources
        self.seqs = [fd.seq_desc(1, s0.max_seq_len, s0.gen_len, s0.block_size, 512, k) for k in range(N_BLOCKS)]
        self.fresh = []
        for k in range(N_BLOCKS):
            a = make_attn_inputs(shape_c2(k), "dual", variant=k)
            self.fresh.append((up(a.q), up(a.k_new), up(a.v_new)))
            if k == 0:
                kc, vc = up(a.k_cache), up(a.v_cache)
        ks, vs = make_refresh_src(s0)
        ks, vs = up(ks), up(vs)
        L = args.layers
        self.kc = [kc.clone() for _ in range(L)]
        self.vc = [vc.clone() for _ in range(L)]
        self.ks = [ks.clone() for _ in range(L)]
        self.vs = [vs.clone() for _ in range(L)]
        self.out = [torch.empty_like(self.fresh[k][0]) for k in range(N_BLOCKS)]
        lg = up(make_logits(s0, "peak"))
        self.logits = [lg.clone() for _ in range(args.logit_sets)]
        # pristine decode state per block index
        self.tok0, self.mask0 = [], []
        for k in range(N_BLOCKS):
            t, m = make_decode_state(shape_c2(k))
            self.tok0.append(torch.from_numpy(t).to(dev))
            self.mask0.append(torch.from_numpy(m).to(dev))
        n_calls = (args.warmup + args.steps) * N_BLOCKS
        self.tok_pristine = torch.stack([self.tok0[c % N_BLOCKS] for c in range(n_calls)])
        self.mask_pristine = torch.stack([self.mask0[c % N_BLOCKS] for c in range(n_calls)])
        self.tok = torch.empty_like(self.tok_pristine)
        self.mask = torch.empty_like(self.mask_pristine)
        self.n_dec = torch.zeros(1, dtype=torch.int32, device=dev)
        self.dpos = torch.zeros((1, 32), dtype=torch.int32, device=dev)
        self.done = torch.zeros(1, dtype=torch.int32, device=dev)
        self.n_done = torch.zeros(1, dtype=torch.int32, device=dev)
        ad = fd.attn_desc(32, 32, 128, fd.BF16)
        self.ws_attn = fd.new_workspace(fd.block_attn_workspace(self.seqs[0], ad, "dual", 32))
        self.ws_unmask = fd.new_workspace(fd.unmask_workspace(self.seqs[0], s0.vocab, fd.BF16))
        self.reset_state()
        torch.cuda.synchronize()
        # algorithmic bytes per launch
        d, Hkv, Lfull, B, V = 128, 32, 768, 32, s0.vocab
        self.bytes = {
            "block_attn": 2 * Hkv * Lfull * d * 2 + 2 * 32 * B * d * 2,   # K+V rows read, Q read, out written
            "unmask_threshold": B * V * 2,                                # every masked logits row read once
            "kv_refresh": 2 * 2 * Hkv * Lfull * d * 2,                     # K+V read and written
        }
        self.flops_attn = 4 * 32 * B * Lfull * d

    def reset_state(self):
        self.tok.copy_(self.tok_pristine)
        self.mask.copy_(self.mask_pristine)

    def launches(self, call):
        """The three kernels of block-step number `call` (in launch order)."""
        fd = self.fd
        k = call % N_BLOCKS
        L = self.args.layers
        la, lr = call % L, (call + L // 2) % L
        lg = self.logits[call % len(self.logits)]
        seq = self.seqs[k]
        q, kn, vn = self.fresh[k]
        return [
            ("kv_refresh", lambda: fd.kv_refresh(seq, "dual", self.ks[lr], self.vs[lr], self.kc[lr], self.vc[lr])),
            ("block_attn", lambda: fd.block_attn(seq, "dual", q, kn, vn, self.kc[la], self.vc[la], self.out[k],
                                                 self.ws_attn)),
            ("unmask_threshold", lambda: fd.unmask_threshold(
                seq, lg, TAUS[k % 3], self.tok[call], self.mask[call], self.n_dec, self.dpos, None, self.done,
                self.n_done, self.ws_unmask)),
        ]

    def run_steps(self, first_step, n_steps, events=None):
        """Launch the block-steps; with `events`, every kernel records its own
        start/stop HIP events (kernel n uses events 2n and 2n+1)."""
        names = []
        for st in range(first_step, first_step + n_steps):
            for k in range(N_BLOCKS):
                for name, fn in self.launches(st * N_BLOCKS + k):
                    if events is not None:
                        n = len(names)
                        self.fd.set_timing_events(events.ev[2 * n], events.ev[2 * n + 1])
                    fn()
                    names.append(name)
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decoding hot path is "
              "measured on a single MI355X and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import torch

    b = Bench(args)
    K, W = args.steps, args.warmup
    use_graph = not args.no_graph
    n_k = K * N_BLOCKS * 3
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
    # kernel bracketed by its own start/stop events
    b.reset_state()
    torch.cuda.synchronize()
    names = b.run_steps(W, K, events)
    torch.cuda.synchronize()

    elapsed = t1 - t0
    per = {}
    for n, name in enumerate(names):
        per.setdefault(name, []).append(events.elapsed_s(2 * n, 2 * n + 1))
    events.close()
    kernels = {}
    for name, ts in per.items():
        avg = sum(ts) / len(ts)
        gbs = b.bytes[name] / avg / 1e9
        kernels[name] = {"avg_us": round(avg * 1e6, 3), "launches": len(ts), "bytes": b.bytes[name],
                         "GB_per_s": round(gbs, 1), "frac_of_8TBps": round(gbs * 1e9 / PEAK_HBM_BPS, 4)}
    dom = max(kernels, key=lambda n: kernels[n]["avg_us"])
    dk = kernels[dom]
    block_steps = K * N_BLOCKS
    t_au = (kernels["block_attn"]["avg_us"] + kernels["unmask_threshold"]["avg_us"]) * 1e-6
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
        "config": {"workload": "LLaDA-8B-shaped layer: batch 1, 32 heads x 128 (MHA), prompt 512 + gen 256, "
                               "block 32, DualCache, block index 0..7 swept, tau in {0.7, 0.9, 1.0}, vocab 126464; "
                               "one block-step = refresh + attention + unmask",
                   "block_steps_per_step": N_BLOCKS, "graph": use_graph,
                   "rotating_sets": {"layers": args.layers, "logits": args.logit_sets}},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dk["GB_per_s"], 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(dk["GB_per_s"] / 8000.0, 4), "traffic": None},
        "kernels": kernels,
        "attn_unmask_block_steps_per_s": round(1.0 / t_au, 1),
        "attn_mfma_tflops": round(b.flops_attn / (kernels["block_attn"]["avg_us"] * 1e-6) / 1e12, 2),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
