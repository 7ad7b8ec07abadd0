"""HIP-graph replay of a decoding step built from every kernel variant.

The split-key attention (in-kernel merge through arrival counters), the
8-wave GQA ring with its merge kernel, the refresh (one layer, and two
layers in one launch from the unmask's done list), both unmask rules
(per-sequence arrival counters, the finished-sequence list and the block
advance) and the fused LM head with its finalisation are captured once and
replayed several times, with eager work and
synchronisations between the replays.  Every counter is reset by its last
user, so each replay must reproduce the eager run bit for bit; the eager
run's attention is checked against the oracle too.
"""
import numpy as np
import pytest
import torch

import block_wise_kv_amd as fd
from gpu_util import DEV, check_attn, oracle_attn_subset, require_gpu, say, seq_for, to_dev
from workloads import (make_attn_inputs, make_decode_state, make_lmhead_inputs, make_logits, make_refresh_src,
                       shape_custom)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class _Step:
    """Device state of one step over two shapes (MHA and GQA), with the
    pristine copies to restore it before every run."""

    def __init__(self):
        # MHA, one query tile per head: split-key kernel, 5 key chunks
        self.s1 = shape_custom("g_mha", "bf16", 2, 4, 4, 128, [300, 200], 256, 32, [2, 5], 3000, cfg_id=70)
        # GQA groups of 7: 8-wave ring, 8 key chunks and the merge kernel
        self.s2 = shape_custom("g_gqa", "bf16", 2, 14, 2, 128, [500, 700], 256, 32, [1, 3], 3000, cfg_id=71)
        self.keep = []
        self.bidx2 = torch.from_numpy(self.s2.block_idxs.astype(np.int32)).to(DEV)
        self.seq1 = seq_for(self.s1, True, self.keep)
        self.seq2 = seq_for(self.s2, True, self.keep, self.bidx2)
        self.inp1 = make_attn_inputs(self.s1, "dual")
        self.inp2 = make_attn_inputs(self.s2, "dual")
        d = lambda x: to_dev(x, "bf16")
        self.q1, self.kn1, self.vn1 = d(self.inp1.q), d(self.inp1.k_new), d(self.inp1.v_new)
        self.q2, self.kn2, self.vn2 = d(self.inp2.q), d(self.inp2.k_new), d(self.inp2.v_new)
        self.kc1_0, self.vc1_0 = d(self.inp1.k_cache), d(self.inp1.v_cache)
        self.kc1, self.vc1 = self.kc1_0.clone(), self.vc1_0.clone()
        self.kc2, self.vc2 = d(self.inp2.k_cache), d(self.inp2.v_cache)
        ks, vs = make_refresh_src(self.s1, variant=1)
        self.ks1, self.vs1 = d(ks), d(vs)
        # the done list of s2's unmask refreshes two layer caches in one launch
        ks2, vs2 = make_refresh_src(self.s2, variant=2)
        self.ks2, self.vs2 = d(ks2), d(vs2)
        self.rkc_0 = [self.kc2.clone(), self.kc2.clone() * 0.5]
        self.rvc_0 = [self.vc2.clone(), self.vc2.clone() * 2.0]
        self.rkc = [t.clone() for t in self.rkc_0]
        self.rvc = [t.clone() for t in self.rvc_0]
        self.out1 = torch.zeros_like(self.q1)
        self.out2 = torch.zeros_like(self.q2)
        ad1 = fd.attn_desc(4, 4, 128, fd.BF16)
        ad2 = fd.attn_desc(14, 2, 128, fd.BF16)
        self.ws1 = fd.new_workspace(fd.block_attn_workspace(self.seq1, ad1, "dual", self.q1.shape[1]))
        self.ws2 = fd.new_workspace(fd.block_attn_workspace(self.seq2, ad2, "dual", self.q2.shape[1]))
        assert self.ws1 is not None and self.ws2 is not None  # both split their keys
        # unmask: threshold rule with block advance and done list on s2, top-k on s1
        self.lg1 = d(make_logits(self.s1, "calibrated"))
        self.lg2 = d(make_logits(self.s2, "calibrated"))
        t1, m1 = make_decode_state(self.s1, [32, 7])
        t2, m2 = make_decode_state(self.s2, [1, 32])  # sequence 0 finishes its block
        self.tk1_0, self.mk1_0 = torch.from_numpy(t1).to(DEV), torch.from_numpy(m1).to(DEV)
        self.tk2_0, self.mk2_0 = torch.from_numpy(t2).to(DEV), torch.from_numpy(m2).to(DEV)
        self.bidx2_0 = self.bidx2.clone()
        self.tk1, self.mk1 = self.tk1_0.clone(), self.mk1_0.clone()
        self.tk2, self.mk2 = self.tk2_0.clone(), self.mk2_0.clone()
        b = 2
        self.nd1 = torch.zeros(b, dtype=torch.int32, device=DEV)
        self.dp1 = torch.zeros((b, 32), dtype=torch.int32, device=DEV)
        self.nd2 = torch.zeros(b, dtype=torch.int32, device=DEV)
        self.dp2 = torch.zeros((b, 32), dtype=torch.int32, device=DEV)
        self.cf2 = torch.zeros((b, 32), dtype=torch.float64, device=DEV)
        self.ds2 = torch.zeros(b, dtype=torch.int32, device=DEV)
        self.nn2 = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.uws1 = fd.new_workspace(fd.unmask_workspace(self.seq1, 3000, fd.BF16))
        self.uws2 = fd.new_workspace(fd.unmask_workspace(self.seq2, 3000, fd.BF16))
        # fused LM head on s2's rows (threshold rule, done list), own decode state
        self.lm = make_lmhead_inputs(self.s2, 512)
        self.lx = to_dev(self.lm.x, "bf16")
        self.lwp = fd.lmhead_pack(torch.from_numpy(self.lm.w_codes).to(DEV).to(torch.bfloat16))
        t3, m3 = make_decode_state(self.s2, [0, 20])  # sequence 0 has nothing left to decode
        self.tk3_0, self.mk3_0 = torch.from_numpy(t3).to(DEV), torch.from_numpy(m3).to(DEV)
        self.tk3, self.mk3 = self.tk3_0.clone(), self.mk3_0.clone()
        self.nd3 = torch.zeros(b, dtype=torch.int32, device=DEV)
        self.dp3 = torch.zeros((b, 32), dtype=torch.int32, device=DEV)
        self.ds3 = torch.zeros(b, dtype=torch.int32, device=DEV)
        self.nn3 = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.seq3 = seq_for(self.s2, True, self.keep)
        self.lws = fd.new_workspace(fd.lmhead_unmask_workspace(self.seq3, 3000, 512))

    def restore(self):
        for dst, src in ((self.kc1, self.kc1_0), (self.vc1, self.vc1_0), (self.tk1, self.tk1_0),
                         (self.mk1, self.mk1_0), (self.tk2, self.tk2_0), (self.mk2, self.mk2_0),
                         (self.bidx2, self.bidx2_0), (self.tk3, self.tk3_0), (self.mk3, self.mk3_0),
                         *zip(self.rkc, self.rkc_0), *zip(self.rvc, self.rvc_0)):
            dst.copy_(src)

    def launch(self):
        fd.kv_refresh(self.seq1, "dual", self.ks1, self.vs1, self.kc1, self.vc1)
        fd.block_attn(self.seq1, "dual", self.q1, self.kn1, self.vn1, self.kc1, self.vc1, self.out1, self.ws1)
        fd.block_attn(self.seq2, "dual", self.q2, self.kn2, self.vn2, self.kc2, self.vc2, self.out2, self.ws2)
        fd.unmask_threshold(self.seq2, self.lg2, 0.7, self.tk2, self.mk2, self.nd2, self.dp2, self.cf2,
                            self.ds2, self.nn2, self.uws2, flags=fd.UNMASK_ADVANCE_BLOCK)
        fd.kv_refresh_layers(self.seq2, "dual", [self.ks2] * 2, [self.vs2] * 2, self.rkc, self.rvc, self.ds2,
                             self.nn2)
        fd.unmask_topk(self.seq1, self.lg1, 3, self.tk1, self.mk1, self.nd1, self.dp1, None, None, None,
                       self.uws1)
        fd.lmhead_unmask_threshold(self.seq3, self.lx, self.lwp, 3000, 0.6, self.tk3, self.mk3, self.nd3, self.dp3,
                                   None, self.ds3, self.nn3, self.lws)

    def outputs(self):
        return [t.clone() for t in (self.kc1, self.vc1, self.out1, self.out2, self.tk1, self.mk1, self.nd1,
                                    self.dp1, self.tk2, self.mk2, self.nd2, self.dp2, self.cf2, self.ds2,
                                    self.nn2, self.bidx2, self.tk3, self.mk3, self.nd3, self.dp3, self.ds3,
                                    self.nn3, *self.rkc, *self.rvc)]


def test_graph_replays_match_eager():
    st = _Step()
    st.restore()
    st.launch()
    torch.cuda.synchronize()
    ref = st.outputs()
    # the eager step itself against the oracle (attention after the refresh)
    from workloads import AttnInputs
    ks_t = st.ks1.transpose(1, 2).float().cpu().numpy()
    vs_t = st.vs1.transpose(1, 2).float().cpu().numpy()
    inp1 = AttnInputs(st.s1, "dual", st.inp1.q, st.inp1.k_new, st.inp1.v_new, ks_t, vs_t)
    check_attn(ref[2].float().cpu().numpy().astype(np.float64), oracle_attn_subset(inp1, [0, 1]), inp1,
               seqs=[0, 1], label="graph step mha")
    check_attn(ref[3].float().cpu().numpy().astype(np.float64), oracle_attn_subset(st.inp2, [1]), st.inp2,
               seqs=[1], label="graph step gqa")
    assert int(ref[14].item()) >= 1  # a sequence finished its block and is listed
    # the one-launch refresh of the listed sequences' two layers: listed
    # sequences' rows [0, L) hold the sources, the rest keep their values
    done2 = [int(x) for x in ref[13].cpu().numpy()[:int(ref[14].item())]]
    ks2_t, vs2_t = st.ks2.transpose(1, 2), st.vs2.transpose(1, 2)
    for l in range(2):
        kc_l, vc_l = ref[22 + l], ref[24 + l]
        for i in range(st.s2.batch):
            L = int(st.s2.prompt_lens[i]) + st.s2.gen_len
            if i in done2:
                assert torch.equal(kc_l[i, :, :L], ks2_t[i, :, :L]) and torch.equal(vc_l[i, :, :L], vs2_t[i, :, :L])
                assert torch.equal(kc_l[i, :, L:], st.rkc_0[l][i, :, L:])
            else:
                assert torch.equal(kc_l[i], st.rkc_0[l][i]) and torch.equal(vc_l[i], st.rvc_0[l][i])
    # the fused LM head against the oracle: sequence 0 had nothing masked
    from oracle import lmhead_unmask_ref
    t3, m3 = st.tk3_0.cpu().numpy(), st.mk3_0.cpu().numpy()
    r3 = lmhead_unmask_ref(st.lm.x, st.lm.weight(), t3, m3, st.s2.prompt_lens, st.s2.gen_len, 32,
                           st.s2.block_idxs, threshold=0.6)
    assert not r3.tie_step.any() and not r3.tie_tau.any()
    assert np.array_equal(ref[16].cpu().numpy(), r3.tokens) and np.array_equal(ref[17].cpu().numpy(), r3.mask)
    assert np.array_equal(ref[18].cpu().numpy(), r3.n_decoded) and int(r3.n_decoded[0]) == 0
    assert int(ref[21].item()) == r3.n_done and list(ref[20].cpu().numpy()[:r3.n_done]) == list(r3.done_seqs)
    assert 0 in list(r3.done_seqs)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.restore()
        st.launch()  # warm-up on the capture stream
        with torch.cuda.graph(g, stream=side):
            st.launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        st.restore()
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = st.outputs()
        for k, (a, b_) in enumerate(zip(got, ref)):
            # bitwise (NaN marks unmasked rows in the confidence output)
            assert torch.equal(a.view(torch.uint8), b_.view(torch.uint8)), \
                f"replay {rep}: output {k} differs from the eager run"
        del junk
    say("  graph step: 3 replays equal the eager run bit for bit")
