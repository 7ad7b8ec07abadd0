"""Plain fp64 reference of one Fast-dLLM decoding step (CPU, NumPy).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the package smoke check
and the benchmark's CPU-baseline leg, never by the HIP library.  Slow on
purpose: every step is written out the way the method states it, with NumPy
matmul / exp / max as the only library primitives.

Sources (the method is described in prose only; there are no equations or
listings on the pages):

* [ABS]  Fast-dLLM: Training-free Acceleration of Diffusion LLM by Enabling
         KV Cache and Parallel Decoding -- paper summary page (arXiv
         2505.22618v3), section "Abstract" and the method notes
         ("core idea", "technical framework").
* [NEWS] aibase news article on Fast-dLLM, section "Innovations in the
         Fast-dLLM Framework", items 1 (block-wise approximate KV cache,
         DualCache) and 2 (confidence-aware parallel decoding); section "The
         Challenges and Opportunities" (no-cache recompute, bidirectional
         attention).
* [README] Fast-dLLM project README mirror, section "Key techniques" items
         1 (block-wise KV cache reused across the steps of a block; DualCache
         also caches the masked suffix) and 2 (each step decodes the tokens
         whose confidence exceeds the threshold; the rest stay masked);
         section "Usage" (flags gen_length, block_size, use_cache,
         if_cache_position, threshold).
* [REV]  ICLR reviews of Fast-dLLM, review 4 (refresh recomputes all blocks
         after one completes; 0.9 is the usual threshold).

Notation: sequence i has prompt length P, gen length G, L = P + G, block
size B, block index k; block k covers positions [P + kB, P + (k+1)B).
Heads: Hq query heads, Hkv key/value heads, group size g = Hq / Hkv, head
dim d.  Vocabulary size V, threshold tau.

Readings where the pages are silent (each listed in the design notes):
confidence = max softmax probability and the committed token = argmax with
the lowest id on a tie; "exceeds" is strict (conf > tau); if no masked row
passes, the single most confident masked row is decoded (lowest block offset
on a tie); only masked rows of the current block are candidates; decoded
tokens are never re-masked; softmax scale = d^-1/2, no mask or bias; query
head h reads KV head floor(h / g); the fresh (recomputed) rows per cache mode
are: none -> [0, L), prefix -> [P + kB, L), dual -> [P + kB, P + (k+1)B).
"""
from __future__ import annotations

import dataclasses
from typing import Callable, List, Optional

import numpy as np

# Absolute band inside which a confidence / threshold or top-2 comparison is
# flagged as a near tie and excluded from bit-exact decision parity.
NEAR_TIE = 1e-6


# ---------------------------------------------------------------------------
# Step setup: which rows are recomputed in each cache mode
# ---------------------------------------------------------------------------

def fresh_range(P: int, G: int, B: int, k: int, mode: str):
    """Rows [a0, a1) whose K/V are recomputed this step (also the query rows).

    [NEWS] item 1 and [README] item 1: without a cache everything is
    recomputed every step; the prefix cache keeps the already-decoded prefix
    and recomputes the current block and everything after it; DualCache also
    keeps the still-masked suffix, so only the current block is recomputed.
    """
    L = P + G
    if mode == "none":
        return 0, L
    if mode == "prefix":
        return P + k * B, L
    if mode == "dual":
        return P + k * B, P + (k + 1) * B
    raise ValueError(f"unknown cache mode {mode!r}")


# ---------------------------------------------------------------------------
# (a) block attention
# ---------------------------------------------------------------------------

def attn_ref(q, k_new, v_new, k_cache, v_cache, prompt_lens, gen_len: int,
             block_size: int, block_idxs, mode: str, scale: Optional[float] = None):
    """Bidirectional attention of the fresh rows over [cached | fresh | cached] KV.

    [NEWS] "Challenges": attention is bidirectional, so no causal mask.
    [README] item 1: K/V of the rows outside the recomputed range come from
    the cache built at the last refresh; the recomputed rows use the K/V
    produced this step.

    q        [b][cap][Hq][d]   row r = position a0 + r
    k_new    [b][cap][Hkv][d]  (same row convention)
    v_new    [b][cap][Hkv][d]
    k_cache  [b][Hkv][Lcap][d] (None allowed in mode "none")
    v_cache  [b][Hkv][Lcap][d]
    Returns float64 [b][cap][Hq][d]; rows >= a1 - a0 are NaN (never written).
    """
    q = np.asarray(q, np.float64)
    k_new = np.asarray(k_new, np.float64)
    v_new = np.asarray(v_new, np.float64)
    b, cap, Hq, d = q.shape
    Hkv = k_new.shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.full((b, cap, Hq, d), np.nan)
    for i in range(b):
        P = int(prompt_lens[i])
        k = int(block_idxs[i])
        L = P + gen_len
        a0, a1 = fresh_range(P, gen_len, block_size, k, mode)
        nq = a1 - a0
        for hk in range(Hkv):
            # Assemble the key/value rows 0..L-1 this step reads.
            K = np.empty((L, d))
            Vv = np.empty((L, d))
            for j in range(L):
                if a0 <= j < a1:
                    K[j] = k_new[i, j - a0, hk]
                    Vv[j] = v_new[i, j - a0, hk]
                else:
                    K[j] = np.asarray(k_cache[i, hk, j], np.float64)
                    Vv[j] = np.asarray(v_cache[i, hk, j], np.float64)
            for h in range(hk * g, (hk + 1) * g):
                Q = q[i, :nq, h]                       # [nq][d]
                S = (Q @ K.T) * scale                  # [nq][L]
                S = S - S.max(axis=1, keepdims=True)
                W = np.exp(S)
                W = W / W.sum(axis=1, keepdims=True)
                out[i, :nq, h] = W @ Vv
    return out


# ---------------------------------------------------------------------------
# (b) confidence-aware parallel unmasking
# ---------------------------------------------------------------------------

def row_confidence(row):
    """Confidence and greedy token of one position's logits.

    [ABS] / [README] item 2: a position's confidence is how sure the model is
    of its prediction; read here as the largest softmax probability, with the
    predicted token the argmax (lowest id among equal maxima).
    Returns (conf, tok, m, Z) with m = max logit, Z = sum exp(l - m), conf = 1/Z.
    """
    l = np.asarray(row, np.float64)
    m = l.max()
    tok = int(np.flatnonzero(l == m)[0])
    Z = float(np.exp(l - m).sum())
    return 1.0 / Z, tok, float(m), Z


@dataclasses.dataclass
class UnmaskResult:
    tokens: np.ndarray       # int32 [b][Lcap]
    mask: np.ndarray         # uint8 [b][Lcap]
    n_decoded: np.ndarray    # int32 [b]
    decoded_pos: np.ndarray  # int32 [b][B], ascending block offsets, -1 padded
    conf: np.ndarray         # float64 [b][B], NaN where not masked
    done: np.ndarray         # bool [b]
    done_seqs: np.ndarray    # int32 [n_done], ascending
    block_idxs: np.ndarray   # int32 [b] (advanced when asked)
    fallback: np.ndarray     # bool [b]: no row passed, the single best one was decoded
    tie_tau: np.ndarray      # bool [b][B]: |conf - tau| <= NEAR_TIE
    tie_top2: np.ndarray     # bool [b][B]: top-2 logits within NEAR_TIE
    tie_step: np.ndarray     # bool [b]: the step's decision hinges on a near tie

    @property
    def n_done(self) -> int:
        return int(self.done_seqs.size)


def unmask_ref(logits, tokens, mask, prompt_lens, gen_len: int, block_size: int,
               block_idxs, threshold: float, advance: bool = False) -> UnmaskResult:
    """One confidence-threshold unmasking step over a batch.

    [README] item 2 / [NEWS] item 2: every still-masked position of the
    current block whose confidence exceeds the threshold is decoded in this
    step; the others stay masked for later steps.  When none exceeds it, the
    single most confident masked position is decoded, so each step makes
    progress.

    logits  [b][B][V]; row t belongs to position P + kB + t; rows of
            positions that are not masked are not read.
    tokens  int [b][Lcap], mask uint8 [b][Lcap] (1 = masked); not modified,
            updated copies are returned.
    threshold is a float32 value; the comparison is done in float64.
    """
    tokens = np.array(tokens, np.int32, copy=True)
    mask = np.array(mask, np.uint8, copy=True)
    bidx = np.array(block_idxs, np.int32, copy=True).reshape(-1)
    b = tokens.shape[0]
    B = block_size
    tau = float(np.float32(threshold))
    n_dec = np.zeros(b, np.int32)
    dpos = np.full((b, B), -1, np.int32)
    conf = np.full((b, B), np.nan)
    done = np.zeros(b, bool)
    fb = np.zeros(b, bool)
    t_tau = np.zeros((b, B), bool)
    t_top2 = np.zeros((b, B), bool)
    t_step = np.zeros(b, bool)
    n_blocks = gen_len // B
    for i in range(b):
        start = int(prompt_lens[i]) + int(bidx[i]) * B
        masked = [t for t in range(B) if mask[i, start + t] == 1]
        tok = {}
        for t in masked:
            c, v, m, _ = row_confidence(logits[i][t])
            conf[i, t] = c
            tok[t] = v
            t_tau[i, t] = abs(c - tau) <= NEAR_TIE
            srt = np.sort(np.asarray(logits[i][t], np.float64))
            t_top2[i, t] = srt.size > 1 and (srt[-1] - srt[-2]) <= NEAR_TIE
        chosen = [t for t in masked if conf[i, t] > tau]
        if not chosen and masked:
            best = masked[0]
            for t in masked[1:]:
                if conf[i, t] > conf[i, best]:
                    best = t
            chosen = [best]
            fb[i] = True
            cs = np.sort(conf[i, masked])
            if cs.size > 1 and cs[-1] - cs[-2] <= NEAR_TIE:
                t_step[i] = True
        if masked:
            clearly_above = [t for t in masked if conf[i, t] > tau + NEAR_TIE]
            if not clearly_above and any(t_tau[i, t] for t in masked):
                t_step[i] = True
        for t in chosen:
            tokens[i, start + t] = tok[t]
            mask[i, start + t] = 0
        chosen.sort()
        n_dec[i] = len(chosen)
        dpos[i, :len(chosen)] = chosen
        done[i] = not any(mask[i, start + t] == 1 for t in range(B))
        if advance and done[i] and bidx[i] + 1 < n_blocks:
            bidx[i] += 1
    done_seqs = np.array([i for i in range(b) if done[i]], np.int32)
    return UnmaskResult(tokens, mask, n_dec, dpos, conf, done, done_seqs, bidx, fb,
                        t_tau, t_top2, t_step)


def unmask_topk_ref(logits, tokens, mask, prompt_lens, gen_len: int, block_size: int,
                    block_idxs, k: int, advance: bool = False) -> UnmaskResult:
    """One fixed-step unmasking step: decode the k most confident masked rows.

    [README] section "Usage": the sampling-steps flag fixes the number of
    denoising steps, so a fixed number of tokens is committed per step (gen
    length / steps; one per step with the defaults).  This is the decoding
    the pages use as their baseline ("LLaDA" and "+cache" columns of the
    evaluation table).  Which positions are committed is not on the pages;
    read here as the min(k, m) masked positions of the current block with
    the highest confidence (the same max-probability confidence as the
    threshold rule), the lower block offset first among equal confidences.
    The committed token is the row's argmax, as in the threshold rule.

    Near ties: tie_top2 as in unmask_ref; tie_step marks a sequence whose
    k-th and (k+1)-th largest confidences are within NEAR_TIE (the chosen set
    hinges on that comparison); tie_tau and fallback are always False.
    """
    if int(k) < 1:
        raise ValueError("k must be >= 1")
    tokens = np.array(tokens, np.int32, copy=True)
    mask = np.array(mask, np.uint8, copy=True)
    bidx = np.array(block_idxs, np.int32, copy=True).reshape(-1)
    b = tokens.shape[0]
    B = block_size
    n_dec = np.zeros(b, np.int32)
    dpos = np.full((b, B), -1, np.int32)
    conf = np.full((b, B), np.nan)
    done = np.zeros(b, bool)
    t_top2 = np.zeros((b, B), bool)
    t_step = np.zeros(b, bool)
    n_blocks = gen_len // B
    for i in range(b):
        start = int(prompt_lens[i]) + int(bidx[i]) * B
        masked = [t for t in range(B) if mask[i, start + t] == 1]
        tok = {}
        for t in masked:
            c, v, _, _ = row_confidence(logits[i][t])
            conf[i, t] = c
            tok[t] = v
            srt = np.sort(np.asarray(logits[i][t], np.float64))
            t_top2[i, t] = srt.size > 1 and (srt[-1] - srt[-2]) <= NEAR_TIE
        # rank the masked rows: higher confidence first, lower offset first
        order = sorted(masked, key=lambda t: (-conf[i, t], t))
        chosen = order[:int(k)]
        if len(order) > int(k) and conf[i, order[int(k) - 1]] - conf[i, order[int(k)]] <= NEAR_TIE:
            t_step[i] = True
        for t in chosen:
            tokens[i, start + t] = tok[t]
            mask[i, start + t] = 0
        chosen.sort()
        n_dec[i] = len(chosen)
        dpos[i, :len(chosen)] = chosen
        done[i] = not any(mask[i, start + t] == 1 for t in range(B))
        if advance and done[i] and bidx[i] + 1 < n_blocks:
            bidx[i] += 1
    done_seqs = np.array([i for i in range(b) if done[i]], np.int32)
    z = np.zeros((b, B), bool)
    return UnmaskResult(tokens, mask, n_dec, dpos, conf, done, done_seqs, bidx,
                        np.zeros(b, bool), z, t_top2, t_step)


def tokens_per_step(gen_len: int, block_size: int, steps: int) -> int:
    """Tokens committed per step by the fixed-step schedule.

    [README] "Usage": steps sampling steps over a generation of gen_len
    tokens decoded block by block.  Read as steps / (gen_len / block_size)
    steps per block, each committing the same number of tokens; the pages'
    own settings (gen 128 / steps 128, gen 64 / steps 64, block 32) divide
    evenly, and uneven schedules are rejected rather than guessed.
    """
    n_blocks = gen_len // block_size
    if gen_len % block_size or steps % n_blocks or block_size % (steps // n_blocks):
        raise ValueError("steps must split evenly over the blocks and the block over its steps")
    return block_size // (steps // n_blocks)



# ---------------------------------------------------------------------------
# (b') the step before the confidence pass: logits from the hidden states
# ---------------------------------------------------------------------------

def lmhead_logits_ref(x, w):
    """Logits of the block rows from their final hidden states.

    The pages take a position's logits as given: its confidence is their
    largest softmax probability and its token their argmax ([README] "Key
    techniques" item 2).  A language model produces them by projecting the
    final hidden state onto the vocabulary; read here as
    logits[..., v] = sum_k x[..., k] * w[v, k], with w the [V][H] projection
    weight and no bias.

    x  [..., H] hidden states; w [V][H].  Returns float64 [..., V].
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    return x @ w.T


def lmhead_unmask_ref(x, w, tokens, mask, prompt_lens, gen_len: int, block_size: int,
                      block_idxs, threshold: Optional[float] = None, k: Optional[int] = None,
                      advance: bool = False) -> UnmaskResult:
    """One unmasking step whose logits come from the hidden states.

    x [b][B][H] holds the final hidden states of the current block's rows
    (row t <-> position P + kB + t), w [V][H] the vocabulary projection.
    The logits are lmhead_logits_ref(x, w); the step is then the threshold
    rule (unmask_ref, `threshold`) or the fixed-step rule (unmask_topk_ref,
    `k`) on them, exactly one of the two given.
    """
    if (threshold is None) == (k is None):
        raise ValueError("give exactly one of threshold and k")
    logits = lmhead_logits_ref(x, w)
    if k is None:
        return unmask_ref(logits, tokens, mask, prompt_lens, gen_len, block_size, block_idxs,
                          threshold, advance)
    return unmask_topk_ref(logits, tokens, mask, prompt_lens, gen_len, block_size, block_idxs,
                           k, advance)

# ---------------------------------------------------------------------------
# (c) cache refresh at a block boundary
# ---------------------------------------------------------------------------

def refresh_ref(k_src, v_src, k_cache, v_cache, prompt_lens, gen_len: int,
                block_size: int, block_idxs, mode: str, seq_ids=None):
    """Rewrite the cached K/V from a full forward at a block boundary.

    [REV] review 4 and [NEWS] item 1: once a block is finished the K/V of
    every position are recomputed and stored; the steps of the next block
    reuse them.  DualCache keeps all L rows; the prefix cache keeps the rows
    before the (new) current block; no-cache mode keeps nothing.

    k_src, v_src   [b][Lcap][Hkv][d] token-major K/V of the full forward
    k_cache/v_cache [b][Hkv][Lcap][d]; copies are returned, inputs untouched.
    seq_ids: iterable of sequence indices to refresh (None = all).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    b = kc.shape[0]
    ids = range(b) if seq_ids is None else [int(s) for s in seq_ids]
    for i in ids:
        P = int(prompt_lens[i])
        k = int(block_idxs[i])
        if mode == "dual":
            hi = P + gen_len
        elif mode == "prefix":
            hi = P + k * block_size
        elif mode == "none":
            hi = 0
        else:
            raise ValueError(mode)
        for j in range(hi):
            for h in range(kc.shape[1]):
                kc[i, h, j] = k_src[i, j, h]
                vc[i, h, j] = v_src[i, j, h]
    return kc, vc


# ---------------------------------------------------------------------------
# In-block decode loop (used for step-count invariants)
# ---------------------------------------------------------------------------

def decode_block_ref(logits_for_step: Callable[[int], np.ndarray], tokens, mask,
                     prompt_lens, gen_len: int, block_size: int, block_idxs,
                     threshold: float, max_steps: int = 10_000) -> List[np.ndarray]:
    """Repeat the unmask step with fresh logits until the block is decoded.

    [README] items 1-2: inside a block the model runs several steps, each
    decoding the confident tokens, until no masked position of the block is
    left.  Returns the per-step n_decoded arrays (one [b] array per step).
    """
    per_step = []
    for step in range(max_steps):
        r = unmask_ref(logits_for_step(step), tokens, mask, prompt_lens, gen_len,
                       block_size, block_idxs, threshold)
        tokens, mask = r.tokens, r.mask
        per_step.append(r.n_decoded)
        if r.done.all():
            return per_step
    raise RuntimeError("block did not finish")


def decode_block_topk_ref(logits_for_step: Callable[[int], np.ndarray], tokens, mask,
                          prompt_lens, gen_len: int, block_size: int, block_idxs,
                          k: int, max_steps: int = 10_000) -> List[np.ndarray]:
    """The fixed-step loop: k tokens per step until the block is decoded.

    Same loop as decode_block_ref with the top-k step; returns the per-step
    n_decoded arrays.
    """
    per_step = []
    for step in range(max_steps):
        r = unmask_topk_ref(logits_for_step(step), tokens, mask, prompt_lens, gen_len,
                            block_size, block_idxs, k)
        tokens, mask = r.tokens, r.mask
        per_step.append(r.n_decoded)
        if r.done.all():
            return per_step
    raise RuntimeError("block did not finish")
