"""Seeded synthetic inputs for the Fast-dLLM block-decoding hot path.

This module only draws and quantises input tensors. It holds none of the
method's arithmetic (no attention, no softmax decision, no cache refresh):
both the fp64 oracle and the HIP library receive the arrays it returns, and
neither imports the other.

Shapes follow the LLaDA-8B and Dream-7B workloads named in the Fast-dLLM
project README ("Usage" flags --gen_length, --block_size, --threshold) and
the model families in the paper abstract (arXiv 2505.22618 summary page).
The pages' own benchmarks (GSM8K, MATH, HumanEval, MBPP) are not available,
so seeded normal tensors of the same shapes stand in for model activations.

Conventions (all arrays are numpy):

* float tensors are float32; when ``dtype == "bf16"`` every value has
  already been rounded to bfloat16 (round to nearest, ties to even), so the
  float32 array holds exactly what a bf16 device buffer will hold;
* "N(0, s)" in a recipe means ``standard_normal * s`` (s is the standard
  deviation);
* fresh tensors (q, k_new, v_new) are allocated with a per-sequence row
  *capacity*; rows past the live count of a sequence hold finite junk and are
  never read by a correct implementation;
* caches are head-major ``[b][Hkv][Lcap][d]``; fresh tensors are token-major
  ``[b][rows][H][d]``; logits are ``[b][B][V]``; masks are uint8 with 1 =
  still masked; token ids are int32.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Optional

import numpy as np

MODES = ("none", "prefix", "dual")
MODE_ID = {"none": 0, "prefix": 1, "dual": 2}

# Base seed for every generator; every tensor gets its own stream derived
# from (BASE_SEED, config id, tensor id, extra ids...).
BASE_SEED = 20250528

# tensor ids used in the SeedSequence key
_T_Q, _T_KN, _T_VN, _T_KC, _T_VC, _T_LOG, _T_PEAKTOK, _T_PEAKH, _T_SPIKE, \
    _T_MASK, _T_TOK, _T_PLEN, _T_BIDX, _T_NMASK, _T_SRCK, _T_SRCV, _T_U = range(17)


def rng_for(*ids: int) -> np.random.Generator:
    """Independent generator keyed by (BASE_SEED, *ids)."""
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED, *[int(i) for i in ids]]))


def bf16_round(x: np.ndarray, inplace: bool = False) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs must be finite.  ``inplace`` rounds a C-contiguous float32 array
    in place.
    """
    if not (inplace and x.dtype == np.float32 and x.flags.c_contiguous):
        x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.reshape(-1).view(np.uint32)
    step = 1 << 24
    for s in range(0, u.size, step):   # chunked: bounded temporaries
        c = u[s:s + step]
        lsb = (c >> 16) & np.uint32(1)
        c += np.uint32(0x7FFF)          # finite values cannot overflow 32 bits
        c += lsb
        c &= np.uint32(0xFFFF0000)
    return x


def quantise(x: np.ndarray, dtype: str, inplace: bool = False) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(x, inplace)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


_CHUNK = 1 << 22


def _fill_chunk(flat: np.ndarray, sigma: float, dtype: str, ids, c: int):
    part = flat[c * _CHUNK:(c + 1) * _CHUNK]
    rng_for(*ids, c).standard_normal(out=part, dtype=np.float32)
    if sigma != 1.0:
        part *= np.float32(sigma)
    if dtype == "bf16":
        bf16_round(part, inplace=True)


def normal(shape, sigma: float, dtype: str, *ids: int) -> np.ndarray:
    """N(0, sigma) float32 array quantised to ``dtype``.

    The flattened array is drawn in chunks of 2^22 values; chunk c uses the
    generator keyed by (*ids, c), so the result does not depend on how many
    threads fill it.
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"unknown dtype {dtype!r}")
    x = np.empty(shape, np.float32)
    flat = x.reshape(-1)
    n_chunks = (flat.size + _CHUNK - 1) // _CHUNK
    if n_chunks <= 1:
        for c in range(n_chunks):
            _fill_chunk(flat, sigma, dtype, ids, c)
    else:
        import concurrent.futures
        workers = min(16, len(os.sched_getaffinity(0)), n_chunks)
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda c: _fill_chunk(flat, sigma, dtype, ids, c), range(n_chunks)))
    return x


# --------------------------------------------------------------------------
# Shapes
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Shape:
    """One decoding configuration (a batch of b sequences, one layer)."""
    name: str
    cfg_id: int
    dtype: str            # "bf16" | "f32"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    prompt_lens: np.ndarray   # int32 [b]
    gen_len: int
    block_size: int
    block_idxs: np.ndarray    # int32 [b]
    vocab: int
    max_seq_len: int          # Lcap

    @property
    def uniform(self) -> bool:
        return bool(np.all(self.prompt_lens == self.prompt_lens[0])
                    and np.all(self.block_idxs == self.block_idxs[0]))

    def fresh_capacity(self, mode: str) -> int:
        """Row capacity per sequence of q / k_new / v_new / out.

        A capacity, not the live row count: block rows for dual, the whole
        generation region for prefix, the whole row capacity for none.
        """
        if mode == "dual":
            return self.block_size
        if mode == "prefix":
            return self.gen_len
        if mode == "none":
            return self.max_seq_len
        raise ValueError(mode)


def shape_c1() -> Shape:
    """Tiny fp32 step: 1 x 4 heads x 64, prompt 64 + gen 128, B=32, block 1."""
    return Shape("c1_tiny_f32", 1, "f32", 1, 4, 4, 64,
                 np.array([64], np.int32), 128, 32, np.array([1], np.int32), 1024, 192)


def shape_c2(block_idx: int = 0) -> Shape:
    """LLaDA-8B-shaped layer: 1 x 32 heads x 128 (MHA), prompt 512 + gen 256."""
    return Shape("c2_llada8b_b1", 2, "bf16", 1, 32, 32, 128,
                 np.array([512], np.int32), 256, 32, np.array([block_idx], np.int32), 126464, 768)


def shape_c3(block_idx: int = 0) -> Shape:
    """Dream-7B-shaped GQA layer: 8 x 28 q heads / 4 kv heads x 128, 1024 + 1024."""
    return Shape("c3_dream7b_b8", 3, "bf16", 8, 28, 4, 128,
                 np.full(8, 1024, np.int32), 1024, 32, np.full(8, block_idx, np.int32), 152064, 2048)


def shape_c4(block_size: int = 32, block_idx: int = 0, batch: int = 32) -> Shape:
    """Large-batch LLaDA-8B-shaped layer: 32 x 32 heads x 128, 2048 + 512."""
    return Shape(f"c4_llada8b_b{batch}_B{block_size}", 4, "bf16", batch, 32, 32, 128,
                 np.full(batch, 2048, np.int32), 512, block_size,
                 np.full(batch, block_idx, np.int32), 126464, 2560)


def shape_c5(batch: int = 64) -> Shape:
    """Ragged Dream-7B GQA batch: prompt U(256, 4096) per sequence, gen 512,
    B=32, block index U{0..15} per sequence."""
    g = rng_for(5, _T_PLEN)
    plen = g.integers(256, 4096, size=batch, endpoint=True).astype(np.int32)
    g = rng_for(5, _T_BIDX)
    bidx = g.integers(0, 512 // 32, size=batch).astype(np.int32)
    lcap = int(plen.max()) + 512
    return Shape(f"c5_dream7b_ragged_b{batch}", 5, "bf16", batch, 28, 4, 128,
                 plen, 512, 32, bidx, 152064, lcap)


def shape_custom(name: str, dtype: str, batch: int, hq: int, hkv: int, d: int,
                 prompt_lens, gen_len: int, block_size: int, block_idxs,
                 vocab: int, max_seq_len: Optional[int] = None, cfg_id: int = 99) -> Shape:
    plen = np.asarray(prompt_lens, np.int32).reshape(-1)
    if plen.size == 1 and batch > 1:
        plen = np.full(batch, int(plen[0]), np.int32)
    bidx = np.asarray(block_idxs, np.int32).reshape(-1)
    if bidx.size == 1 and batch > 1:
        bidx = np.full(batch, int(bidx[0]), np.int32)
    lcap = int(max_seq_len) if max_seq_len is not None else int(plen.max()) + gen_len
    return Shape(name, cfg_id, dtype, batch, hq, hkv, d, plen, gen_len, block_size,
                 bidx, vocab, lcap)


# --------------------------------------------------------------------------
# Attention / refresh inputs
# --------------------------------------------------------------------------

@dataclasses.dataclass
class AttnInputs:
    shape: Shape
    mode: str
    q: np.ndarray        # [b][cap][Hq][d]
    k_new: np.ndarray    # [b][cap][Hkv][d]
    v_new: np.ndarray    # [b][cap][Hkv][d]
    k_cache: Optional[np.ndarray]  # [b][Hkv][Lcap][d]
    v_cache: Optional[np.ndarray]


def make_attn_inputs(shape: Shape, mode: str, variant: int = 0, caches: bool = True) -> AttnInputs:
    """Q, fresh K/V and cached K/V ~ N(0, 1), quantised to the shape's dtype.

    The fresh rows are drawn independently of the cache (they stand for the
    block's tokens after some were decoded since the last refresh).
    ``variant`` selects another independent draw of the same shape;
    ``caches=False`` skips drawing the caches.
    """
    s = shape
    cap = s.fresh_capacity(mode)
    ids = (s.cfg_id, variant, MODE_ID[mode])
    q = normal((s.batch, cap, s.n_q_heads, s.head_dim), 1.0, s.dtype, *ids, _T_Q)
    kn = normal((s.batch, cap, s.n_kv_heads, s.head_dim), 1.0, s.dtype, *ids, _T_KN)
    vn = normal((s.batch, cap, s.n_kv_heads, s.head_dim), 1.0, s.dtype, *ids, _T_VN)
    if mode == "none" or not caches:
        kc = vc = None
    else:
        kc = normal((s.batch, s.n_kv_heads, s.max_seq_len, s.head_dim), 1.0, s.dtype,
                    s.cfg_id, variant, _T_KC)
        vc = normal((s.batch, s.n_kv_heads, s.max_seq_len, s.head_dim), 1.0, s.dtype,
                    s.cfg_id, variant, _T_VC)
    return AttnInputs(s, mode, q, kn, vn, kc, vc)


def make_refresh_src(shape: Shape, variant: int = 0):
    """Token-major K/V of a full forward: ``[b][Lcap][Hkv][d]`` each, N(0, 1)."""
    s = shape
    shp = (s.batch, s.max_seq_len, s.n_kv_heads, s.head_dim)
    return (normal(shp, 1.0, s.dtype, s.cfg_id, variant, _T_SRCK),
            normal(shp, 1.0, s.dtype, s.cfg_id, variant, _T_SRCV))


# --------------------------------------------------------------------------
# Unmask inputs
# --------------------------------------------------------------------------

def make_logits(shape: Shape, recipe: str = "auto", step: int = 0, variant: int = 0,
                dtype: Optional[str] = None) -> np.ndarray:
    """Logits ``[b][B][V]`` for one decoding step of the current block.

    Recipes (one row per block position, each row independent):

    * ``"spike"`` (tiny fp32 case): N(0, 2); with probability 0.4 a seeded
      token gets +8.
    * ``"peak"`` (LLaDA / Dream shapes): N(0, 3); a seeded token gets
      +h, h ~ U(0, 12).
    * ``"calibrated"``: N(0, 3) background, then the seeded token's logit is
      set so that its softmax probability is u ~ U(0.5, 1) before
      quantisation.  This makes threshold sweeps decode meaningful numbers
      of tokens; ``calibrated_targets`` returns the u values.
    * ``"auto"``: ``spike`` for config 1, ``peak`` otherwise.

    Row r = i * B + t draws its background from the generator keyed by
    (config, variant, step, r).
    """
    s = shape
    dt = dtype or s.dtype
    if recipe == "auto":
        recipe = "spike" if s.cfg_id == 1 else "peak"
    if recipe not in ("spike", "peak", "calibrated"):
        raise ValueError(recipe)
    ids = (s.cfg_id, variant, step)
    b, B, V = s.batch, s.block_size, s.vocab
    sigma = np.float32(2.0 if recipe == "spike" else 3.0)
    x = np.empty((b, B, V), np.float32)
    rows = x.reshape(b * B, V)
    tok = rng_for(*ids, _T_PEAKTOK).integers(0, V, size=(b, B)).reshape(-1)
    if recipe == "spike":
        on = rng_for(*ids, _T_SPIKE).random(size=(b, B)).reshape(-1) < 0.4
        add = np.where(on, np.float32(8.0), np.float32(0.0)).astype(np.float32)
    elif recipe == "peak":
        add = rng_for(*ids, _T_PEAKH).uniform(0.0, 12.0, size=(b, B)).astype(np.float32).reshape(-1)
    else:
        u = calibrated_targets(s, step, variant).reshape(-1)

    def fill(r):
        row = rows[r]
        rng_for(*ids, _T_LOG, r).standard_normal(out=row, dtype=np.float32)
        row *= sigma
        if recipe == "calibrated":
            row[tok[r]] = -np.inf
            m = float(row.max())
            rest = m + np.log(np.exp(row.astype(np.float64) - m).sum())
            row[tok[r]] = np.float32(rest + np.log(u[r] / (1.0 - u[r])))
        else:
            row[tok[r]] += add[r]
        if dt == "bf16":
            bf16_round(row, inplace=True)

    n = b * B
    if n * V <= (1 << 22):
        for r in range(n):
            fill(r)
    else:
        import concurrent.futures
        workers = min(16, len(os.sched_getaffinity(0)))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(n)))
    return x


def calibrated_targets(shape: Shape, step: int = 0, variant: int = 0) -> np.ndarray:
    """The u ~ U(0.5, 1) targets of the ``calibrated`` recipe, ``[b][B]``."""
    s = shape
    return rng_for(s.cfg_id, variant, step, _T_U).uniform(0.5, 1.0, size=(s.batch, s.block_size))


def peak_tokens(shape: Shape, step: int = 0, variant: int = 0) -> np.ndarray:
    """The seeded peak token id per row, ``[b][B]`` (same draw as make_logits)."""
    s = shape
    return rng_for(s.cfg_id, variant, step, _T_PEAKTOK).integers(0, s.vocab, size=(s.batch, s.block_size))


def make_decode_state(shape: Shape, n_masked: Optional[object] = None, variant: int = 0):
    """Token ids and mask bitmap ``[b][Lcap]`` at the first step of the
    current block.

    Positions before the block hold decoded ids (mask 0); the block holds
    ``n_masked`` masked positions chosen uniformly without replacement
    (an int, an array per sequence, or None = all B); positions after the
    block are masked (mask 1); positions past L_i are padding (mask 0,
    token -1).  Masked positions hold the id ``mask_id`` = vocab (one past
    the real vocabulary, like a dedicated mask token).
    """
    s = shape
    b, B, Lcap = s.batch, s.block_size, s.max_seq_len
    tokens = rng_for(s.cfg_id, variant, _T_TOK).integers(0, s.vocab, size=(b, Lcap)).astype(np.int32)
    mask = np.zeros((b, Lcap), np.uint8)
    g = rng_for(s.cfg_id, variant, _T_MASK)
    if n_masked is None:
        nm = np.full(b, B, np.int64)
    elif np.isscalar(n_masked):
        nm = np.full(b, int(n_masked), np.int64)
    else:
        nm = np.asarray(n_masked, np.int64).reshape(b)
    for i in range(b):
        P = int(s.prompt_lens[i]); L = P + s.gen_len
        start = P + int(s.block_idxs[i]) * B
        sel = g.choice(B, size=int(nm[i]), replace=False)
        mask[i, start + sel] = 1
        mask[i, start + B:L] = 1
        tokens[i, L:] = -1
    tokens[mask == 1] = s.vocab
    return tokens, mask


def n_masked_c5(shape: Shape) -> np.ndarray:
    """Masked positions per sequence for the ragged case: U{1..32}."""
    return rng_for(shape.cfg_id, _T_NMASK).integers(1, shape.block_size, size=shape.batch,
                                                    endpoint=True)


# --------------------------------------------------------------------------
# LM-head inputs: final hidden states of the block rows and the vocabulary
# projection weight
# --------------------------------------------------------------------------

_T_LMX, _T_LMW, _T_LME = 17, 18, 19

# Model width of each config's model (LLaDA-8B: 4096, Dream-7B: 3584).
HIDDEN = {1: 256, 2: 4096, 3: 3584, 4: 4096, 5: 3584}


@dataclasses.dataclass
class LmheadInputs:
    shape: Shape
    hidden: int
    recipe: str
    x: np.ndarray                  # float32 [b][B][H], bf16-exact
    w_codes: Optional[np.ndarray]  # int8 [V][H] ("grid": w == w_codes exactly), else None
    w: Optional[np.ndarray]        # float32 [V][H], bf16-exact ("normal"), else None
    row_exp: Optional[np.ndarray]  # int [b][B]: "grid" rows are x = codes * 2^-row_exp

    def weight(self, v0: int = 0, v1: Optional[int] = None) -> np.ndarray:
        """Rows [v0, v1) of the weight as float64."""
        src = self.w_codes if self.w_codes is not None else self.w
        return np.asarray(src[v0:v1], np.float64)


def _int_chunk(flat: np.ndarray, lo: int, hi: int, ids, c: int):
    part = flat[c * _CHUNK:(c + 1) * _CHUNK]
    part[:] = rng_for(*ids, c).integers(lo, hi, size=part.size, endpoint=True, dtype=np.int8)


def small_ints(shape, lo: int, hi: int, *ids: int) -> np.ndarray:
    """int8 array of integers uniform in [lo, hi], drawn in chunks of 2^22
    (chunk c keyed by (*ids, c))."""
    x = np.empty(shape, np.int8)
    flat = x.reshape(-1)
    n_chunks = (flat.size + _CHUNK - 1) // _CHUNK
    if n_chunks <= 1:
        for c in range(n_chunks):
            _int_chunk(flat, lo, hi, ids, c)
    else:
        import concurrent.futures
        workers = min(16, len(os.sched_getaffinity(0)), n_chunks)
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda c: _int_chunk(flat, lo, hi, ids, c), range(n_chunks)))
    return x


def make_lmhead_inputs(shape: Shape, hidden: Optional[int] = None, recipe: str = "grid",
                       variant: int = 0) -> LmheadInputs:
    """Hidden states ``x [b][B][H]`` of the current block's rows and the
    projection weight ``w [V][H]`` (bf16 values; logits = x w^T).

    * ``"grid"``: w = integers uniform in [-3, 3]; row r of x = integers
      uniform in [-3, 3] times 2^-e_r, e_r in {e0 - 1, e0, e0 + 1} (seeded
      per row), e0 = round(log2(sqrt(H))).  A logit then has standard
      deviation about 8, 4 or 2 (so rows range from unsure to confident),
      and it is an integer multiple of 2^-e_r smaller than 9 H 2^-e_r in
      magnitude: below 2^24 units, every fp32 sum of the products, in any
      order, is exact.
    * ``"normal"``: x ~ N(0, 1), w ~ N(0, 3 / sqrt(H)), both rounded to
      bf16 (logit standard deviation about 3; fp32 accumulation rounds).
    """
    s = shape
    H = int(hidden if hidden is not None else HIDDEN[s.cfg_id])
    b, B, V = s.batch, s.block_size, s.vocab
    ids = (s.cfg_id, variant, H)
    if recipe == "grid":
        e0 = int(round(0.5 * np.log2(H)))
        e = e0 + rng_for(*ids, _T_LME).integers(-1, 1, size=(b, B), endpoint=True)
        cx = small_ints((b, B, H), -3, 3, *ids, _T_LMX).astype(np.float32)
        x = (cx * np.exp2(-e.astype(np.float32))[:, :, None]).astype(np.float32)
        wc = small_ints((V, H), -3, 3, *ids, _T_LMW)
        return LmheadInputs(s, H, recipe, x, wc, None, e)
    if recipe == "normal":
        x = normal((b, B, H), 1.0, "bf16", *ids, _T_LMX)
        w = normal((V, H), 3.0 / np.sqrt(H), "bf16", *ids, _T_LMW)
        return LmheadInputs(s, H, recipe, x, None, w, None)
    raise ValueError(recipe)
