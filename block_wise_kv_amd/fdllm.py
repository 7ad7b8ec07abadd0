"""ctypes binding of libfdllm (the C ABI in include/fdllm.h).

Argument marshalling only: tensors are passed as device pointers together
with torch's current HIP stream; every step of the path runs in the HIP
kernels of libfdllm.so.  Importing this module does not require a GPU, but
loading fails loudly when libfdllm.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfdllm.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH = range(5)
MODE = {"none": 0, "prefix": 1, "dual": 2}
BF16, F32 = 0, 1
UNMASK_ADVANCE_BLOCK = 1


class FdllmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class SeqDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("gen_len", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("prompt_len", ctypes.c_int32),
        ("block_idx", ctypes.c_int32),
        ("prompt_lens", ctypes.c_void_p),
        ("block_idxs", ctypes.c_void_p),
        ("max_prompt_len", ctypes.c_int32),
    ]


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


_lib = None

# (name, restype, argtypes) for every function declared in include/fdllm.h
_P = ctypes.c_void_p
_SIGS = [
    ("fdllm_block_attn_workspace", ctypes.c_size_t,
     [ctypes.POINTER(SeqDesc), ctypes.POINTER(AttnDesc), ctypes.c_int32, ctypes.c_int32]),
    ("fdllm_block_attn", ctypes.c_int32,
     [ctypes.POINTER(SeqDesc), ctypes.POINTER(AttnDesc), ctypes.c_int32, ctypes.c_int32,
      _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("fdllm_unmask_workspace", ctypes.c_size_t,
     [ctypes.POINTER(SeqDesc), ctypes.c_int32, ctypes.c_int32]),
    ("fdllm_unmask_threshold", ctypes.c_int32,
     [ctypes.POINTER(SeqDesc), ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int64,
      ctypes.c_float, ctypes.c_uint32, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("fdllm_unmask_threshold_static", ctypes.c_int32,
     [ctypes.POINTER(SeqDesc), ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int64,
      ctypes.c_float, ctypes.c_uint32, _P, _P, _P, _P, _P, _P, _P, _P]),
    ("fdllm_unmask_topk", ctypes.c_int32,
     [ctypes.POINTER(SeqDesc), ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int64,
      ctypes.c_int32, ctypes.c_uint32, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("fdllm_lmhead_packed_bytes", ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    ("fdllm_lmhead_pack", ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]),
    ("fdllm_lmhead_unmask_workspace", ctypes.c_size_t,
     [ctypes.POINTER(SeqDesc), ctypes.c_int32, ctypes.c_int32]),
    ("fdllm_lmhead_unmask_threshold", ctypes.c_int32,
     [ctypes.POINTER(SeqDesc), ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int64, _P,
      ctypes.c_float, ctypes.c_uint32, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("fdllm_lmhead_unmask_topk", ctypes.c_int32,
     [ctypes.POINTER(SeqDesc), ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int64, _P,
      ctypes.c_int32, ctypes.c_uint32, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    ("fdllm_set_lmhead_tuning", ctypes.c_int32, [ctypes.c_int32]),
    ("fdllm_kv_refresh", ctypes.c_int32,
     [ctypes.POINTER(SeqDesc), ctypes.POINTER(AttnDesc), ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P]),
    ("fdllm_kv_refresh_layers", ctypes.c_int32,
     [ctypes.POINTER(SeqDesc), ctypes.POINTER(AttnDesc), ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P, _P,
      _P]),
    ("fdllm_workspace_init", ctypes.c_int32, [_P, ctypes.c_size_t, _P]),
    ("fdllm_set_debug", ctypes.c_int32, [ctypes.c_int32]),
    ("fdllm_set_timing_events", ctypes.c_int32, [_P, _P]),
    ("fdllm_set_tuning", ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    ("fdllm_status_string", ctypes.c_char_p, [ctypes.c_int32]),
    ("fdllm_last_error", ctypes.c_char_p, []),
    ("fdllm_version", ctypes.c_int32, []),
]


def lib():
    """Load libfdllm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        try:  # share torch's HIP runtime (same soname) when torch is present
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_wise_kv_amd.build` "
                               "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGS:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != OK:
        L = lib()
        raise FdllmError(status, f"{L.fdllm_status_string(status).decode()}: {L.fdllm_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def seq_desc(batch: int, max_seq_len: int, gen_len: int, block_size: int, prompt_len: int = 0,
             block_idx: int = 0, prompt_lens=None, block_idxs=None,
             max_prompt_len: Optional[int] = None) -> SeqDesc:
    """Sequence descriptor; prompt_lens / block_idxs are int32 device tensors (ragged) or None."""
    if max_prompt_len is None:
        max_prompt_len = prompt_len
    return SeqDesc(batch, max_seq_len, gen_len, block_size, prompt_len, block_idx,
                   _ptr(prompt_lens), _ptr(block_idxs), max_prompt_len)


def attn_desc(n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: int, scale: float = 0.0) -> AttnDesc:
    return AttnDesc(n_q_heads, n_kv_heads, head_dim, dtype, scale)


# ---------------------------------------------------------------------------
# workspaces
# ---------------------------------------------------------------------------

def workspace_init(ws, stream=None):
    if ws is None or ws.numel() == 0:
        return
    _check(lib().fdllm_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def new_workspace(nbytes: int, device="cuda", stream=None):
    """A zeroed workspace buffer (torch uint8 tensor), or None when nbytes == 0."""
    if nbytes == 0:
        return None
    import torch
    ws = torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device)
    workspace_init(ws, stream)
    return ws


def block_attn_workspace(seq: SeqDesc, ad: AttnDesc, mode: str, fresh_rows: int) -> int:
    return int(lib().fdllm_block_attn_workspace(ctypes.byref(seq), ctypes.byref(ad), MODE[mode], fresh_rows))


def unmask_workspace(seq: SeqDesc, vocab: int, dtype: int) -> int:
    return int(lib().fdllm_unmask_workspace(ctypes.byref(seq), vocab, dtype))


# ---------------------------------------------------------------------------
# the three calls
# ---------------------------------------------------------------------------

def block_attn(seq: SeqDesc, mode: str, q, k_new, v_new, k_cache, v_cache, out, workspace=None,
               scale: float = 0.0, stream=None):
    """fdllm_block_attn; shapes q/out [b][rows][Hq][d], k_new/v_new [b][rows][Hkv][d],
    caches [b][Hkv][Lcap][d]."""
    ad = attn_desc(q.shape[2], k_new.shape[2], q.shape[3], _dtype_code(q), scale)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fdllm_block_attn(ctypes.byref(seq), ctypes.byref(ad), MODE[mode], q.shape[1],
                                  _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(out), _ptr(workspace), nbytes, _stream(stream)))


def unmask_threshold(seq: SeqDesc, logits, threshold: float, tokens, mask, n_decoded,
                     decoded_pos=None, conf=None, done_seqs=None, n_done=None, workspace=None,
                     flags: int = 0, stream=None):
    """fdllm_unmask_threshold; logits [b][B][V] (any strides, last dim contiguous)."""
    assert logits.stride(2) == 1
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fdllm_unmask_threshold(ctypes.byref(seq), logits.shape[2], _dtype_code(logits), _ptr(logits),
                                        logits.stride(0), logits.stride(1), float(threshold), flags,
                                        _ptr(tokens), _ptr(mask), _ptr(n_decoded), _ptr(decoded_pos),
                                        _ptr(conf), _ptr(done_seqs), _ptr(n_done), _ptr(workspace), nbytes,
                                        _stream(stream)))


def unmask_threshold_static(seq: SeqDesc, logits, threshold: float, tokens, mask, n_decoded,
                            decoded_pos=None, conf=None, done_seqs=None, n_done=None, flags: int = 0, stream=None):
    """fdllm_unmask_threshold_static: the threshold step on the library's
    static scratch (no workspace argument, nothing allocated)."""
    assert logits.stride(2) == 1
    _check(lib().fdllm_unmask_threshold_static(ctypes.byref(seq), logits.shape[2], _dtype_code(logits),
                                               _ptr(logits), logits.stride(0), logits.stride(1), float(threshold),
                                               flags, _ptr(tokens), _ptr(mask), _ptr(n_decoded),
                                               _ptr(decoded_pos), _ptr(conf), _ptr(done_seqs), _ptr(n_done),
                                               _stream(stream)))


def unmask_topk(seq: SeqDesc, logits, k: int, tokens, mask, n_decoded, decoded_pos=None, conf=None,
                done_seqs=None, n_done=None, workspace=None, flags: int = 0, stream=None):
    """fdllm_unmask_topk; logits [b][B][V] (any strides, last dim contiguous)."""
    assert logits.stride(2) == 1
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fdllm_unmask_topk(ctypes.byref(seq), logits.shape[2], _dtype_code(logits), _ptr(logits),
                                   logits.stride(0), logits.stride(1), int(k), flags,
                                   _ptr(tokens), _ptr(mask), _ptr(n_decoded), _ptr(decoded_pos),
                                   _ptr(conf), _ptr(done_seqs), _ptr(n_done), _ptr(workspace), nbytes,
                                   _stream(stream)))


def lmhead_packed_bytes(vocab: int, hidden: int) -> int:
    return int(lib().fdllm_lmhead_packed_bytes(vocab, hidden))


def lmhead_pack(w, w_packed=None, stream=None):
    """fdllm_lmhead_pack: w bf16 [V][H] contiguous -> packed weight (a new
    uint8 device tensor unless `w_packed` is given)."""
    assert w.dim() == 2 and w.is_contiguous()
    V, H = w.shape
    nbytes = lmhead_packed_bytes(V, H)
    if w_packed is None:
        import torch
        w_packed = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=w.device)
    _check(lib().fdllm_lmhead_pack(V, H, _ptr(w), _ptr(w_packed), w_packed.numel() * w_packed.element_size(),
                                   _stream(stream)))
    return w_packed


def lmhead_unmask_workspace(seq: SeqDesc, vocab: int, hidden: int) -> int:
    return int(lib().fdllm_lmhead_unmask_workspace(ctypes.byref(seq), vocab, hidden))


def _lmhead_call(fn, seq, x, w_packed, vocab, rule_arg, tokens, mask, n_decoded, decoded_pos, conf, done_seqs,
                 n_done, workspace, flags, stream):
    assert x.stride(2) == 1
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(ctypes.byref(seq), vocab, x.shape[2], _ptr(x), x.stride(0), x.stride(1), _ptr(w_packed), rule_arg,
              flags, _ptr(tokens), _ptr(mask), _ptr(n_decoded), _ptr(decoded_pos), _ptr(conf), _ptr(done_seqs),
              _ptr(n_done), _ptr(workspace), nbytes, _stream(stream)))


def lmhead_unmask_threshold(seq: SeqDesc, x, w_packed, vocab: int, threshold: float, tokens, mask, n_decoded,
                            decoded_pos=None, conf=None, done_seqs=None, n_done=None, workspace=None,
                            flags: int = 0, stream=None):
    """fdllm_lmhead_unmask_threshold; x bf16 [b][B][H] (last dim contiguous)."""
    _lmhead_call(lib().fdllm_lmhead_unmask_threshold, seq, x, w_packed, vocab, float(threshold), tokens, mask,
                 n_decoded, decoded_pos, conf, done_seqs, n_done, workspace, flags, stream)


def lmhead_unmask_topk(seq: SeqDesc, x, w_packed, vocab: int, k: int, tokens, mask, n_decoded,
                       decoded_pos=None, conf=None, done_seqs=None, n_done=None, workspace=None,
                       flags: int = 0, stream=None):
    """fdllm_lmhead_unmask_topk; x bf16 [b][B][H] (last dim contiguous)."""
    _lmhead_call(lib().fdllm_lmhead_unmask_topk, seq, x, w_packed, vocab, int(k), tokens, mask,
                 n_decoded, decoded_pos, conf, done_seqs, n_done, workspace, flags, stream)


def set_lmhead_tuning(vt: int = 0):
    """fdllm_set_lmhead_tuning: vocabulary tiles per wave (0 = automatic)."""
    _check(lib().fdllm_set_lmhead_tuning(int(vt)))


def kv_refresh(seq: SeqDesc, mode: str, k_src, v_src, k_cache, v_cache, seq_ids=None, n_seq=None,
               stream=None):
    """fdllm_kv_refresh; src [b][Lcap][Hkv][d] token-major, caches [b][Hkv][Lcap][d]."""
    ad = attn_desc(0, k_src.shape[2], k_src.shape[3], _dtype_code(k_src))
    _check(lib().fdllm_kv_refresh(ctypes.byref(seq), ctypes.byref(ad), MODE[mode], _ptr(k_src), _ptr(v_src),
                                  _ptr(k_cache), _ptr(v_cache), _ptr(seq_ids), _ptr(n_seq), _stream(stream)))


def kv_refresh_layers(seq: SeqDesc, mode: str, k_srcs, v_srcs, k_caches, v_caches, seq_ids=None, n_seq=None,
                      stream=None):
    """fdllm_kv_refresh_layers: one launch refreshing every layer l from k_srcs[l] / v_srcs[l] into
    k_caches[l] / v_caches[l] (lists of tensors laid out as for kv_refresh)."""
    n = len(k_srcs)
    if not (len(v_srcs) == len(k_caches) == len(v_caches) == n):
        raise ValueError("kv_refresh_layers needs the same number of k_srcs, v_srcs, k_caches and v_caches")
    ad = attn_desc(0, k_srcs[0].shape[2], k_srcs[0].shape[3], _dtype_code(k_srcs[0])) if n else attn_desc(0, 1, 64, F32)
    arr = lambda ts: (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in ts])
    ks, vs, kc, vc = arr(k_srcs), arr(v_srcs), arr(k_caches), arr(v_caches)
    _check(lib().fdllm_kv_refresh_layers(ctypes.byref(seq), ctypes.byref(ad), MODE[mode], n, ks, vs, kc, vc,
                                         _ptr(seq_ids), _ptr(n_seq), _stream(stream)))


def set_debug(on: bool):
    """fdllm_set_debug: validate device-resident per-sequence arrays before each call."""
    _check(lib().fdllm_set_debug(1 if on else 0))


def set_timing_events(start_event, stop_event):
    """Arm the measurement hook: the next launch records these hipEvent_t handles (ints)."""
    _check(lib().fdllm_set_timing_events(start_event, stop_event))


def set_tuning(attn_qt: int = 0, attn_wgs: int = 0, unmask_wgs: int = 0):
    """fdllm_set_tuning: launch-planner overrides (0 = automatic)."""
    _check(lib().fdllm_set_tuning(int(attn_qt), int(attn_wgs), int(unmask_wgs)))


def version() -> int:
    return int(lib().fdllm_version())
