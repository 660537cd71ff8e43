"""Python binding of libcpattn (include/cp_attn.h): argument marshalling only.

Every computation runs in the HIP library; this module only turns torch
tensors into pointers and sizes, passes torch's current HIP stream, and turns
a non-zero status into an exception. There is no CPU fallback: if the built
library is missing, importing this package raises.

Entry points (same names as the C ABI, without the ``cp_`` prefix):
  attn_chunk_partial   one ring hop: (O_c, LSE_c) of Q over one K/V chunk
  lse_merge            merge of P fp32 partials into full attention
  ring_attention       one ring rank: Q over P chunks in visit order, fused fp32 merge
  ring_attention_noalloc
                       the same with the library's static scratch (allocates nothing)
  ulysses_seq2head     Ulysses regrouping before attention (all P ranks)
  ulysses_head2seq     Ulysses regrouping after attention (inverse)
                       (both also take a stack of tensors, e.g. Q, K, V, in one launch)
  ulysses_anything_seq2head / ulysses_anything_head2seq
                       the same with uneven per-rank token and head counts
  kv_gather            the K/V all-gather's unpack (sequence shards joined)
  attn_backward_delta  Delta_i = <dO_i, O_i>, the backward's per-row statistic
  attn_chunk_backward  one K/V chunk's share of dQ, dK, dV from the saved LSE
  ring_attention_backward
                       one ring rank's backward: dQ over all its chunks, each
                       chunk's dK/dV share
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python -c 'import __graft_entry__ as g; g.build()'` "
        "(or `python context_attention_dit_amd/_build.py`). There is no fallback path.")

_lib = ctypes.CDLL(LIB_PATH)

CP_BF16, CP_F32 = 0, 1
STATUS = {0: "CP_OK", 1: "CP_E_INVALID", 2: "CP_E_UNSUPPORTED", 3: "CP_E_DIVISIBILITY",
          4: "CP_E_WORKSPACE", 5: "CP_E_HIP"}
MAX_RING_CHUNKS = 64
NOALLOC_SCRATCH_BYTES = 64 << 20  # CP_NOALLOC_SCRATCH_BYTES
BWD_ACCUMULATE_DQ, BWD_ACCUMULATE_DKV = 1, 2

_i64, _vp, _f32, _int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int


class KVChunk(ctypes.Structure):
    _fields_ = [("k", _vp), ("v", _vp), ("len", _i64), ("pos0", _i64)]


class KVGrad(ctypes.Structure):
    _fields_ = [("dk", _vp), ("dv", _vp)]


def _sig(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_chunk_partial = _sig("cp_attn_chunk_partial", [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                                _i64, _int, _int, _f32, _int, _i64, _i64, _vp])
_chunk_partial_vt = _sig("cp_attn_chunk_partial_vt",
                         [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _f32,
                          _int, _i64, _i64, _vp])
_lse_merge = _sig("cp_lse_merge", [_vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp])
_ring_ws = _sig("cp_ring_attention_workspace_bytes", [_i64] * 5, ctypes.c_size_t)
_ring = _sig("cp_ring_attention", [_vp, ctypes.POINTER(KVChunk), _i64, _vp, _vp, _i64, _i64, _i64,
                                   _i64, _int, _f32, _int, _i64, _vp, ctypes.c_size_t, _vp])
_ring_noalloc = _sig("cp_ring_attention_noalloc",
                     [_vp, ctypes.POINTER(KVChunk), _i64, _vp, _vp, _i64, _i64, _i64, _i64, _int,
                      _f32, _int, _i64, _vp])
_seq2head = _sig("cp_ulysses_seq2head", [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _vp])
_head2seq = _sig("cp_ulysses_head2seq", [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _vp])
_kv_gather_vt = _sig("cp_kv_gather_vt", [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _vp])
_seq2head_vt = _sig("cp_ulysses_seq2head_vt", [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _vp])
_seq2head_n = _sig("cp_ulysses_seq2head_n", [_vp, _vp] + [_i64] * 6 + [_int, _vp])
_head2seq_n = _sig("cp_ulysses_head2seq_n", [_vp, _vp] + [_i64] * 6 + [_int, _vp])
_any_seq2head = _sig("cp_ulysses_anything_seq2head",
                     [_vp, _vp, _i64, _i64, _vp, _vp, _i64, _int, _vp])
_any_head2seq = _sig("cp_ulysses_anything_head2seq",
                     [_vp, _vp, _i64, _i64, _vp, _vp, _i64, _int, _vp])
_any_seq2head_n = _sig("cp_ulysses_anything_seq2head_n",
                       [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _int, _vp])
_any_head2seq_n = _sig("cp_ulysses_anything_head2seq_n",
                       [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _int, _vp])
_kv_gather = _sig("cp_kv_gather", [_vp, _vp, _i64, _i64, _vp, _i64, _i64, _int, _vp])
_kv_gather_n = _sig("cp_kv_gather_n", [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _int, _vp])
_bwd_delta = _sig("cp_attn_backward_delta", [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp])
_chunk_bwd = _sig("cp_attn_chunk_backward", [_vp] * 9 + [_i64] * 5 +
                  [_int, _f32, _int, _i64, _i64, _int, _vp])
_ring_bwd = _sig("cp_ring_attention_backward",
                 [_vp, ctypes.POINTER(KVChunk), _i64, _vp, _vp, _vp, _vp, ctypes.POINTER(KVGrad),
                  _i64, _i64, _i64, _i64, _int, _f32, _int, _i64, _int, _vp])
_last_error = _sig("cp_last_error", [], ctypes.c_char_p)
_abi_version = _sig("cp_abi_version", [])


class CpAttnError(RuntimeError):
    """A cp_* call returned a non-zero status."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise CpAttnError(fn, status, (_last_error() or b"").decode())


def last_error() -> str:
    return (_last_error() or b"").decode()


def abi_version() -> int:
    return _abi_version()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return CP_BF16
    if t == torch.float32:
        return CP_F32
    raise TypeError(f"unsupported dtype {t} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


def _want(t: torch.Tensor, name: str, shape, dtype, device) -> torch.Tensor:
    """A buffer the library reads or writes as `shape` elements of `dtype`: the
    C ABI sees only its address, so its size, type and device are checked here."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, "
                         f"got {t.dtype} of shape {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


def _bshd(x: torch.Tensor, name: str) -> Tuple[int, int, int, int]:
    if x.dim() != 4:
        raise ValueError(f"{name} must be [B][S][H][D], got shape {tuple(x.shape)}")
    return tuple(x.shape)  # type: ignore[return-value]


def attn_chunk_partial(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, *,
                       scale: Optional[float] = None, causal: bool = False, q_pos0: int = 0,
                       kv_pos0: int = 0, out_dtype: torch.dtype = torch.float32,
                       stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(O_c, LSE_c) of ``q`` over one K/V chunk; see cp_attn_chunk_partial in include/cp_attn.h."""
    B, Sq, H, D = _bshd(q, "q")
    Bk, Skv, Hk, Dk = _bshd(k, "k")
    if (Bk, Hk, Dk) != (B, H, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k, v shapes disagree")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    _want(k, "k", k.shape, q.dtype, q.device)
    _want(v, "v", k.shape, q.dtype, q.device)
    if o is None:
        o = torch.empty((B, Sq, H, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _want(o, "o", (B, Sq, H, D), o.dtype, q.device)
    _want(lse, "lse", (B, H, Sq), torch.float32, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check("cp_attn_chunk_partial", _chunk_partial(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq, Skv, D, _dtype_code(q.dtype),
        _dtype_code(o.dtype), scale, int(causal), q_pos0, kv_pos0, _stream(stream)))
    return o, lse


def attn_chunk_partial_vt(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor,
                          o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, *,
                          scale: Optional[float] = None, causal: bool = False, q_pos0: int = 0,
                          kv_pos0: int = 0, out_dtype: torch.dtype = torch.float32,
                          stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """As attn_chunk_partial with V key-contiguous in 64-key tiles,
    ``vt [B][H][ceil(Skv/64)][D][64]``; see cp_attn_chunk_partial_vt in include/cp_attn.h."""
    B, Sq, H, D = _bshd(q, "q")
    Bk, Skv, Hk, Dk = _bshd(k, "k")
    if (Bk, Hk, Dk) != (B, H, D):
        raise ValueError("q, k shapes disagree")
    if k.dtype != q.dtype or vt.dtype != q.dtype:
        raise TypeError("q, k, vt must share one dtype")
    _want(k, "k", k.shape, q.dtype, q.device)
    _want(vt, "vt", (B, H, (Skv + 63) // 64, D, 64), q.dtype, q.device)
    if o is None:
        o = torch.empty((B, Sq, H, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _want(o, "o", (B, Sq, H, D), o.dtype, q.device)
    _want(lse, "lse", (B, H, Sq), torch.float32, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check("cp_attn_chunk_partial_vt", _chunk_partial_vt(
        _ptr(q), _ptr(k), _ptr(vt), _ptr(o), _ptr(lse), B, H, Sq, Skv, D, _dtype_code(q.dtype),
        _dtype_code(o.dtype), scale, int(causal), q_pos0, kv_pos0, _stream(stream)))
    return o, lse


def lse_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, o: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, *, out_dtype: torch.dtype = torch.float32,
              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge ``o_parts [P][B][Sq][H][D]`` / ``lse_parts [P][B][H][Sq]`` (fp32); see cp_lse_merge."""
    if o_parts.dim() != 5 or lse_parts.dim() != 4:
        raise ValueError("o_parts must be [P][B][Sq][H][D] and lse_parts [P][B][H][Sq]")
    P, B, Sq, H, D = o_parts.shape
    if tuple(lse_parts.shape) != (P, B, H, Sq):
        raise ValueError("lse_parts shape disagrees with o_parts")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partials must be float32")
    _want(lse_parts, "lse_parts", (P, B, H, Sq), torch.float32, o_parts.device)
    if o is None:
        o = torch.empty((B, Sq, H, D), dtype=out_dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=o_parts.device)
    _want(o, "o", (B, Sq, H, D), o.dtype, o_parts.device)
    _want(lse, "lse", (B, H, Sq), torch.float32, o_parts.device)
    _check("cp_lse_merge", _lse_merge(_ptr(o_parts), _ptr(lse_parts), P, _ptr(o), _ptr(lse), B, H,
                                      Sq, D, _dtype_code(o.dtype), _stream(stream)))
    return o, lse


def ring_attention_workspace_bytes(P: int, B: int, H: int, Sq: int, D: int) -> int:
    return int(_ring_ws(P, B, H, Sq, D))


def ring_attention(q: torch.Tensor, chunks: Sequence[Tuple[torch.Tensor, torch.Tensor, int]],
                   o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, *,
                   scale: Optional[float] = None, causal: bool = False, q_pos0: int = 0,
                   workspace: Optional[torch.Tensor] = None,
                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One ring rank: ``q`` over ``chunks = [(k_c, v_c, pos0_c), ...]`` in visit order.

    Output O has q's dtype; LSE is fp32 ``[B][H][Sq]``. See cp_ring_attention.
    """
    B, Sq, H, D = _bshd(q, "q")
    arr = (KVChunk * max(1, len(chunks)))()
    for c, (k, v, pos0) in enumerate(chunks):
        Bk, L, Hk, Dk = _bshd(k, "k")
        if (Bk, Hk, Dk) != (B, H, D) or tuple(v.shape) != tuple(k.shape):
            raise ValueError(f"chunk {c} shape disagrees with q")
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise TypeError(f"chunk {c} dtype disagrees with q")
        _want(k, f"chunk {c} k", k.shape, q.dtype, q.device)
        _want(v, f"chunk {c} v", k.shape, q.dtype, q.device)
    if o is None:
        o = torch.empty((B, Sq, H, D), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _want(o, "o", (B, Sq, H, D), q.dtype, q.device)
    _want(lse, "lse", (B, H, Sq), torch.float32, q.device)
    for c, (k, v, pos0) in enumerate(chunks):
        arr[c] = KVChunk(_ptr(k), _ptr(v), k.shape[1], int(pos0))
    need = ring_attention_workspace_bytes(len(chunks), B, H, Sq, D)
    own_ws = workspace is None and need > 0 and q.dtype == torch.bfloat16
    if own_ws:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None and workspace.device != q.device:
        raise ValueError(f"workspace must be on {q.device}")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check("cp_ring_attention", _ring(
        _ptr(q), arr, len(chunks), _ptr(o), _ptr(lse), B, H, Sq, D, _dtype_code(q.dtype), scale,
        int(causal), q_pos0, _ptr(workspace), ws_bytes, _stream(stream)))
    if own_ws and stream is not None:
        # the workspace was allocated on the current stream but is used on `stream`:
        # keep the caching allocator from reusing it before that work is done
        workspace.record_stream(stream)
    return o, lse


def ring_attention_noalloc(q: torch.Tensor,
                           chunks: Sequence[Tuple[torch.Tensor, torch.Tensor, int]],
                           o: torch.Tensor, lse: torch.Tensor, *, scale: Optional[float] = None,
                           causal: bool = False, q_pos0: int = 0,
                           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """``ring_attention`` through cp_ring_attention_noalloc: the library keeps the
    key-split partials in its static device scratch, so the call allocates
    nothing (``o`` and ``lse`` are required). Calls that overlap on one GPU race."""
    B, Sq, H, D = _bshd(q, "q")
    arr = (KVChunk * max(1, len(chunks)))()
    for c, (k, v, pos0) in enumerate(chunks):
        Bk, L, Hk, Dk = _bshd(k, "k")
        if (Bk, Hk, Dk) != (B, H, D) or tuple(v.shape) != tuple(k.shape):
            raise ValueError(f"chunk {c} shape disagrees with q")
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise TypeError(f"chunk {c} dtype disagrees with q")
        _want(k, f"chunk {c} k", k.shape, q.dtype, q.device)
        _want(v, f"chunk {c} v", k.shape, q.dtype, q.device)
        arr[c] = KVChunk(_ptr(k), _ptr(v), k.shape[1], int(pos0))
    _want(o, "o", (B, Sq, H, D), q.dtype, q.device)
    _want(lse, "lse", (B, H, Sq), torch.float32, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    _check("cp_ring_attention_noalloc", _ring_noalloc(
        _ptr(q), arr, len(chunks), _ptr(o), _ptr(lse), B, H, Sq, D, _dtype_code(q.dtype), scale,
        int(causal), q_pos0, _stream(stream)))
    return o, lse


def ulysses_seq2head(x: torch.Tensor, P: int, out: Optional[torch.Tensor] = None, *,
                     stream=None) -> torch.Tensor:
    """``[P][B][S_l][H][D]`` -> ``[P][B][P*S_l][H/P][D]``; see cp_ulysses_seq2head.

    A 6-D ``x`` of shape ``[n][P][B][S_l][H][D]`` (for example a rank's Q, K and
    V stacked) is regrouped tensor by tensor in one launch (cp_ulysses_seq2head_n).
    """
    if x.dim() not in (5, 6) or x.shape[-5] != P:
        raise ValueError("x must be [P][B][S_local][H][D] or [n][P][B][S_local][H][D]")
    _, B, S_l, H, D = x.shape[-5:]
    lead = tuple(x.shape[:-5])
    if out is None:
        out = torch.empty(lead + (P, B, P * S_l, H // P, D), dtype=x.dtype, device=x.device)
    _want(out, "out", lead + (P, B, P * S_l, H // P, D), x.dtype, x.device)
    if x.dim() == 6:
        _check("cp_ulysses_seq2head_n", _seq2head_n(_ptr(x), _ptr(out), x.shape[0], P, B, S_l,
                                                    H, D, _dtype_code(x.dtype), _stream(stream)))
    else:
        _check("cp_ulysses_seq2head", _seq2head(_ptr(x), _ptr(out), P, B, S_l, H, D,
                                                _dtype_code(x.dtype), _stream(stream)))
    return out


def ulysses_seq2head_vt(x: torch.Tensor, P: int, out: Optional[torch.Tensor] = None, *,
                        stream=None) -> torch.Tensor:
    """``[P][B][S_l][H][D]`` -> ``[P][B][H/P][ceil(P*S_l/64)][D][64]`` (V delivered
    key-contiguous per head in 64-token tiles); see cp_ulysses_seq2head_vt."""
    if x.dim() != 5 or x.shape[0] != P:
        raise ValueError("x must be [P][B][S_local][H][D]")
    _, B, S_l, H, D = x.shape
    shape = (P, B, H // P, (P * S_l + 63) // 64, D, 64)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    _want(out, "out", shape, x.dtype, x.device)
    _check("cp_ulysses_seq2head_vt", _seq2head_vt(_ptr(x), _ptr(out), P, B, S_l, H, D,
                                                  _dtype_code(x.dtype), _stream(stream)))
    return out


def kv_gather_vt(x: torch.Tensor, out: Optional[torch.Tensor] = None, *,
                 stream=None) -> torch.Tensor:
    """``[P][B][S_l][H][D]`` (P equal shards) -> ``[B][H][ceil(P*S_l/64)][D][64]`` (the
    gathered V, key-contiguous in 64-token tiles); see cp_kv_gather_vt."""
    if x.dim() != 5:
        raise ValueError("x must be [P][B][S_local][H][D]")
    P, B, S_l, H, D = x.shape
    shape = (B, H, (P * S_l + 63) // 64, D, 64)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    _want(out, "out", shape, x.dtype, x.device)
    _check("cp_kv_gather_vt", _kv_gather_vt(_ptr(x), _ptr(out), P, B, S_l, H, D,
                                            _dtype_code(x.dtype), _stream(stream)))
    return out


def ulysses_head2seq(y: torch.Tensor, P: int, out: Optional[torch.Tensor] = None, *,
                     stream=None) -> torch.Tensor:
    """``[P][B][P*S_l][H_l][D]`` -> ``[P][B][S_l][P*H_l][D]``; see cp_ulysses_head2seq.

    A 6-D ``y`` (``[n][P][B][P*S_l][H_l][D]``) is regrouped tensor by tensor in
    one launch (cp_ulysses_head2seq_n)."""
    if y.dim() not in (5, 6) or y.shape[-5] != P or y.shape[-3] % P != 0:
        raise ValueError("y must be [P][B][P*S_local][H/P][D] or [n][P][B][P*S_local][H/P][D]")
    _, B, S, H_l, D = y.shape[-5:]
    lead = tuple(y.shape[:-5])
    if out is None:
        out = torch.empty(lead + (P, B, S // P, H_l * P, D), dtype=y.dtype, device=y.device)
    _want(out, "out", lead + (P, B, S // P, H_l * P, D), y.dtype, y.device)
    if y.dim() == 6:
        _check("cp_ulysses_head2seq_n", _head2seq_n(_ptr(y), _ptr(out), y.shape[0], P, B, S // P,
                                                    H_l * P, D, _dtype_code(y.dtype),
                                                    _stream(stream)))
    else:
        _check("cp_ulysses_head2seq", _head2seq(_ptr(y), _ptr(out), P, B, S // P, H_l * P, D,
                                                _dtype_code(y.dtype), _stream(stream)))
    return out


def _counts(xs):
    arr = (ctypes.c_int64 * max(1, len(xs)))(*[int(v) for v in xs])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def _packed(x: torch.Tensor, n: int) -> int:
    """Tensor count of a packed input: 1 for a flat tensor of n elements, or
    the leading size of a 2-D [count][n] stack."""
    if not x.is_contiguous() or x.dim() not in (1, 2) or x.shape[-1] != n:
        raise ValueError(f"expected a contiguous packed tensor of {n} elements, or a 2-D "
                         f"[count][{n}] stack of them")
    return 1 if x.dim() == 1 else x.shape[0]


def _anything(names, fns, x, s_lens, h_counts, B, D, out, stream):
    P = len(s_lens)
    if len(h_counts) != P:
        raise ValueError("s_lens and h_counts need one entry per rank")
    n = B * sum(s_lens) * sum(h_counts) * D
    count = _packed(x, n)
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    _want(out, "out", x.shape, x.dtype, x.device)
    sa, sp = _counts(s_lens)
    ha, hp = _counts(h_counts)
    if x.dim() == 2:
        _check(names[1], fns[1](_ptr(x), _ptr(out), count, P, B, sp, hp, D, _dtype_code(x.dtype),
                                _stream(stream)))
    else:
        _check(names[0], fns[0](_ptr(x), _ptr(out), P, B, sp, hp, D, _dtype_code(x.dtype),
                                _stream(stream)))
    return out


def ulysses_anything_seq2head(x: torch.Tensor, s_lens, h_counts, B: int, D: int,
                              out: Optional[torch.Tensor] = None, *, stream=None) -> torch.Tensor:
    """Packed sequence shards (shard q = [B][s_lens[q]][H][D]) -> packed head
    groups (group p = [B][S][h_counts[p]][D]); see cp_ulysses_anything_seq2head.
    Returns a flat tensor of B*S*H*D elements. A 2-D ``x`` of shape
    ``[n][B*S*H*D]`` (a rank's Q, K and V, say) is regrouped tensor by tensor in
    one launch (cp_ulysses_anything_seq2head_n)."""
    return _anything(("cp_ulysses_anything_seq2head", "cp_ulysses_anything_seq2head_n"),
                     (_any_seq2head, _any_seq2head_n), x, s_lens, h_counts, B, D, out, stream)


def ulysses_anything_head2seq(y: torch.Tensor, s_lens, h_counts, B: int, D: int,
                              out: Optional[torch.Tensor] = None, *, stream=None) -> torch.Tensor:
    """Packed head groups -> packed sequence shards; the inverse of
    ulysses_anything_seq2head (see cp_ulysses_anything_head2seq). A 2-D ``y``
    is a stack of such inputs (cp_ulysses_anything_head2seq_n)."""
    return _anything(("cp_ulysses_anything_head2seq", "cp_ulysses_anything_head2seq_n"),
                     (_any_head2seq, _any_head2seq_n), y, s_lens, h_counts, B, D, out, stream)


def kv_gather(x: torch.Tensor, s_lens, B: int, H: int, D: int,
              out: Optional[torch.Tensor] = None, *, stream=None) -> torch.Tensor:
    """Packed sequence shards (shard q = [B][s_lens[q]][H][D]) -> the gathered
    [B][S][H][D] tensor; see cp_kv_gather. A 2-D ``x`` of shape
    ``[n][B*S*H*D]`` (K and V, say) gives ``[n][B][S][H][D]`` in one launch
    (cp_kv_gather_n)."""
    S = sum(s_lens)
    count = _packed(x, B * S * H * D)
    lead = (count,) if x.dim() == 2 else ()
    if out is None:
        out = torch.empty(lead + (B, S, H, D), dtype=x.dtype, device=x.device)
    _want(out, "out", lead + (B, S, H, D), x.dtype, x.device)
    sa, sp = _counts(s_lens)
    if x.dim() == 2:
        _check("cp_kv_gather_n", _kv_gather_n(_ptr(x), _ptr(out), count, len(s_lens), B, sp, H,
                                              D, _dtype_code(x.dtype), _stream(stream)))
    else:
        _check("cp_kv_gather", _kv_gather(_ptr(x), _ptr(out), len(s_lens), B, sp, H, D,
                                          _dtype_code(x.dtype), _stream(stream)))
    return out


def attn_backward_delta(o: torch.Tensor, dout: torch.Tensor, delta: Optional[torch.Tensor] = None,
                        *, stream=None) -> torch.Tensor:
    """``delta [B][H][Sq]`` fp32 = <dO_i, O_i> per row; see cp_attn_backward_delta."""
    B, Sq, H, D = _bshd(o, "o")
    if tuple(dout.shape) != tuple(o.shape) or dout.dtype != o.dtype:
        raise ValueError("o and dout must share shape and dtype")
    _want(dout, "dout", o.shape, o.dtype, o.device)
    if delta is None:
        delta = torch.empty((B, H, Sq), dtype=torch.float32, device=o.device)
    _want(delta, "delta", (B, H, Sq), torch.float32, o.device)
    _check("cp_attn_backward_delta", _bwd_delta(_ptr(o), _ptr(dout), _ptr(delta), B, H, Sq, D,
                                                _dtype_code(o.dtype), _stream(stream)))
    return delta


def attn_chunk_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
                        lse: torch.Tensor, delta: torch.Tensor, dq: Optional[torch.Tensor] = None,
                        dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None, *,
                        scale: Optional[float] = None, causal: bool = False, q_pos0: int = 0,
                        kv_pos0: int = 0, accumulate_dq: bool = False,
                        accumulate_dkv: bool = False,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """One K/V chunk's share of (dQ, dK, dV) in fp32; see cp_attn_chunk_backward.

    With ``accumulate_dq`` / ``accumulate_dkv`` the given buffers hold running
    sums and the share is added to them; otherwise they are overwritten (and
    allocated when not given)."""
    B, Sq, H, D = _bshd(q, "q")
    Bk, Skv, Hk, Dk = _bshd(k, "k")
    if (Bk, Hk, Dk) != (B, H, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("q, k, v shapes disagree")
    if tuple(dout.shape) != tuple(q.shape):
        raise ValueError("dout must have q's shape")
    if tuple(lse.shape) != (B, H, Sq) or tuple(delta.shape) != (B, H, Sq):
        raise ValueError("lse and delta must be [B][H][Sq]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    for name, t, shape, dt in (("k", k, k.shape, q.dtype), ("v", v, k.shape, q.dtype),
                               ("dout", dout, q.shape, q.dtype),
                               ("lse", lse, (B, H, Sq), torch.float32),
                               ("delta", delta, (B, H, Sq), torch.float32)):
        _want(t, name, shape, dt, q.device)
    if (accumulate_dq and dq is None) or (accumulate_dkv and (dk is None or dv is None)):
        raise ValueError("accumulating needs the running-sum buffers")
    f32 = torch.float32
    dq = torch.empty((B, Sq, H, D), dtype=f32, device=q.device) if dq is None else dq
    dk = torch.empty((B, Skv, H, D), dtype=f32, device=q.device) if dk is None else dk
    dv = torch.empty((B, Skv, H, D), dtype=f32, device=q.device) if dv is None else dv
    for name, t, shape in (("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, k.shape)):
        _want(t, name, shape, f32, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    flags = (BWD_ACCUMULATE_DQ if accumulate_dq else 0) | \
        (BWD_ACCUMULATE_DKV if accumulate_dkv else 0)
    _check("cp_attn_chunk_backward", _chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk),
        _ptr(dv), B, H, Sq, Skv, D, _dtype_code(q.dtype), scale, int(causal), q_pos0, kv_pos0,
        flags, _stream(stream)))
    return dq, dk, dv


def ring_attention_backward(q: torch.Tensor,
                            chunks: Sequence[Tuple[torch.Tensor, torch.Tensor, int]],
                            dout: torch.Tensor, lse: torch.Tensor, delta: torch.Tensor,
                            dq: Optional[torch.Tensor] = None,
                            grads: Optional[Sequence[Tuple[torch.Tensor, torch.Tensor]]] = None,
                            *, scale: Optional[float] = None, causal: bool = False,
                            q_pos0: int = 0, accumulate_dq: bool = False,
                            accumulate_dkv: bool = False, stream=None):
    """One ring rank's backward over ``chunks = [(k_c, v_c, pos0_c), ...]``; see
    cp_ring_attention_backward. Returns ``(dq, [(dk_c, dv_c), ...])`` in fp32."""
    B, Sq, H, D = _bshd(q, "q")
    if tuple(dout.shape) != tuple(q.shape):
        raise ValueError("dout must have q's shape")
    if tuple(lse.shape) != (B, H, Sq) or tuple(delta.shape) != (B, H, Sq):
        raise ValueError("lse and delta must be [B][H][Sq]")
    for name, t, shape, dt in (("dout", dout, q.shape, q.dtype),
                               ("lse", lse, (B, H, Sq), torch.float32),
                               ("delta", delta, (B, H, Sq), torch.float32)):
        _want(t, name, shape, dt, q.device)
    if (accumulate_dq and dq is None) or (accumulate_dkv and grads is None):
        raise ValueError("accumulating needs the running-sum buffers")
    f32 = torch.float32
    if dq is None:
        dq = torch.empty((B, Sq, H, D), dtype=f32, device=q.device)
    if grads is None:
        grads = [(torch.empty(k.shape, dtype=f32, device=q.device),
                  torch.empty(k.shape, dtype=f32, device=q.device)) for k, _, _ in chunks]
    if len(grads) != len(chunks):
        raise ValueError("one (dk, dv) pair per chunk")
    n = max(1, len(chunks))
    arr, garr = (KVChunk * n)(), (KVGrad * n)()
    for c, ((k, v, pos0), (dk, dv)) in enumerate(zip(chunks, grads)):
        Bk, L, Hk, Dk = _bshd(k, "k")
        if (Bk, Hk, Dk) != (B, H, D) or tuple(v.shape) != tuple(k.shape):
            raise ValueError(f"chunk {c} shape disagrees with q")
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise TypeError(f"chunk {c} dtype disagrees with q")
        _want(k, f"chunk {c} k", k.shape, q.dtype, q.device)
        _want(v, f"chunk {c} v", k.shape, q.dtype, q.device)
        for name, t in (("dk", dk), ("dv", dv)):
            _want(t, f"chunk {c} {name}", k.shape, f32, q.device)
        arr[c] = KVChunk(_ptr(k), _ptr(v), L, int(pos0))
        garr[c] = KVGrad(_ptr(dk), _ptr(dv))
    _want(dq, "dq", (B, Sq, H, D), f32, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    flags = (BWD_ACCUMULATE_DQ if accumulate_dq else 0) | \
        (BWD_ACCUMULATE_DKV if accumulate_dkv else 0)
    _check("cp_ring_attention_backward", _ring_bwd(
        _ptr(q), arr, len(chunks), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq), garr, B, H, Sq,
        D, _dtype_code(q.dtype), scale, int(causal), q_pos0, flags, _stream(stream)))
    return dq, list(grads)


__all__ = ["attn_chunk_partial", "attn_chunk_partial_vt", "ulysses_seq2head_vt", "kv_gather_vt", "lse_merge", "ring_attention", "ring_attention_workspace_bytes",
           "ulysses_seq2head", "ulysses_head2seq", "ulysses_anything_seq2head",
           "ulysses_anything_head2seq", "kv_gather", "attn_backward_delta",
           "attn_chunk_backward", "ring_attention_backward", "KVGrad", "BWD_ACCUMULATE_DQ",
           "BWD_ACCUMULATE_DKV", "last_error", "abi_version", "CpAttnError", "KVChunk",
           "LIB_PATH"]
