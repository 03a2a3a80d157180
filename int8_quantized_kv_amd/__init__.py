"""Split-KV decode attention for MI355X (gfx950): Python binding of libdattn.so.

The functions here have the names of the C entry points in include/dattn.h and
only marshal arguments: they check tensor dtypes, devices and shapes, fill the
``dattn_params`` struct, allocate the caller-side outputs and workspace with
torch when the caller did not pass them, and call the library on torch's
current HIP stream.  Every step of the attention runs in the HIP kernels; when
the library is missing, loading fails with an error instead of falling back.

Cache layouts (C-contiguous):
  q                 [B, H, D]                  float32
  k_cache, v_cache  [num_blocks, bs, Hkv, D]   float16 or float32
  block_table       [B, max_blocks]            int32
  seq_lens, q_pos   [B]                        int32
  k_hot, v_hot      [B, hot_window, Hkv, D]    float16
  k_cold, v_cold    [num_blocks, bs, Hkv, D/4] int32/uint32 words of 4 int8, LSB first
  k_scale, v_scale  [num_blocks, bs, Hkv]      float16
  k_cold, v_cold    [num_blocks, bs, Hkv, D]   float16 (the tiered f16 cache)
  k_ring, v_ring    [B, W, Hkv, D]             float16 (the window ring, W = sliding window)
  row_ptr           [num_layouts, rows + 1]    int32
  col_idx           [num_layouts, col_stride]  int32
q may also be float16 (converted exactly).
Outputs: out [B, H, D] float32 or float16 (out_dtype), lse [B, H] float32;
want_out=False writes lse only.

Every decode function needs max_seq_len, a host-side upper bound of seq_lens
that sizes the grid: the binding never reads device memory, so a call
enqueues work without synchronising the stream and can be captured in a graph.
Shapes are checked before anything is enqueued: every per-sequence array
(seq_lens, cold_lens, q_pos, block tables) must have one row per sequence.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "DattnError", "DattnParams", "lib", "library_path", "dattn_workspace_size",
    "dattn_decode_paged", "dattn_decode_tiered_int8", "dattn_decode_tiered_int8_static", "dattn_decode_tiered_f16", "dattn_decode_ring_f16",
    "dattn_decode_block_sparse", "dattn_append_tiered_int8", "dattn_append_ring_f16",
    "dattn_stream_read", "dattn_last_error", "dattn_version",
    "KIND_PAGED", "KIND_TIERED_INT8", "KIND_BLOCK_SPARSE", "KIND_TIERED_F16", "KIND_RING_F16",
    "F32", "F16", "PHASE_ALL", "PHASE_SPLIT", "PHASE_COMBINE",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libdattn.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH = 0, -1, -2, -3, -4
F32, F16 = 0, 1
PHASE_ALL, PHASE_SPLIT, PHASE_COMBINE = 0, 1, 2
KIND_PAGED, KIND_TIERED_INT8, KIND_BLOCK_SPARSE, KIND_TIERED_F16, KIND_RING_F16 = 0, 1, 2, 3, 4


class DattnParams(ctypes.Structure):
    """Mirror of ``dattn_params`` in include/dattn.h."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
        ("softcap", ctypes.c_float),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("split_tokens", ctypes.c_int32),
        ("phases", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("query_len", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
    ]


class DattnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"dattn error {code}: {message}")
        self.code = code


_lib = None


def lib():
    """The loaded libdattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is missing: build it first (int8_quantized_kv_amd.build)")
        L = ctypes.CDLL(library_path)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        PP = ctypes.POINTER(DattnParams)
        L.dattn_last_error.restype = ctypes.c_char_p
        L.dattn_version.restype = ctypes.c_char_p
        L.dattn_workspace_size.argtypes = [PP, i32, i32, ctypes.POINTER(sz)]
        L.dattn_decode_paged.argtypes = [PP, P, P, P, i32, P, P, P, P, P, P, sz, P]
        L.dattn_decode_tiered_int8.argtypes = [PP, P, P, P, i32, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.dattn_decode_tiered_int8_static.argtypes = [PP, P, P, P, i32, P, P, P, P, P, P, P, P, P, P, P]
        L.dattn_decode_tiered_f16.argtypes = [PP, P, P, P, i32, P, P, P, P, P, P, P, P, P, sz, P]
        L.dattn_decode_ring_f16.argtypes = [PP, P, P, P, P, P, P, P, P, sz, P]
        L.dattn_decode_block_sparse.argtypes = [PP, P, P, P, P, P, P, i32, i32, P, i32, P, i32, P, P, P, sz, P]
        L.dattn_append_tiered_int8.argtypes = [PP, P, P, P, P, i32, P, P, P, P, P, P, P, P]
        L.dattn_append_ring_f16.argtypes = [PP, P, P, P, P, P, P]
        L.dattn_stream_read.argtypes = [P, sz, P, P]
        for f in (L.dattn_workspace_size, L.dattn_decode_paged, L.dattn_decode_tiered_int8,
                  L.dattn_decode_tiered_int8_static,
                  L.dattn_decode_tiered_f16, L.dattn_decode_ring_f16, L.dattn_decode_block_sparse,
                  L.dattn_append_tiered_int8, L.dattn_append_ring_f16, L.dattn_stream_read):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def dattn_last_error() -> str:
    return lib().dattn_last_error().decode()


def dattn_version() -> str:
    return lib().dattn_version().decode()


def _check(rc: int):
    if rc != OK:
        raise DattnError(rc, dattn_last_error())


def dattn_workspace_size(params: DattnParams, kind: int, sparse_block: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dattn_workspace_size(ctypes.byref(params), kind, sparse_block, ctypes.byref(n)))
    return int(n.value)


# ------------------------------------------------------------ torch side

def _torch():
    import torch
    return torch


def _need(t, name, dtypes, ndim, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _rows(B, **tensors):
    """Every per-sequence array has one row per sequence: the kernels index
    row b of each for every b < B, so a short array would be read past its end."""
    for name, t in tensors.items():
        if t is not None and t.shape[0] != B:
            raise ValueError(f"{name} has {t.shape[0]} rows, expected one per sequence ({B})")


def _on_gpu(t, name):
    """Checked after the shapes: every other array was required to be on t's device."""
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device}); the library reads device memory only")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _out_code(out_dtype):
    torch = _torch()
    if out_dtype not in (torch.float32, torch.float16):
        raise TypeError(f"out_dtype must be torch.float32 or torch.float16, got {out_dtype}")
    return F16 if out_dtype == torch.float16 else F32


def _params(q, Hkv, D, bs, max_blocks, num_blocks, max_seq_len, scale, causal, sliding_window, softcap,
            split_tokens, phases=PHASE_ALL, out_dtype=None):
    """q is [B, H, D], or [B, Qn, H, D] for Qn queries per sequence."""
    B, H = q.shape[0], q.shape[-2]
    qn = q.shape[1] if q.dim() == 4 else 1
    code = F32 if out_dtype is None else _out_code(out_dtype)
    torch = _torch()
    return DattnParams(B, H, Hkv, D, float(scale), int(causal), int(sliding_window), float(softcap), bs, max_blocks,
                       num_blocks, int(max_seq_len), int(split_tokens), int(phases), code, qn,
                       F16 if q.dtype == torch.float16 else F32)


def _outputs(q, out, lse, want_lse, workspace, ws_bytes, out_dtype=None, want_out=True):
    torch = _torch()
    oshape, lshape = tuple(q.shape), tuple(q.shape[:-1])
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    if not want_out:
        if out is not None:
            raise ValueError("out given with want_out=False")
        if lse is None and not want_lse:
            raise ValueError("want_out=False needs lse")
    elif out is None:
        out = torch.empty(oshape, dtype=out_dtype, device=q.device)
    else:
        _need(out, "out", (out_dtype,), len(oshape), q.device)
        if tuple(out.shape) != oshape:
            raise ValueError(f"out must have shape {oshape}")
    if lse is None and want_lse:
        lse = torch.empty(lshape, dtype=torch.float32, device=q.device)
    elif lse is not None:
        _need(lse, "lse", (torch.float32,), len(lshape), q.device)
        if tuple(lse.shape) != lshape:
            raise ValueError(f"lse must have shape {lshape}")
    if workspace is None and ws_bytes is not None:   # ws_bytes None: the call takes no workspace
        workspace = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=q.device)
    return out, lse, workspace


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _max_len(max_seq_len):
    """max_seq_len sizes the grid on the host; it is a required argument because
    reading it from the device array seq_lens would synchronise the stream (and
    break graph capture)."""
    if max_seq_len is None:
        raise ValueError("max_seq_len is required (an upper bound of seq_lens known on the host)")
    if int(max_seq_len) < 0:
        raise ValueError(f"max_seq_len must be >= 0 (got {max_seq_len})")
    return int(max_seq_len)


def dattn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, *, q_pos=None, scale: float = 0.0,
                       causal: bool = True, sliding_window: int = 0, softcap: float = 0.0,
                       max_seq_len: Optional[int] = None, split_tokens: int = 0, out=None, lse=None,
                       want_lse: bool = True, workspace=None, stream=None, phases: int = PHASE_ALL,
                       out_dtype=None, want_out: bool = True):
    """Decode attention over a paged f16/f32 cache; returns (out, lse).  q [B, Qn, H, D]
    asks for Qn queries per sequence (query i at q_pos[b] + i, q_pos defaulting to
    seq_lens - Qn); out and lse then carry the Qn axis too."""
    torch = _torch()
    dev = q.device
    _need(q, "q", (torch.float32, torch.float16), q.dim() if q.dim() in (3, 4) else 3, dev)
    _need(k_cache, "k_cache", (torch.float16, torch.float32), 4, dev)
    _need(v_cache, "v_cache", (k_cache.dtype,), 4, dev)
    _need(block_table, "block_table", (torch.int32,), 2, dev)
    _need(seq_lens, "seq_lens", (torch.int32,), 1, dev)
    if q_pos is not None:
        _need(q_pos, "q_pos", (torch.int32,), 1, dev)
    NB, bs, Hkv, D = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or q.shape[-1] != D:
        raise ValueError("k_cache, v_cache and q disagree on shape")
    _rows(q.shape[0], block_table=block_table, seq_lens=seq_lens, q_pos=q_pos)
    max_seq_len = _max_len(max_seq_len)
    _on_gpu(q, "q")
    p = _params(q, Hkv, D, bs, block_table.shape[1], NB, max_seq_len, scale, causal,
                sliding_window, softcap, split_tokens, phases, out_dtype)
    ws = dattn_workspace_size(p, KIND_PAGED)
    out, lse, workspace = _outputs(q, out, lse, want_lse, workspace, ws, out_dtype, want_out)
    kv_dtype = F16 if k_cache.dtype == torch.float16 else F32
    _check(lib().dattn_decode_paged(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), kv_dtype,
                                    _ptr(block_table), _ptr(seq_lens), _ptr(q_pos), _ptr(out), _ptr(lse),
                                    _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def dattn_decode_tiered_int8(q, k_hot, v_hot, k_cold, v_cold, k_scale, v_scale, cold_block_table, seq_lens,
                             cold_lens, *, q_pos=None, scale: float = 0.0, causal: bool = True,
                             sliding_window: int = 0, softcap: float = 0.0, max_seq_len: Optional[int] = None,
                             split_tokens: int = 0, out=None, lse=None, want_lse: bool = True, workspace=None,
                             stream=None, phases: int = PHASE_ALL, out_dtype=None, want_out: bool = True):
    """Decode attention over an int8 cold pool + f16 hot ring; returns (out, lse).
    q [B, Qn, H, D] asks for Qn queries per sequence, as for dattn_decode_paged."""
    torch = _torch()
    dev = q.device
    _need(q, "q", (torch.float32, torch.float16), q.dim() if q.dim() in (3, 4) else 3, dev)
    _need(k_hot, "k_hot", (torch.float16,), 4, dev)
    _need(v_hot, "v_hot", (torch.float16,), 4, dev)
    _need(k_cold, "k_cold", (torch.int32, torch.uint32), 4, dev)
    _need(v_cold, "v_cold", (k_cold.dtype,), 4, dev)
    _need(k_scale, "k_scale", (torch.float16,), 3, dev)
    _need(v_scale, "v_scale", (torch.float16,), 3, dev)
    _need(cold_block_table, "cold_block_table", (torch.int32,), 2, dev)
    _need(seq_lens, "seq_lens", (torch.int32,), 1, dev)
    _need(cold_lens, "cold_lens", (torch.int32,), 1, dev)
    if q_pos is not None:
        _need(q_pos, "q_pos", (torch.int32,), 1, dev)
    B, D = q.shape[0], q.shape[-1]
    _, hot_window, Hkv, Dh = k_hot.shape
    NB, bs, Hkv2, W4 = k_cold.shape
    if Dh != D or Hkv2 != Hkv or W4 * 4 != D or tuple(v_hot.shape) != tuple(k_hot.shape) \
            or tuple(v_cold.shape) != tuple(k_cold.shape) or tuple(k_scale.shape) != (NB, bs, Hkv) \
            or tuple(v_scale.shape) != (NB, bs, Hkv) or k_hot.shape[0] != B:
        raise ValueError("tiered cache tensors disagree on shape")
    _rows(B, cold_block_table=cold_block_table, seq_lens=seq_lens, cold_lens=cold_lens, q_pos=q_pos)
    max_seq_len = _max_len(max_seq_len)
    _on_gpu(q, "q")
    p = _params(q, Hkv, D, bs, cold_block_table.shape[1], NB, max_seq_len, scale, causal,
                sliding_window, softcap, split_tokens, phases, out_dtype)
    ws = dattn_workspace_size(p, KIND_TIERED_INT8)
    out, lse, workspace = _outputs(q, out, lse, want_lse, workspace, ws, out_dtype, want_out)
    _check(lib().dattn_decode_tiered_int8(ctypes.byref(p), _ptr(q), _ptr(k_hot), _ptr(v_hot), hot_window,
                                          _ptr(k_cold), _ptr(v_cold), _ptr(k_scale), _ptr(v_scale),
                                          _ptr(cold_block_table), _ptr(seq_lens), _ptr(cold_lens), _ptr(q_pos),
                                          _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))
    return out, lse


def dattn_decode_tiered_int8_static(q, k_hot, v_hot, k_cold, v_cold, k_scale, v_scale, cold_block_table, seq_lens,
                                    cold_lens, *, q_pos=None, scale: float = 0.0, causal: bool = True,
                                    sliding_window: int = 0, softcap: float = 0.0,
                                    max_seq_len: Optional[int] = None, split_tokens: int = 0, out=None, lse=None,
                                    want_lse: bool = True, stream=None, phases: int = PHASE_ALL, out_dtype=None,
                                    want_out: bool = True):
    """dattn_decode_tiered_int8 with the split partials in the library's static
    device scratch (32 MiB per device) instead of a workspace: for callers that
    cannot allocate device memory.  Calls that overlap on one device race; out
    and lse are allocated here only when the caller does not pass them."""
    torch = _torch()
    dev = q.device
    _need(q, "q", (torch.float32, torch.float16), q.dim() if q.dim() in (3, 4) else 3, dev)
    _need(k_hot, "k_hot", (torch.float16,), 4, dev)
    _need(v_hot, "v_hot", (torch.float16,), 4, dev)
    _need(k_cold, "k_cold", (torch.int32, torch.uint32), 4, dev)
    _need(v_cold, "v_cold", (k_cold.dtype,), 4, dev)
    _need(k_scale, "k_scale", (torch.float16,), 3, dev)
    _need(v_scale, "v_scale", (torch.float16,), 3, dev)
    _need(cold_block_table, "cold_block_table", (torch.int32,), 2, dev)
    _need(seq_lens, "seq_lens", (torch.int32,), 1, dev)
    _need(cold_lens, "cold_lens", (torch.int32,), 1, dev)
    if q_pos is not None:
        _need(q_pos, "q_pos", (torch.int32,), 1, dev)
    B, D = q.shape[0], q.shape[-1]
    _, hot_window, Hkv, Dh = k_hot.shape
    NB, bs, Hkv2, W4 = k_cold.shape
    if Dh != D or Hkv2 != Hkv or W4 * 4 != D or tuple(v_hot.shape) != tuple(k_hot.shape) \
            or tuple(v_cold.shape) != tuple(k_cold.shape) or tuple(k_scale.shape) != (NB, bs, Hkv) \
            or tuple(v_scale.shape) != (NB, bs, Hkv) or k_hot.shape[0] != B:
        raise ValueError("tiered cache tensors disagree on shape")
    _rows(B, cold_block_table=cold_block_table, seq_lens=seq_lens, cold_lens=cold_lens, q_pos=q_pos)
    max_seq_len = _max_len(max_seq_len)
    _on_gpu(q, "q")
    p = _params(q, Hkv, D, bs, cold_block_table.shape[1], NB, max_seq_len, scale, causal, sliding_window, softcap,
                split_tokens, phases, out_dtype)
    out, lse, _ = _outputs(q, out, lse, want_lse, None, None, out_dtype, want_out)
    _check(lib().dattn_decode_tiered_int8_static(ctypes.byref(p), _ptr(q), _ptr(k_hot), _ptr(v_hot), hot_window,
                                                 _ptr(k_cold), _ptr(v_cold), _ptr(k_scale), _ptr(v_scale),
                                                 _ptr(cold_block_table), _ptr(seq_lens), _ptr(cold_lens),
                                                 _ptr(q_pos), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def dattn_decode_tiered_f16(q, k_hot, v_hot, k_cold, v_cold, cold_block_table, seq_lens, cold_lens, *, q_pos=None,
                            scale: float = 0.0, causal: bool = True, sliding_window: int = 0, softcap: float = 0.0,
                            max_seq_len: Optional[int] = None, split_tokens: int = 0, out=None, lse=None,
                            want_lse: bool = True, workspace=None, stream=None, phases: int = PHASE_ALL,
                            out_dtype=None, want_out: bool = True):
    """Decode attention over an f16 paged cold pool + f16 hot ring; returns (out, lse).
    q [B, Qn, H, D] asks for Qn queries per sequence, as for dattn_decode_paged."""
    torch = _torch()
    dev = q.device
    _need(q, "q", (torch.float32, torch.float16), q.dim() if q.dim() in (3, 4) else 3, dev)
    _need(k_hot, "k_hot", (torch.float16,), 4, dev)
    _need(v_hot, "v_hot", (torch.float16,), 4, dev)
    _need(k_cold, "k_cold", (torch.float16,), 4, dev)
    _need(v_cold, "v_cold", (torch.float16,), 4, dev)
    _need(cold_block_table, "cold_block_table", (torch.int32,), 2, dev)
    _need(seq_lens, "seq_lens", (torch.int32,), 1, dev)
    _need(cold_lens, "cold_lens", (torch.int32,), 1, dev)
    if q_pos is not None:
        _need(q_pos, "q_pos", (torch.int32,), 1, dev)
    B, D = q.shape[0], q.shape[-1]
    _, hot_window, Hkv, Dh = k_hot.shape
    NB, bs, Hkv2, Dc = k_cold.shape
    if Dh != D or Dc != D or Hkv2 != Hkv or tuple(v_hot.shape) != tuple(k_hot.shape) \
            or tuple(v_cold.shape) != tuple(k_cold.shape) or k_hot.shape[0] != B:
        raise ValueError("tiered cache tensors disagree on shape")
    _rows(B, cold_block_table=cold_block_table, seq_lens=seq_lens, cold_lens=cold_lens, q_pos=q_pos)
    max_seq_len = _max_len(max_seq_len)
    _on_gpu(q, "q")
    p = _params(q, Hkv, D, bs, cold_block_table.shape[1], NB, max_seq_len, scale, causal,
                sliding_window, softcap, split_tokens, phases, out_dtype)
    ws = dattn_workspace_size(p, KIND_TIERED_F16)
    out, lse, workspace = _outputs(q, out, lse, want_lse, workspace, ws, out_dtype, want_out)
    _check(lib().dattn_decode_tiered_f16(ctypes.byref(p), _ptr(q), _ptr(k_hot), _ptr(v_hot), hot_window,
                                         _ptr(k_cold), _ptr(v_cold), _ptr(cold_block_table), _ptr(seq_lens),
                                         _ptr(cold_lens), _ptr(q_pos), _ptr(out), _ptr(lse), _ptr(workspace),
                                         workspace.numel(), _stream(stream)))
    return out, lse


def dattn_decode_ring_f16(q, k_ring, v_ring, seq_lens, *, q_pos=None, scale: float = 0.0, causal: bool = True,
                          softcap: float = 0.0, max_seq_len: Optional[int] = None, split_tokens: int = 0, out=None,
                          lse=None, want_lse: bool = True, workspace=None, stream=None, phases: int = PHASE_ALL,
                          out_dtype=None, want_out: bool = True):
    """Decode attention over a sliding-window ring [B, W, Hkv, D] f16 (the window is W,
    the ring's slot count); returns (out, lse).  q [B, Qn, H, D] asks for Qn queries
    per sequence, as for dattn_decode_paged."""
    torch = _torch()
    dev = q.device
    _need(q, "q", (torch.float32, torch.float16), q.dim() if q.dim() in (3, 4) else 3, dev)
    _need(k_ring, "k_ring", (torch.float16,), 4, dev)
    _need(v_ring, "v_ring", (torch.float16,), 4, dev)
    _need(seq_lens, "seq_lens", (torch.int32,), 1, dev)
    if q_pos is not None:
        _need(q_pos, "q_pos", (torch.int32,), 1, dev)
    B, D = q.shape[0], q.shape[-1]
    Bk, W, Hkv, Dk = k_ring.shape
    if Bk != B or Dk != D or tuple(v_ring.shape) != tuple(k_ring.shape):
        raise ValueError("ring tensors disagree on shape")
    _rows(B, seq_lens=seq_lens, q_pos=q_pos)
    max_seq_len = _max_len(max_seq_len)
    _on_gpu(q, "q")
    p = _params(q, Hkv, D, 1, 1, 1, max_seq_len, scale, causal, W, softcap, split_tokens,
                phases, out_dtype)
    ws = dattn_workspace_size(p, KIND_RING_F16)
    out, lse, workspace = _outputs(q, out, lse, want_lse, workspace, ws, out_dtype, want_out)
    _check(lib().dattn_decode_ring_f16(ctypes.byref(p), _ptr(q), _ptr(k_ring), _ptr(v_ring), _ptr(seq_lens),
                                       _ptr(q_pos), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                       _stream(stream)))
    return out, lse


def dattn_append_tiered_int8(k_new, v_new, k_hot, v_hot, k_cold, v_cold, k_scale, v_scale, cold_block_table,
                             seq_lens, cold_lens, *, stream=None):
    """Append one token per sequence (k_new, v_new [B, Hkv, D] f16) to a tiered cache in place,
    quantising the oldest hot token into the cold tier when the ring is full; seq_lens and
    cold_lens (device int32) advance in place."""
    torch = _torch()
    dev = k_new.device
    _need(k_new, "k_new", (torch.float16,), 3, dev)
    _need(v_new, "v_new", (torch.float16,), 3, dev)
    _need(k_hot, "k_hot", (torch.float16,), 4, dev)
    _need(v_hot, "v_hot", (torch.float16,), 4, dev)
    _need(k_cold, "k_cold", (torch.int32, torch.uint32), 4, dev)
    _need(v_cold, "v_cold", (k_cold.dtype,), 4, dev)
    _need(k_scale, "k_scale", (torch.float16,), 3, dev)
    _need(v_scale, "v_scale", (torch.float16,), 3, dev)
    _need(cold_block_table, "cold_block_table", (torch.int32,), 2, dev)
    _need(seq_lens, "seq_lens", (torch.int32,), 1, dev)
    _need(cold_lens, "cold_lens", (torch.int32,), 1, dev)
    B, Hkv, D = k_new.shape
    _, hot_window, Hkv2, Dh = k_hot.shape
    NB, bs, Hkv3, W4 = k_cold.shape
    if tuple(v_new.shape) != (B, Hkv, D) or k_hot.shape[0] != B or Hkv2 != Hkv or Dh != D or Hkv3 != Hkv \
            or W4 * 4 != D or tuple(v_hot.shape) != tuple(k_hot.shape) or tuple(v_cold.shape) != tuple(k_cold.shape) \
            or tuple(k_scale.shape) != (NB, bs, Hkv) or tuple(v_scale.shape) != (NB, bs, Hkv) \
            or cold_block_table.shape[0] != B or seq_lens.shape[0] != B or cold_lens.shape[0] != B:
        raise ValueError("tiered cache tensors disagree on shape")
    _on_gpu(k_new, "k_new")
    p = DattnParams(B, Hkv, Hkv, D, 0.0, 0, 0, 0.0, bs, cold_block_table.shape[1], NB, 0, 0, 0)
    _check(lib().dattn_append_tiered_int8(ctypes.byref(p), _ptr(k_new), _ptr(v_new), _ptr(k_hot), _ptr(v_hot),
                                          hot_window, _ptr(k_cold), _ptr(v_cold), _ptr(k_scale), _ptr(v_scale),
                                          _ptr(cold_block_table), _ptr(seq_lens), _ptr(cold_lens),
                                          _stream(stream)))


def dattn_decode_block_sparse(q, k_cache, v_cache, block_table, seq_lens, sparse_block: int, row_ptr, col_idx, *,
                              q_pos=None, scale: float = 0.0, causal: bool = True, sliding_window: int = 0,
                              softcap: float = 0.0, max_seq_len: Optional[int] = None, split_tokens: int = 0,
                              out=None, lse=None, want_lse: bool = True, workspace=None, stream=None,
                              phases: int = PHASE_ALL, out_dtype=None, want_out: bool = True):
    """Decode attention over the paged f16 cache restricted by per-head CSR block masks;
    q [B, Qn, H, D] gives Qn queries per sequence, each with its own CSR row."""
    torch = _torch()
    dev = q.device
    _need(q, "q", (torch.float32, torch.float16), q.dim() if q.dim() in (3, 4) else 3, dev)
    _need(k_cache, "k_cache", (torch.float16,), 4, dev)
    _need(v_cache, "v_cache", (torch.float16,), 4, dev)
    _need(block_table, "block_table", (torch.int32,), 2, dev)
    _need(seq_lens, "seq_lens", (torch.int32,), 1, dev)
    _need(row_ptr, "row_ptr", (torch.int32,), 2, dev)
    _need(col_idx, "col_idx", (torch.int32,), 2, dev)
    if q_pos is not None:
        _need(q_pos, "q_pos", (torch.int32,), 1, dev)
    NB, bs, Hkv, D = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or q.shape[-1] != D:
        raise ValueError("k_cache, v_cache and q disagree on shape")
    if row_ptr.shape[0] != col_idx.shape[0]:
        raise ValueError("row_ptr and col_idx must have one row per layout")
    _rows(q.shape[0], block_table=block_table, seq_lens=seq_lens, q_pos=q_pos)
    max_seq_len = _max_len(max_seq_len)
    _on_gpu(q, "q")
    p = _params(q, Hkv, D, bs, block_table.shape[1], NB, max_seq_len, scale, causal,
                sliding_window, softcap, split_tokens, phases, out_dtype)
    ws = dattn_workspace_size(p, KIND_BLOCK_SPARSE, sparse_block)
    out, lse, workspace = _outputs(q, out, lse, want_lse, workspace, ws, out_dtype, want_out)
    _check(lib().dattn_decode_block_sparse(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                           _ptr(block_table), _ptr(seq_lens), _ptr(q_pos), int(sparse_block),
                                           row_ptr.shape[0], _ptr(row_ptr), row_ptr.shape[1], _ptr(col_idx),
                                           col_idx.shape[1], _ptr(out), _ptr(lse), _ptr(workspace),
                                           workspace.numel(), _stream(stream)))
    return out, lse


def dattn_append_ring_f16(k_new, v_new, k_ring, v_ring, seq_lens, *, stream=None):
    """Append one token per sequence (k_new, v_new [B, Hkv, D] f16) to a window ring
    [B, W, Hkv, D] in place, at slot seq_len mod W; seq_lens (device int32) advance in place."""
    torch = _torch()
    dev = k_new.device
    _need(k_new, "k_new", (torch.float16,), 3, dev)
    _need(v_new, "v_new", (torch.float16,), 3, dev)
    _need(k_ring, "k_ring", (torch.float16,), 4, dev)
    _need(v_ring, "v_ring", (torch.float16,), 4, dev)
    _need(seq_lens, "seq_lens", (torch.int32,), 1, dev)
    B, Hkv, D = k_new.shape
    if tuple(v_new.shape) != (B, Hkv, D) or tuple(v_ring.shape) != tuple(k_ring.shape) or k_ring.shape[0] != B \
            or k_ring.shape[2] != Hkv or k_ring.shape[3] != D or seq_lens.shape[0] != B:
        raise ValueError("ring tensors disagree on shape")
    _on_gpu(k_new, "k_new")
    p = DattnParams(B, Hkv, Hkv, D, 0.0, 0, int(k_ring.shape[1]), 0.0, 1, 1, 1, 0, 0, 0)
    _check(lib().dattn_append_ring_f16(ctypes.byref(p), _ptr(k_new), _ptr(v_new), _ptr(k_ring), _ptr(v_ring),
                                       _ptr(seq_lens), _stream(stream)))


def dattn_stream_read(src, sink, *, stream=None):
    """Measurement helper: stream-read the bytes of the contiguous GPU tensor `src`
    (sink: a 1-element int32 GPU tensor) -- the measured read ceiling."""
    torch = _torch()
    _need(sink, "sink", (torch.int32,), 1, src.device)
    _on_gpu(src, "src")
    if not src.is_contiguous() or src.device.type != "cuda":
        raise ValueError("src must be a contiguous GPU tensor")
    _check(lib().dattn_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)))
