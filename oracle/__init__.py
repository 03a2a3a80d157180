"""fp64 CPU oracle for decode attention (paged, tiered int8/f16, block-sparse)
and for the tiered cache's quantise-on-evict write path.

TEST INFRASTRUCTURE ONLY: the product library never imports this package.
Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, two-pass
softmax, OpenMP over (sequence, head) pairs); this module compiles it with gcc
and marshals numpy arrays into it.  Every entry takes an optional list of flat
pair indices ``b * num_heads + h`` so that very large workloads can be checked
on a sample of heads; the outputs are then ``[len(pairs), D]`` and
``[len(pairs)]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, F16 = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
             _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


class _Params(ctypes.Structure):
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
        ("query_len", ctypes.c_int32),
    ]


@dataclass
class Params:
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float = 0.0
    causal: int = 1
    sliding_window: int = 0
    softcap: float = 0.0
    block_size: int = 16
    max_blocks_per_seq: int = 0
    num_blocks: int = 0
    query_len: int = 1

    def c(self) -> _Params:
        return _Params(self.num_seqs, self.num_heads, self.num_kv_heads, self.head_dim,
                       self.scale, self.causal, self.sliding_window, self.softcap,
                       self.block_size, self.max_blocks_per_seq, self.num_blocks, self.query_len)


_libs = {}


def load(path: str = _LIB):
    """ctypes handle of a compiled oracle library (the default one unless a path is given)."""
    if path in _libs:
        return _libs[path]
    if path == _LIB and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f64.restype = ctypes.c_double
    lib.orc_int8_lane.argtypes = [ctypes.c_uint32, i32]
    lib.orc_int8_lane.restype = i32
    lib.orc_key_visible.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, i32, i32]
    lib.orc_key_visible.restype = i32
    lib.orc_ring_slot.argtypes = [ctypes.c_int64, i32]
    lib.orc_ring_slot.restype = ctypes.c_int64
    lib.orc_max_threads.restype = ctypes.c_int
    lib.orc_decode_paged.argtypes = [ctypes.POINTER(_Params), P, P, P, i32, P, P, P, P, i32, i32, P, P]
    lib.orc_decode_tiered_int8.argtypes = [ctypes.POINTER(_Params), P, P, P, i32, P, P, P, P, P, P, P, P,
                                           P, i32, i32, P, P]
    lib.orc_decode_block_sparse.argtypes = [ctypes.POINTER(_Params), P, P, P, P, P, P, i32, i32, P, i32, P,
                                            i32, P, i32, i32, P, P]
    lib.orc_decode_tiered_f16.argtypes = [ctypes.POINTER(_Params), P, P, P, i32, P, P, P, P, P, P, P, i32, i32,
                                          P, P]
    lib.orc_decode_ring_f16.argtypes = [ctypes.POINTER(_Params), P, P, P, P, P, P, i32, i32, P, P]
    for f in (lib.orc_decode_paged, lib.orc_decode_tiered_int8, lib.orc_decode_tiered_f16, lib.orc_decode_ring_f16,
              lib.orc_decode_block_sparse):
        f.restype = ctypes.c_int
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_quantize_row.argtypes = [P, i32, P, P]
    lib.orc_quantize_row.restype = None
    lib.orc_append_tiered_int8.argtypes = [ctypes.POINTER(_Params), P, P, P, P, i32, P, P, P, P, P, P, P]
    lib.orc_append_tiered_int8.restype = ctypes.c_int
    lib.orc_append_ring_f16.argtypes = [ctypes.POINTER(_Params), P, P, P, P, P]
    lib.orc_append_ring_f16.restype = ctypes.c_int
    _libs[path] = lib
    return lib


def _load(lib=None):
    if lib is not None:
        return lib
    # a planted-mistake build of the oracle can be swapped in for the pin tests
    return load(os.environ.get("ORACLE_LIB_OVERRIDE", _LIB))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _arr(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _pairs(p: Params, pairs):
    if pairs is None:
        return None, p.num_seqs * max(1, p.query_len) * p.num_heads
    pa = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32))
    return pa, int(pa.size)


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def f16_to_f64(bits: int, lib=None) -> float:
    return _load(lib).orc_f16_to_f64(bits)


def int8_lane(word: int, lane: int, lib=None) -> int:
    return _load(lib).orc_int8_lane(word, lane)


def key_visible(t: int, q: int, L: int, causal: int, window: int, lib=None) -> bool:
    return bool(_load(lib).orc_key_visible(t, q, L, causal, window))


def ring_slot(t: int, hot_window: int, lib=None) -> int:
    return _load(lib).orc_ring_slot(t, hot_window)


def max_threads() -> int:
    return _load().orc_max_threads()


def decode_paged(p: Params, q, k_cache, v_cache, block_table, seq_lens, q_pos=None, pairs=None, nthreads=0, lib=None):
    """Paged cache [num_blocks, block_size, Hkv, D] of float32 or float16."""
    lib = _load(lib)
    q = _arr(q, np.float32)
    if k_cache.dtype == np.float16:
        dt = F16
        k_cache = _arr(k_cache, np.float16)
        v_cache = _arr(v_cache, np.float16)
    else:
        dt = F32
        k_cache = _arr(k_cache, np.float32)
        v_cache = _arr(v_cache, np.float32)
    bt = _arr(block_table, np.int32)
    sl = _arr(seq_lens, np.int32)
    qp = _arr(q_pos, np.int32)
    pa, n = _pairs(p, pairs)
    out = np.zeros((n, p.head_dim), np.float64)
    lse = np.zeros((n,), np.float64)
    cp = p.c()
    rc = lib.orc_decode_paged(ctypes.byref(cp), _ptr(q), _ptr(k_cache), _ptr(v_cache), dt, _ptr(bt), _ptr(sl),
                              _ptr(qp), _ptr(pa), n, nthreads, _ptr(out), _ptr(lse))
    _check(rc, "orc_decode_paged")
    return out, lse


def decode_tiered_int8(p: Params, q, k_hot, v_hot, hot_window, k_cold, v_cold, k_scale, v_scale,
                       cold_block_table, seq_lens, cold_lens, q_pos=None, pairs=None, nthreads=0, lib=None):
    """Hot ring [B, hot_window, Hkv, D] f16; cold pool [Nc, bs, Hkv, D/4] u32 with f16 scales [Nc, bs, Hkv]."""
    lib = _load(lib)
    q = _arr(q, np.float32)
    kh = _arr(k_hot, np.float16)
    vh = _arr(v_hot, np.float16)
    kc = _arr(k_cold, np.uint32)
    vc = _arr(v_cold, np.uint32)
    ks = _arr(k_scale, np.float16)
    vs = _arr(v_scale, np.float16)
    bt = _arr(cold_block_table, np.int32)
    sl = _arr(seq_lens, np.int32)
    cl = _arr(cold_lens, np.int32)
    qp = _arr(q_pos, np.int32)
    pa, n = _pairs(p, pairs)
    out = np.zeros((n, p.head_dim), np.float64)
    lse = np.zeros((n,), np.float64)
    cp = p.c()
    rc = lib.orc_decode_tiered_int8(ctypes.byref(cp), _ptr(q), _ptr(kh), _ptr(vh), int(hot_window), _ptr(kc),
                                    _ptr(vc), _ptr(ks), _ptr(vs), _ptr(bt), _ptr(sl), _ptr(cl), _ptr(qp),
                                    _ptr(pa), n, nthreads, _ptr(out), _ptr(lse))
    _check(rc, "orc_decode_tiered_int8")
    return out, lse


def decode_tiered_f16(p: Params, q, k_hot, v_hot, hot_window, k_cold, v_cold, cold_block_table, seq_lens,
                      cold_lens, q_pos=None, pairs=None, nthreads=0, lib=None):
    """Hot ring [B, hot_window, Hkv, D] f16; cold pool [Nc, bs, Hkv, D] f16 read through cold_block_table."""
    lib = _load(lib)
    q = _arr(q, np.float32)
    kh = _arr(k_hot, np.float16)
    vh = _arr(v_hot, np.float16)
    kc = _arr(k_cold, np.float16)
    vc = _arr(v_cold, np.float16)
    bt = _arr(cold_block_table, np.int32)
    sl = _arr(seq_lens, np.int32)
    cl = _arr(cold_lens, np.int32)
    qp = _arr(q_pos, np.int32)
    pa, n = _pairs(p, pairs)
    out = np.zeros((n, p.head_dim), np.float64)
    lse = np.zeros((n,), np.float64)
    cp = p.c()
    rc = lib.orc_decode_tiered_f16(ctypes.byref(cp), _ptr(q), _ptr(kh), _ptr(vh), int(hot_window), _ptr(kc),
                                   _ptr(vc), _ptr(bt), _ptr(sl), _ptr(cl), _ptr(qp), _ptr(pa), n, nthreads,
                                   _ptr(out), _ptr(lse))
    _check(rc, "orc_decode_tiered_f16")
    return out, lse


def decode_ring_f16(p: Params, q, k_ring, v_ring, seq_lens, q_pos=None, pairs=None, nthreads=0, lib=None):
    """Ring [B, W, Hkv, D] f16 with W = p.sliding_window: token t at slot t mod W, the last W resident."""
    lib = _load(lib)
    q = _arr(q, np.float32)
    kr = _arr(k_ring, np.float16)
    vr = _arr(v_ring, np.float16)
    sl = _arr(seq_lens, np.int32)
    qp = _arr(q_pos, np.int32)
    pa, n = _pairs(p, pairs)
    out = np.zeros((n, p.head_dim), np.float64)
    lse = np.zeros((n,), np.float64)
    cp = p.c()
    rc = lib.orc_decode_ring_f16(ctypes.byref(cp), _ptr(q), _ptr(kr), _ptr(vr), _ptr(sl), _ptr(qp), _ptr(pa), n,
                                 nthreads, _ptr(out), _ptr(lse))
    _check(rc, "orc_decode_ring_f16")
    return out, lse


def decode_block_sparse(p: Params, q, k_cache, v_cache, block_table, seq_lens, sparse_block, num_layouts,
                        row_ptr, col_idx, q_pos=None, pairs=None, nthreads=0, lib=None):
    """CSR row_ptr [NL, R+1], col_idx [NL, col_stride]; paged f16 cache."""
    lib = _load(lib)
    q = _arr(q, np.float32)
    kc = _arr(k_cache, np.float16)
    vc = _arr(v_cache, np.float16)
    bt = _arr(block_table, np.int32)
    sl = _arr(seq_lens, np.int32)
    qp = _arr(q_pos, np.int32)
    rp = _arr(row_ptr, np.int32)
    ci = _arr(col_idx, np.int32)
    pa, n = _pairs(p, pairs)
    out = np.zeros((n, p.head_dim), np.float64)
    lse = np.zeros((n,), np.float64)
    cp = p.c()
    rc = lib.orc_decode_block_sparse(ctypes.byref(cp), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(sl), _ptr(qp),
                                     int(sparse_block), int(num_layouts), _ptr(rp), int(rp.shape[1]), _ptr(ci),
                                     int(ci.shape[1]), _ptr(pa), n, nthreads, _ptr(out), _ptr(lse))
    _check(rc, "orc_decode_block_sparse")
    return out, lse


def run(case, pairs=None, nthreads=0, lib=None):
    """Dispatch on a synthetic case object (attributes as laid out by the input generators)."""
    p = Params(**case.params)
    if case.kind == "paged":
        return decode_paged(p, case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens, case.q_pos,
                            pairs, nthreads, lib)
    if case.kind == "tiered":
        return decode_tiered_int8(p, case.q, case.k_hot, case.v_hot, case.hot_window, case.k_cold, case.v_cold,
                                  case.k_scale, case.v_scale, case.cold_block_table, case.seq_lens, case.cold_lens,
                                  case.q_pos, pairs, nthreads, lib)
    if case.kind == "tiered_f16":
        return decode_tiered_f16(p, case.q, case.k_hot, case.v_hot, case.hot_window, case.k_cold, case.v_cold,
                                 case.cold_block_table, case.seq_lens, case.cold_lens, case.q_pos, pairs, nthreads,
                                 lib)
    if case.kind == "ring":
        return decode_ring_f16(p, case.q, case.k_hot, case.v_hot, case.seq_lens, case.q_pos, pairs, nthreads, lib)
    if case.kind == "sparse":
        return decode_block_sparse(p, case.q, case.k_cache, case.v_cache, case.block_table, case.seq_lens,
                                   case.sparse_block, case.num_layouts, case.row_ptr, case.col_idx, case.q_pos,
                                   pairs, nthreads, lib)
    raise ValueError(case.kind)


def f32_to_f16(x: float, lib=None) -> int:
    """IEEE binary16 bits of the f32 value x, rounded to nearest even."""
    return int(_load(lib).orc_f32_to_f16(float(np.float32(x))))


def quantize_row(x_f16, lib=None):
    """One row of D f16 values -> (D/4 packed u32 words, f16 scale bits)."""
    lib = _load(lib)
    x = _arr(np.asarray(x_f16).view(np.float16).reshape(-1), np.float16)
    D = int(x.size)
    words = np.zeros(D // 4, np.uint32)
    sc = np.zeros(1, np.uint16)
    lib.orc_quantize_row(_ptr(x), D, _ptr(words), _ptr(sc))
    return words, int(sc[0])


def append_tiered_int8(p: Params, k_new, v_new, k_hot, v_hot, hot_window, k_cold, v_cold, k_scale, v_scale,
                       cold_block_table, seq_lens, cold_lens, lib=None):
    """Append one token per sequence (k_new, v_new [B, Hkv, D] f16) to a tiered cache.
    Works on copies and returns (k_hot, v_hot, k_cold, v_cold, k_scale, v_scale, seq_lens, cold_lens)."""
    lib = _load(lib)
    kn = _arr(k_new, np.float16)
    vn = _arr(v_new, np.float16)
    kh = np.array(_arr(k_hot, np.float16), copy=True)
    vh = np.array(_arr(v_hot, np.float16), copy=True)
    kc = np.array(_arr(k_cold, np.uint32), copy=True)
    vc = np.array(_arr(v_cold, np.uint32), copy=True)
    ks = np.array(_arr(k_scale, np.float16), copy=True)
    vs = np.array(_arr(v_scale, np.float16), copy=True)
    bt = _arr(cold_block_table, np.int32)
    sl = np.array(_arr(seq_lens, np.int32), copy=True)
    cl = np.array(_arr(cold_lens, np.int32), copy=True)
    cp = p.c()
    rc = lib.orc_append_tiered_int8(ctypes.byref(cp), _ptr(kn), _ptr(vn), _ptr(kh), _ptr(vh), int(hot_window),
                                    _ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs), _ptr(bt), _ptr(sl), _ptr(cl))
    _check(rc, "orc_append_tiered_int8")
    return kh, vh, kc, vc, ks, vs, sl, cl


def append_ring_f16(p: Params, k_new, v_new, k_ring, v_ring, seq_lens, lib=None):
    """One token per sequence into a window ring [B, W, Hkv, D] f16 (W = p.sliding_window),
    at slot seq_len mod W; returns copies (k_ring, v_ring, seq_lens)."""
    lib = _load(lib)
    kn, vn = _arr(k_new, np.float16), _arr(v_new, np.float16)
    kr, vr = np.array(k_ring, np.float16, copy=True), np.array(v_ring, np.float16, copy=True)
    sl = np.array(seq_lens, np.int32, copy=True)
    cp = p.c()
    _check(lib.orc_append_ring_f16(ctypes.byref(cp), _ptr(kn), _ptr(vn), _ptr(kr), _ptr(vr), _ptr(sl)),
           "orc_append_ring_f16")
    return kr, vr, sl
