"""CPU checks of the C-ABI library: it loads, exports what include/dattn.h
declares, lays out dattn_params as the binding does, and rejects every bad
argument the host can see with the documented code before touching HIP."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dattn.h")

dk = pytest.importorskip("int8_quantized_kv_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dk.library_path):
        pytest.skip("libdattn.so not built")
    return dk.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dattn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dattn_decode_paged", "dattn_decode_tiered_int8", "dattn_decode_tiered_f16", "dattn_decode_ring_f16",
              "dattn_decode_block_sparse",
              "dattn_append_tiered_int8", "dattn_append_ring_f16", "dattn_workspace_size", "dattn_last_error",
              "dattn_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", dk.library_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dattn_[a-z0-9_]+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_params_layout_matches_the_header(tmp_path):
    fields = [f[0] for f in dk.DattnParams._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "dattn.h"\nint main(void){\n'
                   + "".join(f'printf("%zu\\n", offsetof(dattn_params, {f}));\n' for f in fields)
                   + 'printf("%zu\\n", sizeof(dattn_params));\nreturn 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [getattr(dk.DattnParams, f).offset for f in fields] + [ctypes.sizeof(dk.DattnParams)]
    assert got == want


def test_fastdiv_is_exact(tmp_path):
    src = tmp_path / "fd.cpp"
    src.write_text(r'''
#include "fastdiv.h"
#include <cstdio>
#include <random>
int main() {
  std::mt19937_64 r(7); long bad = 0;
  for (uint32_t d = 1; d < 3000; ++d) {
    auto f = dattn::make_fastdiv(d);
    for (int k = 0; k < 500; ++k) { uint32_t x = (uint32_t)(r() & 0x7fffffff); bad += dattn::fdiv(x, f) != x / d; }
    for (uint32_t x = 0; x < 4 * d + 5; ++x) bad += dattn::fdiv(x, f) != x / d || dattn::fmod_(x, f) != x % d;
    for (uint32_t x = 0x7fffffff - 2 * d; x < 0x7fffffff; ++x) bad += dattn::fdiv(x, f) != x / d;
  }
  for (int k = 0; k < 100000; ++k) {
    uint32_t d = (uint32_t)(r() % 0x7fffffff) + 1, x = (uint32_t)(r() & 0x7fffffff);
    auto f = dattn::make_fastdiv(d); bad += dattn::fdiv(x, f) != x / d;
  }
  printf("%ld\n", bad); return bad != 0;
}''')
    exe = tmp_path / "fd"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "int8_quantized_kv_amd", "csrc"), str(src),
                    "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "0"


def good_params(**kw):
    p = dict(num_seqs=2, num_heads=8, num_kv_heads=2, head_dim=128, scale=0.0, causal=1, sliding_window=0,
             softcap=0.0, block_size=16, max_blocks_per_seq=8, num_blocks=16, max_seq_len=100, split_tokens=0,
             phases=0, out_dtype=0)
    p.update(kw)
    return dk.DattnParams(**p)


def ws_size(lib, p, kind=0, sb=0):
    n = ctypes.c_size_t(0)
    rc = lib.dattn_workspace_size(ctypes.byref(p) if p is not None else None, kind, sb, ctypes.byref(n))
    return rc, n.value, lib.dattn_last_error().decode()


BAD = [
    (dict(num_seqs=-1), dk.ERR_INVALID, "num_seqs"),
    (dict(num_heads=0), dk.ERR_INVALID, "num_heads"),
    (dict(num_heads=6, num_kv_heads=4), dk.ERR_INVALID, "multiple"),
    (dict(num_heads=32, num_kv_heads=2), dk.ERR_UNSUPPORTED, "GQA"),
    (dict(num_heads=6, num_kv_heads=2), dk.ERR_UNSUPPORTED, "GQA"),
    (dict(head_dim=96), dk.ERR_UNSUPPORTED, "head_dim"),
    (dict(scale=float("nan")), dk.ERR_INVALID, "scale"),
    (dict(softcap=float("inf")), dk.ERR_INVALID, "softcap"),
    (dict(causal=2), dk.ERR_INVALID, "causal"),
    (dict(sliding_window=-3), dk.ERR_INVALID, "sliding_window"),
    (dict(block_size=0), dk.ERR_INVALID, "block_size"),
    (dict(max_blocks_per_seq=0), dk.ERR_INVALID, "max_blocks_per_seq"),
    (dict(num_blocks=0), dk.ERR_INVALID, "num_blocks"),
    (dict(max_seq_len=-1), dk.ERR_INVALID, "max_seq_len"),
    (dict(max_seq_len=129), dk.ERR_INVALID, "exceeds"),
    (dict(split_tokens=24), dk.ERR_INVALID, "split_tokens"),
    (dict(split_tokens=-16), dk.ERR_INVALID, "split_tokens"),
    (dict(phases=7), dk.ERR_INVALID, "phases"),
    (dict(out_dtype=2), dk.ERR_INVALID, "out_dtype"),
    (dict(num_seqs=70000), dk.ERR_UNSUPPORTED, "num_seqs"),
    (dict(query_len=-1), dk.ERR_INVALID, "query_len"),
    (dict(query_len=33), dk.ERR_UNSUPPORTED, "128"),           # 33 queries x group 4 = 132 rows
    (dict(query_len=129, num_heads=2, num_kv_heads=2), dk.ERR_UNSUPPORTED, "128"),
]


@pytest.mark.parametrize("kw,code,word", BAD)
def test_workspace_size_rejects(lib, kw, code, word):
    rc, _, msg = ws_size(lib, good_params(**kw))
    assert rc == code and word in msg, (rc, msg)


def test_workspace_size_null_arguments(lib):
    rc, _, msg = ws_size(lib, None)
    assert rc == dk.ERR_INVALID and "NULL" in msg
    assert lib.dattn_workspace_size(ctypes.byref(good_params()), 0, 0, None) == dk.ERR_INVALID
    rc, _, msg = ws_size(lib, good_params(), kind=9)
    assert rc == dk.ERR_INVALID and "kind" in msg


def test_workspace_size_values(lib):
    # the library-chosen split (split_tokens = 0) also sizes the balanced schedule's slots
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # slots: one resident round of at most 4096 waves, i.e. 4096 / Hkv workers per kv-head group, plus B
    for hkv, n_heads in ((2, 8), (1, 8), (8, 32)):
        rc, n0, _ = ws_size(lib, good_params(num_kv_heads=hkv, num_heads=n_heads))
        slots = 4096 // hkv + 2
        assert rc == 0 and n0 == up(slots * n_heads * 128 * 4) + up(slots * n_heads * 8) + up(5 * 4), hkv
    rc, n, _ = ws_size(lib, good_params(split_tokens=32))
    assert rc == 0
    S, B, H, D = 4, 2, 8, 128          # ceil(100 / 32) splits
    acc = B * H * S * D * 4
    ml = B * H * S * 8
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert n == up(acc) + up(ml)
    # the tiered table only maps the cold prefix: max_seq_len may exceed it
    assert ws_size(lib, good_params(max_seq_len=500), kind=dk.KIND_TIERED_INT8)[0] == 0
    assert ws_size(lib, good_params(max_seq_len=500), kind=dk.KIND_TIERED_F16)[0] == 0
    assert ws_size(lib, good_params(), kind=dk.KIND_TIERED_F16)[1] == ws_size(lib, good_params(),
                                                                              kind=dk.KIND_TIERED_INT8)[1]
    # multi-query: slots and rows grow with the row blocks (query_len * group / 16 waves per kv head)
    for qn, hkv, n_heads in ((32, 2, 8), (8, 8, 32), (128, 1, 1)):
        rc, n0, _ = ws_size(lib, good_params(num_kv_heads=hkv, num_heads=n_heads, query_len=qn))
        slots = 4096 // (hkv * -(-qn * n_heads // hkv // 16)) + 2
        rows = slots * n_heads * qn
        assert rc == 0 and n0 == up(rows * 128 * 4) + up(rows * 8) + up(5 * 4), (qn, hkv)
    assert ws_size(lib, good_params(query_len=32), kind=dk.KIND_BLOCK_SPARSE, sb=32)[0] == 0
    assert ws_size(lib, good_params(query_len=33), kind=dk.KIND_BLOCK_SPARSE, sb=32)[0] == dk.ERR_UNSUPPORTED
    # sparse: sparse_block must be a positive multiple of block_size
    assert ws_size(lib, good_params(), kind=dk.KIND_BLOCK_SPARSE, sb=24)[0] == dk.ERR_INVALID
    assert ws_size(lib, good_params(), kind=dk.KIND_BLOCK_SPARSE, sb=32)[0] == 0


def test_decode_calls_validate_before_any_hip_call(lib):
    p = good_params()
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced: every call below fails validation
    # bad dtype
    rc = lib.dattn_decode_paged(ctypes.byref(p), fake, fake, fake, 5, fake, fake, None, fake, None, fake, 1 << 20, None)
    assert rc == dk.ERR_INVALID and "kv_dtype" in dk.dattn_last_error()
    # NULL input
    rc = lib.dattn_decode_paged(ctypes.byref(p), None, fake, fake, dk.F16, fake, fake, None, fake, None, fake, 1 << 20,
                                None)
    assert rc == dk.ERR_INVALID and "NULL" in dk.dattn_last_error()
    # workspace too small / NULL / misaligned
    rc = lib.dattn_decode_paged(ctypes.byref(p), fake, fake, fake, dk.F16, fake, fake, None, fake, None, fake, 16, None)
    assert rc == dk.ERR_WORKSPACE and "smaller" in dk.dattn_last_error()
    rc = lib.dattn_decode_paged(ctypes.byref(p), fake, fake, fake, dk.F16, fake, fake, None, fake, None, None, 1 << 20,
                                None)
    assert rc == dk.ERR_WORKSPACE
    rc = lib.dattn_decode_paged(ctypes.byref(p), fake, fake, fake, dk.F16, fake, fake, None, fake, None, P(0x1004),
                                1 << 40, None)
    assert rc == dk.ERR_WORKSPACE and "aligned" in dk.dattn_last_error()
    # tiered: hot_window
    rc = lib.dattn_decode_tiered_int8(ctypes.byref(p), fake, fake, fake, 0, fake, fake, fake, fake, fake, fake, fake,
                                      None, fake, None, fake, 1 << 20, None)
    assert rc == dk.ERR_INVALID and "hot_window" in dk.dattn_last_error()
    # sparse: layouts / strides
    for args, word in (((64, 0, fake, 5, fake, 5), "num_layouts"), ((64, 2, fake, 1, fake, 5), "row_stride"),
                       ((64, 2, fake, 5, fake, 0), "col_stride"), ((20, 2, fake, 5, fake, 5), "sparse_block")):
        rc = lib.dattn_decode_block_sparse(ctypes.byref(p), fake, fake, fake, fake, fake, None, *args, fake, None,
                                           fake, 1 << 20, None)
        assert rc == dk.ERR_INVALID and word in dk.dattn_last_error()
    # tiered f16: hot_window, NULL cold pool
    rc = lib.dattn_decode_tiered_f16(ctypes.byref(p), fake, fake, fake, 0, fake, fake, fake, fake, fake, None, fake,
                                     None, fake, 1 << 20, None)
    assert rc == dk.ERR_INVALID and "hot_window" in dk.dattn_last_error()
    rc = lib.dattn_decode_tiered_f16(ctypes.byref(p), fake, fake, fake, 16, None, fake, fake, fake, fake, None, fake,
                                     None, fake, 1 << 20, None)
    assert rc == dk.ERR_INVALID and "NULL" in dk.dattn_last_error()
    # window ring: needs a window (its slot count); pool fields are ignored
    for kw, word in ((dict(sliding_window=0), "sliding_window"), (dict(sliding_window=64, head_dim=80), "head_dim")):
        pr = good_params(**kw)
        rc = lib.dattn_decode_ring_f16(ctypes.byref(pr), fake, fake, fake, fake, None, fake, None, fake, 1 << 20, None)
        assert rc in (dk.ERR_INVALID, dk.ERR_UNSUPPORTED) and word in dk.dattn_last_error(), kw
    pr = good_params(sliding_window=64, block_size=0, num_blocks=0, max_blocks_per_seq=0, max_seq_len=5000)
    rc, n, _ = ws_size(lib, pr, kind=dk.KIND_RING_F16)
    assert rc == 0 and n > 0
    rc = lib.dattn_decode_ring_f16(ctypes.byref(pr), fake, None, fake, fake, None, fake, None, fake, 1 << 30, None)
    assert rc == dk.ERR_INVALID and "NULL" in dk.dattn_last_error()
    # combine-only phase does not need the inputs, but needs out or lse
    pc = good_params(phases=dk.PHASE_COMBINE)
    rc = lib.dattn_decode_paged(ctypes.byref(pc), None, None, None, dk.F16, None, None, None, None, None, fake,
                                1 << 20, None)
    assert rc == dk.ERR_INVALID and "out and lse" in dk.dattn_last_error()
    # out_dtype is checked on every entry point
    po = good_params(out_dtype=3)
    rc = lib.dattn_decode_paged(ctypes.byref(po), fake, fake, fake, dk.F16, fake, fake, None, fake, None, fake,
                                1 << 20, None)
    assert rc == dk.ERR_INVALID and "out_dtype" in dk.dattn_last_error()


def test_empty_batch_is_a_no_op(lib):
    p = good_params(num_seqs=0)
    rc = lib.dattn_decode_paged(ctypes.byref(p), None, None, None, dk.F16, None, None, None, None, None, None, 0, None)
    assert rc == 0 and dk.dattn_last_error() == ""


def test_binding_refuses_host_tensors(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros((1, 4, 64), dtype=torch.float32)
    k = torch.zeros((1, 16, 2, 64), dtype=torch.float16)
    bt = torch.zeros((1, 1), dtype=torch.int32)
    sl = torch.ones((1,), dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        dk.dattn_decode_paged(q, k, k, bt, sl, max_seq_len=1)
    with pytest.raises(TypeError):
        dk.dattn_decode_paged(q.double(), k, k, bt, sl, max_seq_len=1)


def _host_decode_args(B=2, H=4, Hkv=2, D=64, bs=16, nb=4, mb=2, hw=16):
    """Host tensors of consistent shapes for every decode wrapper (never launched:
    the wrappers check shapes before they look at the device)."""
    torch = pytest.importorskip("torch")
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)  # noqa: E731
    f16 = lambda *s: torch.zeros(s, dtype=torch.float16)  # noqa: E731
    return dict(q=torch.zeros((B, H, D), dtype=torch.float32), k_cache=f16(nb, bs, Hkv, D), block_table=i32(B, mb),
                seq_lens=i32(B), cold_lens=i32(B), q_pos=i32(B), k_hot=f16(B, hw, Hkv, D),
                k_cold=i32(nb, bs, Hkv, D // 4), k_scale=f16(nb, bs, Hkv), k_cold16=f16(nb, bs, Hkv, D),
                k_ring=f16(B, hw, Hkv, D), row_ptr=i32(4, 3), col_idx=i32(4, 8))


def _decode_calls(a):
    """name -> (callable taking the per-sequence arrays as keywords)."""
    def paged(block_table, seq_lens, q_pos, **_):
        return dk.dattn_decode_paged(a["q"], a["k_cache"], a["k_cache"], block_table, seq_lens, q_pos=q_pos,
                                     max_seq_len=16)

    def tiered(block_table, seq_lens, q_pos, cold_lens, **_):
        return dk.dattn_decode_tiered_int8(a["q"], a["k_hot"], a["k_hot"], a["k_cold"], a["k_cold"], a["k_scale"],
                                           a["k_scale"], block_table, seq_lens, cold_lens, q_pos=q_pos,
                                           max_seq_len=16)

    def tiered_f16(block_table, seq_lens, q_pos, cold_lens, **_):
        return dk.dattn_decode_tiered_f16(a["q"], a["k_hot"], a["k_hot"], a["k_cold16"], a["k_cold16"], block_table,
                                          seq_lens, cold_lens, q_pos=q_pos, max_seq_len=16)

    def ring(seq_lens, q_pos, **_):
        return dk.dattn_decode_ring_f16(a["q"], a["k_ring"], a["k_ring"], seq_lens, q_pos=q_pos, max_seq_len=16)

    def sparse(block_table, seq_lens, q_pos, **_):
        return dk.dattn_decode_block_sparse(a["q"], a["k_cache"], a["k_cache"], block_table, seq_lens, 16,
                                            a["row_ptr"], a["col_idx"], q_pos=q_pos, max_seq_len=16)

    return dict(paged=(paged, ("block_table", "seq_lens", "q_pos")),
                tiered=(tiered, ("block_table", "seq_lens", "q_pos", "cold_lens")),
                tiered_f16=(tiered_f16, ("block_table", "seq_lens", "q_pos", "cold_lens")),
                ring=(ring, ("seq_lens", "q_pos")),
                sparse=(sparse, ("block_table", "seq_lens", "q_pos")))


def test_binding_checks_rows_per_sequence(lib):
    """A per-sequence array with fewer (or more) rows than q has sequences is
    refused before anything is enqueued; the kernels would read row b of it for
    every b < B.  With every shape right the call fails only on the device check
    (host tensors), so the row checks come first."""
    a = _host_decode_args()
    for name, (fn, arrays) in _decode_calls(a).items():
        good = {k: a[k] for k in ("block_table", "seq_lens", "q_pos", "cold_lens")}
        with pytest.raises(ValueError, match="GPU"):
            fn(**good)
        for arr in arrays:
            for rows in (1, 3):
                bad = dict(good)
                t = good[arr]
                bad[arr] = t.new_zeros((rows,) + tuple(t.shape[1:]))
                with pytest.raises(ValueError, match="rows"):
                    fn(**bad)


def test_binding_needs_max_seq_len(lib):
    """max_seq_len sizes the grid on the host; the binding never reads it from
    the device array (that would synchronise), so leaving it out is an error."""
    a = _host_decode_args()
    with pytest.raises(ValueError, match="max_seq_len"):
        dk.dattn_decode_paged(a["q"], a["k_cache"], a["k_cache"], a["block_table"], a["seq_lens"])
    with pytest.raises(ValueError, match="max_seq_len"):
        dk.dattn_decode_ring_f16(a["q"], a["k_ring"], a["k_ring"], a["seq_lens"])
    assert not hasattr(dk, "default_scale")


def test_append_validates_before_any_hip_call(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced: every call below fails validation or is empty
    args = [fake] * 4 + [8] + [fake] * 7 + [None]
    for kw, code, word in ((dict(head_dim=96), dk.ERR_UNSUPPORTED, "head_dim"),
                           (dict(num_kv_heads=0), dk.ERR_INVALID, "num_kv_heads"),
                           (dict(block_size=0), dk.ERR_INVALID, "block_size"),
                           (dict(num_blocks=0), dk.ERR_INVALID, "num_blocks"),
                           (dict(num_seqs=-1), dk.ERR_INVALID, "num_seqs")):
        p = good_params(**kw)
        rc = lib.dattn_append_tiered_int8(ctypes.byref(p), *args)
        assert rc == code and word in dk.dattn_last_error(), kw
    p = good_params()
    bad_hw = list(args)
    bad_hw[4] = 0
    rc = lib.dattn_append_tiered_int8(ctypes.byref(p), *bad_hw)
    assert rc == dk.ERR_INVALID and "hot_window" in dk.dattn_last_error()
    null = list(args)
    null[7] = None
    rc = lib.dattn_append_tiered_int8(ctypes.byref(p), *null)
    assert rc == dk.ERR_INVALID and "NULL" in dk.dattn_last_error()
    p0 = good_params(num_seqs=0)
    rc = lib.dattn_append_tiered_int8(ctypes.byref(p0), *([None] * 4 + [8] + [None] * 8))
    assert rc == 0 and dk.dattn_last_error() == ""


def test_ring_append_validates_before_any_hip_call(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced: every call below fails validation or is empty
    for kw, code, word in ((dict(sliding_window=0), dk.ERR_INVALID, "sliding_window"),
                           (dict(sliding_window=8, head_dim=96), dk.ERR_UNSUPPORTED, "head_dim"),
                           (dict(sliding_window=8, num_kv_heads=0), dk.ERR_INVALID, "num_kv_heads")):
        p = good_params(**kw)
        rc = lib.dattn_append_ring_f16(ctypes.byref(p), fake, fake, fake, fake, fake, None)
        assert rc == code and word in dk.dattn_last_error(), kw
    p = good_params(sliding_window=8)
    rc = lib.dattn_append_ring_f16(ctypes.byref(p), fake, fake, None, fake, fake, None)
    assert rc == dk.ERR_INVALID and "NULL" in dk.dattn_last_error()
    rc = lib.dattn_append_ring_f16(ctypes.byref(good_params(num_seqs=0, sliding_window=8)), None, None, None, None,
                                   None, None)
    assert rc == 0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_stream_read_validates(lib):
    P = ctypes.c_void_p
    assert lib.dattn_stream_read(None, 64, P(0x1000), None) == dk.ERR_INVALID
    assert lib.dattn_stream_read(P(0x1000), 60, P(0x1000), None) == dk.ERR_INVALID
    assert lib.dattn_stream_read(P(0x1004), 64, P(0x1000), None) == dk.ERR_INVALID
    assert lib.dattn_stream_read(P(0x1000), 0, P(0x1000), None) == 0
