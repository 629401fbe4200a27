"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import pytest

import decode_attention_11_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(["mla_status_string", "mla_decode_workspace_size", "mla_decode",
                                           "mla_merge_lse", "cp_local_slot", "mla_profile_attention_events",
                                           "mla_kv_write", "mla_decode_interleaved", "mla_decode_varlen",
                                           "mla_decode_fp8", "mla_kv_write_fp8", "mla_decode_noalloc",
                                           "mla_probe_mfma"])


def test_library_exports_every_declared_symbol():
    lib = mla.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(mla.exported_symbols()) == declared_functions()


def test_status_strings():
    lib = mla.load_library()
    assert lib.mla_status_string(0) == b"ok"
    assert lib.mla_status_string(1) == b"invalid argument"
    assert lib.mla_status_string(3) == b"HIP launch failure"
    assert lib.mla_status_string(99) == b"unknown status"


def _decode(**kw):
    lib = mla.load_library()
    a = dict(q=1, kv=1, bt=1, sl=1, gl=None, B=2, Q=1, H=16, nblk=4, bs=64, maxb=2, maxlen=128, W=1, r=0,
             causal=1, scale=0.1, base=0, out=1, lse=1, ws=1, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.mla_decode(a["q"], a["kv"], a["bt"], a["sl"], a["gl"], a["B"], a["Q"], a["H"], a["nblk"], a["bs"],
                          a["maxb"], a["maxlen"], a["W"], a["r"], a["causal"], ctypes.c_float(a["scale"]), a["base"],
                          a["out"], a["lse"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("bad", [
    dict(Q=0), dict(H=0), dict(B=-1), dict(r=1), dict(r=-1), dict(W=0), dict(W=8, r=8),
    dict(W=8, r=3, gl=None), dict(base=2), dict(causal=2), dict(scale=float("nan")), dict(scale=float("inf")),
    dict(bs=0), dict(nblk=0), dict(maxb=0), dict(maxlen=-1),
    dict(q=None), dict(kv=None), dict(bt=None), dict(sl=None), dict(out=None), dict(ws=None), dict(wsb=0),
])
def test_decode_rejects_bad_arguments(bad):
    assert _decode(**bad) == 1


def test_decode_empty_batch_is_a_noop():
    assert _decode(B=0, q=None, kv=None, out=None) == 0


def test_noncausal_dcp_needs_no_global():
    # non-causal draft blocks use the local length only; only the workspace check fails here
    assert _decode(W=2, r=1, causal=0, gl=None, wsb=0) == 1


def test_workspace_size():
    n1 = mla.mla_decode_workspace_size(64, 1, 16, 8192)
    assert n1 > 0
    assert mla.mla_decode_workspace_size(0, 1, 16, 8192) == 0
    assert mla.mla_decode_workspace_size(2, 0, 16, 100) == 0


def _merge(**kw):
    lib = mla.load_library()
    a = dict(parts=(ctypes.c_void_p * 2)(1, 1), lses=(ctypes.c_void_p * 2)(1, 1), n=2, rows=4, H=2, base=0,
             out=1, lse=1, stream=None)
    a.update(kw)
    return lib.mla_merge_lse(ctypes.cast(a["parts"], ctypes.c_void_p) if a["parts"] is not None else None,
                             ctypes.cast(a["lses"], ctypes.c_void_p) if a["lses"] is not None else None,
                             a["n"], a["rows"], a["H"], a["base"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("bad", [dict(n=0), dict(n=65), dict(rows=-1), dict(H=0), dict(base=5),
                                 dict(parts=None), dict(lses=None), dict(out=None),
                                 dict(parts=(ctypes.c_void_p * 2)(1, None))])
def test_merge_rejects_bad_arguments(bad):
    assert _merge(**bad) == 1


def _slot(**kw):
    lib = mla.load_library()
    a = dict(pos=1, nv=None, B=2, n=16, bt=1, maxb=4, bs=64, W=2, r=1, I=1, slots=1, stream=None)
    a.update(kw)
    return lib.cp_local_slot(a["pos"], a["nv"], a["B"], a["n"], a["bt"], a["maxb"], a["bs"], a["W"], a["r"],
                             a["I"], a["slots"], a["stream"])


@pytest.mark.parametrize("bad", [dict(B=-1), dict(n=-1), dict(maxb=0), dict(bs=0), dict(W=0), dict(r=2),
                                 dict(r=-1), dict(I=0), dict(bs=64, I=3), dict(pos=None), dict(bt=None),
                                 dict(slots=None)])
def test_slot_rejects_bad_arguments(bad):
    assert _slot(**bad) == 1


def test_slot_empty_is_a_noop():
    assert _slot(B=0, pos=None, bt=None, slots=None) == 0


def test_profile_events_need_both_or_neither():
    lib = mla.load_library()
    assert lib.mla_profile_attention_events(1, None) == 1
    assert lib.mla_profile_attention_events(None, 1) == 1
    assert lib.mla_profile_attention_events(None, None) == 0


def _kv_write(**kw):
    lib = mla.load_library()
    a = dict(rows=256, slots=256, n=4, cache=256, nblk=4, bs=64, stream=None)
    a.update(kw)
    return lib.mla_kv_write(a["rows"], a["slots"], a["n"], a["cache"], a["nblk"], a["bs"], a["stream"])


@pytest.mark.parametrize("bad", [dict(n=-1), dict(nblk=0), dict(bs=0), dict(rows=None), dict(slots=None),
                                 dict(cache=None), dict(rows=258), dict(cache=264)])
def test_kv_write_rejects_bad_arguments(bad):
    assert _kv_write(**bad) == 1


def test_kv_write_empty_is_a_noop():
    assert _kv_write(n=0, rows=None, slots=None, cache=None) == 0


def _decode_il(I, **kw):
    lib = mla.load_library()
    a = dict(q=1, kv=1, bt=1, sl=1, gl=1, B=2, Q=1, H=16, nblk=4, bs=64, maxb=2, maxlen=128, W=2, r=1,
             causal=1, scale=0.1, base=0, out=1, lse=1, ws=1, wsb=0, stream=None)
    a.update(kw)
    return lib.mla_decode_interleaved(a["q"], a["kv"], a["bt"], a["sl"], a["gl"], a["B"], a["Q"], a["H"], a["nblk"],
                                      a["bs"], a["maxb"], a["maxlen"], a["W"], a["r"], I, a["causal"],
                                      ctypes.c_float(a["scale"]), a["base"], a["out"], a["lse"], a["ws"], a["wsb"],
                                      a["stream"])


@pytest.mark.parametrize("I,kw", [(0, {}), (-2, {}), (1 << 29, dict(W=4, r=1)), (2, dict(r=2)), (2, dict(gl=None))])
def test_interleaved_decode_rejects_bad_arguments(I, kw):
    # every case fails a host check (the last ones also have a zero-size workspace)
    assert _decode_il(I, **kw) == 1


def test_varlen_decode_needs_token_offsets():
    lib = mla.load_library()
    args = [1, None, 4, 1, 1, 1, None, 2, 16, 4, 64, 2, 128, 1, 0, 1, 1, ctypes.c_float(0.1), 0, 1, 1, 1, 1 << 40, None]
    assert lib.mla_decode_varlen(*args) == 1          # no query_start_loc
    args[1] = 1
    args[2] = 0
    assert lib.mla_decode_varlen(*args) == 1          # max_q_len < 1



def _decode_fp8(kv_scale, **kw):
    lib = mla.load_library()
    a = dict(q=1, kv=1, bt=1, sl=1, gl=None, B=2, Q=1, H=16, nblk=4, bs=64, maxb=2, maxlen=128, W=1, r=0, I=1,
             causal=1, scale=0.1, base=0, out=1, lse=1, ws=1, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.mla_decode_fp8(a["q"], a["kv"], ctypes.c_float(kv_scale), a["bt"], a["sl"], a["gl"], a["B"], a["Q"],
                              a["H"], a["nblk"], a["bs"], a["maxb"], a["maxlen"], a["W"], a["r"], a["I"], a["causal"],
                              ctypes.c_float(a["scale"]), a["base"], a["out"], a["lse"], a["ws"], a["wsb"],
                              a["stream"])


@pytest.mark.parametrize("kv_scale,kw", [
    (0.0, {}), (-1.0, {}), (float("nan"), {}), (float("inf"), {}), (1e-3, dict(I=0)), (1e-3, dict(Q=0)),
    (1e-3, dict(kv=None)), (1e-3, dict(wsb=0)),
])
def test_fp8_decode_rejects_bad_arguments(kv_scale, kw):
    assert _decode_fp8(kv_scale, **kw) == 1


def test_fp8_decode_empty_batch_is_a_noop():
    assert _decode_fp8(0.5, B=0, q=None, kv=None, out=None) == 0


def _kv_write_fp8(kv_scale, n=4, rows=16, slots=16, cache=16, nblk=2, bs=64):
    return mla.load_library().mla_kv_write_fp8(rows, slots, n, ctypes.c_float(kv_scale), cache, nblk, bs, None)


@pytest.mark.parametrize("kv_scale,kw", [
    (0.0, {}), (-2.0, {}), (float("nan"), {}), (float("inf"), {}), (1.0, dict(n=-1)), (1.0, dict(nblk=0)),
    (1.0, dict(bs=0)), (1.0, dict(rows=None)), (1.0, dict(slots=None)), (1.0, dict(cache=None)),
    (1.0, dict(rows=8)), (1.0, dict(cache=8)),
])
def test_kv_write_fp8_rejects_bad_arguments(kv_scale, kw):
    assert _kv_write_fp8(kv_scale, **kw) == 1


def test_kv_write_fp8_empty_is_a_noop():
    assert _kv_write_fp8(0.5, n=0, rows=None, slots=None, cache=None) == 0


def _noalloc(**kw):
    lib = mla.load_library()
    a = dict(q=1, kv=1, bt=1, sl=1, gl=None, B=2, Q=1, H=16, nblk=4, bs=64, maxb=2, maxlen=128, W=1, r=0,
             causal=1, scale=0.1, base=0, out=1, lse=1, stream=None)
    a.update(kw)
    return lib.mla_decode_noalloc(a["q"], a["kv"], a["bt"], a["sl"], a["gl"], a["B"], a["Q"], a["H"], a["nblk"],
                                  a["bs"], a["maxb"], a["maxlen"], a["W"], a["r"], a["causal"],
                                  ctypes.c_float(a["scale"]), a["base"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("bad", [dict(Q=0), dict(H=0), dict(B=-1), dict(maxlen=-1),
                                 # more partial slots than the fixed array holds
                                 dict(B=4096, Q=16, H=128, maxlen=1 << 20), dict(B=64, Q=16, H=128, maxlen=1 << 18)])
def test_noalloc_rejects_bad_arguments_and_sizes_beyond_its_array(bad):
    assert _noalloc(**bad) == 1


def test_noalloc_array_size_is_the_documented_one():
    src = open(HEADER).read()
    assert "#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)96 * 1024 * 1024)" in src
    assert mla.NOALLOC_SCRATCH_BYTES == 96 * 1024 * 1024
    # the largest benchmark workload (B 16, q_len 16, H 128, 131072-key bound) fits
    assert mla.mla_decode_workspace_size(16, 16, 128, 131072) <= mla.NOALLOC_SCRATCH_BYTES


def test_probe_refuses_bad_sizes_without_launching():
    lib = mla.load_library()
    assert lib.mla_probe_mfma(0, 10, None, None) == 1
    assert lib.mla_probe_mfma(4, 0, None, None) == 1
    assert lib.mla_probe_mfma(4, 10, None, None) == 1  # NULL out
