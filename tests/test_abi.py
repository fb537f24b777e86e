"""CPU checks of the C ABI: libqsa.so loads, exports every function qsa.h
declares, and refuses bad arguments with the documented status before any
HIP call (so these run without a GPU; nothing here launches a kernel)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")
LIB = os.path.join(ROOT, "sparse_attention_block_qsa_amd", "libqsa.so")

OK, ARG, UNSUP, HIP, TOO_LARGE = 0, 1, 2, 3, 4
A16 = 0x10000          # a fake, 16-byte aligned device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):   # CPU container only: hipcc cross-compiles gfx950
        import importlib.util  # by path: the package __init__ needs the built library
        spec = importlib.util.spec_from_file_location(
            "_qsa_build_lib", os.path.join(ROOT, "sparse_attention_block_qsa_amd", "build_lib.py"))
        build_lib = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(build_lib)
        build_lib.build()
    L = ctypes.CDLL(LIB)
    vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    L.qsa_block_scores.argtypes = [vp, i64, vp, i64, vp, i64, i32, i32, i32, i32, i64, i32, u32,
                                   vp]
    L.qsa_select_topk.argtypes = [vp, i64, i64, i32, i32, vp, i64, vp, vp]
    L.qsa_convert_f32_f16.argtypes = [vp, vp, i64, vp]
    L.qsa_select_phase.argtypes = [vp, vp, i64, vp, i64, vp, i64, vp, i64, vp, i32, i32, i32,
                                   i32, i64, i32, i32, i64, u32, vp]
    L.qsa_select_phase_noalloc.argtypes = [vp, vp, i64, vp, i64, vp, i64, vp, i32, i32, i32,
                                           i32, i64, i32, i32, i64, u32, vp]
    L.qsa_block_keys.argtypes = [vp, i64, vp, i64, i32, i32, i64, i32, vp]
    L.qsa_sparse_attention.argtypes = [vp, i64, vp, vp, i64, vp, i64, vp, i64, i32, i32, i32,
                                       i32, i64, i32, i32, vp, i64, vp]
    L.qsa_sparse_attention_ws_floats.argtypes = [i32, i32, i32, i32, i32, i32]
    L.qsa_sparse_attention_ws_floats.restype = ctypes.c_int64
    L.qsa_status_string.argtypes = [ctypes.c_int]
    L.qsa_status_string.restype = ctypes.c_char_p
    return L


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["qsa_abi_version", "qsa_status_string", "qsa_convert_f32_f16", "qsa_block_keys",
         "qsa_block_scores", "qsa_select_topk", "qsa_select_phase", "qsa_select_phase_noalloc",
         "qsa_sparse_attention", "qsa_sparse_attention_ws_floats"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    hdr = open(HEADER).read()
    ver = int(re.search(r"#define QSA_ABI_VERSION (\d+)", hdr).group(1))
    assert lib.qsa_abi_version() == ver
    for st in (OK, ARG, UNSUP, HIP, TOO_LARGE, 99):
        assert lib.qsa_status_string(st)


def test_python_binding_exports_match_header():
    src = open(os.path.join(ROOT, "sparse_attention_block_qsa_amd", "__init__.py")).read()
    names = re.search(r"EXPORTS = \((.*?)\)", src, re.S).group(1)
    assert sorted(re.findall(r'"(qsa_\w+)"', names)) == declared_functions()


def scores_call(lib, **kw):
    a = dict(q16=A16, qts=8 * 128, kblk=A16, khs=64 * 128, scores=A16, ld_s=64, G=1, nq=256,
             H=8, D=128, n_kv=4096, bs=64, flags=0)
    a.update(kw)
    return lib.qsa_block_scores(a["q16"], a["qts"], a["kblk"], a["khs"], a["scores"], a["ld_s"],
                                a["G"], a["nq"], a["H"], a["D"], a["n_kv"], a["bs"], a["flags"],
                                None)


@pytest.mark.parametrize("kw,want", [
    (dict(D=96), UNSUP), (dict(D=32), UNSUP), (dict(H=0), UNSUP), (dict(H=17), UNSUP),
    (dict(bs=0), UNSUP), (dict(n_kv=-1), ARG), (dict(G=-1), ARG), (dict(nq=-5), ARG),
    (dict(q16=None), ARG), (dict(kblk=None), ARG), (dict(scores=None), ARG),
    (dict(ld_s=63), ARG), (dict(qts=8 * 128 - 8), ARG), (dict(khs=63 * 128), ARG),
    (dict(q16=A16 + 2), UNSUP), (dict(qts=8 * 128 + 4), UNSUP), (dict(kblk=A16 + 8), UNSUP),
    (dict(khs=64 * 128 + 2), UNSUP), (dict(scores=A16 + 2), UNSUP),
    (dict(ld_s=1 << 62, nq=8), ARG),          # row extent overflows int64
    (dict(flags=2), ARG), (dict(flags=4), ARG), (dict(flags=0xFFFFFFFF), ARG),   # only QSA_FORCE_TAIL is defined
    (dict(flags=3, n_kv=0), ARG),             # refused before the empty early return
])
def test_block_scores_refusals(lib, kw, want):
    assert scores_call(lib, **kw) == want


@pytest.mark.parametrize("kw", [dict(n_kv=0), dict(nq=0), dict(G=0),
                                dict(n_kv=0, q16=None, kblk=None, scores=None)])
def test_block_scores_empty_is_ok_without_launch(lib, kw):
    assert scores_call(lib, **kw) == OK


def topk_call(lib, **kw):
    a = dict(scores=A16, ld_s=2048, rows=256, nb=2048, k=64, ids=A16, ld_ids=64, vals=None)
    a.update(kw)
    return lib.qsa_select_topk(a["scores"], a["ld_s"], a["rows"], a["nb"], a["k"], a["ids"],
                               a["ld_ids"], a["vals"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(k=65), UNSUP), (dict(k=-1), ARG), (dict(rows=-1), ARG), (dict(nb=-1), ARG),
    (dict(ids=None), ARG), (dict(scores=None), ARG), (dict(ld_ids=63), ARG),
    (dict(ld_s=2047), ARG), (dict(ids=A16 + 2), UNSUP), (dict(vals=A16 + 1), UNSUP),
])
def test_select_topk_refusals(lib, kw, want):
    assert topk_call(lib, **kw) == want


@pytest.mark.parametrize("kw", [dict(k=0), dict(rows=0), dict(k=0, ids=None)])
def test_select_topk_empty_is_ok_without_launch(lib, kw):
    assert topk_call(lib, **kw) == OK


def test_convert_refusals(lib):
    assert lib.qsa_convert_f32_f16(A16, A16, -1, None) == ARG
    assert lib.qsa_convert_f32_f16(None, A16, 8, None) == ARG
    assert lib.qsa_convert_f32_f16(A16, None, 8, None) == ARG
    assert lib.qsa_convert_f32_f16(A16 + 1, A16, 8, None) == UNSUP
    assert lib.qsa_convert_f32_f16(None, None, 0, None) == OK


def phase_call(lib, **kw):
    a = dict(q32=A16, q16=A16, qts=8 * 128, kblk=A16, khs=64 * 128, ws=A16, ld_s=64, ids=A16,
             ld_ids=16, vals=None, G=1, nq=256, H=8, D=128, n_kv=4096, bs=64, k=16, q_chunk=0,
             flags=0)
    a.update(kw)
    return lib.qsa_select_phase(a["q32"], a["q16"], a["qts"], a["kblk"], a["khs"], a["ws"],
                                a["ld_s"], a["ids"], a["ld_ids"], a["vals"], a["G"], a["nq"],
                                a["H"], a["D"], a["n_kv"], a["bs"], a["k"], a["q_chunk"],
                                a["flags"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q_chunk=-1), ARG), (dict(k=65), UNSUP), (dict(D=80), UNSUP), (dict(ids=None), ARG),
    (dict(q16=None, q32=None), ARG), (dict(ws=None), ARG), (dict(ld_ids=8), ARG),
    (dict(ld_s=10), ARG), (dict(q32=A16 + 2), UNSUP), (dict(H=20), UNSUP),
    # no fp16 buffer: the fp32 rows must be 16-byte aligned
    (dict(q16=None, q32=A16 + 4), UNSUP), (dict(q16=None, qts=8 * 128 + 2), UNSUP),
    # QSA_FORCE_TAIL | QSA_FUSED_SELECT | QSA_STREAM_SELECT only
    (dict(flags=8), ARG), (dict(flags=1 << 31), ARG),
])
def test_select_phase_refusals(lib, kw, want):
    assert phase_call(lib, **kw) == want


def test_select_phase_empty_is_ok_without_launch(lib):
    assert phase_call(lib, nq=0) == OK
    assert phase_call(lib, G=0) == OK


def noalloc_call(lib, **kw):
    a = dict(q32=A16, q16=None, qts=8 * 128, kblk=A16, khs=64 * 128, ids=A16, ld_ids=16,
             vals=None, G=1, nq=256, H=8, D=128, n_kv=4096, bs=64, k=16, q_chunk=0, flags=0)
    a.update(kw)
    return lib.qsa_select_phase_noalloc(a["q32"], a["q16"], a["qts"], a["kblk"], a["khs"],
                                        a["ids"], a["ld_ids"], a["vals"], a["G"], a["nq"],
                                        a["H"], a["D"], a["n_kv"], a["bs"], a["k"],
                                        a["q_chunk"], a["flags"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(q_chunk=-1), ARG), (dict(G=-1), ARG), (dict(nq=-1), ARG), (dict(n_kv=-1), ARG),
    (dict(bs=0), UNSUP), (dict(flags=8), ARG),
    # one query's score row (17M blocks of one token, 68 MB) exceeds the 64 MiB array
    (dict(n_kv=17 << 20, bs=1, khs=(17 << 20) * 128), TOO_LARGE),
    # four KV heads of 2049 blocks fit 2016 queries per pass, not 4096
    (dict(G=4, qts=4 * 1024, n_kv=131077, khs=2049 * 128, nq=4096, q_chunk=4096), TOO_LARGE),
])
def test_select_phase_noalloc_refusals(lib, kw, want):
    assert noalloc_call(lib, **kw) == want


def test_select_phase_noalloc_empty_is_ok_without_launch(lib):
    assert noalloc_call(lib, nq=0) == OK
    assert noalloc_call(lib, G=0) == OK


def keys_call(lib, **kw):
    a = dict(k=A16, ts=4 * 128, kb=A16, khs=2049 * 128, G=4, D=128, n_kv=131077, bs=64)
    a.update(kw)
    return lib.qsa_block_keys(a["k"], a["ts"], a["kb"], a["khs"], a["G"], a["D"], a["n_kv"],
                              a["bs"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(G=-1), ARG), (dict(n_kv=-1), ARG), (dict(ts=-8), ARG), (dict(bs=0), UNSUP),
    (dict(bs=8193), UNSUP), (dict(D=96), UNSUP), (dict(k=None), ARG), (dict(kb=None), ARG),
    (dict(ts=4 * 128 - 8), ARG), (dict(khs=2048 * 128), ARG), (dict(k=A16 + 2), UNSUP),
    (dict(ts=4 * 128 + 4), UNSUP), (dict(kb=A16 + 8), UNSUP), (dict(khs=2049 * 128 + 2), UNSUP),
    (dict(ts=1 << 50), ARG),                  # token extent overflows int64
])
def test_block_keys_refusals(lib, kw, want):
    assert keys_call(lib, **kw) == want


@pytest.mark.parametrize("kw", [dict(G=0), dict(n_kv=0), dict(n_kv=0, k=None, kb=None)])
def test_block_keys_empty_is_ok_without_launch(lib, kw):
    assert keys_call(lib, **kw) == OK


def attn_call(lib, **kw):
    a = dict(q=A16, qts=8 * 128, k=A16, v=A16, kvts=128, ids=A16, ld=64, out=A16, ots=8 * 128,
             G=1, nq=256, H=8, D=128, n_kv=131072, bs=64, kk=64, ws=None, wsf=0)
    a.update(kw)
    return lib.qsa_sparse_attention(a["q"], a["qts"], a["k"], a["v"], a["kvts"], a["ids"], a["ld"],
                                    a["out"], a["ots"], a["G"], a["nq"], a["H"], a["D"],
                                    a["n_kv"], a["bs"], a["kk"], a["ws"], a["wsf"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(G=-1), ARG), (dict(nq=-1), ARG), (dict(n_kv=-1), ARG), (dict(kk=-1), ARG),
    (dict(bs=0), UNSUP), (dict(D=96), UNSUP), (dict(H=0), UNSUP), (dict(H=17), UNSUP),
    (dict(kk=65, ld=65), UNSUP), (dict(q=None), ARG), (dict(out=None), ARG), (dict(ids=None), ARG),
    (dict(k=None), ARG), (dict(v=None), ARG), (dict(qts=8 * 128 - 1), ARG),
    (dict(ots=8 * 128 - 1), ARG), (dict(ld=63), ARG), (dict(kvts=127), ARG),
    (dict(k=A16 + 2), UNSUP), (dict(v=A16 + 8), UNSUP), (dict(kvts=132), UNSUP),
    (dict(q=A16 + 1), UNSUP), (dict(out=A16 + 2), UNSUP), (dict(ids=A16 + 2), UNSUP),
    (dict(ots=1 << 60), ARG), (dict(wsf=-1), ARG), (dict(ws=A16 + 2, wsf=100), UNSUP),
    # past QSA_ATTENTION_MAX_KV_STRIDE (64 value rows addressed with 32-bit offsets)
    (dict(kvts=(16 << 20) + 8, n_kv=4), UNSUP),
])
def test_sparse_attention_refusals(lib, kw, want):
    assert attn_call(lib, **kw) == want


def test_sparse_attention_empty_is_ok_without_launch(lib):
    assert attn_call(lib, nq=0) == OK
    assert attn_call(lib, G=0) == OK


def test_sparse_attention_workspace_size(lib):
    f = lib.qsa_sparse_attention_ws_floats
    # a decode step: 8 rows of 64 chunks split 8 ways (one chunk per wave)
    assert f(8, 1, 8, 128, 64, 64) == 8 * 8 * 8 * 130
    # 256 rows fill the CUs alone: no split
    assert f(1, 256, 8, 128, 64, 64) == 0
    # 64 rows: four workgroups each
    assert f(1, 64, 8, 128, 64, 64) == 4 * 64 * 8 * 130
    # enough rows to fill the chip alone: no split, no workspace
    assert f(4, 16384, 8, 128, 64, 64) == 0
    assert f(0, 1, 8, 128, 64, 64) == 0 and f(1, 1, 17, 128, 64, 64) == 0
