"""C-ABI checks that need no GPU: the library loads, exports every function that
include/flashprefill.h declares, and rejects invalid arguments on the host before
anything is enqueued (these calls never reach a kernel launch)."""
import ctypes
import math
import os
import re

import pytest

from block_sparse_long_pooled_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashprefill.h")

# A fake but 16-byte aligned "device" address: validation never dereferences pointers.
P = 0x10000
EINVAL, EUNSUP = _lib.FP_EINVAL, _lib.FP_EUNSUPPORTED


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(fp_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_hot_path():
    names = declared_functions()
    for n in ["fp_discover", "fp_threshold_compact", "fp_sparse_attn", "fp_dense_attn",
              "fp_discover_paged", "fp_threshold_compact_varlen", "fp_sparse_attn_paged"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(_lib.EXPORTED)


def test_status_strings_and_helpers():
    lib = _lib.load()
    assert lib.fp_status_string(0) == b"FP_OK"
    assert lib.fp_status_string(1) == b"FP_EINVAL"
    assert lib.fp_abi_version() == _lib.ABI_VERSION
    assert lib.fp_num_blocks(131072, 128) == 1024
    assert lib.fp_num_blocks(1000, 128) == 8
    assert lib.fp_idx_capacity(32, 1024) == 32 * 1024 * 1025 // 2


def discover(**kw):
    a = dict(q=P, k=P, dtype=0, qs=None, ks=None, L=4096, hq=4, hkv=2, d=128, block=128,
             qst=512, qsh=128, kst=256, ksh=128, pq=P, pk=P, stream=None)
    a.update(kw)
    return _lib.status_of("fp_discover", a["q"], a["k"], a["dtype"], a["qs"], a["ks"], a["L"], a["hq"], a["hkv"],
                          a["d"], a["block"], a["qst"], a["qsh"], a["kst"], a["ksh"], a["pq"], a["pk"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=64), EUNSUP), (dict(block=64), EUNSUP), (dict(dtype=7), EUNSUP),
    (dict(hq=3, hkv=2), EINVAL), (dict(hkv=0), EINVAL), (dict(q=None), EINVAL), (dict(pk=None), EINVAL),
    (dict(q=P + 2), EINVAL), (dict(qst=511), EINVAL), (dict(ksh=-128), EINVAL), (dict(L=-1), EINVAL),
    (dict(dtype=1), EINVAL),  # fp8 without scales
    (dict(dtype=1, qs=P, ks=P, qst=520), EINVAL),  # fp8 rows need 16-element alignment
])
def test_discover_rejects(kw, code):
    assert discover(**kw) == code
    assert _lib.load().fp_last_error()


def select(**kw):
    a = dict(pq=P, pk=P, nb=32, hq=4, hkv=2, d=128, scale=1 / math.sqrt(128), alpha=0.1, ns=1, nl=2,
             idx=P, cnt=P, scores=None, stream=None)
    a.update(kw)
    return _lib.status_of("fp_threshold_compact", a["pq"], a["pk"], a["nb"], a["hq"], a["hkv"], a["d"],
                          a["scale"], a["alpha"], a["ns"], a["nl"], a["idx"], a["cnt"], a["scores"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(alpha=-0.1), EINVAL), (dict(alpha=float("nan")), EINVAL), (dict(alpha=float("inf")), EINVAL),
    (dict(nl=0), EINVAL), (dict(ns=-1), EINVAL), (dict(scale=0.0), EINVAL), (dict(idx=None), EINVAL),
    (dict(cnt=None), EINVAL), (dict(d=96), EUNSUP), (dict(hq=5, hkv=2), EINVAL), (dict(nb=-3), EINVAL),
    (dict(scores=P + 4), EINVAL),
])
def test_threshold_rejects(kw, code):
    assert select(**kw) == code


def attn(name="fp_sparse_attn", **kw):
    a = dict(q=P, k=P, v=P, dtype=0, qs=None, ks=None, vs=None, L=1024, hq=4, hkv=2, d=128, block=128,
             st=[512, 128, 256, 128, 256, 128, 512, 128], idx=P, cnt=P, scale=0.088, out=P, lse=None, stream=None)
    a.update(kw)
    args = [a["q"], a["k"], a["v"], a["dtype"], a["qs"], a["ks"], a["vs"], a["L"], a["hq"], a["hkv"], a["d"],
            a["block"], *a["st"]]
    if name in ("fp_sparse_attn", "fp_sparse_attn_grouped"):
        args += [a["idx"], a["cnt"]]
    elif name == "fp_sparse_attn_masked":
        args += [a["idx"]]
    args += [a["scale"], a["out"], a["lse"], a["stream"]]
    return _lib.status_of(name, *args)


@pytest.mark.parametrize("kw,code", [
    (dict(idx=None), EINVAL), (dict(out=None), EINVAL), (dict(v=P + 8), EINVAL),
    (dict(scale=-1.0), EINVAL), (dict(scale=float("nan")), EINVAL), (dict(dtype=1), EINVAL),
    (dict(st=[512, 128, 256, 128, 256, 128, 512, 4]), EINVAL), (dict(lse=P + 2), EINVAL),
    (dict(d=256), EUNSUP), (dict(hq=4, hkv=3), EINVAL),
])
def test_sparse_attn_rejects(kw, code):
    assert attn(**kw) == code


@pytest.mark.parametrize("kw,msg", [
    (dict(L=2**31 - 1, hq=2048, hkv=2), b"grid too large"),   # hq * nb work items in a 1-D grid
    (dict(hq=4097, hkv=1), b"too large"),
    (dict(st=[2**24, 128, 256, 128, 256, 128, 512, 128]), b"32-bit tile offsets"),  # Q stride
    (dict(st=[512, 128, 2**24, 128, 256, 128, 512, 128]), b"32-bit tile offsets"),  # K stride
])
def test_sparse_attn_size_limits(kw, msg):
    assert attn(**kw) == EINVAL and msg in _lib.load().fp_last_error()


def test_dense_attn_rejects():
    assert attn("fp_dense_attn", out=None) == EINVAL
    assert attn("fp_dense_attn", block=256) == EUNSUP


def test_mask_words():
    lib = _lib.load()
    assert [lib.fp_mask_words(n) for n in (0, 1, 31, 32, 33, 1024, 2048)] == [0, 1, 1, 1, 2, 32, 64]


def mask_select(**kw):
    a = dict(pq=P, pk=P, nb=32, hq=4, hkv=2, d=128, scale=1 / math.sqrt(128), alpha=0.1, ns=1, nl=2,
             mask=P, stream=None)
    a.update(kw)
    return _lib.status_of("fp_threshold_mask", a["pq"], a["pk"], a["nb"], a["hq"], a["hkv"], a["d"],
                          a["scale"], a["alpha"], a["ns"], a["nl"], a["mask"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), EINVAL), (dict(mask=P + 2), EINVAL), (dict(alpha=-1.0), EINVAL), (dict(nl=0), EINVAL),
    (dict(pq=None), EINVAL), (dict(d=64), EUNSUP), (dict(hq=3, hkv=2), EINVAL),
])
def test_threshold_mask_rejects(kw, code):
    assert mask_select(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(idx=None), EINVAL), (dict(idx=P + 2), EINVAL), (dict(out=None), EINVAL), (dict(dtype=1), EINVAL),
    (dict(block=64), EUNSUP), (dict(scale=0.0), EINVAL),
])
def test_sparse_attn_masked_rejects(kw, code):
    assert attn("fp_sparse_attn_masked", **kw) == code


def test_paged_rejects():
    lib = _lib.load()
    # page table given but max_pages smaller than ceil(max_seqlen / 128)
    rc = lib.fp_sparse_attn_paged(P, P, P, 0, None, None, None, P, 2, 1000, 1500, 12, 78, P, 3, 20, 4, 2, 128, 128,
                                  512, 128, 32768, 256, 128, 32768, 256, 128, 512, 128, P, P, 0.088, P, None, None)
    assert rc == EINVAL and b"max_pages" in lib.fp_last_error()
    # no cu_seqlens
    rc = lib.fp_discover_paged(P, P, 0, None, None, None, 2, 1000, 1500, 12, None, 0, 0, 4, 2, 128, 128,
                               512, 128, 0, 256, 128, P, P, None)
    assert rc == EINVAL
    # n_seqs out of range
    rc = lib.fp_threshold_compact_varlen(P, P, P, 0, 1000, 12, 78, 4, 2, 128, 0.088, 0.1, 1, 1, P, P, None)
    assert rc == EINVAL


def test_chunked_rejects():
    lib = _lib.load()
    # no query lengths
    rc = lib.fp_threshold_compact_chunked(P, P, None, P, 2, 300, 1000, 12, 16, 200, 4, 2, 128, 0.088, 0.1, 1, 1,
                                          P, P, None)
    assert rc == EINVAL and b"cu_seqlens_q" in lib.fp_last_error()
    # negative query extent
    rc = lib.fp_discover_chunked(P, P, 0, None, None, P, P, 2, 300, 1000, -1, 1500, 12, 16, None, 0, 0, 4, 2, 128,
                                 128, 512, 128, 0, 256, 128, P, P, None)
    assert rc == EINVAL
    # page table narrower than the key blocks
    rc = lib.fp_sparse_attn_chunked(P, P, P, 0, None, None, None, P, P, 2, 300, 1000, 400, 1500, 12, 16, 200,
                                    P, 3, 20, 4, 2, 128, 128, 512, 128, 32768, 256, 128, 32768, 256, 128, 512, 128,
                                    P, P, 0.088, P, None, None)
    assert rc == EINVAL and b"max_pages" in lib.fp_last_error()
    # bad head dimension
    rc = lib.fp_sparse_attn_chunked(P, P, P, 0, None, None, None, P, P, 2, 300, 1000, 400, 1500, 12, 16, 200,
                                    None, 0, 0, 4, 2, 64, 128, 512, 128, 0, 256, 128, 0, 256, 128, 512, 128,
                                    P, P, 0.088, P, None, None)
    assert rc == EUNSUP


def test_grouped_rejects():
    lib = _lib.load()
    assert lib.fp_union_compact(None, 32, 4, 2, P, P, None) == EINVAL
    assert lib.fp_union_compact(P + 2, 32, 4, 2, P, P, None) == EINVAL
    assert lib.fp_union_compact(P, 32, 5, 2, P, P, None) == EINVAL
    assert lib.fp_union_compact(P, 0, 4, 2, P, P, None) == _lib.FP_OK
    assert attn("fp_sparse_attn_grouped", idx=None) == EINVAL
    assert attn("fp_sparse_attn_grouped", d=64) == EUNSUP


def test_pool_and_mean_correct_reject():
    lib = _lib.load()
    assert lib.fp_pool(None, 0, None, 256, 2, 128, 128, 256, 128, P, None) == EINVAL
    assert lib.fp_pool(P, 1, None, 256, 2, 128, 128, 256, 128, P, None) == EINVAL  # fp8 without scale
    assert lib.fp_pool(P, 0, None, 256, 2, 64, 128, 256, 128, P, None) == EUNSUP
    assert lib.fp_pool(P, 0, None, 0, 2, 128, 128, 256, 128, P, None) == _lib.FP_OK
    ws = lib.fp_mean_correct_workspace_bytes(1024, 2)
    assert ws == 2 * 1 * 3 * 32 * 256  # 2 KV heads x 1 tile of 32 pooled keys x 24 KB
    assert lib.fp_mean_correct_workspace_bytes(-1, 2) == -1 and lib.fp_mean_correct_workspace_bytes(1024, 0) == -1
    args = [P, 0, None, P, P, 1024, 4, 2, 128, 128, 512, 128, 512, 128, P, P, 0.088, P, P, P, ws, None]
    # the pointers are fake, so only reject paths are exercised
    bad_lse = list(args); bad_lse[18] = None
    assert lib.fp_mean_correct(*bad_lse) == EINVAL and b"lse" in lib.fp_last_error()
    bad_pk = list(args); bad_pk[3] = None
    assert lib.fp_mean_correct(*bad_pk) == EINVAL
    bad_pk = list(args); bad_pk[4] = P + 8
    assert lib.fp_mean_correct(*bad_pk) == EINVAL and b"aligned" in lib.fp_last_error()
    bad_d = list(args); bad_d[8] = 96
    assert lib.fp_mean_correct(*bad_d) == EUNSUP
    bad_ws = list(args); bad_ws[19] = None
    assert lib.fp_mean_correct(*bad_ws) == EINVAL and b"workspace" in lib.fp_last_error()
    bad_ws = list(args); bad_ws[20] = ws - 1
    assert lib.fp_mean_correct(*bad_ws) == EINVAL and b"workspace" in lib.fp_last_error()
    too_long = list(args); too_long[5] = 65536 * 128 + 1
    too_long[20] = lib.fp_mean_correct_workspace_bytes(too_long[5], 2)
    assert lib.fp_mean_correct(*too_long) == EUNSUP


def test_mean_correct_noalloc_rejects():
    """The static-scratch variant rejects, before touching a GPU, calls whose tile
    images exceed its 8 MiB scratch, and the usual malformed arguments."""
    lib = _lib.load()
    args = [P, 0, None, P, P, 1024, 4, 2, 128, 128, 512, 128, 512, 128, P, P, 0.088, P, P, None]
    big = list(args); big[5] = 400 * 1024; big[7] = 4  # 4 KV heads x 98 tiles x 24 KB > 8 MiB
    assert lib.fp_mean_correct_workspace_bytes(big[5], 4) > 8 << 20
    assert lib.fp_mean_correct_noalloc(*big) == EUNSUP
    assert b"scratch" in lib.fp_last_error() and b"8388608" in lib.fp_last_error()
    bad_lse = list(args); bad_lse[18] = None
    assert lib.fp_mean_correct_noalloc(*bad_lse) == EINVAL and b"lse" in lib.fp_last_error()
    bad_d = list(args); bad_d[8] = 96
    assert lib.fp_mean_correct_noalloc(*bad_d) == EUNSUP
    empty = list(args); empty[5] = 0
    assert lib.fp_mean_correct_noalloc(*empty) == _lib.FP_OK


def test_mean_correct_varlen_and_pool_varlen_reject():
    lib = _lib.load()
    assert lib.fp_mean_correct_varlen_workspace_bytes(100, 3, 2) == 2 * (4 + 3) * 3 * 32 * 256
    assert lib.fp_mean_correct_varlen_workspace_bytes(-1, 3, 2) == -1
    assert lib.fp_mean_correct_varlen_workspace_bytes(10, 0, 2) == -1
    ws = lib.fp_mean_correct_varlen_workspace_bytes(20, 2, 2)
    args = [P, 0, None, P, P, P, 2, 1300, 2000, 20, 200, 4, 2, 128, 128, 512, 128, 512, 128, P, P, 0.088,
            P, P, P, ws, None]
    short = list(args); short[25] = ws - 1
    assert lib.fp_mean_correct_varlen(*short) == EINVAL and b"workspace" in lib.fp_last_error()
    no_cu = list(args); no_cu[5] = None
    assert lib.fp_mean_correct_varlen(*no_cu) == EINVAL
    no_lse = list(args); no_lse[23] = None
    assert lib.fp_mean_correct_varlen(*no_lse) == EINVAL
    empty = list(args); empty[8] = 0
    assert lib.fp_mean_correct_varlen(*empty) == _lib.FP_OK
    pargs = [P, 0, None, P, 2, 1300, 2000, 20, None, 0, 0, 2, 128, 128, 0, 256, 128, P, None]
    assert lib.fp_pool_varlen(*pargs[:17], None, None) == EINVAL  # no output
    bad = list(pargs); bad[3] = None
    assert lib.fp_pool_varlen(*bad) == EINVAL
    bad = list(pargs); bad[1] = 1  # fp8 without a scale
    assert lib.fp_pool_varlen(*bad) == EINVAL
    paged = list(pargs); paged[8] = P; paged[9] = 5; paged[10] = 8  # max_pages 5 < 11 blocks
    assert lib.fp_pool_varlen(*paged) == EINVAL and b"max_pages" in lib.fp_last_error()


def test_empty_inputs_are_a_no_op():
    """L = 0 validates and returns FP_OK without launching anything."""
    assert discover(L=0) == _lib.FP_OK
    assert select(nb=0) == _lib.FP_OK
    assert attn(L=0) == _lib.FP_OK
    assert mask_select(nb=0) == _lib.FP_OK
    assert attn("fp_sparse_attn_masked", L=0) == _lib.FP_OK
