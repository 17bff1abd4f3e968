"""The C-ABI library loads, exports every declared symbol, and rejects bad calls on
the host before touching a device (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcs.h")


def lib():
    from long_context_self_amd import lcs
    if not os.path.exists(lcs.lib_path()):
        pytest.skip("liblcs.so not built")
    return lcs, lcs.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lcs_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lcs, L = lib()
    names = declared_symbols()
    assert {"lcs_verify_attn", "lcs_select_topk", "lcs_sparse_draft_attn", "lcs_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert lcs.version().startswith("lcs ")


def fake_kv(lcs, **kw):
    d = dict(k=0x1000, v=0x2000, block_table=0x3000, num_pages=10, page_size=16, max_pages=4, Hkv=2, d=128)
    d.update(kw)
    return lcs.PagedKVDesc(**d)


def verify(lcs, L, kv, **kw):
    a = dict(q=0x4000, B=1, n_q=5, Hq=4, prefix_len=0x5000, max_len=40, tree=None, scale=0.1, r0=0, r1=4,
             out=0x6000, logits=0x7000, ld=40, lse=None, ws=0x8000, wsb=1 << 20)
    a.update(kw)
    return L.lcs_verify_attn(ctypes.byref(kv), a["q"], a["B"], a["n_q"], a["Hq"], a["prefix_len"], a["max_len"],
                             a["tree"], a["scale"], a["r0"], a["r1"], a["out"], a["logits"], a["ld"], a["lse"],
                             a["ws"], a["wsb"], None)


def test_verify_host_errors():
    lcs, L = lib()
    kv = fake_kv(lcs)
    assert verify(lcs, L, fake_kv(lcs, d=96)) == lcs.LCS_E_UNSUPPORTED
    assert b"head dim" in L.lcs_last_error()
    assert verify(lcs, L, fake_kv(lcs, page_size=12)) == lcs.LCS_E_UNSUPPORTED
    assert verify(lcs, L, fake_kv(lcs, k=0)) == lcs.LCS_E_ARG
    assert verify(lcs, L, kv, Hq=3) == lcs.LCS_E_SHAPE
    assert verify(lcs, L, kv, n_q=65) == lcs.LCS_E_UNSUPPORTED
    assert verify(lcs, L, kv, n_q=0) == lcs.LCS_E_SHAPE
    assert verify(lcs, L, fake_kv(lcs, Hkv=1), Hq=65) == lcs.LCS_E_UNSUPPORTED    # G = 65
    assert verify(lcs, L, kv, q=0) == lcs.LCS_E_ARG
    assert verify(lcs, L, kv, q=0x4002) == lcs.LCS_E_ARG          # misaligned
    assert verify(lcs, L, kv, r1=5) == lcs.LCS_E_ARG
    assert verify(lcs, L, kv, ld=39) == lcs.LCS_E_SHAPE
    assert verify(lcs, L, kv, max_len=60) == lcs.LCS_E_SHAPE       # 60 + 5 > 4 pages * 16
    assert verify(lcs, L, kv, max_len=-1) == lcs.LCS_E_SHAPE
    assert verify(lcs, L, kv, scale=float("inf")) == lcs.LCS_E_ARG
    assert verify(lcs, L, kv, wsb=0) == lcs.LCS_E_WORKSPACE
    assert verify(lcs, L, kv, B=0) == lcs.LCS_OK                   # empty batch: nothing launched
    assert verify(lcs, L, kv, B=0, q=0, out=0, prefix_len=0) == lcs.LCS_OK


def test_verify_rows_host_errors():
    lcs, L = lib()
    kv = fake_kv(lcs)

    def vr(**kw):
        a = dict(q=0x4000, B=1, n_q=5, Hq=4, prefix_len=0x5000, max_len=40, tree=None, scale=0.1, mask=0b10001,
                 out=0x6000, logits=0x7000, ld=40, lse=None, ws=0x8000, wsb=1 << 20)
        a.update(kw)
        return L.lcs_verify_attn_rows(ctypes.byref(kv), a["q"], a["B"], a["n_q"], a["Hq"], a["prefix_len"],
                                      a["max_len"], a["tree"], a["scale"], a["mask"], a["out"], a["logits"],
                                      a["ld"], a["lse"], a["ws"], a["wsb"], None)

    assert vr(mask=0) == lcs.LCS_E_ARG                    # logits without rows
    assert b"collect_mask" in L.lcs_last_error()
    assert vr(mask=1 << 5) == lcs.LCS_E_ARG               # row 5 of 5
    assert vr(n_q=65) == lcs.LCS_E_UNSUPPORTED
    assert vr(ld=39) == lcs.LCS_E_SHAPE
    assert vr(wsb=0) == lcs.LCS_E_WORKSPACE
    assert vr(B=0, q=0, out=0, prefix_len=0) == lcs.LCS_OK
    assert lcs.rows_mask([4, 0, 2]) == 0b10101


def test_select_rows_host_errors():
    lcs, L = lib()

    def sr(**kw):
        a = dict(lg=0x1000, ld=100, n=3, kind=0, lse=None, n_q=0, rm=0, B=1, Hq=4, Hkv=2, pl=0x2000, maxL=100,
                 mode=0, k=10, ns=4, nr=8, bs=0, idx=0x3000, cnt=0x4000, cap=22, ws=0x5000, wsb=1 << 24)
        a.update(kw)
        return L.lcs_select_topk_rows(a["lg"], a["ld"], a["n"], a["kind"], a["lse"], a["n_q"], a["rm"], a["B"],
                                      a["Hq"], a["Hkv"], a["pl"], a["maxL"], a["mode"], a["k"], a["ns"], a["nr"],
                                      a["bs"], a["idx"], a["cnt"], a["cap"], a["ws"], a["wsb"], None)

    assert sr(n=0) == lcs.LCS_E_ARG
    assert sr(n=65) == lcs.LCS_E_ARG
    assert sr(kind=2) == lcs.LCS_E_ARG
    assert sr(kind=1, lse=None, n_q=9, rm=0b111) == lcs.LCS_E_ARG          # no lse
    assert sr(kind=1, lse=0x6000, n_q=9, rm=0b11) == lcs.LCS_E_ARG         # 2 rows named, n = 3
    assert sr(kind=1, lse=0x6000, n_q=2, rm=0b111) == lcs.LCS_E_ARG        # row 2 of 2
    assert sr(kind=1, lse=0x6000, n_q=9, rm=0b111, B=0) == lcs.LCS_OK
    assert sr(cap=21) == lcs.LCS_E_SHAPE
    assert sr(wsb=10) == lcs.LCS_E_WORKSPACE


def test_select_host_errors():
    lcs, L = lib()

    def sel(**kw):
        a = dict(lg=0x1000, ld=100, B=1, Hq=4, Hkv=2, pl=0x2000, maxL=100, mode=0, k=10, ns=4, nr=8, bs=0,
                 idx=0x3000, cnt=0x4000, cap=22, ws=0x5000, wsb=1 << 24)
        a.update(kw)
        return L.lcs_select_topk(a["lg"], a["ld"], a["B"], a["Hq"], a["Hkv"], a["pl"], a["maxL"], a["mode"],
                                 a["k"], a["ns"], a["nr"], a["bs"], a["idx"], a["cnt"], a["cap"], a["ws"],
                                 a["wsb"], None)

    assert sel(B=0) == lcs.LCS_OK
    assert sel(B=0, lg=0, idx=0, cnt=0, pl=0) == lcs.LCS_OK
    assert sel(mode=7) == lcs.LCS_E_ARG
    assert sel(lg=0) == lcs.LCS_E_ARG
    assert sel(Hq=5) == lcs.LCS_E_SHAPE
    assert sel(k=-1) == lcs.LCS_E_ARG
    assert sel(cap=21) == lcs.LCS_E_SHAPE
    assert sel(ld=99) == lcs.LCS_E_SHAPE
    assert sel(mode=2, bs=12) == lcs.LCS_E_UNSUPPORTED
    assert sel(maxL=1 << 24, ld=1 << 24) == lcs.LCS_E_UNSUPPORTED
    assert sel(wsb=10) == lcs.LCS_E_WORKSPACE
    assert L.lcs_select_workspace_bytes(1, 4, 2, 0, 100, 0) > 0


def test_sparse_host_errors():
    lcs, L = lib()
    kv = fake_kv(lcs)

    def sp(kvd=kv, **kw):
        a = dict(q=0x1000, B=1, n_q=1, Hq=4, mode=0, idx=0x2000, cnt=0x3000, cap=10, tb=0x4000, tl=0x5000,
                 mtl=4, tm=None, scale=0.1, out=0x6000, lse=None, ws=0x7000, wsb=1 << 24)
        a.update(kw)
        return L.lcs_sparse_draft_attn(ctypes.byref(kvd), a["q"], a["B"], a["n_q"], a["Hq"], a["mode"], a["idx"],
                                       a["cnt"], a["cap"], a["tb"], a["tl"], a["mtl"], a["tm"], a["scale"],
                                       a["out"], a["lse"], a["ws"], a["wsb"], None)

    assert sp(B=0) == lcs.LCS_OK
    assert sp(mode=3) == lcs.LCS_E_ARG
    assert sp(tb=0) == lcs.LCS_E_ARG
    assert sp(idx=0) == lcs.LCS_E_ARG
    assert sp(n_q=65) == lcs.LCS_E_UNSUPPORTED
    assert sp(tm=0x8000, mtl=65) == lcs.LCS_E_UNSUPPORTED
    assert sp(mode=2) == lcs.LCS_E_UNSUPPORTED          # page 16 is not a multiple of 32
    assert sp(fake_kv(lcs, page_size=64), mode=2, ws=None) == lcs.LCS_E_WORKSPACE
    assert sp(wsb=0, cap=100000, mtl=100) == lcs.LCS_E_WORKSPACE


def test_sparse_noalloc_host_errors():
    """The static-scratch variant checks its arguments like the workspace variant, and
    refuses a call whose workspace need exceeds its 32 MiB scratch, all before touching
    a device."""
    lcs, L = lib()
    kv = fake_kv(lcs)

    def sp(kvd=kv, **kw):
        a = dict(q=0x1000, B=1, n_q=1, Hq=4, mode=0, idx=0x2000, cnt=0x3000, cap=10, tb=0x4000, tl=0x5000,
                 mtl=4, tm=None, scale=0.1, out=0x6000, lse=None)
        a.update(kw)
        return L.lcs_sparse_draft_attn_noalloc(ctypes.byref(kvd), a["q"], a["B"], a["n_q"], a["Hq"], a["mode"],
                                               a["idx"], a["cnt"], a["cap"], a["tb"], a["tl"], a["mtl"], a["tm"],
                                               a["scale"], a["out"], a["lse"], None)

    assert sp(B=0) == lcs.LCS_OK
    assert sp(mode=3) == lcs.LCS_E_ARG
    assert sp(q=0) == lcs.LCS_E_ARG
    assert sp(n_q=65) == lcs.LCS_E_UNSUPPORTED
    # block mode, 4 x 2 pairs x 64 rows x 100000 blocks: far beyond 32 MiB of union plan
    big = fake_kv(lcs, page_size=64)
    need = L.lcs_sparse_workspace_bytes(4, 64, 4, ctypes.byref(big), 2, 100000, 4)
    assert need > 32 << 20
    assert sp(big, B=4, n_q=64, mode=2, cap=100000) == lcs.LCS_E_WORKSPACE
    assert b"static scratch" in L.lcs_last_error()


def test_workspace_queries_are_deterministic():
    lcs, L = lib()
    kv = fake_kv(lcs, page_size=16, max_pages=4096, num_pages=4096 * 8, Hkv=8)
    a = L.lcs_verify_workspace_bytes(1, 9, 32, ctypes.byref(kv), 32768)
    b = L.lcs_verify_workspace_bytes(1, 9, 32, ctypes.byref(kv), 32768)
    assert a == b and a > 0
    assert L.lcs_verify_workspace_bytes(1, 9, 33, ctypes.byref(kv), 32768) == 0


def test_scores_host_errors():
    lcs, L = lib()
    kv = fake_kv(lcs)

    def vs(kvd=kv, **kw):
        a = dict(q=0x4000, B=1, n_q=5, Hq=4, prefix_len=0x5000, max_len=40, tree=None, scale=0.1, r0=0, r1=4,
                 out=0x6000, sc=0x7000, ld=40, lse=None, ws=0x8000, wsb=1 << 20)
        a.update(kw)
        return L.lcs_verify_attn_scores(ctypes.byref(kvd), a["q"], a["B"], a["n_q"], a["Hq"], a["prefix_len"],
                                        a["max_len"], a["tree"], a["scale"], a["r0"], a["r1"], a["out"], a["sc"],
                                        a["ld"], a["lse"], a["ws"], a["wsb"], None)

    assert vs(sc=0) == lcs.LCS_E_ARG
    assert vs(ld=39) == lcs.LCS_E_SHAPE
    assert vs(r1=5) == lcs.LCS_E_ARG
    big = fake_kv(lcs, max_pages=64, num_pages=200)
    assert vs(big, n_q=13, Hq=8) == lcs.LCS_E_UNSUPPORTED      # 52 rows: two row chunks
    many = fake_kv(lcs, Hkv=1, d=64)
    assert vs(many, n_q=1, Hq=16, r1=0) == lcs.LCS_E_UNSUPPORTED   # G = 16 > d/32 * 1 tile
    assert vs(B=0, q=0, out=0, prefix_len=0, sc=0) == lcs.LCS_OK

    def ss(**kw):
        a = dict(sc=0x1000, ld=100, B=1, Hkv=2, pl=0x2000, maxL=100, mode=0, k=10, ns=4, nr=8, bs=0,
                 idx=0x3000, cnt=0x4000, cap=22, ws=0x5000, wsb=1 << 24)
        a.update(kw)
        return L.lcs_select_topk_scores(a["sc"], a["ld"], a["B"], a["Hkv"], a["pl"], a["maxL"], a["mode"], a["k"],
                                        a["ns"], a["nr"], a["bs"], a["idx"], a["cnt"], a["cap"], a["ws"], a["wsb"],
                                        None)

    assert ss(sc=0) == lcs.LCS_E_ARG
    assert ss(ld=99) == lcs.LCS_E_SHAPE
    assert ss(mode=9) == lcs.LCS_E_ARG
    assert ss(B=0) == lcs.LCS_OK


def test_row_ld_avoids_power_of_two_strides():
    """lcs.row_ld: at least n, a multiple of 4 (16-byte rows for the fast write path),
    and 32 floats past a multiple of 64, so no row stride is a power of two."""
    from long_context_self_amd import lcs
    for n in (1, 5, 63, 64, 65, 4096, 32768, 65536, 131072, 131073):
        ld = lcs.row_ld(n)
        assert ld >= n and ld % 4 == 0 and ld % 64 == 32
        assert ld & (ld - 1) != 0
        assert ld - n < 96
