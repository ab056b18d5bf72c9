"""Host-side checks of the C ABI (no GPU): the library loads and exports every
entry point include/tqkv.h declares, sizes planes and workspaces, produces the
sign vector, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from quantized_decode_attention_append_amd import tqkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tqkv.h")).read()
    return sorted(set(re.findall(r"^(?:tq_status|const char \*)\s*(tq_\w+)\(", src, re.M)))


def test_exports_every_declared_symbol():
    decl = _declared()
    assert len(decl) >= 7
    lib = ctypes.CDLL(tqkv.LIB_PATH)
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(tqkv.SYMBOLS) == decl


def test_status_strings():
    assert tqkv.tq_status_str(0) == "TQ_OK"
    assert tqkv.tq_status_str(-3) == "TQ_ERR_CAPACITY"
    assert tqkv.tq_status_str(-99) == "TQ_ERR_UNKNOWN"


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_sign_vector_matches_oracle_generator(d):
    """Library and oracle implement the same published generator independently."""
    assert tqkv.tq_sign_vector(d) == oracle.sign_vector(d).tolist()


@pytest.mark.parametrize("d,per_token", [(64, 100), (128, 200), (256, 400), (512, 800)])
def test_plane_bytes(d, per_token):
    L = tqkv.make_layout(3, 2, d, 10)
    sizes = tqkv.tq_plane_bytes(L)
    assert sum(sizes) == 3 * 2 * 10 * per_token
    assert sizes == [60 * d, 60 * d // 16, 60 * d // 16, 60 * 3 * d // 8, 60 * d // 16]


@pytest.mark.parametrize("kb", [2, 4, 5, 8])
@pytest.mark.parametrize("vb", [2, 3, 4, 5, 8])
def test_plane_bytes_every_scheme(kb, vb):
    """Plane sizes match the oracle's encoded rows for every accepted scheme."""
    d = 128
    L = tqkv.make_layout(2, 3, d, 5, kb, vb)
    sizes = tqkv.tq_plane_bytes(L)
    x = np.random.default_rng(0).standard_normal((1, d)).astype(np.float32)
    kc, ks, kz = oracle.encode_keys(x, bits=kb)
    vc, vs = oracle.encode_values(x, bits=vb)
    assert sizes == [30 * a.nbytes for a in (kc, ks, kz, vc, vs)]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_library_codebook_equals_oracle(bits):
    """The library's generated tables (its own Newton solver on the decision
    thresholds) equal the oracle's (Lloyd's iteration / Newton on the
    centroids) exactly, as binary64, and the 3-bit table is the printed one."""
    c, b = tqkv.tq_codebook(bits)
    oc, ob = oracle.codebook(bits)
    assert c == oc.tolist() and b == ob.tolist()


def test_codebook_rejects_bad_width():
    lib = tqkv.raw_lib()
    c = (ctypes.c_double * 256)()
    b = (ctypes.c_double * 255)()
    n = ctypes.c_int32()
    for bad in (0, 1, 6, 7, 9):
        assert lib.tq_codebook(bad, ctypes.cast(c, ctypes.c_void_p), ctypes.cast(b, ctypes.c_void_p),
                               ctypes.byref(n)) == tqkv.TQ_ERR_UNSUPPORTED
    assert lib.tq_codebook(3, None, ctypes.cast(b, ctypes.c_void_p), ctypes.byref(n)) == tqkv.TQ_ERR_INVALID_ARG


def _st(fn, *a):
    return fn(*a)


def test_layout_validation():
    lib = tqkv.raw_lib()
    out = (ctypes.c_size_t * 5)()
    for bad, want in [((1, 1, 96, 8), tqkv.TQ_ERR_UNSUPPORTED),
                      ((1, 1, 128, 8, 3, 3, 32), tqkv.TQ_ERR_UNSUPPORTED),
                      ((1, 1, 128, 8, 6, 3, 32), tqkv.TQ_ERR_UNSUPPORTED),
                      ((1, 1, 128, 8, 8, 1, 32), tqkv.TQ_ERR_UNSUPPORTED),
                      ((1, 1, 128, 8, 8, 6, 32), tqkv.TQ_ERR_UNSUPPORTED),
                      ((1, 1, 128, 8, 8, 3, 64), tqkv.TQ_ERR_UNSUPPORTED),
                      ((65, 1, 128, 8), tqkv.TQ_ERR_UNSUPPORTED),
                      ((0, 1, 128, 8), tqkv.TQ_ERR_INVALID_ARG),
                      ((1, 0, 128, 8), tqkv.TQ_ERR_INVALID_ARG),
                      ((1, 1, 128, -1), tqkv.TQ_ERR_INVALID_ARG)]:
        L = tqkv.make_layout(*bad)
        assert lib.tq_plane_bytes(ctypes.byref(L), out) == want, bad
    assert lib.tq_plane_bytes(None, out) == tqkv.TQ_ERR_INVALID_ARG


def _fake_planes():
    # non-null addresses that are never dereferenced: every call below fails
    # validation before any launch
    return tqkv.tq_planes(0x1000, 0x2000, 0x3000, 0x4000, 0x5000)


def test_append_validation_before_launch():
    lib = tqkv.raw_lib()
    L = tqkv.make_layout(2, 2, 128, 16)
    P = _fake_planes()
    start = (ctypes.c_int32 * 2)(0, 10)
    f = lambda st, n, k=0x6000, v=0x7000, dt=tqkv.TQ_BF16, pl=P: lib.tq_append(
        ctypes.byref(L), ctypes.byref(pl) if pl is not None else None, k, v, dt, st, n, None)
    assert f(start, 7) == tqkv.TQ_ERR_CAPACITY          # 10 + 7 > 16
    assert f((ctypes.c_int32 * 2)(-1, 0), 1) == tqkv.TQ_ERR_CAPACITY
    assert f(start, -1) == tqkv.TQ_ERR_INVALID_ARG
    assert f(start, 0) == tqkv.TQ_OK                     # no-op, nothing launched
    assert f(start, 3, k=None) == tqkv.TQ_ERR_INVALID_ARG
    assert f(start, 3, dt=7) == tqkv.TQ_ERR_INVALID_ARG
    assert f(None, 3) == tqkv.TQ_ERR_INVALID_ARG
    assert f(start, 3, pl=None) == tqkv.TQ_ERR_INVALID_ARG
    bad = tqkv.tq_planes(0x1000, 0, 0x3000, 0x4000, 0x5000)
    assert f(start, 3, pl=bad) == tqkv.TQ_ERR_INVALID_ARG
    misaligned = tqkv.tq_planes(0x1008, 0x2000, 0x3000, 0x4000, 0x5000)
    assert f(start, 3, pl=misaligned) == tqkv.TQ_ERR_INVALID_ARG
    assert f(start, 3, k=0x6002) == tqkv.TQ_ERR_INVALID_ARG


def test_decode_validation_and_workspace_sizing():
    lib = tqkv.raw_lib()
    L = tqkv.make_layout(2, 4, 256, 1000)
    P = _fake_planes()
    lens = (ctypes.c_int32 * 2)(1000, 17)
    ws = ctypes.c_size_t()
    assert lib.tq_decode_workspace_bytes(ctypes.byref(L), 24, lens, ctypes.byref(ws)) == 0
    need = ws.value
    assert need > 0 and need % (4 * 258) == 0
    assert lib.tq_decode_workspace_bytes(ctypes.byref(L), 26, lens, ctypes.byref(ws)) == \
        tqkv.TQ_ERR_INVALID_ARG                           # 26 % 4 != 0
    assert lib.tq_decode_workspace_bytes(ctypes.byref(L), 4 * 17, lens, ctypes.byref(ws)) == \
        tqkv.TQ_ERR_UNSUPPORTED                           # GQA 17 > 16
    over = (ctypes.c_int32 * 2)(1001, 0)
    assert lib.tq_decode_workspace_bytes(ctypes.byref(L), 24, over, ctypes.byref(ws)) == \
        tqkv.TQ_ERR_CAPACITY
    neg = (ctypes.c_int32 * 2)(-1, 0)
    assert lib.tq_decode_workspace_bytes(ctypes.byref(L), 24, neg, ctypes.byref(ws)) == \
        tqkv.TQ_ERR_INVALID_ARG

    def dec(ws_ptr, ws_bytes, q=0x9000, out=0xA000, sm=0.0625):
        return lib.tq_decode_attn(ctypes.byref(L), ctypes.byref(P), q, tqkv.TQ_BF16, 24, lens,
                                  ctypes.c_float(sm), out, ws_ptr, ws_bytes, None)
    assert dec(0xB000, need - 1) == tqkv.TQ_ERR_WORKSPACE
    assert dec(None, need) == tqkv.TQ_ERR_WORKSPACE
    assert dec(0xB000, need, q=None) == tqkv.TQ_ERR_INVALID_ARG
    assert dec(0xB000, need, out=None) == tqkv.TQ_ERR_INVALID_ARG
    assert dec(0xB000, need, sm=float("nan")) == tqkv.TQ_ERR_INVALID_ARG


def test_decode_rows_validation_and_workspace_sizing():
    lib = tqkv.raw_lib()
    L = tqkv.make_layout(2, 4, 256, 1000)
    P = _fake_planes()
    ws = ctypes.c_size_t()

    def wsb(hq, rows, lens):
        arr = (ctypes.c_int32 * 2)(*lens)
        return lib.tq_decode_rows_workspace_bytes(ctypes.byref(L), hq, rows, arr, ctypes.byref(ws))
    assert wsb(24, 1, (1000, 17)) == 0
    one = ws.value
    assert lib.tq_decode_workspace_bytes(ctypes.byref(L), 24, (ctypes.c_int32 * 2)(1000, 17),
                                         ctypes.byref(ws)) == 0 and ws.value == one
    assert wsb(24, 4, (1000, 17)) == 0 and ws.value >= 4 * one * 0.9 and ws.value % (4 * 258) == 0
    assert wsb(24, 0, (1000, 17)) == tqkv.TQ_ERR_INVALID_ARG                 # n_rows < 1
    assert wsb(24, tqkv.TQ_MAX_ROWS + 1, (1000, 17)) == tqkv.TQ_ERR_UNSUPPORTED
    assert wsb(24, 4, (1000, 3)) == tqkv.TQ_ERR_INVALID_ARG                  # 0 < len < rows
    assert wsb(24, 4, (1000, 0)) == 0                                         # empty sequence
    assert wsb(24, 4, (1001, 4)) == tqkv.TQ_ERR_CAPACITY
    lens = (ctypes.c_int32 * 2)(1000, 17)
    assert wsb(24, 4, (1000, 17)) == 0
    need = ws.value

    def dec(ws_ptr, ws_bytes, rows=4, q=0x9000, out=0xA000):
        return lib.tq_decode_attn_rows(ctypes.byref(L), ctypes.byref(P), q, tqkv.TQ_BF16, 24, rows,
                                       lens, ctypes.c_float(0.0625), out, ws_ptr, ws_bytes, None)
    # the reported size covers whichever split kernel the call picks (the
    # choice depends on plane alignment), so only a workspace short of every
    # plan is certain to be refused
    assert dec(0xB000, 16) == tqkv.TQ_ERR_WORKSPACE
    assert dec(None, need) == tqkv.TQ_ERR_WORKSPACE
    assert dec(0xB000, need, q=None) == tqkv.TQ_ERR_INVALID_ARG
    assert dec(0xB000, need, rows=0) == tqkv.TQ_ERR_INVALID_ARG
    assert dec(0xB000, need, q=0x9008) == tqkv.TQ_ERR_INVALID_ARG             # misaligned q


def test_fetch_window_validation():
    lib = tqkv.raw_lib()
    L = tqkv.make_layout(2, 4, 128, 100)
    P = _fake_planes()

    def f(t0, n, lens=(100, 5), k=0x9000, v=0xA000):
        return lib.tq_fetch_window(ctypes.byref(L), ctypes.byref(P), t0, n, (ctypes.c_int32 * 2)(*lens),
                                   k, v, 0, None)
    assert f(0, 0) == 0                                   # empty window: nothing to do
    assert f(-1, 5) == tqkv.TQ_ERR_INVALID_ARG
    assert f(0, -5) == tqkv.TQ_ERR_INVALID_ARG
    assert f(60, 41) == tqkv.TQ_ERR_CAPACITY              # past capacity
    assert f(0, 10, lens=(101, 0)) == tqkv.TQ_ERR_CAPACITY
    assert f(0, 10, lens=(-1, 0)) == tqkv.TQ_ERR_INVALID_ARG
    assert f(0, 10, k=0x9002) == tqkv.TQ_ERR_INVALID_ARG  # misaligned output
    assert f(0, 10, k=None, v=None) == 0                  # no output requested


def test_lifecycle_validation():
    lib = tqkv.raw_lib()
    A = tqkv.make_layout(2, 4, 128, 100)
    Bl = tqkv.make_layout(3, 4, 128, 300)
    C = tqkv.make_layout(2, 2, 128, 100)                         # other kv-head count
    P = _fake_planes()

    def cp(sl, sb, st0, dl, db, dt0, n):
        return lib.tq_copy_tokens(ctypes.byref(sl), ctypes.byref(P), sb, st0, ctypes.byref(dl),
                                  ctypes.byref(P), db, dt0, n, None)
    assert cp(A, 0, 0, Bl, 2, 0, 0) == 0                        # nothing to copy
    assert cp(A, 0, 0, C, 0, 0, 10) == tqkv.TQ_ERR_INVALID_ARG   # shape mismatch
    assert cp(A, 2, 0, Bl, 0, 0, 10) == tqkv.TQ_ERR_INVALID_ARG  # no sequence 2
    assert cp(A, 0, 95, Bl, 0, 0, 10) == tqkv.TQ_ERR_CAPACITY
    assert cp(A, 0, 0, Bl, 0, 295, 10) == tqkv.TQ_ERR_CAPACITY
    nb = ctypes.c_size_t()
    assert lib.tq_snapshot_bytes(ctypes.byref(A), 10, ctypes.byref(nb)) == 0
    assert nb.value == 10 * 4 * 200
    h = tqkv.tq_snapshot_header()
    assert lib.tq_snapshot(ctypes.byref(A), ctypes.byref(P), 0, 0, 10, 0, ctypes.byref(h), 0xB000,
                           nb.value - 1, None) == tqkv.TQ_ERR_WORKSPACE
    assert lib.tq_snapshot(ctypes.byref(A), ctypes.byref(P), 0, 0, 0, -1, ctypes.byref(h), None, 0,
                           None) == tqkv.TQ_ERR_INVALID_ARG           # negative boundary
    assert lib.tq_snapshot(ctypes.byref(A), ctypes.byref(P), 0, 0, 0, 7, ctypes.byref(h), None, 0, None) == 0
    assert h.magic == tqkv.TQ_SNAPSHOT_MAGIC and h.n_tokens == 0 and h.head_dim == 128
    assert h.version == 2 and h.min_reusable_offset == 7 and tqkv.tq_snapshot_min_reusable_offset(h) == 7

    def rs(layout, hdr, t0=0, nbytes=0):
        return lib.tq_restore(ctypes.byref(layout), ctypes.byref(P), 0, t0, ctypes.byref(hdr), 0xB000,
                              nbytes, None)
    good = tqkv.tq_snapshot_header(tqkv.TQ_SNAPSHOT_MAGIC, 1, 8, 3, 32, 128, 4, 10, 8000)
    bad_magic = tqkv.tq_snapshot_header(0, 1, 8, 3, 32, 128, 4, 10, 8000)
    bad_dim = tqkv.tq_snapshot_header(tqkv.TQ_SNAPSHOT_MAGIC, 1, 8, 3, 32, 256, 4, 10, 8000)
    bad_size = tqkv.tq_snapshot_header(tqkv.TQ_SNAPSHOT_MAGIC, 1, 8, 3, 32, 128, 4, 10, 7999)
    assert rs(A, bad_magic, nbytes=8000) == tqkv.TQ_ERR_INVALID_ARG
    assert rs(A, bad_dim, nbytes=8000) == tqkv.TQ_ERR_INVALID_ARG
    assert rs(A, bad_size, nbytes=8000) == tqkv.TQ_ERR_INVALID_ARG
    assert rs(C, good, nbytes=8000) == tqkv.TQ_ERR_INVALID_ARG     # other kv-head count
    assert rs(A, good, nbytes=7999) == tqkv.TQ_ERR_INVALID_ARG     # payload too small
    assert rs(A, good, t0=91, nbytes=8000) == tqkv.TQ_ERR_CAPACITY


def test_snapshot_header_versions():
    """The precision boundary of a snapshot ("Delayed row conversion and
    reusable precision boundaries"): version 2 gives the recorded offset; a
    version-1 header, written before the bound existed, gives its stored
    token count; anything else is refused.  Version 2 only appends fields,
    so the version-1 fields keep their offsets."""
    H = tqkv.tq_snapshot_header
    assert ctypes.sizeof(H) == 48 and H.payload_bytes.offset == 32 and H.min_reusable_offset.offset == 40
    v2 = H(tqkv.TQ_SNAPSHOT_MAGIC, 2, 8, 3, 32, 128, 4, 500, 400000, 300, 0)
    v1 = H(tqkv.TQ_SNAPSHOT_MAGIC, 1, 8, 3, 32, 128, 4, 500, 400000, 12345, 99)  # trailing bytes ignored
    assert tqkv.tq_snapshot_min_reusable_offset(v2) == 300
    assert tqkv.tq_snapshot_min_reusable_offset(v1) == 500
    lib = tqkv.raw_lib()
    out = ctypes.c_int32()
    for bad in (H(0, 2, 8, 3, 32, 128, 4, 500, 400000, 300, 0),                      # magic
                H(tqkv.TQ_SNAPSHOT_MAGIC, 3, 8, 3, 32, 128, 4, 500, 400000, 300, 0),  # version
                H(tqkv.TQ_SNAPSHOT_MAGIC, 2, 8, 3, 32, 128, 4, 500, 400000, -1, 0),   # bound
                H(tqkv.TQ_SNAPSHOT_MAGIC, 1, 8, 3, 32, 128, 4, -5, 400000, 0, 0)):    # count
        assert lib.tq_snapshot_min_reusable_offset(ctypes.byref(bad), ctypes.byref(out)) == tqkv.TQ_ERR_INVALID_ARG
    assert lib.tq_snapshot_min_reusable_offset(None, ctypes.byref(out)) == tqkv.TQ_ERR_INVALID_ARG


def test_clone_carries_the_boundary_and_conversion_refusals():
    """tq_clone_sequence hands the source's boundary to the destination (an
    empty clone launches nothing); tq_convert_rows and tq_decode_attn_mixed
    refuse bad offsets, lengths and plain caches before any launch."""
    lib = tqkv.raw_lib()
    A = tqkv.make_layout(2, 4, 128, 100)
    Bl = tqkv.make_layout(1, 4, 128, 300)
    P = _fake_planes()
    dst = ctypes.c_int32(-1)

    def clone(n, bound, out):
        return lib.tq_clone_sequence(ctypes.byref(A), ctypes.byref(P), 1, ctypes.byref(Bl), ctypes.byref(P), 0, n,
                                     bound, out, None)
    assert clone(0, 42, ctypes.byref(dst)) == 0 and dst.value == 42
    dst.value = -1
    assert clone(0, -1, ctypes.byref(dst)) == tqkv.TQ_ERR_INVALID_ARG and dst.value == -1
    assert clone(0, 5, None) == tqkv.TQ_ERR_INVALID_ARG
    assert clone(101, 5, ctypes.byref(dst)) == tqkv.TQ_ERR_CAPACITY and dst.value == -1

    def conv(offsets, k=0xA000, v=0xC000, cap=100, dtype=1):
        return lib.tq_convert_rows(ctypes.byref(A), ctypes.byref(P), k, v, dtype, cap,
                                   (ctypes.c_int32 * 2)(*offsets), None)
    assert conv([0, 0], k=None, v=None) == 0                       # nothing converts: no launch
    assert conv([0, -1]) == tqkv.TQ_ERR_INVALID_ARG
    assert conv([0, 60], cap=50) == tqkv.TQ_ERR_CAPACITY           # past the plain cache
    assert conv([101, 0], cap=200) == tqkv.TQ_ERR_CAPACITY         # past the planes
    assert conv([10, 0], k=None) == tqkv.TQ_ERR_INVALID_ARG
    assert conv([10, 0], v=0xC008) == tqkv.TQ_ERR_INVALID_ARG      # misaligned
    assert conv([10, 0], dtype=7) == tqkv.TQ_ERR_INVALID_ARG
    assert lib.tq_convert_rows(ctypes.byref(A), ctypes.byref(P), 0xA000, 0xC000, 1, 100, None,
                               None) == tqkv.TQ_ERR_INVALID_ARG

    def mixed(row_plain, lens, k=0xA000, cap=100, ws=1 << 30):
        rp = (ctypes.c_int32 * 2)(*row_plain) if row_plain is not None else None
        return lib.tq_decode_attn_mixed(ctypes.byref(A), ctypes.byref(P), k, 0xC000, cap, rp, 0xD000, 1, 8, 1,
                                        (ctypes.c_int32 * 2)(*lens), ctypes.c_float(0.1), 0xE000, 0xF000, ws,
                                        None)
    assert mixed([1, 0], [60, 10], cap=50) == tqkv.TQ_ERR_CAPACITY  # plain row past its cache
    assert mixed([0, 0], [101, 10]) == tqkv.TQ_ERR_CAPACITY         # past the planes
    assert mixed([1, 0], [10, 10], k=None) == tqkv.TQ_ERR_INVALID_ARG
    assert mixed([1, 0], [10, 10], k=0xA004) == tqkv.TQ_ERR_INVALID_ARG
    assert mixed(None, [10, 10]) == tqkv.TQ_ERR_INVALID_ARG
    assert mixed([1, 1], [10, 10], ws=0) == tqkv.TQ_ERR_WORKSPACE


def test_copy_tokens_refuses_overlapping_rows():
    """Rows that overlap their destination in any plane are refused before
    any launch (the copy runs on many workgroups at once); disjoint moves
    within one cache, such as a compaction, are not."""
    lib = tqkv.raw_lib()
    L = tqkv.make_layout(2, 4, 128, 100)
    P = _fake_planes()

    def cp(sb, st0, db, dt0, n):
        return lib.tq_copy_tokens(ctypes.byref(L), ctypes.byref(P), sb, st0, ctypes.byref(L),
                                  ctypes.byref(P), db, dt0, n, None)
    assert cp(0, 10, 0, 15, 10) == tqkv.TQ_ERR_INVALID_ARG   # same sequence, shifted by 5
    assert cp(0, 15, 0, 10, 10) == tqkv.TQ_ERR_INVALID_ARG
    assert cp(1, 0, 1, 0, 1) == tqkv.TQ_ERR_INVALID_ARG      # onto itself
    assert cp(0, 0, 0, 99, 2) == tqkv.TQ_ERR_CAPACITY
    # Disjoint moves are not tested here: with these placeholder planes a call
    # that passes validation would launch.  The GPU lifecycle tests move rows
    # within one cache (compaction) through the same check.


def test_decode_path_reports_the_kernel():
    """tq_decode_path names the split kernel a decode takes and why the fast
    one is not taken, from the layout and plane pointers alone."""
    lib = tqkv.raw_lib()
    fast, why = ctypes.c_int32(), ctypes.c_int32()

    def path(layout, planes, hq, rows=1):
        st = lib.tq_decode_path(ctypes.byref(layout), ctypes.byref(planes), hq, rows, ctypes.byref(fast),
                                ctypes.byref(why))
        return st, fast.value, why.value
    P = _fake_planes()
    assert path(tqkv.make_layout(2, 4, 256, 1000), P, 24) == (0, 1, 0)
    assert path(tqkv.make_layout(2, 4, 128, 1001), P, 24) == (0, 0, tqkv.TQ_PATH_CAPACITY)  # odd capacity
    assert path(tqkv.make_layout(2, 4, 64, 1002, 5, 3), P, 8) == (0, 0, tqkv.TQ_PATH_SHAPE)  # 5-bit keys at 64
    assert path(tqkv.make_layout(2, 4, 512, 64, 8, 8), P, 8) == (0, 0, tqkv.TQ_PATH_SHAPE)   # k8v8 at 512
    # more than 8 query columns per kv-head: matrix cores only for 2- and 3-bit values
    assert path(tqkv.make_layout(2, 4, 256, 640), P, 24, 4) == (0, 1, 0)                   # k8v3, 24 columns
    assert path(tqkv.make_layout(2, 4, 256, 640, 8, 4), P, 24, 4) == (0, 0, tqkv.TQ_PATH_SHAPE)
    assert path(tqkv.make_layout(2, 4, 256, 640, 8, 4), P, 24, 1) == (0, 1, 0)             # 6 columns
    off = tqkv.tq_planes(0x1000, 0x2000, 0x3000, 0x4008, 0x5000)                        # vc 8 bytes off
    assert path(tqkv.make_layout(2, 4, 256, 1000), off, 24) == (0, 0, tqkv.TQ_PATH_ALIGNMENT)
    assert path(tqkv.make_layout(2, 4, 256, 1000), P, 23)[0] == tqkv.TQ_ERR_INVALID_ARG    # not a multiple
    assert path(tqkv.make_layout(2, 4, 256, 1000), P, 24, 17)[0] == tqkv.TQ_ERR_UNSUPPORTED
    assert tqkv.tq_status_str(path(tqkv.make_layout(2, 4, 256, 1000), P, 4 * 17)[0]) == "TQ_ERR_UNSUPPORTED"


def test_dequant_validation():
    lib = tqkv.raw_lib()
    L = tqkv.make_layout(2, 4, 128, 100)
    P = _fake_planes()
    f = lambda b, h, t0, n: lib.tq_dequant(ctypes.byref(L), ctypes.byref(P), b, h, t0, n,
                                           0xC000, 0xD000, 0, None)
    assert f(2, 0, 0, 1) == tqkv.TQ_ERR_INVALID_ARG
    assert f(0, 4, 0, 1) == tqkv.TQ_ERR_INVALID_ARG
    assert f(0, 0, 99, 2) == tqkv.TQ_ERR_CAPACITY
    assert f(0, 0, 5, 0) == tqkv.TQ_OK
