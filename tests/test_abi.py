"""The C-ABI library builds, loads, exports what include/dualkv.h declares and
rejects bad arguments before touching the GPU (no compute calls here: every
call below fails argument checks, so no HIP API is reached)."""
import ctypes
import os
import re

import pytest

from exact_shared_prefix_amd import binding, metrics
from exact_shared_prefix_amd.binding import (ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, OK,
                                             Packing)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dualkv.h")
FAKE = 0x100000  # aligned, never dereferenced: every call here fails validation first


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dualkv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    nm = os.popen(f"nm -D --defined-only {binding.LIB_PATH}").read()
    for name in declared_symbols():
        assert re.search(rf"\bT {name}\b", nm), name


def test_library_has_gfx950_code_object():
    data = open(binding.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_status_strings(lib):
    for s in range(5):
        assert binding.status_string(s)
    assert binding.status_string(99) == "unknown status"


def _fwd(lib, P=16, R=8, N=2, offsets=None, Hq=4, Hkv=2, d=128, scale=0.1, ws=FAKE,
         ws_bytes=1 << 20, q=FAKE, lse=FAKE):
    offp = None
    if offsets is not None:
        arr = (ctypes.c_int32 * len(offsets))(*offsets)
        offp = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return lib.dualkv_fwd(q, FAKE, FAKE, FAKE, lse, P, R, N, offp, Hq, Hkv, d, scale, ws,
                          ws_bytes, None)


def _bwd(lib, P=16, R=8, N=2, Hq=4, Hkv=2, d=128, scale=0.1, det=0, ws=FAKE, ws_bytes=1 << 20,
         dq=FAKE):
    return lib.dualkv_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, P, R, N, None, Hq,
                          Hkv, d, scale, det, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), ERR_INVALID_ARG),
    (dict(P=-1), ERR_INVALID_ARG),
    (dict(R=-3), ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), ERR_INVALID_ARG),
    (dict(Hkv=0), ERR_INVALID_ARG),
    (dict(d=96), ERR_UNSUPPORTED),
    (dict(d=256), ERR_UNSUPPORTED),
    (dict(scale=-1.0), ERR_INVALID_ARG),
    (dict(scale=float("nan")), ERR_INVALID_ARG),
    (dict(scale=float("inf")), ERR_INVALID_ARG),
    (dict(q=None), ERR_INVALID_ARG),
    (dict(q=FAKE + 2), ERR_INVALID_ARG),          # misaligned
    (dict(lse=None), ERR_INVALID_ARG),
    (dict(offsets=[15, 20, 30], N=2), ERR_INVALID_ARG),  # offsets[0] != P
    (dict(offsets=[16, 30, 20], N=2), ERR_INVALID_ARG),  # decreasing
    (dict(R=1 << 12, N=1 << 20), ERR_INVALID_ARG),  # T >= 2^31
    (dict(P=1 << 30, Hq=64, Hkv=8, d=128, R=0), ERR_INVALID_ARG),  # T*Hq*d >= 2^40
    (dict(ws=None), ERR_WORKSPACE),
    (dict(ws_bytes=1), ERR_WORKSPACE),
])
def test_fwd_rejects_bad_arguments(lib, kw, status):
    assert _fwd(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(det=1, ws_bytes=16), ERR_WORKSPACE),
    (dict(N=0), ERR_INVALID_ARG),
    (dict(Hq=3, Hkv=2), ERR_INVALID_ARG),
    (dict(d=32), ERR_UNSUPPORTED),
    (dict(scale=-0.5), ERR_INVALID_ARG),
    (dict(dq=None), ERR_INVALID_ARG),
    (dict(dq=FAKE + 8), ERR_INVALID_ARG),
    (dict(ws_bytes=16), ERR_WORKSPACE),
])
def test_bwd_rejects_bad_arguments(lib, kw, status):
    assert _bwd(lib, **kw) == status


@pytest.mark.parametrize("mask,status", [(0, ERR_INVALID_ARG), (16, ERR_INVALID_ARG),
                                         (-1, ERR_INVALID_ARG), (2, ERR_WORKSPACE),
                                         (8, ERR_WORKSPACE)])
def test_bwd_phases_rejects_bad_mask(lib, mask, status):
    r = lib.dualkv_bwd_phases(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, 8, 2, None,
                              4, 2, 128, 0.1, 0, FAKE, 16, None, mask)
    assert r == status


def test_workspace_sizes(lib):
    pk = Packing(128, R=64, N=4)
    nf = binding.fwd_workspace_bytes(pk, 4, 2, 64)
    nb = binding.bwd_workspace_bytes(pk, 4, 2, 64)
    assert nf >= 16 and nf % 256 == 0
    T = pk.T
    # bwd holds at least the {-LSE log2 e, D} pairs [Hq,T] and fp32 dK/dV accumulators
    # (dQ is written directly)
    assert nb >= 4 * (2 * 4 * T + 2 * T * 2 * 64)
    assert nb < 4 * (2 * 4 * T + 2 * T * 2 * 64) + 4 * T * 4 * 64
    # deterministic mode holds per-item dK/dV partials instead of the accumulators
    nd = binding.bwd_workspace_bytes(pk, 4, 2, 64, deterministic=True)
    assert nd > 0 and nd % 256 == 0 and nd != nb
    with pytest.raises(binding.DualKVError):
        binding.fwd_workspace_bytes(pk, 4, 3, 64)
    # ragged offsets are accepted and size like the uniform case of equal T
    rag = Packing(128, lengths=[10, 100, 0, 146])
    assert binding.fwd_workspace_bytes(rag, 4, 2, 64) > 0
    assert not rag.uniform and pk.uniform


def _arr(xs):
    if xs is None:
        return None
    a = (ctypes.c_int32 * max(1, len(xs)))(*xs)
    return ctypes.cast(a, ctypes.POINTER(ctypes.c_int32))


def _fwd_groups(lib, B=2, gP=(16, 8), gN=(2, 1), R=(8, 4, 5), Hq=4, Hkv=2, d=128, scale=0.1,
                ws=FAKE, ws_bytes=1 << 20):
    return lib.dualkv_fwd_groups(FAKE, FAKE, FAKE, FAKE, FAKE, B, _arr(gP), _arr(gN), _arr(R), Hq,
                                 Hkv, d, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), ERR_INVALID_ARG),
    (dict(gP=None), ERR_INVALID_ARG),
    (dict(gN=None), ERR_INVALID_ARG),
    (dict(R=None), ERR_INVALID_ARG),
    (dict(gN=(2, 0)), ERR_INVALID_ARG),        # a group without responses
    (dict(gP=(16, -1)), ERR_INVALID_ARG),
    (dict(R=(8, -4, 5)), ERR_INVALID_ARG),
    (dict(R=(8, 1 << 30, 1 << 30)), ERR_INVALID_ARG),   # T >= 2^31
    (dict(Hq=3), ERR_INVALID_ARG),
    (dict(d=96), ERR_UNSUPPORTED),
    (dict(scale=-1.0), ERR_INVALID_ARG),
    (dict(ws_bytes=16), ERR_WORKSPACE),
])
def test_fwd_groups_rejects_bad_arguments(lib, kw, status):
    assert _fwd_groups(lib, **kw) == status


def test_bwd_groups_rejects_bad_arguments(lib):
    gP, gN, R = _arr((16, 8)), _arr((2, 1)), _arr((8, 4, 5))
    call = lambda B, ws_bytes, det=0: lib.dualkv_bwd_groups(  # noqa: E731
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, gP, gN, R, 4, 2, 128, 0.1, det,
        FAKE, ws_bytes, None)
    assert call(0, 1 << 20) == ERR_INVALID_ARG
    assert call(2, 16) == ERR_WORKSPACE
    assert call(2, 16, det=1) == ERR_WORKSPACE


def test_group_workspace_sizes(lib):
    # one group is the single-group problem
    for det in (0, 1):
        one = lib.dualkv_bwd_workspace_bytes_groups(1, _arr((16,)), _arr((3,)), _arr((8, 0, 5)),
                                                    4, 2, 128, det)
        ref = lib.dualkv_bwd_workspace_bytes(16, 0, 3, _arr((16, 24, 24, 29)), 4, 2, 128, det)
        assert one == ref > 0
    one = lib.dualkv_fwd_workspace_bytes_groups(1, _arr((16,)), _arr((3,)), _arr((8, 0, 5)), 4, 2, 128)
    assert one == lib.dualkv_fwd_workspace_bytes(16, 0, 3, _arr((16, 24, 24, 29)), 4, 2, 128) > 0
    two = lib.dualkv_fwd_workspace_bytes_groups(2, _arr((16, 8)), _arr((3, 1)), _arr((8, 0, 5, 4)),
                                                4, 2, 128)
    assert two > one and two % 256 == 0
    assert lib.dualkv_fwd_workspace_bytes_groups(0, _arr((16,)), _arr((3,)), _arr((8,)), 4, 2, 128) == 0


def _fwd_tree(lib, lens=(8, 4, 3, 5), par=(-1, 0, 1, 0), Hq=4, Hkv=2, d=128, ws_bytes=1 << 20):
    return lib.dualkv_fwd_tree(FAKE, FAKE, FAKE, FAKE, FAKE, len(lens) if lens else 0, _arr(lens),
                               _arr(par), Hq, Hkv, d, 0.1, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(lens=()), ERR_INVALID_ARG),
    (dict(par=(-1, 0, 2, 0)), ERR_INVALID_ARG),          # parent not before the segment
    (dict(par=(-1, 0, 1, 2), lens=(8, 4, 3, 5)), OK),    # a chain is fine (checked below with ws)
    (dict(lens=(8, 4, 3, 5, 2), par=(-1, 0, 1, 0, 2)), ERR_INVALID_ARG),   # 2 left the path at 3
    (dict(lens=(8, 4, -3, 5)), ERR_INVALID_ARG),
    (dict(lens=(1, 1, 1, 1, 1), par=(-1, 0, 1, 2, 3)), ERR_INVALID_ARG),   # 4 ancestors
    (dict(d=96), ERR_UNSUPPORTED),
    (dict(ws_bytes=16), ERR_WORKSPACE),
])
def test_fwd_tree_rejects_bad_arguments(lib, kw, status):
    if status == OK:
        kw = dict(kw, ws_bytes=16)
        status = ERR_WORKSPACE   # shape accepted, then the workspace check fails
    assert _fwd_tree(lib, **kw) == status


def test_tree_workspace_matches_single_group(lib):
    # root prompt + leaves is the single-group problem
    for det in (0, 1):
        t = lib.dualkv_bwd_workspace_bytes_tree(4, _arr((16, 8, 0, 5)), _arr((-1, 0, 0, 0)), 4, 2, 128, det)
        g = lib.dualkv_bwd_workspace_bytes(16, 0, 3, _arr((16, 24, 24, 29)), 4, 2, 128, det)
        assert t == g > 0
    t = lib.dualkv_fwd_workspace_bytes_tree(4, _arr((16, 8, 0, 5)), _arr((-1, 0, 0, 0)), 4, 2, 128)
    assert t == lib.dualkv_fwd_workspace_bytes(16, 0, 3, _arr((16, 24, 24, 29)), 4, 2, 128) > 0


def test_pair_accounting_matches_brute_force():
    from oracle import attended_keys
    for P, lengths in ((5, [3, 0, 4]), (0, [6, 2]), (9, [1])):
        brute = sum(len(attended_keys(t, P, lengths)) for t in range(P + sum(lengths)))
        assert metrics.pairs(P, lengths) == brute
        rep = sum(sum(range(1, P + r + 1)) for r in lengths)
        assert metrics.replicated_pairs(P, lengths) == rep


def test_tree_pair_accounting_matches_brute_force():
    from oracle import attended_keys_tree
    for node_len, node_parent in (([7, 3, 0, 5, 4, 2], [-1, 0, 1, 1, 0, -1]), ([4, 2, 3, 1], [-1, 0, 1, 2]),
                                  ([5, 2, 0, 3], [-1, 0, 0, 0])):
        brute = sum(len(attended_keys_tree(t, node_len, node_parent)) for t in range(sum(node_len)))
        assert metrics.tree_pairs(node_len, node_parent) == brute


def _fwd_noalloc(lib, P=16, R=8, N=2, offsets=None, Hq=4, Hkv=2, d=128, scale=0.1, q=FAKE):
    offp = None
    if offsets is not None:
        arr = (ctypes.c_int32 * len(offsets))(*offsets)
        offp = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return lib.dualkv_fwd_noalloc(q, FAKE, FAKE, FAKE, FAKE, P, R, N, offp, Hq, Hkv, d, scale, None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=0), ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), ERR_INVALID_ARG),
    (dict(d=96), ERR_UNSUPPORTED),
    (dict(scale=-1.0), ERR_INVALID_ARG),
    (dict(q=FAKE + 2), ERR_INVALID_ARG),
    (dict(N=257, R=4), ERR_UNSUPPORTED),                      # more responses than travel by value
    (dict(P=1 << 20, Hkv=8, Hq=8, d=128), ERR_WORKSPACE),     # V^T alone is 2 GiB > the fixed array
    (dict(P=1 << 16, R=0, N=1, Hkv=8, Hq=8, d=128), ERR_WORKSPACE),   # 256 tiles fit, V^T (128 MiB) does not
])
def test_fwd_noalloc_rejects_what_exceeds_its_scratch(lib, kw, status):
    assert _fwd_noalloc(lib, **kw) == status


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define DUALKV_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_SCRATCH_BYTES
