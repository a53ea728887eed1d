"""C-ABI boundary checks that need no GPU.

* libmoegmm.so loads and exports every function include/moegmm.h declares.
* Host-side validation returns an error status before anything is enqueued
  (null pointers, sizes out of range, misalignment, small workspace); these
  calls never reach the HIP runtime.
* Workspace size queries.
"""
import ctypes
import os
import re
import subprocess

import pytest

from grouped_gemm_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moegmm.h")

MOE_OK, MOE_ERR_NULL, MOE_ERR_INVALID, MOE_ERR_WORKSPACE = 0, 1, 2, 3


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ["moe_permute", "moe_permute_workspace_size", "gmm_fwd", "gmm_fwd_swiglu", "gmm_bwd_input",
              "gmm_bwd_weight", "gmm_workspace_size", "swiglu", "swiglu_bwd", "moe_unpermute",
              "moe_unpermute_bwd", "moe_permute_bwd", "moe_status_string", "moegmm_abi_version",
              "mx_quantize", "moe_permute_mx", "gmm_mx_fwd", "gmm_mx_fwd_swiglu", "gmm_bwd", "gmm_bwd_swiglu",
              "moe_permute_index", "gmm_fwd_gather", "gmm_fwd_swiglu_gather", "gmm_mx_fwd_swiglu_gather",
              "swiglu_gmm_fwd", "moe_decode_fwd", "moe_decode_fwd_mx"]:
        assert n in names, n


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in _declared_functions():
        assert n in exported, f"{n} declared in moegmm.h but not exported"
        assert hasattr(lib, n)
    assert set(_lib.SIGNATURES) == set(_declared_functions())


def test_abi_version_and_status_strings(lib):
    assert lib.moegmm_abi_version() == _lib.ABI_VERSION
    for s in range(5):
        assert lib.moe_status_string(s).decode().startswith("MOE_")
    assert b"unknown" in lib.moe_status_string(99)


def test_workspace_queries(lib):
    assert lib.moe_permute_workspace_size(4096, 8, 128) >= 32 * 128 * 4
    assert lib.moe_permute_workspace_size(0, 8, 128) >= 0
    assert lib.moe_permute_workspace_size(-1, 8, 128) == 0
    # forward and input gradient need none; the weight gradient its tile queue
    for op in range(2):
        assert lib.gmm_workspace_size(32, 16384, 4096, 3072, op) == 0
    assert lib.gmm_workspace_size(32, 16384, 4096, 3072, 2) == 1152
    assert lib.gmm_workspace_size(32, 16384, 4096, 3072, 3) == 1152
    # a grid of 32 tiles of 256 x 256 on 256 CUs (the count used where no
    # device is visible): the rows split 8 ways, a 256 KiB fp32 partial per
    # (tile, chunk) after the 2048-byte queue area
    assert lib.gmm_workspace_size(1, 32768, 2048, 1024, 2) == 2048 + 32 * 8 * 256 * 256 * 4
    # few rows cap the chunks (one per started 256 rows): 600 rows, 3 chunks;
    # 256 rows, no split
    assert lib.gmm_workspace_size(1, 600, 2048, 1024, 2) == 2048 + 32 * 3 * 256 * 256 * 4
    assert lib.gmm_workspace_size(1, 256, 2048, 1024, 2) == 1152


def test_queue_bytes_constant():
    """The zero-filled prefix of a GMM workspace: the header's value, the
    binding's, and what gmm_bwd asks for agree."""
    import grouped_gemm_moe_amd as moe

    text = open(HEADER).read()
    m = re.search(r"#define MOE_GMM_QUEUE_BYTES (\d+)", text)
    assert m and int(m.group(1)) == moe.GMM_QUEUE_BYTES == 1152


# fake but aligned non-null device addresses: validation must reject the call
# before any of them is touched
A16 = ctypes.c_void_p(0x10000)
A16b = ctypes.c_void_p(0x20000)
A16c = ctypes.c_void_p(0x30000)
MIS = ctypes.c_void_p(0x10002)


def test_gmm_rejects_bad_arguments(lib):
    ws = ctypes.c_void_p(0x40000)
    # null weight / group_list
    assert lib.gmm_fwd(A16, None, A16b, 4, 64, 64, 64, A16c, ws, 0, None, None) == MOE_ERR_NULL
    assert lib.gmm_fwd(A16, A16b, None, 4, 64, 64, 64, A16c, ws, 0, None, None) == MOE_ERR_NULL
    # E out of range, K not a multiple of 8, negative M_cap
    assert lib.gmm_fwd(A16, A16b, A16c, 0, 64, 64, 64, A16c, ws, 0, None, None) == MOE_ERR_INVALID
    assert lib.gmm_fwd(A16, A16b, A16c, 1025, 64, 64, 64, A16c, ws, 0, None, None) == MOE_ERR_INVALID
    assert lib.gmm_fwd(A16, A16b, A16c, 4, 64, 60, 64, A16c, ws, 0, None, None) == MOE_ERR_INVALID
    assert lib.gmm_fwd(A16, A16b, A16c, 4, -1, 64, 64, A16c, ws, 0, None, None) == MOE_ERR_INVALID
    # misaligned bf16 pointer
    assert lib.gmm_fwd(MIS, A16b, A16c, 4, 64, 64, 64, A16c, ws, 0, None, None) == MOE_ERR_INVALID
    assert lib.gmm_bwd_input(A16, MIS, A16c, 4, 64, 64, 64, A16c, ws, 0, None, None) == MOE_ERR_INVALID
    assert lib.gmm_bwd_weight(A16, A16b, A16c, 4, 64, 64, 64, None, ws, 0, None, None) == MOE_ERR_NULL
    assert lib.gmm_bwd_weight(A16, A16b, A16c, 4, 64, 64, 64, MIS, ws, 0, None, None) == MOE_ERR_INVALID
    # the weight gradient's tile queue: missing, short or misaligned workspace
    need = lib.gmm_workspace_size(4, 64, 64, 64, 2)
    assert lib.gmm_bwd_weight(A16, A16b, A16c, 4, 64, 64, 64, A16c, None, need, None, None) == MOE_ERR_WORKSPACE
    assert lib.gmm_bwd_weight(A16, A16b, A16c, 4, 64, 64, 64, A16c, ws, need - 1, None, None) == MOE_ERR_WORKSPACE
    assert lib.gmm_bwd_weight(A16, A16b, A16c, 4, 64, 64, 64, A16c, MIS, need, None, None) == MOE_ERR_INVALID
    # gmm_bwd(x, dy, w, group_list, E, M_cap, K, N, dx, dw, ws, ws_bytes, dev_err, stream)
    need_b = lib.gmm_workspace_size(4, 64, 64, 64, 3)
    assert need_b == need
    D1, D2 = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    assert lib.gmm_bwd(A16, A16b, A16c, A16, 4, 64, 64, 64, None, D2, ws, need, None, None) == MOE_ERR_NULL
    assert lib.gmm_bwd(A16, A16b, A16c, A16, 4, 64, 64, 64, D1, None, ws, need, None, None) == MOE_ERR_NULL
    assert lib.gmm_bwd(None, A16b, A16c, A16, 4, 64, 64, 64, D1, D2, ws, need, None, None) == MOE_ERR_NULL
    assert lib.gmm_bwd(A16, A16b, A16c, A16, 4, 64, 64, 64, D1, D2, None, need, None, None) == MOE_ERR_WORKSPACE
    assert lib.gmm_bwd(MIS, A16b, A16c, A16, 4, 64, 64, 64, D1, D2, ws, need, None, None) == MOE_ERR_INVALID
    # outputs overlapping an input or each other
    assert lib.gmm_bwd(A16, A16b, A16c, A16, 4, 64, 64, 64, A16, D2, ws, need, None, None) == MOE_ERR_INVALID
    assert lib.gmm_bwd(A16, A16b, A16c, A16, 4, 64, 64, 64, D1, A16c, ws, need, None, None) == MOE_ERR_INVALID
    assert lib.gmm_bwd(A16, A16b, A16c, A16, 4, 64, 64, 64, D1,
                       ctypes.c_void_p(0x100000 + 64 * 64 * 2 - 16), ws, need, None, None) == MOE_ERR_INVALID
    # gmm_bwd_swiglu(x, dy, w, h, group_list, E, M_cap, K, N, dh, dw, ws, ws_bytes, dev_err, stream)
    Hh = ctypes.c_void_p(0x300000)
    sw = lambda x_, h_, dh_, dw_, ws_=ws, n_=need: lib.gmm_bwd_swiglu(  # noqa: E731
        x_, A16b, A16c, h_, A16, 4, 64, 64, 64, dh_, dw_, ws_, n_, None, None)
    assert sw(A16, Hh, None, D2) == MOE_ERR_NULL
    assert sw(A16, None, D1, D2) == MOE_ERR_NULL
    assert sw(A16, Hh, D1, D2, ws_=None) == MOE_ERR_WORKSPACE
    assert sw(A16, ctypes.c_void_p(0x300008), D1, D2) == MOE_ERR_INVALID   # misaligned h
    # dh may be h exactly, but not a shifted view of it, nor an input or dw
    assert sw(A16, Hh, ctypes.c_void_p(0x300000 + 256), D2) == MOE_ERR_INVALID
    assert sw(A16, Hh, A16b, D2) == MOE_ERR_INVALID
    assert sw(A16, Hh, D1, ctypes.c_void_p(0x100000 + 1024)) == MOE_ERR_INVALID
    assert sw(A16, Hh, D1, Hh) == MOE_ERR_INVALID
    # rows longer than 32-bit tile offsets can address, and oversized products
    big = 1 << 22
    assert lib.gmm_fwd(A16, A16b, A16c, 4, 64, big, 64, A16c, ws, 0, None, None) == MOE_ERR_INVALID
    assert lib.gmm_bwd_input(A16, A16b, A16c, 4, 64, 64, big, A16c, ws, 0, None, None) == MOE_ERR_INVALID
    assert lib.gmm_fwd(A16, A16b, A16c, 1024, 64, 1 << 21, 1 << 21, A16c, ws, 0, None, None) == MOE_ERR_INVALID


def test_permute_rejects_bad_arguments(lib):
    need = lib.moe_permute_workspace_size(64, 8, 256)
    ws = ctypes.c_void_p(0x50000)
    args = dict(x=A16, ids=A16b, T=64, k=8, H=2048, E=256, xp=A16c, rmap=A16, ss=A16b, tpe=A16c)

    def call(**kw):
        a = dict(args, **kw)
        return lib.moe_permute(a["x"], a["ids"], a["T"], a["k"], a["H"], a["E"], a["xp"], a["rmap"],
                               a["ss"], a["tpe"], kw.get("ws", ws), kw.get("wsb", need), None, None)

    assert call(x=None) == MOE_ERR_NULL
    assert call(tpe=None) == MOE_ERR_NULL
    assert call(ws=None) == MOE_ERR_NULL
    assert call(k=0) == MOE_ERR_INVALID
    assert call(k=33) == MOE_ERR_INVALID
    assert call(E=0) == MOE_ERR_INVALID
    assert call(E=1025) == MOE_ERR_INVALID
    assert call(H=100) == MOE_ERR_INVALID
    assert call(T=-1) == MOE_ERR_INVALID
    assert call(x=MIS) == MOE_ERR_INVALID
    assert call(wsb=need - 1) == MOE_ERR_WORKSPACE


def test_elementwise_reject_bad_arguments(lib):
    assert lib.swiglu(A16, None, 4, 64, 64, A16b, None) == MOE_ERR_NULL
    assert lib.swiglu(A16, A16c, 4, 64, 60, A16b, None) == MOE_ERR_INVALID
    assert lib.swiglu(MIS, A16c, 4, 64, 64, A16b, None) == MOE_ERR_INVALID
    assert lib.swiglu_bwd(A16, A16b, A16c, 4, 64, 64, None, None) == MOE_ERR_NULL
    assert lib.moe_unpermute(A16, None, A16b, 4, 2, 64, A16c, None, None) == MOE_ERR_NULL
    assert lib.moe_unpermute(A16, A16b, A16c, 4, 33, 64, A16c, None, None) == MOE_ERR_INVALID
    assert lib.moe_unpermute(A16, A16b, A16c, 4, 2, 12, A16c, None, None) == MOE_ERR_INVALID


def test_end_backward_calls_reject_bad_arguments(lib):
    # moe_unpermute_bwd(dout, y_perm, row_id_map, probs, T, top_k, H, dy_perm, dprobs, dev_err, stream)
    good = dict(dout=A16, yp=A16b, rmap=A16c, probs=A16, T=8, k=2, H=64, dyp=A16b, dp=A16c)

    def ub(**kw):
        a = dict(good, **kw)
        return lib.moe_unpermute_bwd(a["dout"], a["yp"], a["rmap"], a["probs"], a["T"], a["k"], a["H"],
                                     a["dyp"], a["dp"], None, None)

    assert ub(dout=None) == MOE_ERR_NULL
    assert ub(dp=None) == MOE_ERR_NULL
    assert ub(k=0) == MOE_ERR_INVALID
    assert ub(k=33) == MOE_ERR_INVALID
    assert ub(H=100) == MOE_ERR_INVALID
    assert ub(T=-1) == MOE_ERR_INVALID
    assert ub(dyp=MIS) == MOE_ERR_INVALID
    assert ub(T=0, dout=None, yp=None, rmap=None, probs=None, dyp=None, dp=None) == MOE_OK
    # moe_permute_bwd(dx_perm, row_id_map, T, top_k, H, dx, dev_err, stream)
    assert lib.moe_permute_bwd(None, A16c, 8, 2, 64, A16, None, None) == MOE_ERR_NULL
    assert lib.moe_permute_bwd(A16, A16c, 8, 2, 64, None, None, None) == MOE_ERR_NULL
    assert lib.moe_permute_bwd(A16, A16c, 8, 0, 64, A16b, None, None) == MOE_ERR_INVALID
    assert lib.moe_permute_bwd(A16, A16c, 8, 2, 12, A16b, None, None) == MOE_ERR_INVALID
    assert lib.moe_permute_bwd(MIS, A16c, 8, 2, 64, A16b, None, None) == MOE_ERR_INVALID
    assert lib.moe_permute_bwd(None, None, 0, 2, 64, None, None, None) == MOE_OK


def test_fused_swiglu_rejects_bad_arguments(lib):
    ws = ctypes.c_void_p(0x40000)
    # gmm_fwd_swiglu(x, w1, group_list, E, M_cap, K, I, a, h, ws, ws_bytes, dev_err, stream)
    assert lib.gmm_fwd_swiglu(A16, None, A16c, 4, 64, 64, 32, A16b, None, ws, 0, None, None) == MOE_ERR_NULL
    assert lib.gmm_fwd_swiglu(A16, A16b, A16c, 4, 64, 64, 12, A16b, None, ws, 0, None, None) == MOE_ERR_INVALID
    assert lib.gmm_fwd_swiglu(A16, A16b, A16c, 4, 64, 64, 1 << 21, A16b, None, ws, 0, None, None) == MOE_ERR_INVALID
    assert lib.gmm_fwd_swiglu(A16, A16b, A16c, 4, 64, 64, 32, MIS, None, ws, 0, None, None) == MOE_ERR_INVALID
    assert lib.gmm_fwd_swiglu(A16, A16b, A16c, 4, 64, 64, 32, A16b, MIS, ws, 0, None, None) == MOE_ERR_INVALID


def test_mx_calls_reject_bad_arguments(lib):
    # mx_quantize(x, rows, K, ld_s, q, s, stream)
    assert lib.mx_quantize(None, 4, 64, 16, A16b, A16c, None) == MOE_ERR_NULL
    assert lib.mx_quantize(A16, 4, 48, 16, A16b, A16c, None) == MOE_ERR_INVALID   # K % 32
    assert lib.mx_quantize(A16, 4, 64, 8, A16b, A16c, None) == MOE_ERR_INVALID    # ld % 16
    assert lib.mx_quantize(A16, 4, 1024, 16, A16b, A16c, None) == MOE_ERR_INVALID  # ld < K/32
    assert lib.mx_quantize(A16, -1, 64, 16, A16b, A16c, None) == MOE_ERR_INVALID
    assert lib.mx_quantize(MIS, 4, 64, 16, A16b, A16c, None) == MOE_ERR_INVALID
    assert lib.mx_quantize(None, 0, 64, 16, None, None, None) == MOE_OK
    # gmm_mx_fwd(xq, xs, ld_xs, wq, ws, ld_ws, gl, E, M_cap, K, N, y, dev_err, stream)
    good = dict(xq=A16, xs=A16b, lx=16, wq=A16c, wsc=A16, lw=16, gl=A16b, E=4, M=64, K=64, N=64,
                y=A16c)

    def g(**kw):
        a = dict(good, **kw)
        return lib.gmm_mx_fwd(a["xq"], a["xs"], a["lx"], a["wq"], a["wsc"], a["lw"], a["gl"], a["E"],
                              a["M"], a["K"], a["N"], a["y"], None, None)

    assert g(wsc=None) == MOE_ERR_NULL
    assert g(y=None) == MOE_ERR_NULL
    assert g(K=48) == MOE_ERR_INVALID
    assert g(lx=8) == MOE_ERR_INVALID
    assert g(lw=0) == MOE_ERR_INVALID
    assert g(xs=MIS) == MOE_ERR_INVALID
    assert g(E=0) == MOE_ERR_INVALID
    assert g(N=1 << 22) == MOE_ERR_INVALID
    # one expert's codes past 31-bit offsets (N * K > 0x7FFF0000), each dim in range
    assert g(K=1 << 16, N=1 << 16, lx=2048, lw=2048) == MOE_ERR_INVALID
    # gmm_mx_fwd_swiglu(..., E, M_cap, K, I, aq, as, ld_as, dev_err, stream)
    sw = dict(good, I=32, aq=A16c, asc=A16, la=16)

    def s(**kw):
        a = dict(sw, **kw)
        return lib.gmm_mx_fwd_swiglu(a["xq"], a["xs"], a["lx"], a["wq"], a["wsc"], a["lw"], a["gl"],
                                     a["E"], a["M"], a["K"], a["I"], a["aq"], a["asc"], a["la"],
                                     None, None)

    assert s(I=48) == MOE_ERR_INVALID   # I % 32
    assert s(la=8) == MOE_ERR_INVALID
    assert s(asc=None) == MOE_ERR_NULL
    assert s(aq=MIS) == MOE_ERR_INVALID
    assert s(K=1 << 16, I=1 << 15, lx=2048, lw=2048, la=1024) == MOE_ERR_INVALID  # 2I * K = 2^32
    # moe_permute_mx(x, ids, T, k, H, E, xq, xs, ld_xs, rmap, ss, tpe, ws, ws_bytes, dev_err, stream)
    need = lib.moe_permute_workspace_size(64, 8, 256)
    ws = ctypes.c_void_p(0x50000)

    def p(H=2048, ld=64, xs=A16c, wsb=need):
        return lib.moe_permute_mx(A16, A16b, 64, 8, H, 256, A16c, xs, ld, A16, A16b, A16c, ws, wsb,
                                  None, None)

    assert p(xs=None) == MOE_ERR_NULL
    assert p(H=2056) == MOE_ERR_INVALID  # H % 32
    assert p(ld=48) == MOE_ERR_INVALID   # ld < H/32
    assert p(wsb=need - 1) == MOE_ERR_WORKSPACE


def test_gathered_calls_reject_bad_arguments(lib):
    """moe_permute_index and the gathered forward GMMs validate their token
    arguments on the host: nulls, top_k, M_cap beyond T*top_k, a token matrix
    of 2^30 or more elements (byte offsets must fit 31 bits), misalignment,
    a short permute workspace."""
    ws = ctypes.c_void_p(0x40000)
    S4 = ctypes.c_void_p(0x50000)  # sorted_slot (int32)
    # gmm_fwd_gather(x, sorted_slot, T, top_k, w, group_list, E, M_cap, K, N, y, ws, ws_bytes, err, stream)
    g = lambda x_=A16, s_=S4, T=16, k=4, M=64, K=64, y_=A16c: lib.gmm_fwd_gather(  # noqa: E731
        x_, s_, T, k, A16b, A16, 4, M, K, 64, y_, ws, 0, None, None)
    assert g(x_=None) == MOE_ERR_NULL
    assert g(s_=None) == MOE_ERR_NULL
    assert g(y_=None) == MOE_ERR_NULL
    assert g(k=0) == MOE_ERR_INVALID
    assert g(k=33) == MOE_ERR_INVALID
    assert g(T=-1) == MOE_ERR_INVALID
    assert g(M=65) == MOE_ERR_INVALID            # more grouped rows than slots
    assert g(T=1 << 17, M=64, K=8192) == MOE_ERR_INVALID  # T*K == 2^30
    assert g(x_=MIS) == MOE_ERR_INVALID
    assert g(s_=ctypes.c_void_p(0x50002)) == MOE_ERR_INVALID
    # gmm_fwd_swiglu_gather(x, sorted_slot, T, top_k, w1, group_list, E, M_cap, K, I, a, h, ws, ws_bytes, ...)
    gs = lambda I=32, h_=None, k=4: lib.gmm_fwd_swiglu_gather(  # noqa: E731
        A16, S4, 16, k, A16b, A16, 4, 64, 64, I, A16c, h_, ws, 0, None, None)
    assert gs(I=30) == MOE_ERR_INVALID
    assert gs(h_=MIS) == MOE_ERR_INVALID
    assert gs(k=0) == MOE_ERR_INVALID
    # moe_permute_index(ids, T, top_k, E, row_id_map, sorted_slot, tpe, ws, ws_bytes, err, stream)
    need = lib.moe_permute_workspace_size(64, 8, 128)
    pi = lambda ids=A16, rm=A16b, ss=A16c, tpe=S4, w=ws, n=need, T=64, k=8, E=128: lib.moe_permute_index(  # noqa: E731
        ids, T, k, E, rm, ss, tpe, w, n, None, None)
    assert pi(w=None) == MOE_ERR_NULL
    assert pi(tpe=None) == MOE_ERR_NULL
    assert pi(ids=None) == MOE_ERR_NULL
    assert pi(ss=None) == MOE_ERR_NULL
    assert pi(n=need - 1) == MOE_ERR_WORKSPACE
    assert pi(E=0) == MOE_ERR_INVALID
    assert pi(k=33) == MOE_ERR_INVALID
    assert pi(tpe=ctypes.c_void_p(0x50004)) == MOE_ERR_INVALID
    # gmm_mx_fwd_swiglu_gather(xq, xs, ld_xs, sorted_slot, T, top_k, w1q, w1s, ld_w1s, group_list,
    #                          E, M_cap, K, I, aq, as, ld_as, err, stream)
    mxg = lambda s_=S4, T=16, k=4, M=64, K=64, I=32: lib.gmm_mx_fwd_swiglu_gather(  # noqa: E731
        A16, A16b, 16, s_, T, k, A16c, A16, 16, A16b, 4, M, K, I, A16c, A16, 16, None, None)
    assert mxg(s_=None) == MOE_ERR_NULL
    assert mxg(M=65) == MOE_ERR_INVALID
    assert mxg(k=0) == MOE_ERR_INVALID
    assert mxg(I=48) == MOE_ERR_INVALID          # I % 32
    assert mxg(T=1 << 17, K=8192) == MOE_ERR_INVALID


def test_swiglu_gmm_fwd_rejects_bad_arguments(lib):
    """swiglu_gmm_fwd(h, w2, group_list, E, M_cap, I, N, a, y, dev_err, stream)."""
    D1, D2, D3 = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)
    f = lambda h=D1, a=D2, y=D3, I=64, M=64: lib.swiglu_gmm_fwd(h, A16b, A16, 4, M, I, 64, a, y, None, None)  # noqa: E731
    assert f(a=None) == MOE_ERR_NULL
    assert f(y=None) == MOE_ERR_NULL
    assert f(I=60) == MOE_ERR_INVALID
    assert f(a=MIS) == MOE_ERR_INVALID
    assert f(a=ctypes.c_void_p(0x100000 + 64 * 128 * 2 - 16)) == MOE_ERR_INVALID  # a overlaps h
    assert f(y=D2) == MOE_ERR_INVALID                                           # y overlaps a


def test_decode_fwd_rejects_bad_arguments(lib):
    """moe_decode_fwd(x, ids, probs, w1, w2, T, top_k, H, I, E, out, row_id_map,
    sorted_slot, tokens_per_expert, h, a, y_perm, dev_err, stream): nothing
    is enqueued for a call validation rejects."""
    T, K, H, I, E = 16, 4, 256, 128, 32
    base = [0x1000000 * (i + 1) for i in range(12)]
    p = [ctypes.c_void_p(b) for b in base]

    def call(*over, T=T, K=K, H=H, I=I, E=E):
        a = list(p)
        for i, v in over:
            a[i] = v
        x, ids, probs, w1, w2, out, rmap, ss, tpe, h, aa, yp = a
        return lib.moe_decode_fwd(x, ids, probs, w1, w2, T, K, H, I, E, out, rmap, ss, tpe, h, aa, yp, None, None)

    assert call((0, None)) == MOE_ERR_NULL          # x
    assert call((8, None)) == MOE_ERR_NULL          # tokens_per_expert
    assert call((11, None)) == MOE_ERR_NULL         # y_perm
    assert call((0, MIS)) == MOE_ERR_INVALID        # misaligned x
    assert call(K=0) == MOE_ERR_INVALID
    assert call(H=60) == MOE_ERR_INVALID
    assert call(T=80) == MOE_ERR_INVALID            # 320 slots > 8 per expert: not a decode shape
    assert call(H=8192) == MOE_ERR_INVALID          # staged rows past 32 KiB
    assert call((5, p[0])) == MOE_ERR_INVALID       # out on top of x
    assert call((11, ctypes.c_void_p(base[10] + 16))) == MOE_ERR_INVALID  # y_perm overlapping a
