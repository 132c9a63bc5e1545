"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and its host-only logic (layer map, argument validation,
workspace sizes) behaves as documented.  No kernel is launched here: every
call below returns before the first HIP runtime call."""
import ctypes
import os
import re

import numpy as np
import pytest

from cross_model_kv_kvx_amd import kvx
from oracle import kvx_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvx.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvx_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    L = kvx.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(kvx.EXPORTS)
    out = os.popen(f"nm -D --defined-only {kvx.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_status_strings():
    assert kvx.status_string(0) == "ok"
    assert "positive definite" in kvx.status_string(4)
    assert kvx.status_string(99) == "unknown status"


@pytest.mark.parametrize("ls,lr,nt,stride", [(36, 32, 3, 4), (32, 80, 1, 4), (7, 3, 3, 2), (1, 4, 3, 4),
                                             (10, 1, 1, 4), (3, 5, 5, 1)])
def test_layer_map_matches_oracle(ls, lr, nt, stride):
    got = kvx.layer_map(ls, lr, nt, stride)
    assert np.array_equal(got, O.layer_taps(ls, lr, nt, stride))


def test_layer_map_rejects_bad_arguments():
    out = (ctypes.c_int32 * 64)()
    L = kvx.lib()
    assert L.kvx_layer_map(36, 32, 2, 4, out) == kvx.ERR_INVALID   # even tap count
    assert L.kvx_layer_map(0, 32, 3, 4, out) == kvx.ERR_INVALID
    assert L.kvx_layer_map(36, 32, 9, 4, out) == kvx.ERR_INVALID
    assert L.kvx_layer_map(36, 32, 3, 4, None) == kvx.ERR_INVALID


def desc(L, N, H, d, dt=kvx.BF16, rope=0.0):
    return kvx.CacheDesc(L, N, H, d, dt, rope)


def test_translate_validation_before_launch():
    L = kvx.lib()
    s, r = desc(36, 100, 8, 128), desc(32, 120, 8, 128)
    taps = kvx.layer_map(36, 32, 3, 4)
    tp = taps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    fake = ctypes.c_void_p(0x1000)
    args = dict(k_send=fake, v_send=fake, k_recv=fake, v_recv=fake, map=fake, wk=fake, wv=fake)

    def call(sd=s, rd=r, taps_p=tp, n_taps=3, per_head=0, w_dtype=kvx.BF16, ws=fake, ws_bytes=1 << 40, **kw):
        a = dict(args, **kw)
        return L.kvx_translate(ctypes.byref(sd), a["k_send"], a["v_send"], ctypes.byref(rd), a["k_recv"],
                               a["v_recv"], a["map"], taps_p, n_taps, per_head, w_dtype, a["wk"], a["wv"], None,
                               None, ws, ws_bytes, None)

    assert call(w_dtype=7) == kvx.ERR_INVALID
    assert call(n_taps=0) == kvx.ERR_INVALID
    assert call(taps_p=None) == kvx.ERR_INVALID
    assert call(k_send=None) == kvx.ERR_INVALID                  # K output without K input
    assert call(wv=None) == kvx.ERR_INVALID
    assert call(map=None) == kvx.ERR_INVALID
    bad = taps.copy()
    bad[3, 1] = 36                                               # tap past the last sender layer
    assert call(taps_p=bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))) == kvx.ERR_INVALID
    assert call(per_head=1) == kvx.ERR_SHAPE                     # per head needs one tap
    assert call(rd=desc(32, 120, 8, 128, kvx.F32)) == kvx.ERR_UNSUPPORTED
    assert call(ws=None) == kvx.ERR_WORKSPACE
    assert call(ws_bytes=16) == kvx.ERR_WORKSPACE
    assert call(sd=desc(0, 100, 8, 128)) == kvx.ERR_INVALID
    assert call(sd=desc(36, 100, 8, 127, rope=1e4)) == kvx.ERR_INVALID  # odd head dim with rotation
    kn = desc(32, 120, 8, 128)
    kn.k_norm = 0x2000
    kn.k_norm_eps = -1.0
    assert call(rd=kn) == kvx.ERR_INVALID                       # negative eps of the key norm
    kn.k_norm_eps = 1e-6
    ph = desc(32, 120, 8, 128)
    assert call(sd=desc(32, 100, 8, 128), rd=kn, taps_p=kvx.layer_map(32, 32, 1).ctypes.data_as(
        ctypes.POINTER(ctypes.c_int32)), n_taps=1, per_head=1) == kvx.ERR_UNSUPPORTED  # key norm: flattened only
    assert call(sd=desc(32, 100, 8, 128), rd=ph, taps_p=kvx.layer_map(32, 32, 1).ctypes.data_as(
        ctypes.POINTER(ctypes.c_int32)), n_taps=1, per_head=1, ws_bytes=16) == kvx.ERR_WORKSPACE
    assert call(rd=desc(32, 0, 8, 128)) == kvx.OK                # nothing to translate
    assert call(k_recv=None, v_recv=None) == kvx.OK              # no role requested

    noev = (ctypes.c_void_p * 3)(0x1000, 0, 0x1000)
    assert L.kvx_translate_recorded(ctypes.byref(s), fake, fake, ctypes.byref(r), fake, fake, fake, tp, 3, 0,
                                    kvx.BF16, fake, fake, None, None, fake, 1 << 40, None, noev) == kvx.ERR_INVALID

    def call8(sd=s, rd=r, sk=fake, sv=fake, ws_bytes=1 << 40):
        return L.kvx_translate_fp8(ctypes.byref(sd), fake, fake, ctypes.byref(rd), fake, fake, fake, tp, 3, fake,
                                   fake, sk, sv, None, None, fake, ws_bytes, None, None)

    assert call8(sk=None) == kvx.ERR_INVALID                     # fp8 maps need their scales
    assert call8(sv=None) == kvx.ERR_INVALID
    assert call8(sd=desc(36, 100, 8, 128, kvx.F32), rd=desc(32, 120, 8, 128, kvx.F32)) == kvx.ERR_UNSUPPORTED
    assert call8(ws_bytes=16) == kvx.ERR_WORKSPACE
    assert call8(rd=desc(32, 0, 8, 128)) == kvx.OK


def test_workspace_sizes_are_monotone_and_cover_the_key_rows():
    s, r = desc(36, 25000, 8, 128, rope=5e5), desc(32, 32768, 8, 128, rope=1e6)
    big = kvx.translate_workspace_size(s, r, 3, False)
    # rotated-back unique key rows: sender layers x min(N_R, N_S) rows x 2 KB
    assert big >= 36 * 25000 * 1024 * 2
    plain = kvx.translate_workspace_size(desc(36, 25000, 8, 128), desc(32, 32768, 8, 128), 3, False)
    assert plain < big
    assert kvx.translate_workspace_size(desc(32, 4096, 8, 128), desc(80, 4096, 8, 128), 1, True) >= 0
    L = kvx.lib()
    assert L.kvx_fit_ridge_workspace_size(3072, 1024) > 3072 * 3072 * 8
    assert L.kvx_fit_ridge_workspace_size(0, 1024) == 0
    assert L.kvx_align_workspace_size(1 << 20) > L.kvx_align_workspace_size(1000)


def test_other_entry_points_validate_before_launch():
    L = kvx.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.kvx_align_tokens(fake, 5, fake, 0, fake, None, 0, None) == kvx.OK   # empty receiver
    assert L.kvx_align_tokens(fake, 0, fake, 5, fake, fake, 1 << 30, None) == kvx.ERR_SHAPE
    assert L.kvx_align_tokens(fake, 5, fake, 5, fake, None, 0, None) == kvx.ERR_WORKSPACE
    assert L.kvx_align_tokens(None, 5, fake, 5, fake, fake, 1 << 30, None) == kvx.ERR_INVALID
    assert L.kvx_fit_ridge(fake, 64, fake, 64, kvx.BF16, 10, 64, 64, -1.0, 0.0, 0, fake, None, fake,
                           1 << 40, None) == kvx.ERR_INVALID
    assert L.kvx_fit_ridge(fake, 32, fake, 64, kvx.BF16, 10, 64, 64, 0.0, 0.0, 0, fake, None, fake,
                           1 << 40, None) == kvx.ERR_SHAPE
    assert L.kvx_fit_ridge(fake, 64, fake, 64, kvx.BF16, 10, 60, 64, 0.0, 0.0, 0, fake, None, fake,
                           1 << 40, None) == kvx.ERR_UNSUPPORTED
    assert L.kvx_fit_ridge(fake, 64, fake, 64, kvx.BF16, 10, 64, 64, 0.0, 0.0, 1, fake, None, fake,
                           1 << 40, None) == kvx.ERR_INVALID                     # intercept needs b_out
    assert L.kvx_fit_ridge(fake, 64, fake, 64, kvx.BF16, 10, 64, 64, 0.0, 0.0, 0, fake, None, fake,
                           16, None) == kvx.ERR_WORKSPACE
    arr = ctypes.c_void_p * 1
    ptrs = arr(0x1000)
    nul = arr(0)

    def recolor(count=1, ldx=64, f_in=64, f_out=64, dt=kvx.BF16, rx=1e-3, ry=0.0, w=ptrs, b=ptrs, ws=1 << 40):
        return L.kvx_fit_recolor(count, ptrs, ldx, ptrs, 64, dt, 10, f_in, f_out, rx, ry, w, b, None, None, fake,
                                 ws, None)

    assert recolor(count=0) == kvx.OK
    assert recolor(rx=-1.0) == kvx.ERR_INVALID
    assert recolor(b=nul) == kvx.ERR_INVALID                  # the bias is always written
    assert recolor(ldx=32) == kvx.ERR_SHAPE
    assert recolor(f_in=32, ldx=64) == kvx.ERR_UNSUPPORTED     # f_in < f_out
    assert recolor(f_in=60, f_out=56) == kvx.ERR_UNSUPPORTED   # bf16 rows in 16-byte pieces
    assert recolor(ws=16) == kvx.ERR_WORKSPACE
    assert L.kvx_fit_recolor_workspace_size(64, 3072, 1024) > 64 * 8 * (3072 * 3072 + 2 * 3072 * 1024)
    assert L.kvx_fit_recolor_workspace_size(0, 3072, 1024) == 0
    assert kvx.status_string(kvx.ERR_NOT_CONVERGED) == "iteration did not converge"
    assert L.kvx_quantize_fp8(fake, 0, 16, 16, fake, fake, None) == kvx.OK
    assert L.kvx_quantize_fp8(fake, 4, 0, 16, fake, fake, None) == kvx.ERR_INVALID
    assert L.kvx_quantize_fp8(fake, 4, 16, 0, fake, fake, None) == kvx.ERR_INVALID
    assert L.kvx_quantize_fp8(fake, 4, 16, 16, None, fake, None) == kvx.ERR_INVALID
    assert L.kvx_align_tokens_async(fake, 5, fake, 5, fake, None, fake, 1 << 30, None) == kvx.ERR_INVALID
    assert L.kvx_align_tokens_async(fake, 5, fake, 5, fake, fake, None, 0, None) == kvx.ERR_WORKSPACE
    assert L.kvx_align_tokens_async(fake, 5, fake, 0, fake, None, None, 0, None) == kvx.OK   # empty receiver
    assert L.kvx_fold_lowrank(fake, fake, fake, 0, 8, 8, 2, fake, kvx.BF16, None) == kvx.OK
    assert L.kvx_fold_lowrank(fake, None, fake, 1, 8, 8, 2, fake, kvx.BF16, None) == kvx.ERR_INVALID
    assert L.kvx_fold_lowrank(fake, fake, fake, 1, 8, 8, 2, fake, 5, None) == kvx.ERR_INVALID
    s = desc(4, 10, 2, 8)
    tp = np.array([0, 1], np.int32).ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert L.kvx_gather_features(ctypes.byref(s), fake, 1, fake, 3, tp, 2, fake, None) == kvx.ERR_INVALID
    bad = np.array([0, 4], np.int32).ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert L.kvx_gather_features(ctypes.byref(s), fake, 0, fake, 3, bad, 2, fake, None) == kvx.ERR_INVALID
    assert L.kvx_gather_features(ctypes.byref(s), fake, 0, fake, 0, tp, 2, fake, None) == kvx.OK


def test_prepared_maps_sizes_and_validation():
    """Sizes of the kernel layout of prepared maps (16-bit operands for the
    flattened bf16 path, hi|lo halves for fp32 maps, the map's own type per
    head and for fp32 caches) and argument checks before anything runs."""
    L = kvx.lib()
    fake = ctypes.c_void_p(0x1000)
    s, r = desc(36, 25000, 8, 128, rope=5e5), desc(32, 32768, 8, 128, rope=1e6)
    n = 32 * 3072 * 1024
    size = lambda *a: L.kvx_prepared_maps_size(ctypes.byref(a[0]), ctypes.byref(a[1]), *a[2:])
    assert size(s, r, 3, 0, 0, kvx.BF16) == 2 * n          # fp16 keys
    assert size(s, r, 3, 0, 1, kvx.BF16) == 2 * n          # bf16 values
    assert size(s, r, 3, 0, 0, kvx.F32) == 4 * n           # hi|lo halves
    ps, pr = desc(32, 4096, 8, 128), desc(80, 4096, 8, 128)
    assert size(ps, pr, 1, 1, 0, kvx.F32) == 80 * 8 * 128 * 128 * 4
    assert size(ps, pr, 1, 1, 1, kvx.BF16) == 80 * 8 * 128 * 128 * 2
    fs, fr = desc(5, 100, 2, 64, kvx.F32), desc(3, 90, 2, 64, kvx.F32)
    assert size(fs, fr, 3, 0, 0, kvx.F32) == 3 * 384 * 128 * 4
    assert size(s, r, 3, 0, 2, kvx.BF16) == 0              # no such role
    assert size(s, r, 3, 0, 0, 5) == 0
    prep = lambda *a, **k: L.kvx_prepare_maps(ctypes.byref(a[0]), ctypes.byref(a[1]), *a[2:])
    assert prep(s, r, 3, 0, 0, kvx.BF16, fake, fake, 16, None) == kvx.ERR_WORKSPACE
    assert prep(s, r, 3, 0, 0, kvx.BF16, None, fake, 1 << 40, None) == kvx.ERR_INVALID
    assert prep(s, r, 3, 1, 0, kvx.BF16, fake, fake, 1 << 40, None) == kvx.ERR_SHAPE   # per head: one tap
    assert prep(s, r, 3, 0, 3, kvx.BF16, fake, fake, 1 << 40, None) == kvx.ERR_INVALID
    taps = kvx.layer_map(36, 32, 3, 4)
    tp = taps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    ws_prep = L.kvx_translate_prepared_workspace_size(ctypes.byref(s), ctypes.byref(r), 3, 0, 0)
    assert 0 < ws_prep < kvx.translate_workspace_size(s, r, 3, False)   # no maps in it

    def tpp(w_dtype=kvx.BF16, ws_bytes=1 << 40, events=None):
        return L.kvx_translate_prepared(ctypes.byref(s), fake, fake, ctypes.byref(r), fake, fake, fake, tp, 3, 0,
                                        w_dtype, fake, fake, None, None, fake, ws_bytes, None, None, events)

    assert tpp(w_dtype=2) == kvx.ERR_INVALID
    assert tpp(ws_bytes=16) == kvx.ERR_WORKSPACE
    assert tpp(events=(ctypes.c_void_p * 3)(0x1000, 0, 0x1000)) == kvx.ERR_INVALID


def test_fit_from_caches_validation():
    """kvx_fit_ridge_caches: sizes and argument checks before anything runs."""
    L = kvx.lib()
    fake = ctypes.c_void_p(0x1000)
    s, r = desc(36, 50000, 8, 128), desc(32, 65536, 8, 128)
    taps = kvx.layer_map(36, 32, 3, 4)
    tp = taps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    size = kvx.fit_ridge_caches_workspace_size(s, r, 3)
    # the fp64 systems of 64 problems at least
    assert size > 64 * 8 * (3072 * 3072 + 3072 * 1024)
    assert kvx.fit_ridge_caches_workspace_size(s, desc(32, 0, 8, 128), 3) == 0
    assert kvx.fit_ridge_caches_workspace_size(s, r, 0) == 0

    def call(sd=s, rd=r, taps_p=tp, n_taps=3, lam=1e-3, wk=fake, wv=fake, ws=1 << 40, ks=fake, kr=fake,
             m=fake):
        return L.kvx_fit_ridge_caches(ctypes.byref(sd), ks, fake, ctypes.byref(rd), kr, fake, m, taps_p, n_taps,
                                      0.0, lam, wk, wv, None, fake, ws, None)

    assert call(wk=None, wv=None) == kvx.ERR_INVALID             # no role
    assert call(lam=-1.0) == kvx.ERR_INVALID
    assert call(ks=None) == kvx.ERR_INVALID                      # K output without K caches
    assert call(kr=None) == kvx.ERR_INVALID
    assert call(m=None) == kvx.ERR_INVALID
    assert call(taps_p=None) == kvx.ERR_INVALID
    bad = taps.copy()
    bad[5, 2] = 36
    assert call(taps_p=bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))) == kvx.ERR_INVALID
    # rotated keys are turned back 8 pairs at a time: head_dim a multiple of 16
    assert call(sd=desc(36, 50000, 32, 8, rope=1e4)) == kvx.ERR_UNSUPPORTED
    assert call(rd=desc(32, 65536, 32, 8, rope=1e6)) == kvx.ERR_UNSUPPORTED
    assert call(sd=desc(36, 50000, 8, 128, kvx.F32), rd=desc(32, 65536, 8, 128, kvx.F32)) == kvx.ERR_UNSUPPORTED
    assert call(sd=desc(36, 50000, 3, 64)) == kvx.ERR_UNSUPPORTED    # sender rows not a multiple of 256
    assert call(ks=ctypes.c_void_p(0x1008)) == kvx.ERR_UNSUPPORTED  # 16-byte pieces
    assert call(rd=desc(32, 0, 8, 128)) == kvx.ERR_SHAPE
    assert call(ws=16) == kvx.ERR_WORKSPACE


def test_recolor_from_caches_validation():
    """kvx_fit_recolor_caches: sizes and argument checks before anything runs."""
    L = kvx.lib()
    fake = ctypes.c_void_p(0x1000)
    s, r = desc(36, 50000, 8, 128), desc(32, 65536, 8, 128)
    taps = kvx.layer_map(36, 32, 3, 4)
    tp = taps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    size = kvx.fit_recolor_caches_workspace_size(s, r, 3)
    # more than the ridge fit's: the solve keeps Y^T Y, its factor and the
    # polar iterates per problem besides
    assert size > kvx.fit_ridge_caches_workspace_size(s, r, 3)
    assert size > 64 * 8 * (3072 * 3072 + 3072 * 1024 + 5 * 1024 * 1024)
    assert kvx.fit_recolor_caches_workspace_size(s, desc(32, 0, 8, 128), 3) == 0
    assert kvx.fit_recolor_caches_workspace_size(s, r, 0) == 0

    def call(sd=s, rd=r, taps_p=tp, n_taps=3, rho=1e-3, wk=fake, wv=fake, bk=fake, bv=fake, ws=1 << 40, ks=fake,
             m=fake):
        return L.kvx_fit_recolor_caches(ctypes.byref(sd), ks, fake, ctypes.byref(rd), fake, fake, m, taps_p,
                                        n_taps, rho, 0.0, wk, wv, bk, bv, None, None, fake, ws, None)

    assert call(wk=None, wv=None) == kvx.ERR_INVALID             # no role
    assert call(rho=-1.0) == kvx.ERR_INVALID
    assert call(rho=float("nan")) == kvx.ERR_INVALID
    assert call(bk=None) == kvx.ERR_INVALID                      # a fitted role needs its bias
    assert call(ks=None) == kvx.ERR_INVALID
    assert call(m=None) == kvx.ERR_INVALID
    assert call(taps_p=None) == kvx.ERR_INVALID
    assert call(sd=desc(36, 50000, 32, 8, rope=1e4)) == kvx.ERR_UNSUPPORTED
    assert call(sd=desc(36, 50000, 3, 64)) == kvx.ERR_UNSUPPORTED
    # F_in < F_out: one tap of a 2 x 128 sender row against 8 x 128 targets
    one = np.zeros((32, 1), dtype=np.int32)
    assert call(sd=desc(36, 50000, 2, 128), taps_p=one.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                n_taps=1) == kvx.ERR_UNSUPPORTED
    assert call(rd=desc(32, 0, 8, 128)) == kvx.ERR_SHAPE
    assert call(ws=16) == kvx.ERR_WORKSPACE
