"""The calibration workload at its configured size, through the C-ABI.

Ridge fit of every receiver layer and role of the 36 -> 32 cross-family
pair: 64 problems, each 65536 calibration rows of 3072 gathered bf16 sender
features (taps -4/0/+4) -> 1024 receiver outputs, G = X^T X and X^T Y
accumulated in fp32 on matrix cores, lambda = 1e-3 trace(G)/3072, one batched
call (the left-looking factorisation and solves that a full chip of problems
takes).  Then a fresh 16384-token cache is translated with the fitted fp32
maps ("Cross-Model KV Cache Transfer in Production", The Closed-Form Ridge
Mapping Pipeline, stage 2: W = (X^T X + lambda I)^-1 X^T Y; stage 4: the maps
applied to new caches).

Checks:
* W of layers 0, 15 and 31 (both roles; 0 and 31 carry duplicated taps) vs
  the oracle's fp64 fit on the oracle's own features, element by element;
* every one of the 64 fits against its normal equations (G + lambda I) W r =
  X^T Y r on random probe vectors r, with G and X^T Y formed exactly (fp64
  products of the bf16 data), so the residual measures only the fit's own
  rounding;
* the fresh cache translated with the fitted maps, 256 sampled receiver rows,
  layers 0, 15 and 31, vs the oracle translating with the oracle's fits.
"""
import sys

import numpy as np
import pytest
import torch

from cross_model_kv_kvx_amd import kvx, synth
from oracle import kvx_oracle as O
from tests.kvx_cases import TOL_BF16, bf16_floor, rows_of, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CAL = 65536
N_FRESH = 16384
LAM_REL = 1e-3
CHECK_LAYERS = (0, 15, 31)

# Freivalds bound.  With W_gpu solving (G + dG + lambda' I) W = C + dC in fp64,
# the exact residual is (G + lambda I) W - C = dC - (dG + (lambda' - lambda) I) W.
# dG, dC come from fp32 accumulation of 65536 products per entry, two row
# halves accumulated separately by the matrix cores (each MFMA adds 16 exact
# products into an fp32 accumulator: about 2048 roundings of a running sum per
# half) and added in fp64.  A running sum of s terms of mean-square size m
# rounds with relative error u = 2^-24 at each step, so one half contributes
# about u sqrt(2048) |partial sum| per entry.  Diagonal entries grow linearly
# (|sum| ~ 32768 for unit features): |dG_ii| ~ 6e-8 * 45 * 32768 / sqrt(3) ~
# 0.05; off-diagonal sums are random walks (|sum| ~ 181): |dG_ij| ~ 6e-8 * 45
# * 120 ~ 3e-4, a random matrix of norm ~ 3e-4 * 2 sqrt(3072) ~ 0.03.  So
# ||dG|| ~ 0.1 against eigenvalues of G + lambda I of about 4e4 .. 1e5 in the
# directions C occupies (C = X^T Y lies in the range of X^T), giving a
# relative residual of order 1e-6.  The bound below leaves a factor of 10
# for the outlier-free tail of the estimate.
FREIVALDS_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=DEV)


@pytest.fixture(scope="module")
def cal():
    """The calibration inputs (as the synthetic recipe of this workload
    draws them), every problem's gathered features on the device, and the
    64 fits of one batched call."""
    c = synth.CONFIGS[5]
    seed = c["seed"]
    send_end, recv_end = synth.token_ends(N_CAL, seed)
    shp = synth.CacheShape(36, len(send_end), 8, 128)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap = kvx.align_tokens(dev_i32(send_end), dev_i32(recv_end))
    tmap_o = O.token_align(send_end, recv_end)
    assert np.array_equal(tmap.cpu().numpy(), tmap_o)
    d = dict(send_end=send_end, recv_end=recv_end, taps=taps, tmap_o=tmap_o, tmap=tmap)
    xs, ys = [], []
    for r, role in enumerate(("k", "v")):
        d[f"{role}_send"] = synth.sender_cache(shp, seed * 100 + r, DEV)
        d[f"{role}_recv"] = synth.receiver_cache(synth.CacheShape(32, N_CAL, 8, 128), seed * 100 + 50 + r, DEV)
        for l in range(32):
            xs.append(kvx.gather_features(d[f"{role}_send"], tmap, taps[l]))
            ys.append(d[f"{role}_recv"][l].reshape(N_CAL, 1024))
    say(f"calibration: {len(xs)} problems, {N_CAL} rows, U = {1 + np.count_nonzero(np.diff(tmap_o))}")
    st = []
    ws, _ = kvx.fit_ridge_batched(xs, ys, lambda_rel=LAM_REL, status=st)
    torch.cuda.synchronize()
    assert st == [kvx.OK] * 64
    d["xs"], d["ys"], d["ws"] = xs, ys, ws
    d["oracle_w"] = {}
    yield d
    d.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def problem(role, l):
    return (0 if role == "k" else 32) + l


def test_cfg5_fit_vs_oracle(cal):
    """W of layers 0 / 15 / 31, K and V, vs the oracle's fp64 ridge fit on
    the oracle's own features (65536 x 3072 -> 1024 each)."""
    for role in ("k", "v"):
        for l in CHECK_LAYERS:
            x = O.features(cal[f"{role}_send"], cal["tmap_o"], cal["taps"][l])
            y = O.as_f64(cal[f"{role}_recv"][l]).reshape(N_CAL, 1024)
            wo, _, lam = O.ridge_fit(x, y, lam_rel=LAM_REL)
            cal["oracle_w"][(role, l)] = wo
            del x, y
            w = cal["ws"][problem(role, l)].cpu().numpy().astype(np.float64)
            err = O.rel_err(w, wo)
            say(f"  {role} layer {l}: W max|err|/RMS = {err:.3e} (lambda {lam:.5g})")
            assert err <= TOL_BF16


def test_cfg5_fit_normal_equations_all_problems(cal):
    """Every fit of the batched call against its normal equations on three
    random probes: ||(G + lambda I) W r - X^T Y r|| / ||X^T Y r||, with G r and
    X^T Y r formed as fp64 products of the bf16 data."""
    rng = np.random.default_rng(55)
    worst = 0.0
    for p in range(64):
        xd = cal["xs"][p].double()
        yd = cal["ys"][p].double()
        lam = LAM_REL * float((xd * xd).sum()) / 3072
        w = cal["ws"][p].double()  # [3072][1024], y = x W
        for _ in range(3):
            r = torch.as_tensor(rng.standard_normal(1024), device=DEV)
            wr = w @ r
            lhs = xd.T @ (xd @ wr) + lam * wr
            rhs = xd.T @ (yd @ r)
            res = float(torch.linalg.norm(lhs - rhs) / torch.linalg.norm(rhs))
            worst = max(worst, res)
            assert res <= FREIVALDS_TOL, f"problem {p}: residual {res:.3e}"
        del xd, yd
    say(f"  worst normal-equation residual over 64 problems: {worst:.3e}")


def test_cfg5_fit_from_caches(cal):
    """The same 64 fits by kvx_fit_ridge_caches straight from the caches (the
    Gram from the alignment's runs): layers 0 / 15 / 31 of both roles vs the
    oracle's fits, and every fit against its normal equations formed exactly
    from the gathered bf16 features, as for the batched call."""
    st = []
    wk, wv = kvx.fit_ridge_caches(cal["k_send"], cal["v_send"], cal["k_recv"], cal["v_recv"], cal["tmap"],
                                  cal["taps"], lambda_rel=LAM_REL, status=st)
    torch.cuda.synchronize()
    assert st == [kvx.OK] * 64
    for role, w in (("k", wk), ("v", wv)):
        for l in CHECK_LAYERS:
            wo = cal["oracle_w"].get((role, l))
            if wo is None:
                x = O.features(cal[f"{role}_send"], cal["tmap_o"], cal["taps"][l])
                y = O.as_f64(cal[f"{role}_recv"][l]).reshape(N_CAL, 1024)
                wo = O.ridge_fit(x, y, lam_rel=LAM_REL)[0]
                cal["oracle_w"][(role, l)] = wo
                del x, y
            err = O.rel_err(w[l].cpu().numpy().astype(np.float64), wo)
            say(f"  from caches, {role} layer {l}: W max|err|/RMS = {err:.3e}")
            assert err <= TOL_BF16
    rng = np.random.default_rng(56)
    worst = 0.0
    for p in range(64):
        xd = cal["xs"][p].double()
        yd = cal["ys"][p].double()
        lam = LAM_REL * float((xd * xd).sum()) / 3072
        w = (wk if p < 32 else wv)[p % 32].double()
        for _ in range(3):
            r = torch.as_tensor(rng.standard_normal(1024), device=DEV)
            wr = w @ r
            res = float(torch.linalg.norm(xd.T @ (xd @ wr) + lam * wr - xd.T @ (yd @ r)) /
                        torch.linalg.norm(xd.T @ (yd @ r)))
            worst = max(worst, res)
            assert res <= FREIVALDS_TOL, f"problem {p}: residual {res:.3e}"
        del xd, yd
    say(f"  from caches: worst normal-equation residual over 64 problems: {worst:.3e}")
    del wk, wv
    torch.cuda.empty_cache()


def test_cfg5_recolor_from_caches(cal):
    """The 64 Recolor fits of the workload by kvx_fit_recolor_caches (rho_x =
    1e-3: layers 0 and 31 repeat a tap): K layer 15 and V layer 31 vs the
    oracle's Recolor fit on its own features, and all 64 (W and b) vs
    kvx_fit_recolor on the gathered features."""
    st, info = [], {}
    wk, wv, bk, bv = kvx.fit_recolor_caches(cal["k_send"], cal["v_send"], cal["k_recv"], cal["v_recv"],
                                            cal["tmap"], cal["taps"], rho_x=1e-3, status=st, info=info)
    torch.cuda.synchronize()
    assert st == [kvx.OK] * 64
    say(f"  recolor from caches: {info['iters']} polar iterations")
    for role, l in (("k", 15), ("v", 31)):
        x = O.features(cal[f"{role}_send"], cal["tmap_o"], cal["taps"][l])
        y = O.as_f64(cal[f"{role}_recv"][l]).reshape(N_CAL, 1024)
        wo, bo = O.recolor_fit(x, y, rho_x=1e-3)
        del x, y
        w, b = (wk, bk) if role == "k" else (wv, bv)
        ew = O.rel_err(w[l].cpu().numpy().astype(np.float64), wo)
        eb = O.rel_err(b[l].cpu().numpy().astype(np.float64), bo)
        say(f"  recolor from caches, {role} layer {l}: W {ew:.3e}, b {eb:.3e} vs the oracle")
        assert ew <= TOL_BF16 and eb <= TOL_BF16
    wf, bf = kvx.fit_recolor(cal["xs"], cal["ys"], rho_x=1e-3)
    worst = 0.0
    for p in range(64):
        w, b = (wk, bk) if p < 32 else (wv, bv)
        gw = O.rel_err(w[p % 32].cpu().numpy().astype(np.float64), wf[p].cpu().numpy().astype(np.float64))
        gb = O.rel_err(b[p % 32].cpu().numpy().astype(np.float64), bf[p].cpu().numpy().astype(np.float64))
        worst = max(worst, gw, gb)
        assert gw <= 5e-3 and gb <= 5e-3, f"problem {p}: W {gw:.3e}, b {gb:.3e}"
    say(f"  recolor from caches vs the features path, worst over 64 problems: {worst:.3e}")
    del wk, wv, bk, bv, wf, bf
    torch.cuda.empty_cache()


def test_cfg5_translate_fresh_cache_with_fitted_maps(cal):
    """A fresh 16384-token cache (its own string and sender caches) aligned
    and translated with the fitted fp32 maps (high and low 16-bit halves in
    the kernel), no bias; layers 0 / 15 / 31 of 256 sampled rows vs the
    oracle translating with the oracle's fits of those layers."""
    if len(cal["oracle_w"]) < 2 * len(CHECK_LAYERS):
        pytest.skip("needs the oracle fits of test_cfg5_fit_vs_oracle")
    c = synth.CONFIGS[5]
    fs = c["fresh_seed"]
    fe, fr = synth.token_ends(N_FRESH, fs)
    shp = synth.CacheShape(36, len(fe), 8, 128)
    taps = cal["taps"]
    tmap = kvx.align_tokens(dev_i32(fe), dev_i32(fr))
    tmap_o = O.token_align(fe, fr)
    assert np.array_equal(tmap.cpu().numpy(), tmap_o)
    caches = {role: synth.sender_cache(shp, fs * 100 + r, DEV) for r, role in enumerate(("k", "v"))}
    maps = {role: torch.stack([cal["ws"][problem(role, l)] for l in range(32)]).contiguous() for role in ("k", "v")}
    k, v = kvx.translate(caches["k"], caches["v"], tmap, taps, maps["k"], maps["v"])
    torch.cuda.synchronize()
    rows = sample_rows(tmap_o, 256, 6)
    sel = np.asarray(CHECK_LAYERS)
    for role, out in (("k", k), ("v", v)):
        wo = [cal["oracle_w"][(role, l)] for l in CHECK_LAYERS]
        want = O.translate_rows(caches[role], tmap_o, taps[sel], wo, None, rows, per_head=False, recv_heads=8,
                                recv_head_dim=128)
        got = rows_of(out, rows)[sel]
        err = O.rel_err(got, want)
        say(f"  fresh cache {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16
