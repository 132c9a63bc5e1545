"""kvx_fit_ridge_caches through the C-ABI: the ridge maps of every receiver
layer and role straight from the calibration caches ("Cross-Model KV Cache
Transfer in Production", The Closed-Form Ridge Mapping Pipeline, stage 2:
W = (X^T X + lambda I)^-1 X^T Y per layer pair; stage 3: the layer map).

The oracle fits on the gathered features of each receiver layer (the plain
definition, 65536-row duplicates and all); the library forms X^T X from the
alignment's runs (bit groups of the run lengths, exact doublings) and X^T Y
from run sums of the targets.  Checks, every element of every map:
* a two-head setting (6 -> 4 layers, taps -2/0/+2, 4096 receiver tokens of
  the synthetic string) vs the oracle, and vs kvx_fit_ridge_batched on the
  gathered features;
* a token map with one run of 33000 tokens (past 2^15: the top bit group
  repeats a run) followed by 2000 short runs, a revisited sender token and a
  clamped entry, vs the oracle on the clamped map;
* one role alone (the skipped role's statuses OK);
* zero feature columns with lambda 0 reported per problem as not positive
  definite.

kvx_fit_recolor_caches through the C-ABI: the moment-matched maps ("Prefill-
Free Cross-Family KV Cache Transfer ...", Methodology 3) of every receiver
layer and role from the same caches (feature moments from the runs, the
feature column sums weighted by run length).  Checks, every element of
every W and b:
* the two-head setting vs the oracle's Recolor fit on the gathered
  features, and vs kvx_fit_recolor on the gathered features;
* the long-run map (both roles, layers 1 and 2) vs the oracle;
* one role alone, a constant receiver column with rho_y 0 (not positive
  definite for that problem only) and, on a map with fewer distinct sender
  rows than outputs, every problem reported not converged.

Both fits: receiver rows of 3 heads x 64 (a partial output tile), and keys
stored rotated (rotated back at the sender and receiver positions) against
the oracle and the features path.
"""
import sys

import numpy as np
import pytest
import torch

from cross_model_kv_kvx_amd import kvx, synth
from oracle import kvx_oracle as O
from tests.kvx_cases import TOL_BF16

pytestmark = pytest.mark.gpu
DEV = "cuda"
LAM_REL = 1e-3
RHO_X = 1e-3      # duplicated taps (receiver layers 0 and 3 of 6 -> 4) make S_xx singular


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=DEV)


def small_setting(n_recv, seed, send_layers=6, recv_layers=4, stride=2):
    send_end, recv_end = synth.token_ends(n_recv, seed)
    sshape = synth.CacheShape(send_layers, len(send_end), 2, 128)
    rshape = synth.CacheShape(recv_layers, n_recv, 2, 128)
    d = {"taps": kvx.layer_map(send_layers, recv_layers, 3, stride),
         "tmap": kvx.align_tokens(dev_i32(send_end), dev_i32(recv_end)),
         "tmap_o": O.token_align(send_end, recv_end)}
    for r, role in enumerate(("k", "v")):
        d[f"{role}_send"] = synth.sender_cache(sshape, seed * 10 + r, DEV)
        d[f"{role}_recv"] = synth.receiver_cache(rshape, seed * 10 + 5 + r, DEV)
    return d


def oracle_fit(d, role, l, src_rows, lam_rel=LAM_REL):
    x = O.features(d[f"{role}_send"], src_rows, d["taps"][l])
    y = O.as_f64(d[f"{role}_recv"][l]).reshape(x.shape[0], -1)
    return O.ridge_fit(x, y, lam_rel=lam_rel)[0]


def test_fit_caches_vs_oracle_and_features_path():
    d = small_setting(4096, 31)
    wk, wv = kvx.fit_ridge_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"], d["taps"],
                                  lambda_rel=LAM_REL)
    torch.cuda.synchronize()
    L_R = d["taps"].shape[0]
    for role, w in (("k", wk), ("v", wv)):
        xs = [kvx.gather_features(d[f"{role}_send"], d["tmap"], d["taps"][l]) for l in range(L_R)]
        ys = [d[f"{role}_recv"][l].reshape(4096, -1) for l in range(L_R)]
        wb, _ = kvx.fit_ridge_batched(xs, ys, lambda_rel=LAM_REL)
        for l in range(L_R):
            wo = oracle_fit(d, role, l, d["tmap_o"])
            got = w[l].cpu().numpy().astype(np.float64)
            err = O.rel_err(got, wo)
            gap = O.rel_err(got, wb[l].cpu().numpy().astype(np.float64))
            say(f"  {role} layer {l}: max|err|/RMS vs oracle {err:.3e}, vs the features path {gap:.3e}")
            assert err <= TOL_BF16
            # both are fp32-accumulated solutions of one system: they agree
            # to far better than either's bound against the oracle
            assert gap <= 1e-3


def test_fit_caches_long_run_and_arbitrary_map():
    rng = np.random.default_rng(7)
    lens = [33000] + list(rng.integers(1, 40, size=2000))
    n = int(sum(lens))
    n_send = len(lens) + 5
    vals = np.arange(len(lens), dtype=np.int64)
    vals[1200] = vals[100]                # a sender token visited by two separate runs
    vals[-1] = n_send + 7                 # past the sender: clamped to n_send - 1
    tmap_h = np.repeat(vals, lens).astype(np.int32)
    clamped = np.clip(tmap_h, 0, n_send - 1)
    sshape = synth.CacheShape(6, n_send, 2, 128)
    rshape = synth.CacheShape(4, n, 2, 128)
    d = {"taps": kvx.layer_map(6, 4, 3, 2)}
    for r, role in enumerate(("k", "v")):
        d[f"{role}_send"] = synth.sender_cache(sshape, 70 + r, DEV)
        d[f"{role}_recv"] = synth.receiver_cache(rshape, 75 + r, DEV)
    st = []
    wk, wv = kvx.fit_ridge_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], dev_i32(tmap_h), d["taps"],
                                  lambda_rel=LAM_REL, status=st)
    torch.cuda.synchronize()
    assert st == [kvx.OK] * 8
    # receiver layers 1 and 2 (taps 0/2/4 and 1/3/5): layers 0 and 3 repeat a
    # tap, which leaves only lambda in some directions, and beside the
    # 33000-token run that system's condition number is near 1e6, past what
    # fp32 sums resolve to the parity bar for any accumulation order
    for role, w in (("k", wk), ("v", wv)):
        for l in (1, 2):
            wo = oracle_fit(d, role, l, clamped)
            err = O.rel_err(w[l].cpu().numpy().astype(np.float64), wo)
            say(f"  long run, {role} layer {l}: max|err|/RMS {err:.3e}")
            assert err <= TOL_BF16


def test_fit_caches_one_role_and_singular_status():
    d = small_setting(1500, 33)
    L_R = d["taps"].shape[0]
    st = []
    wk, wv = kvx.fit_ridge_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"], d["taps"],
                                  lambda_rel=LAM_REL, roles=("v",), status=st)
    torch.cuda.synchronize()
    assert wk is None and st == [kvx.OK] * (2 * L_R)
    for l in range(L_R):
        err = O.rel_err(wv[l].cpu().numpy().astype(np.float64), oracle_fit(d, "v", l, d["tmap_o"]))
        assert err <= TOL_BF16
    # sender layer 0 zeroed and lambda 0: the receiver layers that tap it
    # (layers 0 and 1 of the 6 -> 4 map) have zero feature columns, so an
    # exact zero pivot, in both roles
    for role in ("k", "v"):
        d[f"{role}_send"][0].zero_()
    assert all(0 in d["taps"][l] for l in (0, 1))
    st = []
    kvx.fit_ridge_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"], d["taps"],
                         lambda_rel=0.0, status=st)
    torch.cuda.synchronize()
    for z in (0, 1, L_R, L_R + 1):
        assert st[z] == kvx.ERR_NOT_SPD, st
    assert all(v in (kvx.OK, kvx.ERR_NOT_SPD) for v in st)
    with pytest.raises(kvx.KvxError):
        kvx.fit_ridge_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"], d["taps"],
                             lambda_rel=0.0)


def oracle_recolor(d, role, l, src_rows, rho_x=RHO_X):
    x = O.features(d[f"{role}_send"], src_rows, d["taps"][l])
    y = O.as_f64(d[f"{role}_recv"][l]).reshape(x.shape[0], -1)
    return O.recolor_fit(x, y, rho_x=rho_x)


def recolor_err(w, b, wo, bo):
    return (O.rel_err(w.cpu().numpy().astype(np.float64), wo),
            O.rel_err(b.cpu().numpy().astype(np.float64), bo))


def test_recolor_caches_vs_oracle_and_features_path():
    d = small_setting(4096, 31)
    st, info = [], {}
    wk, wv, bk, bv = kvx.fit_recolor_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"],
                                            d["taps"], rho_x=RHO_X, status=st, info=info)
    torch.cuda.synchronize()
    L_R = d["taps"].shape[0]
    assert st == [kvx.OK] * (2 * L_R)
    say(f"  recolor from caches: {info['iters']} polar iterations")
    for role, w, b in (("k", wk, bk), ("v", wv, bv)):
        xs = [kvx.gather_features(d[f"{role}_send"], d["tmap"], d["taps"][l]) for l in range(L_R)]
        ys = [d[f"{role}_recv"][l].reshape(4096, -1) for l in range(L_R)]
        wf, bf = kvx.fit_recolor(xs, ys, rho_x=RHO_X)
        for l in range(L_R):
            wo, bo = oracle_recolor(d, role, l, d["tmap_o"])
            ew, eb = recolor_err(w[l], b[l], wo, bo)
            gw, gb = recolor_err(w[l], b[l], wf[l].cpu().numpy().astype(np.float64),
                                 bf[l].cpu().numpy().astype(np.float64))
            say(f"  {role} layer {l}: W {ew:.3e}, b {eb:.3e} vs the oracle; W {gw:.3e}, b {gb:.3e} vs the "
                f"features path")
            assert ew <= TOL_BF16 and eb <= TOL_BF16
            # both solve one fp64 problem from fp32-accumulated moments that
            # differ only in summation order
            assert gw <= 5e-3 and gb <= 5e-3


def test_recolor_caches_long_run():
    rng = np.random.default_rng(7)
    lens = [33000] + list(rng.integers(1, 40, size=2000))
    n = int(sum(lens))
    n_send = len(lens) + 5
    vals = np.arange(len(lens), dtype=np.int64)
    vals[1200] = vals[100]
    vals[-1] = n_send + 7
    tmap_h = np.repeat(vals, lens).astype(np.int32)
    clamped = np.clip(tmap_h, 0, n_send - 1)
    sshape = synth.CacheShape(6, n_send, 2, 128)
    rshape = synth.CacheShape(4, n, 2, 128)
    d = {"taps": kvx.layer_map(6, 4, 3, 2)}
    for r, role in enumerate(("k", "v")):
        d[f"{role}_send"] = synth.sender_cache(sshape, 80 + r, DEV)
        d[f"{role}_recv"] = synth.receiver_cache(rshape, 85 + r, DEV)
    st = []
    wk, wv, bk, bv = kvx.fit_recolor_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], dev_i32(tmap_h),
                                            d["taps"], rho_x=RHO_X, status=st)
    torch.cuda.synchronize()
    for role, w, b in (("k", wk, bk), ("v", wv, bv)):
        for l in (1, 2):
            assert st[(0 if role == "k" else 4) + l] == kvx.OK
            wo, bo = oracle_recolor(d, role, l, clamped)
            ew, eb = recolor_err(w[l], b[l], wo, bo)
            say(f"  long run, {role} layer {l}: W {ew:.3e}, b {eb:.3e}")
            assert ew <= TOL_BF16 and eb <= TOL_BF16


def test_recolor_caches_one_role_and_statuses():
    d = small_setting(4096, 34)
    L_R = d["taps"].shape[0]
    # a constant target column of V layer 2: S_yy singular with rho_y = 0
    d["v_recv"][2][:, 1, 5] = 2.0
    st = []
    wk, wv, bk, bv = kvx.fit_recolor_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"],
                                            d["taps"], rho_x=RHO_X, roles=("v",), status=st)
    torch.cuda.synchronize()
    assert wk is None and bk is None
    assert st == [kvx.OK] * L_R + [kvx.OK, kvx.OK, kvx.ERR_NOT_SPD, kvx.OK], st
    for l in (0, 1, 3):
        wo, bo = oracle_recolor(d, "v", l, d["tmap_o"])
        ew, eb = recolor_err(wv[l], bv[l], wo, bo)
        assert ew <= TOL_BF16 and eb <= TOL_BF16
    with pytest.raises(kvx.KvxError) as ei:
        kvx.fit_recolor_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"], d["taps"],
                               rho_x=RHO_X, roles=("v",))
    assert ei.value.status == kvx.ERR_NOT_SPD
    # 100 distinct sender rows for 256 outputs: the whitened cross-covariance
    # has rank below 256, so the Procrustes factor is not determined
    tmap_h = np.repeat(np.arange(100, dtype=np.int32), 15)
    sshape = synth.CacheShape(6, 120, 2, 128)
    rshape = synth.CacheShape(4, tmap_h.size, 2, 128)
    ks, kr = synth.sender_cache(sshape, 90, DEV), synth.receiver_cache(rshape, 91, DEV)
    st = []
    kvx.fit_recolor_caches(ks, None, kr, None, dev_i32(tmap_h), d["taps"], rho_x=RHO_X, roles=("k",), status=st)
    torch.cuda.synchronize()
    assert st == [kvx.ERR_NOT_CONVERGED] * L_R + [kvx.OK] * L_R, st


def test_fit_caches_ragged_output_width():
    """Receiver rows of 3 heads x 64 (F_out = 192: a partial 256-wide output
    tile) from sender rows of 2 x 128 at taps -2/0/+2 (F_in = 768): both fits
    from the caches vs the oracle, every element."""
    n = 3000
    send_end, recv_end = synth.token_ends(n, 41)
    d = {"taps": kvx.layer_map(6, 4, 3, 2), "tmap": kvx.align_tokens(dev_i32(send_end), dev_i32(recv_end)),
         "tmap_o": O.token_align(send_end, recv_end)}
    for r, role in enumerate(("k", "v")):
        d[f"{role}_send"] = synth.sender_cache(synth.CacheShape(6, len(send_end), 2, 128), 410 + r, DEV)
        d[f"{role}_recv"] = synth.receiver_cache(synth.CacheShape(4, n, 3, 64), 415 + r, DEV)
    wk, wv = kvx.fit_ridge_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"], d["taps"],
                                  lambda_rel=LAM_REL)
    st = []
    rk, rv, bk, bv = kvx.fit_recolor_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"],
                                            d["taps"], rho_x=RHO_X, status=st)
    torch.cuda.synchronize()
    assert wk.shape == (4, 768, 192) and bk.shape == (4, 192)
    assert st == [kvx.OK] * 8, st
    for role, w, rw, rb in (("k", wk, rk, bk), ("v", wv, rv, bv)):
        for l in range(4):
            err = O.rel_err(w[l].cpu().numpy().astype(np.float64), oracle_fit(d, role, l, d["tmap_o"]))
            ew, eb = recolor_err(rw[l], rb[l], *oracle_recolor(d, role, l, d["tmap_o"]))
            say(f"  F_out 192, {role} layer {l}: ridge {err:.3e}, Recolor W {ew:.3e} b {eb:.3e}")
            assert err <= TOL_BF16 and ew <= TOL_BF16 and eb <= TOL_BF16


def test_fits_from_rotated_caches():
    """Keys stored rotated (sender base 1e4, receiver base 1e6) in the
    two-head setting at 8192 tokens (about 1860 distinct sender rows for 768
    features): the key rows are rotated back at the sender positions and,
    like the features kvx_gather_features writes, rounded to bf16 for the
    matrix cores; the target keys are rotated back at the receiver positions
    and summed in fp32.  So both fits are checked, every element, against
    the oracle fitted on the features rotated back in fp64 and rounded
    fp64 -> fp32 -> bf16 (a rounding taken in a different precision than the
    kernel's only where the fp32 rotation lands within 2^-24 of a bf16
    rounding boundary: a few elements in 10^5, each one bf16 step) and the
    targets rotated back in fp64; the value maps (never rotated) as without
    rotation; and the key maps against the features path fed the rows
    kvx_gather_features rotates back (which also rounds the targets)."""
    n = 8192
    sb, rb = 1e4, 1e6
    d = small_setting(n, 43)
    L_R = d["taps"].shape[0]
    wk, wv = kvx.fit_ridge_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"], d["taps"],
                                  lambda_rel=LAM_REL, send_rope=sb, recv_rope=rb)
    st = []
    rk, rv, bk, bv = kvx.fit_recolor_caches(d["k_send"], d["v_send"], d["k_recv"], d["v_recv"], d["tmap"],
                                            d["taps"], rho_x=RHO_X, send_rope=sb, recv_rope=rb, status=st)
    torch.cuda.synchronize()
    assert st == [kvx.OK] * (2 * L_R), st
    ident = dev_i32(np.arange(n))
    xs = [kvx.gather_features(d["k_send"], d["tmap"], d["taps"][l], derotate=True, rope_base=sb) for l in range(L_R)]
    ys = [kvx.gather_features(d["k_recv"], ident, [l], derotate=True, rope_base=rb) for l in range(L_R)]
    wf, _ = kvx.fit_ridge_batched(xs, ys, lambda_rel=LAM_REL)
    for l in range(L_R):
        x = O.features(d["k_send"], d["tmap_o"], d["taps"][l], derotate_base=sb)
        x = O.bf16_bits_to_f64(O.f32_to_bf16_bits(x.astype(np.float32)))
        y = O.rope_rotate(O.as_f64(d["k_recv"][l]), np.arange(n), rb, -1).reshape(n, -1)
        err = O.rel_err(wk[l].cpu().numpy().astype(np.float64), O.ridge_fit(x, y, lam_rel=LAM_REL)[0])
        gap = O.rel_err(wk[l].cpu().numpy().astype(np.float64), wf[l].cpu().numpy().astype(np.float64))
        ew, eb = recolor_err(rk[l], bk[l], *O.recolor_fit(x, y, rho_x=RHO_X))
        ev = O.rel_err(wv[l].cpu().numpy().astype(np.float64), oracle_fit(d, "v", l, d["tmap_o"]))
        evr, ebr = recolor_err(rv[l], bv[l], *oracle_recolor(d, "v", l, d["tmap_o"]))
        say(f"  rotated keys, layer {l}: ridge K {err:.3e} (features path {gap:.3e}), Recolor K W {ew:.3e} "
            f"b {eb:.3e}; V ridge {ev:.3e}, Recolor {evr:.3e} / {ebr:.3e}")
        assert max(err, ew, eb, ev, evr, ebr) <= TOL_BF16
        # the features path also rounds the rotated-back targets to bf16
        assert gap <= TOL_BF16
