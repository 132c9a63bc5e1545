"""Pins of the oracle's rotation, feature construction, affine maps, fold and
ridge fit, against closed forms, independent algorithms and brute force.

Sources: llms.blog ridge pipeline stages 1-4 (RoPE strip, per-head ridge
W = (X^T X + lambda I)^-1 X^T Y, layer alignment, RoPE re-application);
HeteroFold summary "Methodology" steps 2-3 (three taps, flattened maps,
rank-16 corrections folded into a fixed affine map).
"""
import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import kvx_oracle as O


# ---------------------------------------------------------------- number formats

def test_bf16_rounding_matches_torch_and_ties_to_even():
    assert O.f32_to_bf16_bits(np.float32(1.0)) == 0x3F80
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa -> 1.0
    assert O.f32_to_bf16_bits(np.float32(1.0 + 2.0 ** -8)) == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6
    assert O.f32_to_bf16_bits(np.float32(1.0 + 3 * 2.0 ** -8)) == 0x3F82
    x = (np.random.default_rng(0).standard_normal(100000) * 10).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(x), ref)
    back = O.bf16_bits_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------- rotation

def test_rope_matches_complex_multiplication_and_rotate_half():
    rng = np.random.default_rng(1)
    n, H, d, base = 37, 3, 16, 10000.0
    x = rng.standard_normal((n, H, d))
    pos = rng.integers(0, 40000, size=n)
    got = O.rope_rotate(x, pos, base, +1)
    # complex form: (a + i b) * exp(i pos theta_j), theta_j = exp(-(2j/d) ln base)
    theta = np.exp(-(2.0 * np.arange(d // 2) / d) * np.log(base))
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * theta)
    assert np.allclose(got, np.concatenate([z.real, z.imag], -1), rtol=0, atol=1e-9)
    # rotate-half form: x cos + rot(x) sin, rot(x) = (-x2, x1), cos/sin repeated
    ang = pos[:, None, None] * np.concatenate([theta, theta])
    rot = np.concatenate([-x[..., d // 2:], x[..., : d // 2]], -1)
    assert np.allclose(got, x * np.cos(ang) + rot * np.sin(ang), rtol=0, atol=1e-9)


def test_rope_identities():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 2, 128))
    pos = rng.integers(0, 32768, size=50)
    y = O.rope_rotate(x, pos, 5e5, +1)
    assert np.max(np.abs(O.rope_rotate(y, pos, 5e5, -1) - x)) < 1e-12
    assert np.array_equal(O.rope_rotate(x, np.zeros(50), 1e6, +1), x)
    # pair norms preserved
    pn = lambda v: v[..., :64] ** 2 + v[..., 64:] ** 2
    assert np.allclose(pn(y), pn(x), rtol=1e-12, atol=1e-12)
    # <R_p q, R_p' k> depends only on p - p'
    q, k = rng.standard_normal((1, 1, 128)), rng.standard_normal((1, 1, 128))
    dots = []
    for p0 in (0, 17, 3000):
        a = O.rope_rotate(q, [p0 + 5], 1e4, +1)
        b = O.rope_rotate(k, [p0], 1e4, +1)
        dots.append(float((a * b).sum()))
    assert np.allclose(dots, dots[0], rtol=1e-9)
    # d = 2 by hand: theta_0 = 1, (1, 0) rotated by position 1 -> (cos 1, sin 1)
    assert np.allclose(O.rope_rotate([[[1.0, 0.0]]], [1], 123.0, +1), [[[np.cos(1), np.sin(1)]]])


# ---------------------------------------------------------------- features / affine / translate

def brute_translate(cache, tmap, taps, w, b, rows, H, d, per_head, sb, rb):
    """Element-by-element loops over a tiny problem (no numpy matmul)."""
    L_R = len(taps)
    out = np.zeros((L_R, len(rows), H * d))
    for li in range(L_R):
        for ri, i in enumerate(rows):
            j = tmap[i]
            feat = []
            for t in taps[li]:
                for h in range(H):
                    v = [float(cache[t][j][h][c]) for c in range(d)]
                    if sb:
                        vv = list(v)
                        for q in range(d // 2):
                            ang = -j * sb ** (-2.0 * q / d)
                            vv[q] = v[q] * np.cos(ang) - v[q + d // 2] * np.sin(ang)
                            vv[q + d // 2] = v[q] * np.sin(ang) + v[q + d // 2] * np.cos(ang)
                        v = vv
                    feat.extend(v)
            y = []
            for o in range(H * d):
                if per_head:
                    h, c = divmod(o, d)
                    s = sum(feat[h * d + f] * w[li][h][f][c] for f in range(d))
                else:
                    s = sum(feat[f] * w[li][f][o] for f in range(len(feat)))
                y.append(s + (b[li][o] if b is not None else 0.0))
            if rb:
                for h in range(H):
                    seg = y[h * d:(h + 1) * d]
                    nw = list(seg)
                    for q in range(d // 2):
                        ang = i * rb ** (-2.0 * q / d)
                        nw[q] = seg[q] * np.cos(ang) - seg[q + d // 2] * np.sin(ang)
                        nw[q + d // 2] = seg[q] * np.sin(ang) + seg[q + d // 2] * np.cos(ang)
                    y[h * d:(h + 1) * d] = nw
            out[li, ri] = y
    return out


@pytest.mark.parametrize("per_head,sb,rb", [(False, 0.0, 0.0), (False, 500.0, 1000.0),
                                            (True, 0.0, 0.0), (True, 50.0, 70.0)])
def test_translate_rows_vs_brute_force(per_head, sb, rb):
    rng = np.random.default_rng(3)
    L_S, N_S, H, d = 5, 9, 2, 4
    n_taps = 1 if per_head else 3
    L_R = 3
    cache = rng.standard_normal((L_S, N_S, H, d))
    taps = O.layer_taps(L_S, L_R, n_taps, 2)
    tmap = np.array([0, 0, 1, 3, 3, 3, 4, 8])
    if per_head:
        w = rng.standard_normal((L_R, H, d, d))
    else:
        w = rng.standard_normal((L_R, n_taps * H * d, H * d))
    b = rng.standard_normal((L_R, H * d))
    rows = np.arange(len(tmap))
    got = O.translate_rows(cache, tmap, taps, w, b, rows, per_head=per_head, recv_heads=H,
                           recv_head_dim=d, send_rope_base=sb, recv_rope_base=rb)
    want = brute_translate(cache, tmap, taps, w, b, rows, H, d, per_head, sb, rb)
    assert np.max(np.abs(got - want)) < 1e-12


def test_one_row_by_hand():
    # H=1, d=2, one tap: x = (1, 2), W = [[1, 2], [3, 4]] (y = x W), b = (0.5, -1)
    # y = (1*1 + 2*3, 1*2 + 2*4) + b = (7.5, 9)
    cache = np.array([[[[1.0, 2.0]]]])
    W = np.array([[1.0, 2.0], [3.0, 4.0]])
    y = O.translate_rows(cache, [0], [[0]], [W], [[0.5, -1.0]], [0], per_head=False,
                         recv_heads=1, recv_head_dim=2)
    assert np.array_equal(y, [[[7.5, 9.0]]])


def test_identity_maps_reproduce_input_exactly():
    rng = np.random.default_rng(4)
    L, N, H, d = 3, 11, 2, 8
    cache = rng.standard_normal((L, N, H, d)).astype(np.float32)
    eye = np.broadcast_to(np.eye(d), (L, H, d, d))
    y = O.translate_rows(cache, np.arange(N), O.layer_taps(L, L, 1), eye, None, np.arange(N),
                         per_head=True, recv_heads=H, recv_head_dim=d)
    assert np.array_equal(y, cache.reshape(L, N, H * d).astype(np.float64))
    # flattened [0; I; 0] selects the centre tap exactly
    F = H * d
    sel = np.zeros((L, 3 * F, F))
    sel[:, F:2 * F, :] = np.eye(F)
    taps = O.layer_taps(L, L, 3, 1)
    y3 = O.translate_rows(cache, np.arange(N), taps, sel, None, np.arange(N), per_head=False,
                          recv_heads=H, recv_head_dim=d)
    assert np.array_equal(y3, cache.reshape(L, N, F).astype(np.float64))
    # rotated keys with the same base on both sides and W = I come back unchanged
    pos = np.arange(N)
    rot = np.stack([O.rope_rotate(cache[l], pos, 1e4, +1) for l in range(L)])
    yr = O.translate_rows(rot, np.arange(N), O.layer_taps(L, L, 1), eye, None, pos, per_head=True,
                          recv_heads=H, recv_head_dim=d, send_rope_base=1e4, recv_rope_base=1e4)
    assert np.max(np.abs(yr - rot.reshape(L, N, F))) < 1e-12


def test_key_norm_pins():
    """Receiver key normalisation: with unit weights and eps = 0 every head
    vector comes out with RMS exactly 1; a positive scale of the input
    changes nothing; a hand example; and because a rotation keeps a head
    vector's RMS, normalising then rotating equals rotating then normalising
    when the weights are equal across the pair members."""
    rng = np.random.default_rng(12)
    y = rng.standard_normal((7, 3, 8)) * rng.uniform(0.1, 30.0, size=(7, 3, 1))
    ones = np.ones(8)
    z = O.key_norm(y, ones, 0.0)
    assert np.max(np.abs(np.sqrt(np.mean(z * z, axis=-1)) - 1.0)) < 1e-14
    assert np.max(np.abs(O.key_norm(4.5 * y, ones, 0.0) - z)) < 1e-14
    # (3, 4) with weights (1, 2): mean square 12.5 -> (3, 8) / sqrt(12.5)
    got = O.key_norm(np.array([[[3.0, 4.0]]]), np.array([1.0, 2.0]), 0.0)
    assert np.max(np.abs(got - np.array([[[0.848528137423857, 2.262741699796952]]]))) < 1e-15
    # eps enters the denominator only: a zero vector stays zero
    assert np.array_equal(O.key_norm(np.zeros((1, 1, 4)), ones[:4], 1e-6), np.zeros((1, 1, 4)))
    w = np.tile(rng.uniform(0.5, 1.5, size=4), 2)  # equal weight on c and c + d/2
    pos = np.arange(7) * 37
    a = O.rope_rotate(O.key_norm(y, w, 1e-6), pos, 1e4, +1)
    b = O.key_norm(O.rope_rotate(y, pos, 1e4, +1), w, 1e-6)
    assert np.max(np.abs(a - b)) < 1e-12


def test_translate_rows_with_key_norm():
    """translate_rows with the receiver key norm: per head RMS 1 before the
    receiver rotation with unit weights (also after it, the rotation keeps
    the RMS), and the norm is applied after the bias (a bias-only map gives
    the normalised bias)."""
    rng = np.random.default_rng(13)
    L_S, N_S, H, d = 4, 10, 2, 8
    cache = rng.standard_normal((L_S, N_S, H, d))
    taps = O.layer_taps(L_S, 3, 3, 1)
    wt = rng.standard_normal((3, 3 * H * d, H * d))
    b = rng.standard_normal((3, H * d))
    tmap = np.array([0, 1, 1, 4, 7, 9])
    rows = np.arange(tmap.size)
    kn = np.ones((3, d))
    y = O.translate_rows(cache, tmap, taps, wt, b, rows, per_head=False, recv_heads=H, recv_head_dim=d,
                         recv_rope_base=1e4, recv_key_norm=kn, key_norm_eps=0.0)
    rms = np.sqrt(np.mean(y.reshape(3, rows.size, H, d) ** 2, axis=-1))
    assert np.max(np.abs(rms - 1.0)) < 1e-13
    z = O.translate_rows(cache, tmap, taps, np.zeros_like(wt), b, rows, per_head=False, recv_heads=H,
                         recv_head_dim=d, recv_key_norm=kn, key_norm_eps=0.0)
    bh = b.reshape(3, 1, H, d)
    want = bh / np.sqrt(np.mean(bh * bh, axis=-1, keepdims=True))
    assert np.max(np.abs(z.reshape(3, rows.size, H, d) - want)) < 1e-14


def test_features_layout_and_derotation():
    rng = np.random.default_rng(5)
    cache = rng.standard_normal((4, 6, 2, 4))
    x = O.features(cache, [5, 0], [3, 1, 1])
    assert x.shape == (2, 24)
    assert np.array_equal(x[0, :8], cache[3, 5].ravel())
    assert np.array_equal(x[1, 8:16], cache[1, 0].ravel())
    assert np.array_equal(x[1, 16:], cache[1, 0].ravel())
    content = rng.standard_normal((1, 6, 2, 4))
    stored = O.rope_rotate(content[0], np.arange(6), 77.0, +1)[None]
    back = O.features(stored, np.arange(6), [0], 77.0)
    assert np.max(np.abs(back - content[0].reshape(6, 8))) < 1e-13


# ---------------------------------------------------------------- fold

def test_fold_fp32_order_and_bounds():
    rng = np.random.default_rng(6)
    fo, fi, R = 64, 96, 16
    wt = (rng.standard_normal((fi, fo)) / np.sqrt(fi)).astype(np.float32)
    u = (rng.standard_normal((fi, R)) / np.sqrt(fi)).astype(np.float32)
    v = (rng.standard_normal((R, fo)) * 0.1 / 4).astype(np.float32)
    tot, bits = O.fold_lowrank(wt, u, v)
    exact = O.fold_lowrank_f64(wt, u, v)
    # fp32 running sum of R products then one add: error <= (R+1) u_32 sum|terms|
    bound = (R + 1) * 2.0 ** -24 * (np.abs(wt) + np.abs(u.astype(np.float64)) @ np.abs(v.astype(np.float64)))
    assert np.all(np.abs(tot.astype(np.float64) - exact) <= bound)
    # bf16 of the fp32 fold is within one bf16 ulp of the exact fold
    got = O.bf16_bits_to_f64(bits)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact))) - 7)
    assert np.all(np.abs(got - exact) <= ulp)
    # rank 0 keeps W; small integers fold exactly
    t0, b0 = O.fold_lowrank(wt, u[:, :0], v[:0, :])
    assert np.array_equal(t0, wt) and np.array_equal(b0, O.f32_to_bf16_bits(wt))
    wi = rng.integers(-8, 8, (fi, fo)).astype(np.float32)
    ui = rng.integers(-3, 4, (fi, R)).astype(np.float32)
    vi = rng.integers(-3, 4, (R, fo)).astype(np.float32)
    ti, _ = O.fold_lowrank(wi, ui, vi)
    assert np.array_equal(ti.astype(np.float64), wi + ui.astype(np.float64) @ vi.astype(np.float64))
    # one entry by hand: w = 0.5, a = (1, 2), b = (3, -1) -> 0.5 + 3 - 2 = 1.5
    th, _ = O.fold_lowrank(np.array([[0.5]]), np.array([[1.0, 2.0]]), np.array([[3.0], [-1.0]]))
    assert th[0, 0] == np.float32(1.5)


# ---------------------------------------------------------------- ridge

def well_conditioned(n, f, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, f))


def test_ridge_recovers_planted_map():
    x = well_conditioned(512, 64, 7)
    wtrue = np.random.default_rng(8).standard_normal((64, 48)) / 8
    w, b, lam = O.ridge_fit(x, x @ wtrue, lam_abs=1e-10)
    assert b is None and lam == 1e-10
    assert np.max(np.abs(w - wtrue)) <= 1e-5


def test_ridge_normal_equations_and_qr():
    x = well_conditioned(300, 40, 9)
    y = np.random.default_rng(10).standard_normal((300, 7))
    for lam_abs, lam_rel in ((1e-2, 0.0), (0.0, 1e-3), (3.0, 0.1)):
        w, _, lam = O.ridge_fit(x, y, lam_abs, lam_rel)
        assert np.isclose(lam, lam_abs + lam_rel * np.sum(x * x) / 40, rtol=1e-13)
        g, c = x.T @ x, x.T @ y
        res = np.linalg.norm((g + lam * np.eye(40)) @ w - c) / np.linalg.norm(c)
        assert res <= 1e-12
        # independent algorithm: least squares on the augmented system [X; sqrt(lam) I]
        xa = np.vstack([x, np.sqrt(lam) * np.eye(40)])
        ya = np.vstack([y, np.zeros((40, 7))])
        wq = scipy.linalg.lstsq(xa, ya, lapack_driver="gelsy")[0]
        assert np.max(np.abs(w - wq)) <= 1e-10


def test_ridge_scalar_and_limits():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((200, 1))
    y = 3 * x + rng.standard_normal((200, 1))
    w, _, _ = O.ridge_fit(x, y, lam_abs=2.5)
    assert np.isclose(w[0, 0], (x * y).sum() / ((x * x).sum() + 2.5), rtol=1e-13)
    w_big, _, _ = O.ridge_fit(x, y, lam_abs=1e14)
    assert abs(w_big[0, 0]) < 1e-10


def test_ridge_duplicated_columns_get_equal_rows():
    # the layers whose clamped taps repeat a sender layer feed two identical
    # feature blocks; by symmetry and strict convexity their weights agree
    rng = np.random.default_rng(12)
    a = rng.standard_normal((400, 10))
    x = np.hstack([a, a, rng.standard_normal((400, 10))])
    y = rng.standard_normal((400, 5))
    w, _, _ = O.ridge_fit(x, y, lam_rel=1e-3)
    assert np.max(np.abs(w[:10] - w[10:20])) < 1e-12
    with pytest.raises(np.linalg.LinAlgError):
        np.linalg.cholesky(x.T @ x)  # singular without the penalty


def test_ridge_intercept_is_unpenalised():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((512, 16)) + 3.0
    wtrue = rng.standard_normal((16, 4))
    btrue = rng.standard_normal(4)
    y = x @ wtrue + btrue
    w, b, _ = O.ridge_fit(x, y, lam_abs=1e-10, fit_intercept=True)
    assert np.max(np.abs(w - wtrue)) < 1e-7 and np.max(np.abs(b - btrue)) < 1e-7
    # with a penalty: equals least squares with an unpenalised constant column
    lam = 5.0
    w2, b2, _ = O.ridge_fit(x, y, lam_abs=lam, fit_intercept=True)
    xa = np.vstack([np.hstack([x, np.ones((512, 1))]), np.hstack([np.sqrt(lam) * np.eye(16), np.zeros((16, 1))])])
    ya = np.vstack([y, np.zeros((16, 4))])
    sol = scipy.linalg.lstsq(xa, ya, lapack_driver="gelsy")[0]
    assert np.max(np.abs(w2 - sol[:16])) < 1e-10 and np.max(np.abs(b2 - sol[16])) < 1e-10


def test_rel_err_metric():
    assert O.rel_err([1.0, -1.0], [1.0, -1.0]) == 0.0
    assert np.isclose(O.rel_err([1.5, -1.0], [1.0, -1.0]), 0.5)
