"""HIP path vs the CPU oracle, element by element, through the C-ABI.

Token maps are compared bit for bit; translated K/V by max|err|/RMS per role
against the oracle's unrounded fp64 result (1e-4 for fp32 caches, 2e-2 for
bf16 caches).  Small cases compare every element over several tiles with a
ragged tail; the full workload sizes compare sampled receiver rows (all
layers, heads and channels of each row) or properties that hold at any size.
"""
import math
import sys

import numpy as np
import pytest
import torch

from cross_model_kv_kvx_amd import kvx, synth
from oracle import kvx_oracle as O
from tests.kvx_cases import TOL_BF16, TOL_F32, bf16_floor, host, rows_of, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def dev_i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=DEV)


# ---------------------------------------------------------------- alignment


@pytest.mark.parametrize("n,seed", [(8192, 3), (32768, 4), (65536, 5), (16384, 6), (1, 0), (777, 9), (1025, 2)])
def test_align_bit_exact(n, seed):
    say(f"align n={n} seed={seed}")
    s, r = synth.token_ends(n, seed)
    got = kvx.align_tokens(dev_i32(s), dev_i32(r)).cpu().numpy()
    want = O.token_align(s, r)
    assert np.array_equal(got, want)


def test_align_special_cases():
    rng = np.random.default_rng(0)
    e = np.cumsum(rng.integers(1, 7, size=3000)).astype(np.int32)
    cases = [
        (e, e),                                                     # identical tokenizations
        (np.arange(1, e[-1] + 1, dtype=np.int32), e),               # single-character sender
        (e, np.arange(1, e[-1] + 1, dtype=np.int32)),               # single-character receiver
        (np.array([e[-1]], np.int32), e),                           # one sender token
        (np.array([2, 4, 9], np.int32), np.array([1, 3, 5, 7, 9, 11, 12], np.int32)),  # leading/trailing
    ]
    for s, r in cases:
        say(f"align special n_send={s.size} n_recv={r.size}")
        got = kvx.align_tokens(dev_i32(s), dev_i32(r)).cpu().numpy()
        assert np.array_equal(got, O.token_align(s, r))


def test_align_rejects_non_increasing_offsets():
    for s, r in (([1, 3, 3], [1, 2, 3]), ([1, 2, 3], [2, 1, 3]), ([0, 2], [2]), ([1, 2], [-1, 2])):
        say(f"align invalid {s} {r}")
        with pytest.raises(kvx.KvxError) as ei:
            kvx.align_tokens(dev_i32(s), dev_i32(r))
        assert ei.value.status == kvx.ERR_INVALID


# ---------------------------------------------------------------- fold


def test_fold_bit_exact():
    say("fold 3 maps 1024x3072 rank 16")
    wt, u, v, _ = synth.flat_maps(3, 3072, 1024, 31, "cpu")
    got = kvx.fold_lowrank(wt.to(DEV), u.to(DEV), v.to(DEV), torch.bfloat16)
    got32 = kvx.fold_lowrank(wt.to(DEV), u.to(DEV), v.to(DEV), torch.float32)
    for l in range(3):
        tot, bits = O.fold_lowrank(wt[l].numpy(), u[l].numpy(), v[l].numpy())
        assert np.array_equal(got[l].cpu().view(torch.int16).numpy().view(np.uint16), bits)
        assert np.array_equal(got32[l].cpu().numpy(), tot)


# ---------------------------------------------------------------- cfg1: fp32 per-head fit + translate


def cfg1_receiver(x, w, b, noise):
    """The matched receiver of the fp32 single-layer setting, built on the
    host: y_h = x_h W_true,h + b_h + noise (w[0][h][c][o], row-major)."""
    xs = x.double()
    y = torch.einsum("lnhc,hco->lnho", xs, w[0].double()) + b.double().reshape(1, 1, w.shape[1], -1)
    return (y + noise.double()).float()


def test_cfg1_fit_and_translate_fp32():
    say("cfg1 fp32 fit + per-head translate")
    c = synth.config(1, "cpu")
    H, d = c["heads"], c["head_dim"]
    taps = kvx.layer_map(1, 1, 1)
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    tmap = kvx.align_tokens(dev_i32(c["send_end"]), dev_i32(c["recv_end"]))
    assert np.array_equal(tmap.cpu().numpy(), tmap_o)
    maps_g, maps_o = {}, {}
    for role in ("k", "v"):
        y_cal = cfg1_receiver(c[f"x_cal_{role}"], c[f"w_true_{role}"], c[f"b_true_{role}"], c[f"noise_cal_{role}"])
        xg, yg = c[f"x_cal_{role}"].to(DEV), y_cal.to(DEV)
        wts, bs, wto, bo = [], [], [], []
        for h in range(H):
            w, b = kvx.fit_ridge(xg[0, :, h, :], yg[0, :, h, :], lambda_abs=1e-2, fit_intercept=True)
            wo, bo_h, lam = O.ridge_fit(O.as_f64(c[f"x_cal_{role}"][0, :, h, :]), O.as_f64(y_cal[0, :, h, :]),
                                        lam_abs=1e-2, fit_intercept=True)
            assert O.rel_err(w.cpu().numpy(), wo) <= TOL_F32
            assert O.rel_err(b.cpu().numpy(), bo_h) <= TOL_F32
            wts.append(w)
            bs.append(b)
            wto.append(wo)
            bo.append(bo_h)
        maps_g[role] = (torch.stack(wts)[None].contiguous(), torch.cat(bs)[None].contiguous())
        maps_o[role] = (np.stack(wto)[None], np.concatenate(bo)[None])
    k, v = kvx.translate(c["x_k"].to(DEV), c["x_v"].to(DEV), tmap, taps, maps_g["k"][0], maps_g["v"][0],
                         maps_g["k"][1], maps_g["v"][1], per_head=True)
    for role, out in (("k", k), ("v", v)):
        want = O.translate_rows(c[f"x_{role}"], tmap_o, taps, maps_o[role][0], maps_o[role][1], np.arange(128),
                                per_head=True, recv_heads=H, recv_head_dim=d)
        got = O.as_f64(out).reshape(1, 128, H * d)
        err = O.rel_err(got, want)
        say(f"  cfg1 {role}: max|err|/RMS = {err:.3e}")
        assert err <= TOL_F32


# ---------------------------------------------------------------- cfg2: per-head bf16, 32 -> 80 layers


def run_cfg2(n_tokens, rows=None, seed=2):
    c = synth.config(2, DEV, small=True) if n_tokens == 256 else None
    if c is None:
        cc = dict(synth.CONFIGS[2])
        shp = synth.CacheShape(32, n_tokens, 8, 128)
        c = dict(send_shape=shp)
        c["send_end"], c["recv_end"] = synth.identical_ends(n_tokens, seed)
        for r, role in enumerate(("k", "v")):
            c[f"{role}_send"] = synth.sender_cache(shp, seed * 100 + r, DEV, channel_scale="loguniform")
            c[f"w_{role}"], c[f"b_{role}"] = synth.perhead_maps(80, 8, 128, seed * 100 + 20 + r, DEV)
    taps = kvx.layer_map(32, 80, 1)
    tmap = kvx.align_tokens(dev_i32(c["send_end"]), dev_i32(c["recv_end"]))
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    assert np.array_equal(tmap.cpu().numpy(), tmap_o)
    k, v = kvx.translate(c["k_send"], c["v_send"], tmap, taps, c["w_k"], c["w_v"], c["b_k"], c["b_v"],
                         per_head=True)
    n = tmap_o.size
    rows = np.arange(n) if rows is None else rows
    for role, out in (("k", k), ("v", v)):
        want = O.translate_rows(c[f"{role}_send"], tmap_o, taps, host(c[f"w_{role}"]), host(c[f"b_{role}"]), rows,
                                per_head=True, recv_heads=8, recv_head_dim=128)
        got = rows_of(out, rows)
        err = O.rel_err(got, want)
        say(f"  cfg2 n={n} {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16
    return k, v


def test_cfg2_perhead_small_all_elements():
    say("cfg2 per-head 256 tokens")
    run_cfg2(256)


def test_cfg2_perhead_ragged_all_elements():
    say("cfg2 per-head 300 tokens (ragged chunk)")
    run_cfg2(300, seed=12)


def test_cfg2_perhead_full_sampled_rows():
    say("cfg2 per-head 4096 tokens, sampled rows")
    rows = sample_rows(np.arange(4096), 128, 0)
    run_cfg2(4096, rows)


def perhead_rope_case(n_recv, seed, send_rope, recv_rope, map_dtype, rows=None, L_S=8, L_R=20):
    """Per-head translation of rotated keys: sender keys rotated back at their
    sender positions (fp16 rows), mapped per head, rotated at the receiver
    positions; values mapped without rotation."""
    send_end, recv_end = synth.token_ends(n_recv, seed)
    shp = synth.CacheShape(L_S, len(send_end), 8, 128)
    taps = kvx.layer_map(L_S, L_R, 1)
    tmap_o = O.token_align(send_end, recv_end)
    tm = dev_i32(tmap_o)
    caches, maps, bias = {}, {}, {}
    for r, role in enumerate(("k", "v")):
        # channel scales of the per-head workload (a head's outlier channel
        # would spread over all its outputs and put the bf16 rounding of the
        # result itself above the max|err|/RMS tolerance)
        caches[role] = synth.sender_cache(shp, seed * 10 + r, DEV, channel_scale="loguniform")
        wt, b = synth.perhead_maps(L_R, 8, 128, seed * 10 + 5 + r, DEV)
        maps[role], bias[role] = wt.to(map_dtype), b
    k, v = kvx.translate(caches["k"], caches["v"], tm, taps, maps["k"], maps["v"], bias["k"], bias["v"],
                         per_head=True, send_rope_base=send_rope, recv_rope_base=recv_rope)
    torch.cuda.synchronize()
    rows = np.arange(tmap_o.size) if rows is None else rows
    for role, out in (("k", k), ("v", v)):
        rk = role == "k"
        want = O.translate_rows(caches[role], tmap_o, taps, host(maps[role]).float().numpy().astype(np.float64),
                                host(bias[role]).numpy().astype(np.float64), rows, per_head=True, recv_heads=8,
                                recv_head_dim=128, send_rope_base=send_rope if rk else 0.0,
                                recv_rope_base=recv_rope if rk else 0.0)
        err = O.rel_err(rows_of(out, rows), want)
        say(f"  per-head rope n={tmap_o.size} {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16


@pytest.mark.parametrize("send_rope,recv_rope", [(5e5, 1e6), (0.0, 1e6), (1e4, 0.0)])
@pytest.mark.parametrize("map_dtype", [torch.float32, torch.bfloat16])
def test_perhead_rope_all_elements(send_rope, recv_rope, map_dtype):
    say(f"per-head + RoPE {send_rope:g}->{recv_rope:g} maps {map_dtype}, 300 receiver tokens")
    perhead_rope_case(300, 71, send_rope, recv_rope, map_dtype)


def test_perhead_rope_long_span_all_rows():
    """Several spans of receiver tokens with a ragged last one: with 6
    receiver layers one role's launch is 48 workgroups per span, so the
    launcher splits the 4500 tokens into spans shorter than 4096 to fill its
    rounds, and each span restarts the rotation recurrence at its own first
    token.  Every row is checked, so every span start and end is."""
    say("per-head + RoPE, 4500 receiver tokens, all rows")
    perhead_rope_case(4500, 72, 5e5, 1e6, torch.float32, L_S=4, L_R=6)


# ---------------------------------------------------------------- cfg3/4: flattened maps


class Bf16Maps:
    """Oracle-folded maps kept as bf16 bit patterns; indexing a layer gives
    its float64 values (the oracle reads one layer at a time)."""

    def __init__(self, bits):
        self.bits = bits

    def __len__(self):
        return len(self.bits)

    def __getitem__(self, l):
        return O.bf16_bits_to_f64(self.bits[l])


_MAPS = {}


def flat_maps(k):
    """Maps of a flattened setting, folded by the library (bf16, device) and
    by the oracle (bf16 bits, host); the two folds must agree bit for bit."""
    if k not in _MAPS:
        seed = synth.CONFIGS[k]["seed"]
        out = {}
        for r, role in enumerate(("k", "v")):
            say(f"  folding maps of setting {k} role {role}")
            wt, u, v, b = synth.flat_maps(32, 3072, 1024, seed * 100 + 20 + r, DEV, 16)
            g = kvx.fold_lowrank(wt, u, v, torch.bfloat16)
            wh, uh, vh = host(wt).numpy(), host(u).numpy(), host(v).numpy()
            bits = np.stack([O.fold_lowrank(wh[l], uh[l], vh[l])[1] for l in range(32)])
            assert np.array_equal(host(g).view(torch.int16).numpy().view(np.uint16), bits)
            out[role] = (g, b, Bf16Maps(bits), host(b).numpy().astype(np.float64))
            del wt, u, v
        _MAPS[k] = out
    return _MAPS[k]


def flat_case(k, n_recv=None, seed=None, with_maps=True):
    """Inputs of the flattened settings on the device: token ends and caches
    seeded by ``seed``, maps of setting ``k`` (bf16, unless with_maps is
    false)."""
    cfg = dict(synth.CONFIGS[k])
    seed = cfg["seed"] if seed is None else seed
    nr = cfg["recv_tokens"] if n_recv is None else n_recv
    send_end, recv_end = synth.token_ends(nr, seed)
    shp = synth.CacheShape(36, len(send_end), 8, 128)
    c = dict(send_end=send_end, recv_end=recv_end, shp=shp, n_recv=nr)
    rope = "send_rope" in cfg
    maps = flat_maps(k) if with_maps else None
    for r, role in enumerate(("k", "v")):
        c[f"{role}_send"] = synth.sender_cache(shp, seed * 100 + r, DEV, outlier_frac=cfg.get("outlier_frac", 0.0),
                                               outlier_scale=cfg.get("outlier_scale", 1.0),
                                               outlier_pairs=(role == "k" and rope))
        if maps:
            c[f"wt_{role}"], c[f"b_{role}"], c[f"wt_o_{role}"], c[f"b_o_{role}"] = maps[role]
    c["send_rope"] = cfg.get("send_rope", 0.0)
    c["recv_rope"] = cfg.get("recv_rope", 0.0)
    return c


def check_flat(c, rows=None):
    taps = kvx.layer_map(36, 32, 3, 4)
    assert np.array_equal(taps, O.layer_taps(36, 32, 3, 4))
    tmap = kvx.align_tokens(dev_i32(c["send_end"]), dev_i32(c["recv_end"]))
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    assert np.array_equal(tmap.cpu().numpy(), tmap_o)
    k, v = kvx.translate(c["k_send"], c["v_send"], tmap, taps, c["wt_k"], c["wt_v"], c["b_k"], c["b_v"],
                         send_rope_base=c["send_rope"], recv_rope_base=c["recv_rope"])
    torch.cuda.synchronize()
    n = tmap_o.size
    rows = np.arange(n) if rows is None else rows
    errs = {}
    for role, out in (("k", k), ("v", v)):
        rk = role == "k"
        want = O.translate_rows(c[f"{role}_send"], tmap_o, taps, c[f"wt_o_{role}"], c[f"b_o_{role}"], rows,
                                per_head=False, recv_heads=8, recv_head_dim=128,
                                send_rope_base=c["send_rope"] if rk else 0.0,
                                recv_rope_base=c["recv_rope"] if rk else 0.0)
        got = rows_of(out, rows)
        err = O.rel_err(got, want)
        errs[role] = err
        say(f"  flat n={n} {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16
    return k, v, tmap, errs


def test_cfg3_flat_small_all_elements():
    say("cfg3 flattened, 600 receiver tokens")
    c = flat_case(3, 600, seed=13)
    check_flat(c)


def test_cfg4_flat_rope_small_all_elements():
    say("cfg4 flattened + RoPE, 700 receiver tokens")
    c = flat_case(4, 700, seed=14)
    check_flat(c)


def test_cfg3_flat_full_sampled_rows():
    say("cfg3 flattened, 8192 receiver tokens, sampled rows")
    c = flat_case(3)
    s, r = c["send_end"], c["recv_end"]
    rows = sample_rows(O.token_align(s, r), 256, 3)
    k, v, tmap, _ = check_flat(c, rows)
    # V rows of one run are bitwise equal (one product written to the run)
    m = tmap.cpu().numpy()
    starts = np.flatnonzero(np.diff(m) == 0)[:50]
    for i in starts:
        assert torch.equal(v[:, int(i)], v[:, int(i) + 1])


def test_cfg4_flat_rope_full_sampled_rows():
    say("cfg4 flattened + RoPE, 32768 receiver tokens, sampled rows")
    c = flat_case(4)
    rows = sample_rows(O.token_align(c["send_end"], c["recv_end"]), 256, 4)
    check_flat(c, rows)


class F32Maps:
    """fp32 maps [L][F_in][F_out] (host), handed to the oracle one layer at a
    time as fp64."""

    def __init__(self, a):
        self.a = a

    def __getitem__(self, l):
        return self.a[l].astype(np.float64)


def test_flat_fp32_maps_all_elements():
    """Flattened translation with fp32 maps (the fitted-map path): the kernel
    splits each map into a 16-bit high and low half (fp16 for the
    rotated-back keys, bf16 for the values) and doubles the K extent."""
    say("flattened + RoPE with fp32 maps, 400 receiver tokens")
    cfg = synth.CONFIGS[4]
    send_end, recv_end = synth.token_ends(400, 61)
    shp = synth.CacheShape(36, len(send_end), 8, 128)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap_o = O.token_align(send_end, recv_end)
    tm = dev_i32(tmap_o)
    caches, maps, bias = {}, {}, {}
    for r, role in enumerate(("k", "v")):
        caches[role] = synth.sender_cache(shp, 6100 + r, DEV, outlier_frac=0.01, outlier_scale=20.0,
                                          outlier_pairs=(role == "k"))
        wt, _, _, b = synth.flat_maps(32, 3072, 1024, 6200 + r, DEV, 16)
        maps[role], bias[role] = wt, b
    k, v = kvx.translate(caches["k"], caches["v"], tm, taps, maps["k"], maps["v"], bias["k"], bias["v"],
                         send_rope_base=cfg["send_rope"], recv_rope_base=cfg["recv_rope"])
    torch.cuda.synchronize()
    rows = np.arange(tmap_o.size)
    for role, out in (("k", k), ("v", v)):
        rk = role == "k"
        want = O.translate_rows(caches[role], tmap_o, taps, F32Maps(host(maps[role]).numpy()),
                                host(bias[role]).numpy().astype(np.float64), rows, per_head=False, recv_heads=8,
                                recv_head_dim=128, send_rope_base=cfg["send_rope"] if rk else 0.0,
                                recv_rope_base=cfg["recv_rope"] if rk else 0.0)
        err = O.rel_err(rows_of(out, rows), want)
        say(f"  fp32 maps {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16


def test_perhead_rope_full_size_sampled_rows():
    """The per-head setting with rotated keys at the size the bench times
    (32 -> 80 layers, 4096 tokens, fp32 maps), sampled rows, among them the
    rows around token 2048 (one role per launch: two spans of 2048)."""
    say("per-head + RoPE 32 -> 80 layers, 4096 tokens, sampled rows")
    shp = synth.CacheShape(32, 4096, 8, 128)
    taps = kvx.layer_map(32, 80, 1)
    ident = np.arange(4096)
    rows = np.unique(np.concatenate([sample_rows(ident, 96, 5), np.arange(2040, 2057)]))
    for r, role in enumerate(("k", "v")):
        x = synth.sender_cache(shp, 200 + r, DEV, channel_scale="loguniform")
        wt, b = synth.perhead_maps(80, 8, 128, 220 + r, DEV)
        rk = role == "k"
        kw = dict(send_rope_base=5e5, recv_rope_base=1e6) if rk else {}
        out, _ = kvx.translate(x, None, dev_i32(ident), taps, wt, None, b, None, per_head=True, **kw)
        want = O.translate_rows(x, ident, taps, host(wt).numpy().astype(np.float64),
                                host(b).numpy().astype(np.float64), rows, per_head=True, recv_heads=8,
                                recv_head_dim=128, send_rope_base=5e5 if rk else 0.0,
                                recv_rope_base=1e6 if rk else 0.0)
        err = O.rel_err(rows_of(out, rows), want)
        say(f"  {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16
        del x, wt, out


def test_flat_key_norm_full_size_sampled_rows():
    """Receiver key normalisation on the 32k cross-family setting (the bench's
    key-norm line), sampled rows of the key output."""
    say("flattened + RoPE + key norm, 32768 tokens, sampled rows")
    c = flat_case(4)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    kn = synth.key_norm_weights(32, 128, 430, DEV)
    k, _ = kvx.translate(c["k_send"], None, dev_i32(tmap_o), taps, c["wt_k"], None, c["b_k"], None,
                         send_rope_base=c["send_rope"], recv_rope_base=c["recv_rope"], recv_key_norm=kn,
                         key_norm_eps=1e-6)
    rows = sample_rows(tmap_o, 128, 7)
    want = O.translate_rows(c["k_send"], tmap_o, taps, c["wt_o_k"], c["b_o_k"], rows, per_head=False, recv_heads=8,
                            recv_head_dim=128, send_rope_base=c["send_rope"], recv_rope_base=c["recv_rope"],
                            recv_key_norm=host(kn).numpy(), key_norm_eps=1e-6)
    err = O.rel_err(rows_of(k, rows), want)
    say(f"  k: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
    assert err <= TOL_BF16


@pytest.mark.parametrize("rope", [True, False])
def test_flat_key_norm_all_elements(rope):
    """The receiver's key normalisation in the flattened epilogue (after the
    bias, before the receiver rotation), keys vs the oracle with the norm,
    values vs the oracle without it."""
    say(f"flattened + receiver key norm, rope={rope}, 400 receiver tokens")
    send_end, recv_end = synth.token_ends(400, 81)
    shp = synth.CacheShape(36, len(send_end), 8, 128)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap_o = O.token_align(send_end, recv_end)
    tm = dev_i32(tmap_o)
    caches, maps, bias = {}, {}, {}
    for r, role in enumerate(("k", "v")):
        caches[role] = synth.sender_cache(shp, 8100 + r, DEV, outlier_frac=0.01 if rope else 0.0,
                                          outlier_scale=20.0 if rope else 1.0, outlier_pairs=(rope and role == "k"))
        wt, u, v, b = synth.flat_maps(32, 3072, 1024, 8200 + r, DEV, 16)
        # dense part rounded to bf16 on the host (no fold: the inputs of the
        # oracle never come from the library)
        wb = host(wt).to(torch.bfloat16)
        maps[role] = (wb.to(DEV), Bf16Maps(wb.view(torch.int16).numpy().view(np.uint16)))
        bias[role] = b
        del wt, u, v
    kn = synth.key_norm_weights(32, 128, 8300, DEV)
    kw = dict(send_rope_base=5e5, recv_rope_base=1e6) if rope else {}
    k, v = kvx.translate(caches["k"], caches["v"], tm, taps, maps["k"][0], maps["v"][0], bias["k"], bias["v"],
                         recv_key_norm=kn, key_norm_eps=1e-6, **kw)
    torch.cuda.synchronize()
    rows = np.arange(tmap_o.size)
    for role, out in (("k", k), ("v", v)):
        rk = role == "k"
        want = O.translate_rows(caches[role], tmap_o, taps, maps[role][1], host(bias[role]).numpy().astype(np.float64), rows,
                                per_head=False, recv_heads=8, recv_head_dim=128,
                                send_rope_base=kw.get("send_rope_base", 0.0) if rk else 0.0,
                                recv_rope_base=kw.get("recv_rope_base", 0.0) if rk else 0.0,
                                recv_key_norm=host(kn).numpy() if rk else None, key_norm_eps=1e-6)
        err = O.rel_err(rows_of(out, rows), want)
        say(f"  key norm {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16


def multi_sequence_case(per_head, lengths=(150, 333, 70), seed=91, block=16):
    """Sequences of ragged lengths concatenated, aligned by one batched call,
    translated by one placed call into a shuffled pool of 16-row blocks with
    positions relative to each sequence; each sequence's rows (gathered
    through its slots) against the oracle on that sequence alone, rows of the
    pool no slot names untouched."""
    rng = np.random.default_rng(seed)
    ends = [synth.token_ends(n, seed + q) for q, n in enumerate(lengths)]
    so = np.concatenate([[0], np.cumsum([len(e[0]) for e in ends])]).astype(np.int32)
    ro = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    send_end = dev_i32(np.concatenate([e[0] for e in ends]))
    recv_end = dev_i32(np.concatenate([e[1] for e in ends]))
    tm = kvx.align_tokens_batched(send_end, so, recv_end, ro)
    maps_o = [O.token_align(*e) for e in ends]
    assert np.array_equal(tm.cpu().numpy(), np.concatenate([m + so[q] for q, m in enumerate(maps_o)]))
    L_S, L_R, n_taps = (8, 20, 1) if per_head else (36, 32, 3)
    shp = synth.CacheShape(L_S, int(so[-1]), 8, 128)
    taps = kvx.layer_map(L_S, L_R, n_taps, 4)
    caches, maps, bias = {}, {}, {}
    for r, role in enumerate(("k", "v")):
        caches[role] = synth.sender_cache(shp, seed * 10 + r, DEV, channel_scale="loguniform")
        if per_head:
            wt, b = synth.perhead_maps(L_R, 8, 128, seed * 10 + 5 + r, DEV)
            maps[role] = (wt, host(wt).numpy().astype(np.float64))
        else:
            wt, _, _, b = synth.flat_maps(L_R, 3072, 1024, seed * 10 + 5 + r, DEV, 16)
            wb = host(wt).to(torch.bfloat16)
            maps[role] = (wb.to(DEV), Bf16Maps(wb.view(torch.int16).numpy().view(np.uint16)))
            del wt
        bias[role] = b
    # block tables: every sequence takes shuffled blocks of a pool with spare blocks
    nblk = [(n + block - 1) // block for n in lengths]
    pool_blocks = sum(nblk) + 5
    perm = rng.permutation(pool_blocks)
    slot, used, b0 = [], [], 0
    for q, n in enumerate(lengths):
        table = perm[b0:b0 + nblk[q]]
        b0 += nblk[q]
        j = np.arange(n)
        slot.append(table[j // block] * block + j % block)
    slot = np.concatenate(slot).astype(np.int64)
    pool_rows = pool_blocks * block
    recv_pos = np.concatenate([np.arange(n) for n in lengths]).astype(np.int32)
    send_pos = np.concatenate([np.arange(so[q + 1] - so[q]) for q in range(len(lengths))]).astype(np.int32)
    pos_limit = int(max(max(lengths), int(np.max(np.diff(so)))))
    outs = {role: torch.full((L_R, pool_rows, 8, 128), 7.0, dtype=torch.bfloat16, device=DEV) for role in "kv"}
    kvx.translate(caches["k"], caches["v"], tm, taps, maps["k"][0], maps["v"][0], bias["k"], bias["v"],
                  per_head=per_head, send_rope_base=5e5, recv_rope_base=1e6, k_recv=outs["k"], v_recv=outs["v"],
                  slot=torch.as_tensor(slot, device=DEV), pool_rows=pool_rows,
                  recv_pos=torch.as_tensor(recv_pos, device=DEV), send_pos=torch.as_tensor(send_pos, device=DEV),
                  pos_limit=pos_limit)
    torch.cuda.synchronize()
    free = np.setdiff1d(np.arange(pool_rows), slot)
    for role in ("k", "v"):
        rk = role == "k"
        assert torch.all(outs[role][:, torch.as_tensor(free, device=DEV)] == 7.0)
        for q, n in enumerate(lengths):
            cache_q = caches[role][:, so[q]:so[q + 1]]
            want = O.translate_rows(cache_q, maps_o[q], taps, maps[role][1], host(bias[role]).numpy().astype(np.float64),
                                    np.arange(n), per_head=per_head, recv_heads=8, recv_head_dim=128,
                                    send_rope_base=5e5 if rk else 0.0, recv_rope_base=1e6 if rk else 0.0)
            err = O.rel_err(rows_of(outs[role], slot[ro[q]:ro[q + 1]]), want)
            say(f"  sequence {q} ({n} tokens) {role}: max|err|/RMS = {err:.4e}")
            assert err <= TOL_BF16


@pytest.mark.parametrize("per_head", [False, True])
def test_multi_sequence_into_paged_pool(per_head):
    say(f"three sequences, paged pool, {'per-head' if per_head else 'flattened'} + RoPE")
    multi_sequence_case(per_head)


def test_translate_deterministic_and_identity_maps():
    say("determinism + identity maps")
    c = flat_case(3, 520, seed=23)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap = kvx.align_tokens(dev_i32(c["send_end"]), dev_i32(c["recv_end"]))
    k1, v1 = kvx.translate(c["k_send"], c["v_send"], tmap, taps, c["wt_k"], c["wt_v"], c["b_k"], c["b_v"])
    k2, v2 = kvx.translate(c["k_send"], c["v_send"], tmap, taps, c["wt_k"], c["wt_v"], c["b_k"], c["b_v"])
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    # flattened [0; I; 0] selects the centre tap exactly (bf16 in, bf16 out)
    L, N, F = 6, 300, 1024
    x = synth.sender_cache(synth.CacheShape(L, N, 8, 128), 77, DEV)
    sel = torch.zeros((L, 3 * F, F), dtype=torch.bfloat16, device=DEV)
    sel[:, F:2 * F, :] = torch.eye(F, dtype=torch.bfloat16, device=DEV)
    ident = dev_i32(np.arange(N))
    taps6 = kvx.layer_map(L, L, 3, 1)
    ky, _ = kvx.translate(x, None, ident, taps6, sel, None)
    assert torch.equal(ky, x)
    # per head W = I (fp32 map, hi/lo split) reproduces the input exactly
    eye = torch.eye(128, device=DEV).expand(L, 8, 128, 128).contiguous()
    kp, _ = kvx.translate(x, None, ident, kvx.layer_map(L, L, 1), eye, None, per_head=True)
    assert torch.equal(kp, x)


def test_translate_edge_cases():
    say("edge cases: one receiver token, one run, leading unmatched")
    c = flat_case(3, 64, seed=33)
    taps = kvx.layer_map(36, 32, 3, 4)
    Ns = c["shp"].tokens
    for name, m in (("one row", np.array([5])), ("single run", np.zeros(300, np.int64) + 7),
                    ("long final run", np.minimum(np.arange(257), Ns - 1))):
        say(f"  {name}")
        tm = dev_i32(m)
        k, v = kvx.translate(c["k_send"], c["v_send"], tm, taps, c["wt_k"], c["wt_v"], c["b_k"], c["b_v"])
        for role, out in (("k", k), ("v", v)):
            want = O.translate_rows(c[f"{role}_send"], m, taps, c[f"wt_o_{role}"], c[f"b_o_{role}"], np.arange(m.size),
                                    per_head=False, recv_heads=8, recv_head_dim=128)
            assert O.rel_err(rows_of(out, np.arange(m.size)), want) <= TOL_BF16


# ---------------------------------------------------------------- features and fit (cfg5)


def test_gather_features():
    say("gather features")
    c = flat_case(3, 200, seed=43)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    tm = dev_i32(tmap_o)
    for l in (0, 17, 31):
        x = kvx.gather_features(c["k_send"], tm, taps[l])
        want = O.features(c["k_send"], tmap_o, taps[l])
        assert np.array_equal(O.as_f64(x), want)
    # fp32 cache with rotation undone at the sender position
    kf = synth.sender_cache(synth.CacheShape(5, 300, 2, 64), 9, DEV, torch.float32)
    m = np.sort(np.random.default_rng(1).integers(0, 300, size=150))
    xf = kvx.gather_features(kf, dev_i32(m), [4, 1], derotate=True, rope_base=1e4)
    want = O.features(kf, m, [4, 1], derotate_base=1e4)
    assert O.rel_err(O.as_f64(xf), want) <= 1e-6


def fit_case(n_cal, seed=5):
    send_end, recv_end = synth.token_ends(n_cal, seed)
    shp = synth.CacheShape(36, len(send_end), 8, 128)
    c = dict(send_end=send_end, recv_end=recv_end)
    c["k_send"] = synth.sender_cache(shp, seed * 100, DEV)
    c["recv_k"] = synth.receiver_cache(synth.CacheShape(32, n_cal, 8, 128), seed * 100 + 50, DEV)
    return c


@pytest.mark.parametrize("layer", [0, 15, 31])
def test_fit_ridge_vs_oracle(layer):
    say(f"ridge fit layer {layer}, 4096 calibration rows")
    c = fit_case(4096)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    tm = dev_i32(tmap_o)
    x = kvx.gather_features(c["k_send"], tm, taps[layer])
    y = c["recv_k"][layer].reshape(4096, 1024)
    w, _ = kvx.fit_ridge(x, y, lambda_rel=1e-3)
    xo = O.features(c["k_send"], tmap_o, taps[layer])
    yo = O.as_f64(c["recv_k"][layer]).reshape(4096, 1024)
    wo, _, lam = O.ridge_fit(xo, yo, lam_rel=1e-3)
    err = O.rel_err(w.cpu().numpy(), wo)
    say(f"  W max|err|/RMS = {err:.3e} (lambda {lam:.4g})")
    assert err <= TOL_BF16
    if layer in (0, 31):
        # duplicated taps -> equal weight blocks (exact for the exact solution;
        # the blocked factorisation eliminates the two copies at different
        # steps, so they agree to fp64 rounding amplified by the condition)
        t = taps[layer]
        a, b = [(i, j) for i in range(3) for j in range(i + 1, 3) if t[i] == t[j]][0]
        wn = w.cpu().numpy().astype(np.float64)
        gap = np.max(np.abs(wn[a * 1024:(a + 1) * 1024] - wn[b * 1024:(b + 1) * 1024]))
        say(f"  duplicated-block gap / RMS = {gap / np.sqrt(np.mean(wn * wn)):.3e}")
        assert gap <= 1e-6 * np.sqrt(np.mean(wn * wn))


def test_fit_rejects_singular_gram():
    say("ridge fit lambda 0 on duplicated taps -> not SPD")
    c = fit_case(512, seed=8)
    taps = kvx.layer_map(36, 32, 3, 4)
    tm = kvx.align_tokens(dev_i32(c["send_end"]), dev_i32(c["recv_end"]))
    x = kvx.gather_features(c["k_send"], tm, taps[0])   # taps (0, 0, 4): two equal blocks, 512 < 3072 rows
    y = c["recv_k"][0].reshape(512, 1024)
    with pytest.raises(kvx.KvxError) as ei:
        kvx.fit_ridge(x, y)
    assert ei.value.status == kvx.ERR_NOT_SPD


def test_fit_batched_matches_single_and_oracle():
    """Three layers fitted by one batched call: each result equals the
    single-problem call bit for bit (the same kernels, tile by tile) and the
    oracle's fit within the tolerance."""
    say("batched ridge fit, layers 0 / 15 / 31, 4096 calibration rows")
    c = fit_case(4096)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    tm = dev_i32(tmap_o)
    layers = (0, 15, 31)
    xs = [kvx.gather_features(c["k_send"], tm, taps[l]) for l in layers]
    ys = [c["recv_k"][l].reshape(4096, 1024) for l in layers]
    st = []
    ws, _ = kvx.fit_ridge_batched(xs, ys, lambda_rel=1e-3, status=st)
    assert st == [kvx.OK] * 3
    for l, x, y, w in zip(layers, xs, ys, ws):
        w1, _ = kvx.fit_ridge(x, y, lambda_rel=1e-3)
        assert torch.equal(w, w1), f"layer {l}: batched and single fits differ"
        wo, _, _ = O.ridge_fit(O.features(c["k_send"], tmap_o, taps[l]),
                               O.as_f64(c["recv_k"][l]).reshape(4096, 1024), lam_rel=1e-3)
        err = O.rel_err(w.cpu().numpy(), wo)
        say(f"  layer {l}: W max|err|/RMS = {err:.3e}")
        assert err <= TOL_BF16


def test_fit_batched_many_problems_vs_oracle():
    """32 problems of 776 features -> 1024 outputs in one call (enough
    tiles for the left-looking triangular solves; 776 = three 256-row blocks
    and a ragged block of 8), with an intercept: every problem against the
    oracle's fit, and against the single-problem call (which solves
    right-looking, so the two agree to rounding, not bit for bit)."""
    say("batched ridge fit, 32 problems, 1024 rows, 776 -> 1024, intercept")
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    n, f_in, f_out, count = 1024, 776, 1024, 32
    mix = torch.randn((f_in, f_in), generator=g, device=DEV) / f_in ** 0.5 + torch.eye(f_in, device=DEV)
    xs = [(torch.randn((n, f_in), generator=g, device=DEV) @ mix + 0.5).to(torch.bfloat16) for _ in range(count)]
    a = torch.randn((f_in, f_out), generator=g, device=DEV) / f_in ** 0.5
    ys = [(x.float() @ a + 0.3 * torch.randn((n, f_out), generator=g, device=DEV) - 1.0).to(torch.bfloat16)
          for x in xs]
    st = []
    ws, bs = kvx.fit_ridge_batched(xs, ys, lambda_rel=1e-3, fit_intercept=True, status=st)
    assert st == [kvx.OK] * count
    for i in (0, 13, 31):
        wo, bo, _ = O.ridge_fit(O.as_f64(xs[i]), O.as_f64(ys[i]), lam_rel=1e-3, fit_intercept=True)
        err_w = O.rel_err(ws[i].cpu().numpy(), wo)
        err_b = O.rel_err(bs[i].cpu().numpy(), bo)
        w1, b1 = kvx.fit_ridge(xs[i], ys[i], lambda_rel=1e-3, fit_intercept=True)
        d_w = O.rel_err(ws[i].cpu().numpy(), w1.cpu().numpy().astype(np.float64))
        say(f"  problem {i}: W {err_w:.3e}  b {err_b:.3e}  vs single call {d_w:.3e}")
        assert err_w <= TOL_BF16 and err_b <= TOL_BF16
        assert d_w <= 1e-5


def test_fit_batched_flags_each_problem():
    """lambda = 0 with one rank-deficient problem (half its feature columns
    zero: exact zero pivots) next to a well-posed one: the status of each is
    reported, the well-posed one is still solved (vs the oracle and the
    single-problem call), with the bias of the centred fit."""
    say("batched ridge fit with one singular problem, intercept")
    g = torch.Generator(device=DEV)
    g.manual_seed(91)
    n, f_in, f_out = 1024, 128, 64
    x0 = torch.randn((n, f_in), generator=g, device=DEV).to(torch.bfloat16)
    x1 = torch.randn((n, f_in), generator=g, device=DEV).to(torch.bfloat16)
    x1[:, 64:] = 0
    ys = [torch.randn((n, f_out), generator=g, device=DEV).to(torch.bfloat16) for _ in range(2)]
    st = []
    ws, bs = kvx.fit_ridge_batched([x0, x1], ys, fit_intercept=True, status=st)
    assert st == [kvx.OK, kvx.ERR_NOT_SPD]
    w1, b1 = kvx.fit_ridge(x0, ys[0], fit_intercept=True)
    assert torch.equal(ws[0], w1) and torch.equal(bs[0], b1)
    wo, bo, _ = O.ridge_fit(O.as_f64(x0), O.as_f64(ys[0]), fit_intercept=True)
    err_w = O.rel_err(ws[0].cpu().numpy(), wo)
    err_b = O.rel_err(bs[0].cpu().numpy(), bo)
    say(f"  W max|err|/RMS = {err_w:.3e}, b {err_b:.3e}")
    assert err_w <= TOL_F32 and err_b <= TOL_F32
    with pytest.raises(kvx.KvxError) as ei:
        kvx.fit_ridge_batched([x0, x1], ys, fit_intercept=True)
    assert ei.value.status == kvx.ERR_NOT_SPD


@pytest.mark.parametrize("n,f_in,ld_pad,f_out", [(1000, 264, 16, 72), (77, 64, 0, 8), (4160, 512, 8, 256)])
def test_fit_ragged_shapes(n, f_in, ld_pad, f_out):
    """bf16 fits whose sizes leave partial tiles: rows not a multiple of the
    64-row step (and fewer rows than one split per CU), features not a
    multiple of the 256-wide tile, padded row strides."""
    say(f"ridge fit n={n} f_in={f_in} (row stride {f_in + ld_pad}) f_out={f_out}")
    g = torch.Generator(device=DEV)
    g.manual_seed(n + f_in)
    xb = torch.randn((n, f_in + ld_pad), generator=g, device=DEV).to(torch.bfloat16)
    x = xb[:, :f_in]
    y = torch.randn((n, f_out), generator=g, device=DEV).to(torch.bfloat16)
    w, _ = kvx.fit_ridge(x, y, lambda_rel=1e-3)
    wo, _, _ = O.ridge_fit(O.as_f64(x), O.as_f64(y), lam_rel=1e-3)
    err = O.rel_err(w.cpu().numpy(), wo)
    say(f"  W max|err|/RMS = {err:.3e}")
    assert err <= TOL_F32


def test_fit_full_size_normal_equations():
    """65536 calibration rows, one layer: the fitted W satisfies the normal
    equations (G + lambda I) W = X^T Y, checked on random probe vectors with
    products the oracle's data forms directly (Freivalds)."""
    say("ridge fit 65536 rows: normal-equation residual on probes")
    c = fit_case(65536)
    taps = kvx.layer_map(36, 32, 3, 4)
    tm = kvx.align_tokens(dev_i32(c["send_end"]), dev_i32(c["recv_end"]))
    layer = 20
    x = kvx.gather_features(c["k_send"], tm, taps[layer])
    y = c["recv_k"][layer].reshape(65536, 1024)
    w, _ = kvx.fit_ridge(x, y, lambda_rel=1e-3)
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    X = O.features(c["k_send"], tmap_o, taps[layer])
    Y = O.as_f64(c["recv_k"][layer]).reshape(65536, 1024)
    W = w.cpu().numpy().astype(np.float64)
    lam = 1e-3 * float(np.einsum("ij,ij->", X, X)) / 3072
    rng = np.random.default_rng(0)
    for _ in range(3):
        r = rng.standard_normal(1024)
        wr = W @ r
        lhs = X.T @ (X @ wr) + lam * wr
        rhs = X.T @ (Y @ r)
        res = np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs)
        say(f"  residual {res:.3e}")
        assert res <= 1e-3


# ---------------------------------------------------------------- Recolor fit


def _recolor_err(w, b, wo, bo):
    return O.rel_err(w.cpu().numpy(), wo), O.rel_err(b.cpu().numpy(), bo)


@pytest.mark.parametrize("n,f_in,f_out", [(512, 64, 64), (700, 128, 64), (1000, 264, 72), (2100, 520, 136)])
def test_recolor_f32_vs_oracle(n, f_in, f_out):
    """fp32 calibration rows (moments accumulated in fp64): correlated
    features, a receiver partly explained by them; sizes spanning several
    64- and 256-wide solve blocks with ragged tails."""
    say(f"recolor fp32 n={n} f_in={f_in} f_out={f_out}")
    rng = np.random.default_rng(n + f_in)
    x = rng.standard_normal((n, f_in)) @ (rng.standard_normal((f_in, f_in)) / np.sqrt(f_in)) + 0.5
    y = 0.3 * (x @ rng.standard_normal((f_in, f_out)) / np.sqrt(f_in)) + rng.standard_normal((n, f_out)) - 1.0
    xt = torch.as_tensor(x, dtype=torch.float32, device=DEV)
    yt = torch.as_tensor(y, dtype=torch.float32, device=DEV)
    info = {}
    (w,), (b,) = kvx.fit_recolor([xt], [yt], info=info)
    wo, bo = O.recolor_fit(O.as_f64(xt), O.as_f64(yt))
    ew, eb = _recolor_err(w, b, wo, bo)
    say(f"  W max|err|/RMS = {ew:.3e}, b {eb:.3e}, {info['iters']} polar iterations")
    assert ew <= TOL_F32 and eb <= TOL_F32
    # a well-conditioned whitened cross-covariance converges in a few third-order
    # steps (a broken stopping test would run on to the iteration cap)
    assert 1 <= info["iters"] <= 25
    # moments of the translated calibration rows, from the oracle's data
    t = O.as_f64(xt) @ w.cpu().numpy().astype(np.float64) + b.cpu().numpy()
    ym = O.as_f64(yt)
    assert np.max(np.abs(t.mean(0) - ym.mean(0))) <= 1e-4 * np.sqrt(np.mean(ym * ym))
    ct = np.cov(t.T, bias=True)
    cy = np.cov(ym.T, bias=True)
    assert np.max(np.abs(ct - cy)) <= 1e-4 * np.max(np.abs(cy))


def test_recolor_recovers_planted_map():
    """An exact linear relation y = x A + c is recovered (the whitened
    cross-covariance is already orthonormal)."""
    say("recolor planted map")
    g = torch.Generator(device=DEV)
    g.manual_seed(17)
    n, f_in, f_out = 1500, 192, 64
    x = torch.randn((n, f_in), generator=g, device=DEV, dtype=torch.float64)
    a = torch.randn((f_in, f_out), generator=g, device=DEV, dtype=torch.float64) / np.sqrt(f_in)
    c = torch.randn(f_out, generator=g, device=DEV, dtype=torch.float64)
    xt, yt = x.float(), (x @ a + c).float()
    (w,), (b,) = kvx.fit_recolor([xt], [yt])
    # the relation holds up to the fp32 rounding of y
    an = a.cpu().numpy()
    ea = np.max(np.abs(w.cpu().numpy() - an)) / np.sqrt(np.mean(an * an))
    ec = np.max(np.abs(b.cpu().numpy() - c.cpu().numpy()))
    say(f"  |W - A| / RMS(A) = {ea:.3e}, |b - c| = {ec:.3e}")
    assert ea <= 1e-4 and ec <= 1e-4


@pytest.mark.parametrize("layer", [0, 15, 31])
def test_recolor_bf16_vs_oracle(layer):
    """Gathered bf16 features of 16384 calibration tokens (about 3600
    distinct sender rows; duplicated taps at layers 0 and 31 make S_xx
    singular: rho_x = 1e-3) -> the receiver's keys."""
    say(f"recolor bf16 layer {layer}, 16384 calibration rows")
    c = fit_case(16384)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    x = kvx.gather_features(c["k_send"], dev_i32(tmap_o), taps[layer])
    y = c["recv_k"][layer].reshape(16384, 1024)
    info = {}
    (w,), (b,) = kvx.fit_recolor([x], [y], rho_x=1e-3, info=info)
    wo, bo = O.recolor_fit(O.features(c["k_send"], tmap_o, taps[layer]), O.as_f64(y), rho_x=1e-3)
    ew, eb = _recolor_err(w, b, wo, bo)
    say(f"  W max|err|/RMS = {ew:.3e}, b {eb:.3e}, {info['iters']} polar iterations")
    assert ew <= TOL_BF16 and eb <= TOL_BF16


def test_recolor_too_few_distinct_rows():
    """4096 calibration tokens hold about 900 distinct sender rows, fewer
    than the 1024 outputs: the whitened cross-covariance has rank < 1024 (its
    smallest singular values vanish in the oracle's SVD), the Procrustes
    rotation is not determined, and the fit says so."""
    say("recolor with fewer distinct rows than outputs")
    c = fit_case(4096)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    assert np.unique(tmap_o).size < 1024
    x = kvx.gather_features(c["k_send"], dev_i32(tmap_o), taps[15])
    y = c["recv_k"][15].reshape(4096, 1024)
    st = []
    kvx.fit_recolor([x], [y], rho_x=1e-3, status=st)
    assert st == [kvx.ERR_NOT_CONVERGED]


def test_recolor_batched_statuses():
    """Two problems in one call: one with a constant receiver column (S_yy
    singular, rho_y = 0 -> not positive definite) next to a well-posed one,
    which is still fitted (vs the oracle)."""
    say("recolor batched, one singular receiver covariance")
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    n, f_in, f_out = 900, 128, 64
    xs = [torch.randn((n, f_in), generator=g, device=DEV).to(torch.bfloat16) for _ in range(2)]
    ys = [torch.randn((n, f_out), generator=g, device=DEV).to(torch.bfloat16) for _ in range(2)]
    ys[1][:, 7] = 2.0
    st = []
    ws, bs = kvx.fit_recolor(xs, ys, status=st)
    assert st == [kvx.OK, kvx.ERR_NOT_SPD]
    wo, bo = O.recolor_fit(O.as_f64(xs[0]), O.as_f64(ys[0]))
    ew, eb = _recolor_err(ws[0], bs[0], wo, bo)
    say(f"  W max|err|/RMS = {ew:.3e}, b {eb:.3e}")
    assert ew <= TOL_F32 and eb <= TOL_F32
    with pytest.raises(kvx.KvxError) as ei:
        kvx.fit_recolor(xs, ys)
    assert ei.value.status == kvx.ERR_NOT_SPD


def test_recolor_full_size_vs_oracle():
    """65536 calibration tokens, one layer (3072 -> 1024), the whole fitted
    map against the oracle's."""
    say("recolor 65536 rows, layer 20, vs the oracle")
    c = fit_case(65536)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    layer = 20
    x = kvx.gather_features(c["k_send"], dev_i32(tmap_o), taps[layer])
    y = c["recv_k"][layer].reshape(65536, 1024)
    info = {}
    (w,), (b,) = kvx.fit_recolor([x], [y], rho_x=1e-3, info=info)
    say(f"  {info['iters']} polar iterations; oracle ...")
    wo, bo = O.recolor_fit(O.features(c["k_send"], tmap_o, taps[layer]), O.as_f64(y), rho_x=1e-3)
    ew, eb = _recolor_err(w, b, wo, bo)
    say(f"  W max|err|/RMS = {ew:.3e}, b {eb:.3e}")
    assert ew <= TOL_BF16 and eb <= TOL_BF16


# ---------------------------------------------------------------- fp8 map storage


class Fp8Maps:
    """Oracle-quantised maps (codes [L][F_out][F_in] and scales [L][F_out]:
    one scale per output); indexing a layer gives its float64 map, row-major
    [F_in][F_out]."""

    def __init__(self, q, sc):
        self.q, self.sc = q, sc

    def __len__(self):
        return len(self.q)

    def __getitem__(self, l):
        return O.fp8_dequant(self.q[l], self.sc[l]).T


def oracle_fp8(w):
    """The oracle's fp8 storage of row-major maps w [L][F_in][F_out] (host
    array): each layer's output channels quantised (O.quantize_fp8 of W^T).
    Returns (codes [L][F_out][F_in], scales [L][F_out])."""
    qs = [O.quantize_fp8(np.ascontiguousarray(w[l].T)) for l in range(w.shape[0])]
    return np.stack([q for q, _ in qs]), np.stack([s_ for _, s_ in qs])


_MAPS8 = {}


def fp8_maps(k):
    """Maps of a flattened setting folded in fp32 and stored as fp8 by the
    library (device) and by the oracle (host): codes and scales must agree
    bit for bit."""
    if k not in _MAPS8:
        seed = synth.CONFIGS[k]["seed"]
        out = {}
        for r, role in enumerate(("k", "v")):
            say(f"  folding + quantising maps of setting {k} role {role}")
            wt, u, v, b = synth.flat_maps(32, 3072, 1024, seed * 100 + 20 + r, DEV, 16)
            g = kvx.fold_lowrank(wt, u, v, torch.float32)
            q, sc = kvx.quantize_fp8(g)
            wh, uh, vh = host(wt).numpy(), host(u).numpy(), host(v).numpy()
            qo, so = oracle_fp8(np.stack([O.fold_lowrank(wh[l], uh[l], vh[l])[0] for l in range(32)]))
            assert np.array_equal(host(q).numpy(), qo), "fp8 codes differ from the oracle's"
            assert np.array_equal(host(sc).numpy().view(np.uint32), so.view(np.uint32)), "fp8 scales differ"
            out[role] = (q, sc, b, Fp8Maps(qo, so), host(b).numpy().astype(np.float64))
            del wt, u, v, g
        _MAPS8[k] = out
    return _MAPS8[k]


def check_flat8(c, rows=None):
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap = kvx.align_tokens(dev_i32(c["send_end"]), dev_i32(c["recv_end"]))
    tmap_o = O.token_align(c["send_end"], c["recv_end"])
    m8 = fp8_maps(4)
    k, v = kvx.translate_fp8(c["k_send"], c["v_send"], tmap, taps, m8["k"][0], m8["v"][0], m8["k"][1], m8["v"][1],
                             m8["k"][2], m8["v"][2], send_rope_base=c["send_rope"], recv_rope_base=c["recv_rope"])
    torch.cuda.synchronize()
    n = tmap_o.size
    rows = np.arange(n) if rows is None else rows
    for role, out in (("k", k), ("v", v)):
        rk = role == "k"
        want = O.translate_rows(c[f"{role}_send"], tmap_o, taps, m8[role][3], m8[role][4], rows, per_head=False,
                                recv_heads=8, recv_head_dim=128, send_rope_base=c["send_rope"] if rk else 0.0,
                                recv_rope_base=c["recv_rope"] if rk else 0.0)
        err = O.rel_err(rows_of(out, rows), want)
        say(f"  fp8 maps n={n} {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16


def test_fp8_quantize_special_rows():
    """Zero rows, an outlier, tiny magnitudes (subnormal codes), negative
    zeros and exact ties: codes and scales bit for bit as the oracle's."""
    say("fp8 quantisation of special rows")
    rng = np.random.default_rng(2)
    w = rng.standard_normal((9, 3072)).astype(np.float32)
    w[1] = 0.0
    w[2, 100] = 1e5
    w[3] *= np.float32(3e-3)
    w[4] = -0.0
    w[4, 7] = 1.0
    w[5] = np.float32(448.0) * (np.arange(3072) % 253 - 126).astype(np.float32) / np.float32(126.0)
    w[6, :10] = [448.0, 464.0, 15.5, -15.5, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9, 17.0, 1.0, -0.0]
    # the rows are the output channels of one map W = w^T [3072][9]
    q, sc = kvx.quantize_fp8(torch.as_tensor(np.ascontiguousarray(w.T), device=DEV))
    qo, so = O.quantize_fp8(w)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), so.view(np.uint32))


def test_fp8_every_code_widens_exactly():
    """Every finite E4M3 code reaches the products exactly, as bf16 operands
    (values: one-hot sender rows select one code per output) and as fp16
    operands (keys rotated back at position 0, an identity rotation)."""
    say("fp8 maps: every code, bf16 and fp16 operands")
    val = O.e4m3_values()
    fin = np.isfinite(val)
    n = 1024
    x = torch.zeros((1, n, 8, 128), dtype=torch.bfloat16, device=DEV)
    x.view(n, 1024)[torch.arange(n), torch.arange(n)] = 1.0
    q = ((np.arange(256)[:, None] + np.arange(1024)[None, :]) % 256).astype(np.uint8)
    q[~fin[q]] = 0
    sc = torch.ones((1, 256), dtype=torch.float32, device=DEV)
    taps = np.zeros((1, 1), np.int32)
    _, v = kvx.translate_fp8(None, x, dev_i32(np.arange(n)), taps, None, torch.as_tensor(q[None], device=DEV), None,
                             sc, recv_heads=2, recv_head_dim=128)
    assert np.array_equal(O.as_f64(v).reshape(n, 256), val[q.T])
    kx = torch.randn((1, 4, 8, 128), device=DEV).to(torch.bfloat16)
    kx[0, 0] = 0
    kx[0, 0, 0, 5] = 1.0
    q2 = np.zeros((1, 256, 1024), np.uint8)
    q2[0, :, 5] = np.where(fin, np.arange(256), 0)
    k, _ = kvx.translate_fp8(kx, None, dev_i32(np.zeros(64)), taps, torch.as_tensor(q2, device=DEV), None, sc, None,
                             recv_heads=2, recv_head_dim=128, send_rope_base=1e4)
    got = O.as_f64(k).reshape(64, 256)
    assert np.array_equal(got, np.broadcast_to(val[q2[0, :, 5]], (64, 256)))


def test_fp8_maps_rope_small_all_elements():
    say("fp8 maps, flattened + RoPE, 700 receiver tokens")
    check_flat8(flat_case(4, 700, seed=15, with_maps=False))


def test_fp8_maps_rope_full_sampled_rows():
    say("fp8 maps, flattened + RoPE, 32768 receiver tokens, sampled rows")
    c = flat_case(4, with_maps=False)
    check_flat8(c, sample_rows(O.token_align(c["send_end"], c["recv_end"]), 256, 4))


def test_fp8_maps_key_norm_all_elements():
    """fp8 maps with the receiver's key normalisation and both rotations: the
    per-output scale is applied before the bias and the norm; every element of
    400 receiver tokens vs the oracle on the oracle's own quantised maps."""
    say("fp8 maps + receiver key norm + RoPE, 400 receiver tokens")
    send_end, recv_end = synth.token_ends(400, 83)
    shp = synth.CacheShape(36, len(send_end), 8, 128)
    taps = kvx.layer_map(36, 32, 3, 4)
    tmap_o = O.token_align(send_end, recv_end)
    caches, q8, bias = {}, {}, {}
    for r, role in enumerate(("k", "v")):
        caches[role] = synth.sender_cache(shp, 8400 + r, DEV, outlier_frac=0.01, outlier_scale=20.0,
                                          outlier_pairs=(role == "k"))
        wt, u, v, b = synth.flat_maps(32, 3072, 1024, 8500 + r, DEV, 16)
        q, sc = kvx.quantize_fp8(wt)
        qo, so = oracle_fp8(host(wt).numpy())
        assert np.array_equal(host(q).numpy(), qo)
        assert np.array_equal(host(sc).numpy().view(np.uint32), so.view(np.uint32))
        q8[role] = (q, sc, Fp8Maps(qo, so))
        bias[role] = b
        del wt, u, v
    kn = synth.key_norm_weights(32, 128, 8600, DEV)
    k, v = kvx.translate_fp8(caches["k"], caches["v"], dev_i32(tmap_o), taps, q8["k"][0], q8["v"][0], q8["k"][1],
                             q8["v"][1], bias["k"], bias["v"], send_rope_base=5e5, recv_rope_base=1e6,
                             recv_key_norm=kn, key_norm_eps=1e-6)
    torch.cuda.synchronize()
    rows = np.arange(tmap_o.size)
    for role, out in (("k", k), ("v", v)):
        rk = role == "k"
        want = O.translate_rows(caches[role], tmap_o, taps, q8[role][2], host(bias[role]).numpy().astype(np.float64),
                                rows, per_head=False, recv_heads=8, recv_head_dim=128,
                                send_rope_base=5e5 if rk else 0.0, recv_rope_base=1e6 if rk else 0.0,
                                recv_key_norm=host(kn).numpy() if rk else None, key_norm_eps=1e-6)
        err = O.rel_err(rows_of(out, rows), want)
        say(f"  fp8 + key norm {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16


@pytest.mark.parametrize("n_taps,fp32", [(1, False), (2, False), (3, False), (1, True)])
def test_flat_short_k_all_elements(n_taps, fp32):
    """Two-head caches give K extents of 4, 8 and 12 steps of 64 (fp32 maps
    double them): K loops that are only a tail, and whole groups of five
    steps followed by tails of every length; rotated keys."""
    L_S, L_R, H = 6, 4, 2
    send_end, recv_end = synth.token_ends(300, 90 + n_taps)
    shp = synth.CacheShape(L_S, len(send_end), H, 128)
    if n_taps == 2:  # any tap list is accepted: the matched layer and the next one
        m = kvx.layer_map(L_S, L_R, 1, 1)[:, 0]
        taps = np.stack([m, np.minimum(m + 1, L_S - 1)], axis=1).astype(np.int32)
    else:
        taps = kvx.layer_map(L_S, L_R, n_taps, 1)
    say(f"flattened, {n_taps} taps x {H} heads, fp32 maps {fp32}: K steps {n_taps * H * 128 * (2 if fp32 else 1) // 64}")
    tmap_o = O.token_align(send_end, recv_end)
    caches, maps, bias = {}, {}, {}
    for r, role in enumerate(("k", "v")):
        caches[role] = synth.sender_cache(shp, 9100 + r, DEV)
        wt, u, v, b = synth.flat_maps(L_R, n_taps * H * 128, H * 128, 9200 + r, DEV, 4)
        if fp32:
            maps[role] = (wt, F32Maps(host(wt).numpy()))
        else:
            wb = host(wt).to(torch.bfloat16)
            maps[role] = (wb.to(DEV), Bf16Maps(wb.view(torch.int16).numpy().view(np.uint16)))
        bias[role] = b
        del u, v
    k, v = kvx.translate(caches["k"], caches["v"], dev_i32(tmap_o), taps, maps["k"][0], maps["v"][0], bias["k"],
                         bias["v"], send_rope_base=5e5, recv_rope_base=1e6)
    torch.cuda.synchronize()
    rows = np.arange(tmap_o.size)
    for role, out in (("k", k), ("v", v)):
        rk = role == "k"
        want = O.translate_rows(caches[role], tmap_o, taps, maps[role][1], host(bias[role]).numpy().astype(np.float64),
                                rows, per_head=False, recv_heads=H, recv_head_dim=128,
                                send_rope_base=5e5 if rk else 0.0, recv_rope_base=1e6 if rk else 0.0)
        err = O.rel_err(rows_of(out, rows), want)
        say(f"  {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16



@pytest.mark.parametrize("n_taps,heads", [(1, 2), (2, 2), (3, 2), (2, 4), (5, 2)])
def test_fp8_short_k_all_elements(n_taps, heads):
    """fp8 maps over K extents of 4, 8, 12, 16 and 20 steps of 64: K loops
    that are only a tail, one whole group of twelve steps, and a group
    followed by a tail (W parts of 128 k serve two steps; the tail's dead
    steps load empty ranges); rotated keys, every element vs the oracle on
    the oracle's own quantised maps."""
    L_S, L_R = 6, 4
    send_end, recv_end = synth.token_ends(300, 70 + n_taps + heads)
    shp = synth.CacheShape(L_S, len(send_end), heads, 128)
    taps = np.stack([np.minimum(kvx.layer_map(L_S, L_R, 1, 1)[:, 0] + t, L_S - 1) for t in range(n_taps)],
                    axis=1).astype(np.int32)
    f_in = n_taps * heads * 128
    say(f"fp8 maps, {n_taps} taps x {heads} heads: K steps {f_in // 64}")
    tmap_o = O.token_align(send_end, recv_end)
    caches, q8, bias = {}, {}, {}
    for r, role in enumerate(("k", "v")):
        caches[role] = synth.sender_cache(shp, 9300 + r, DEV)
        wt, u, v, b = synth.flat_maps(L_R, f_in, 256, 9400 + r, DEV, 4)
        q, sc = kvx.quantize_fp8(wt)
        qo, so = oracle_fp8(host(wt).numpy())
        assert np.array_equal(host(q).numpy(), qo)
        q8[role] = (q, sc, Fp8Maps(qo, so))
        bias[role] = b
        del wt, u, v
    k, v = kvx.translate_fp8(caches["k"], caches["v"], dev_i32(tmap_o), taps, q8["k"][0], q8["v"][0], q8["k"][1],
                             q8["v"][1], bias["k"], bias["v"], recv_heads=2, recv_head_dim=128,
                             send_rope_base=5e5, recv_rope_base=1e6)
    torch.cuda.synchronize()
    rows = np.arange(tmap_o.size)
    for role, out in (("k", k), ("v", v)):
        rk = role == "k"
        want = O.translate_rows(caches[role], tmap_o, taps, q8[role][2], host(bias[role]).numpy().astype(np.float64),
                                rows, per_head=False, recv_heads=2, recv_head_dim=128,
                                send_rope_base=5e5 if rk else 0.0, recv_rope_base=1e6 if rk else 0.0)
        err = O.rel_err(rows_of(out, rows), want)
        say(f"  {role}: max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e})")
        assert err <= TOL_BF16


def test_async_align_and_recorded_translate():
    """The entries that do not synchronise: the alignment gives the same map
    and flags invalid offsets on the device; the translation with recorded
    events writes the same outputs, bit for bit, and the events time it."""
    say("asynchronous alignment and translation with recorded events")
    c = flat_case(4, 700, seed=17)
    taps = kvx.layer_map(36, 32, 3, 4)
    se, re_ = dev_i32(c["send_end"]), dev_i32(c["recv_end"])
    inv = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    m_sync = kvx.align_tokens(se, re_)
    m_async = kvx.align_tokens(se, re_, invalid=inv)
    torch.cuda.synchronize()
    assert torch.equal(m_sync, m_async) and int(inv.item()) == 0
    bad = c["recv_end"].copy()
    bad[10] = bad[9]                                    # not strictly increasing
    kvx.align_tokens(se, dev_i32(bad), invalid=inv)
    torch.cuda.synchronize()
    assert int(inv.item()) == 1
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for e in ev:
        e.record()
    kw = dict(send_rope_base=c["send_rope"], recv_rope_base=c["recv_rope"])
    k1, v1 = kvx.translate(c["k_send"], c["v_send"], m_sync, taps, c["wt_k"], c["wt_v"], c["b_k"], c["b_v"], **kw)
    k2, v2 = kvx.translate(c["k_send"], c["v_send"], m_async, taps, c["wt_k"], c["wt_v"], c["b_k"], c["b_v"],
                           events=ev, **kw)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    prep, main = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
    say(f"  recorded phases: preparation {prep:.3f} ms, translation {main:.3f} ms")
    assert prep >= 0.0 and main > 0.0


@pytest.mark.parametrize("case", ["flat_bf16_rope", "flat_f32_rope", "flat_bf16_plain", "perhead_f32_rope",
                                  "perhead_bf16", "f32_caches"])
def test_prepared_maps_equal_raw_maps(case):
    """kvx_prepare_maps + kvx_translate_prepared give the outputs of
    kvx_translate with the same row-major maps, bit for bit (the raw call
    prepares the same layout in its workspace), and the prepared call with a
    placement and events equals the raw placed call."""
    say(f"prepared maps vs raw maps: {case}")
    per_head = case.startswith("perhead")
    f32c = case == "f32_caches"
    rope = "rope" in case or f32c
    n_recv = 300
    send_end, recv_end = synth.token_ends(n_recv, 160)
    tm = dev_i32(O.token_align(send_end, recv_end))
    if f32c:
        L_S, L_R, H, d, n_taps = 5, 3, 2, 64, 3
    elif per_head:
        L_S, L_R, H, d, n_taps = 6, 14, 8, 128, 1
    else:
        L_S, L_R, H, d, n_taps = 10, 8, 8, 128, 3
    shp = synth.CacheShape(L_S, len(send_end), H, d)
    taps = kvx.layer_map(L_S, L_R, n_taps, 2)
    dt = torch.float32 if f32c else torch.bfloat16
    caches, maps, bias = {}, {}, {}
    for r, role in enumerate(("k", "v")):
        caches[role] = synth.sender_cache(shp, 1600 + r, DEV, dt)
        if per_head:
            w, b = synth.perhead_maps(L_R, H, d, 1610 + r, DEV)
        else:
            w, _, _, b = synth.flat_maps(L_R, n_taps * H * d, H * d, 1610 + r, DEV, 2)
        maps[role] = w.to(torch.bfloat16) if "bf16" in case else w
        bias[role] = b
    sb, rb = (1e4, 1e4) if f32c else ((5e5, 1e6) if rope else (0.0, 0.0))
    send = kvx.cache_desc(caches["k"], sb)
    recv = kvx.CacheDesc(L_R, n_recv, H, d, kvx.F32 if f32c else kvx.BF16, rb)
    w_dtype = kvx.BF16 if "bf16" in case else kvx.F32
    pk = kvx.prepare_maps(maps["k"], "k", send, recv, n_taps, per_head)
    pv = kvx.prepare_maps(maps["v"], "v", send, recv, n_taps, per_head)
    kw = dict(per_head=per_head, send_rope_base=sb, recv_rope_base=rb)
    k1, v1 = kvx.translate(caches["k"], caches["v"], tm, taps, maps["k"], maps["v"], bias["k"], bias["v"], **kw)
    k2, v2 = kvx.translate(caches["k"], caches["v"], tm, taps, pk, pv, bias["k"], bias["v"], prepared=True,
                           w_dtype=w_dtype, **kw)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    # the oracle on the same row-major maps
    rows = np.arange(n_recv)
    tol = TOL_F32 if f32c else TOL_BF16
    for role, out in (("k", k2), ("v", v2)):
        rk = role == "k"
        want = O.translate_rows(caches[role], O.token_align(send_end, recv_end), taps, O.as_f64(maps[role]),
                                O.as_f64(bias[role]), rows, per_head=per_head, recv_heads=H, recv_head_dim=d,
                                send_rope_base=sb if rk else 0.0, recv_rope_base=rb if rk else 0.0)
        err = O.rel_err(rows_of(out, rows), want)
        say(f"  {role}: max|err|/RMS = {err:.4e}")
        assert err <= tol
    if f32c:
        return
    # placement and events on the prepared path vs the raw placed call
    pool = n_recv + 40
    slot = torch.as_tensor(np.random.default_rng(3).permutation(pool)[:n_recv], device=DEV)
    outs = {}
    for name, prep in (("raw", False), ("prepared", True)):
        o = {role: torch.full((L_R, pool, H, d), 3.0, dtype=torch.bfloat16, device=DEV) for role in "kv"}
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)] if prep else None
        if ev:
            for e in ev:
                e.record()
        kvx.translate(caches["k"], caches["v"], tm, taps, pk if prep else maps["k"], pv if prep else maps["v"],
                      bias["k"], bias["v"], k_recv=o["k"], v_recv=o["v"], slot=slot, pool_rows=pool,
                      prepared=prep, w_dtype=w_dtype if prep else None, events=ev, **kw)
        outs[name] = o
    torch.cuda.synchronize()
    for role in "kv":
        assert torch.equal(outs["raw"][role], outs["prepared"][role])
