"""Bounds of the translation kernels, through the C-ABI.

* Guard bands: every output cache is the middle of a larger allocation whose
  leading and trailing bands hold a sentinel; after the call the bands are
  unchanged and the middle matches the oracle.  Covers the flattened path
  (bf16 maps, fp32 maps, fp8 maps, rotated keys), the per-head path (bf16 and
  fp32 maps, rotated keys) and the fp32-cache path.
* Clamped token maps: recv_to_send holds -5, n_send + 3 and n_send + 100
  among valid entries.  The sender caches sit in the middle of allocations
  padded on both sides with a different constant, so an unclamped index
  reads padding (and shows as a wrong value) instead of leaving the
  allocation.  The result must equal the oracle on the map clamped into
  [0, n_send).
"""
import sys

import numpy as np
import pytest
import torch

from cross_model_kv_kvx_amd import kvx, synth
from oracle import kvx_oracle as O
from tests.kvx_cases import TOL_BF16, TOL_F32, bf16_floor, rows_of

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENTINEL_BF16 = 0x7F7F          # a finite bf16 bit pattern no translated value here reaches
PAD_FILL = 1000.0               # sender padding: far outside the N(0,1) caches


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=DEV)


def guarded(shape, dtype, pad):
    """(allocation, middle view of `shape`) with `pad` sentinel elements on
    each side of the view."""
    n = int(np.prod(shape))
    if dtype == torch.bfloat16:
        flat = torch.full((n + 2 * pad,), SENTINEL_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    else:
        flat = torch.full((n + 2 * pad,), float("nan"), dtype=dtype, device=DEV)
    return flat, flat[pad:pad + n].view(shape)


def bands_intact(flat, pad):
    head, tail = flat[:pad], flat[flat.numel() - pad:]
    if flat.dtype == torch.bfloat16:
        want = torch.tensor(SENTINEL_BF16, dtype=torch.int16, device=DEV)
        return bool(torch.all(head.view(torch.int16) == want)) and bool(torch.all(tail.view(torch.int16) == want))
    return bool(torch.all(torch.isnan(head))) and bool(torch.all(torch.isnan(tail)))


def padded_sender(cache, pad):
    """`cache` copied into the middle of an allocation padded with PAD_FILL."""
    n = cache.numel()
    flat = torch.full((n + 2 * pad,), PAD_FILL, dtype=cache.dtype, device=DEV)
    mid = flat[pad:pad + n].view(cache.shape)
    mid.copy_(cache)
    return flat, mid


def broken_map(m, n_send):
    """The token map with out-of-range entries planted at the start, in the
    middle and at the end."""
    bad = np.asarray(m, dtype=np.int64).copy()
    bad[0] = -5
    bad[bad.size // 2] = n_send + 3
    bad[-1] = n_send + 100
    return bad


class Maps:
    """Per-layer float64 maps for the oracle from a host tensor."""

    def __init__(self, t):
        self.t = t

    def __len__(self):
        return self.t.shape[0]

    def __getitem__(self, l):
        return O.as_f64(self.t[l])


def flat_setting(map_kind, n_recv=300, seed=120, clamp=False, L_S=10, L_R=8):
    """Flattened translation with rotated keys into guarded outputs (and, with
    `clamp`, a planted out-of-range map over padded senders)."""
    send_end, recv_end = synth.token_ends(n_recv, seed)
    n_send = len(send_end)
    shp = synth.CacheShape(L_S, n_send, 8, 128)
    taps = kvx.layer_map(L_S, L_R, 3, 2)
    tmap_o = O.token_align(send_end, recv_end)
    m_gpu = broken_map(tmap_o, n_send) if clamp else tmap_o
    m_ref = np.clip(m_gpu, 0, n_send - 1)
    pad_s = 256 * 1024
    caches, gcaches, maps, bias = {}, {}, {}, {}
    for r, role in enumerate(("k", "v")):
        caches[role] = synth.sender_cache(shp, seed * 10 + r, DEV, outlier_frac=0.01, outlier_scale=20.0,
                                          outlier_pairs=(role == "k"))
        gcaches[role] = padded_sender(caches[role], pad_s)[1] if clamp else caches[role]
        wt, _, _, b = synth.flat_maps(L_R, 3072, 1024, seed * 10 + 5 + r, DEV, 4)
        if map_kind == "bf16":
            wb = wt.to(torch.bfloat16)
            maps[role] = (wb, Maps(wb.cpu()))
        elif map_kind == "f32":
            maps[role] = (wt, Maps(wt.cpu()))
        else:
            q, sc = kvx.quantize_fp8(wt)
            wh = wt.cpu().numpy()
            qs = [O.quantize_fp8(np.ascontiguousarray(wh[l].T)) for l in range(L_R)]  # one scale per output
            maps[role] = ((q, sc), [O.fp8_dequant(qo, so).T for qo, so in qs])
        bias[role] = b
    pad_o = 64 * 1024
    outs = {role: guarded((L_R, n_recv, 8, 128), torch.bfloat16, pad_o) for role in ("k", "v")}
    kw = dict(send_rope_base=5e5, recv_rope_base=1e6, k_recv=outs["k"][1], v_recv=outs["v"][1])
    if map_kind == "fp8":
        kvx.translate_fp8(gcaches["k"], gcaches["v"], dev_i32(m_gpu), taps, maps["k"][0][0], maps["v"][0][0],
                          maps["k"][0][1], maps["v"][0][1], bias["k"], bias["v"], **kw)
    else:
        kvx.translate(gcaches["k"], gcaches["v"], dev_i32(m_gpu), taps, maps["k"][0], maps["v"][0], bias["k"],
                      bias["v"], **kw)
    torch.cuda.synchronize()
    rows = np.arange(n_recv)
    for role in ("k", "v"):
        rk = role == "k"
        assert bands_intact(outs[role][0], pad_o), f"{role}: guard band overwritten"
        want = O.translate_rows(caches[role], m_ref, taps, maps[role][1], O.as_f64(bias[role]), rows, per_head=False,
                                recv_heads=8, recv_head_dim=128, send_rope_base=5e5 if rk else 0.0,
                                recv_rope_base=1e6 if rk else 0.0)
        err = O.rel_err(rows_of(outs[role][1], rows), want)
        say(f"  flattened {map_kind} maps{' (clamped map)' if clamp else ''} {role}: max|err|/RMS = {err:.4e}")
        assert err <= TOL_BF16


def perhead_setting(map_dtype, n_recv=300, seed=130, clamp=False, L_S=6, L_R=14):
    send_end, recv_end = synth.token_ends(n_recv, seed)
    n_send = len(send_end)
    shp = synth.CacheShape(L_S, n_send, 8, 128)
    taps = kvx.layer_map(L_S, L_R, 1)
    tmap_o = O.token_align(send_end, recv_end)
    m_gpu = broken_map(tmap_o, n_send) if clamp else tmap_o
    m_ref = np.clip(m_gpu, 0, n_send - 1)
    pad_s = 256 * 1024
    caches, gcaches, maps, bias = {}, {}, {}, {}
    for r, role in enumerate(("k", "v")):
        caches[role] = synth.sender_cache(shp, seed * 10 + r, DEV, channel_scale="loguniform")
        gcaches[role] = padded_sender(caches[role], pad_s)[1] if clamp else caches[role]
        wt, b = synth.perhead_maps(L_R, 8, 128, seed * 10 + 5 + r, DEV)
        maps[role] = wt.to(map_dtype)
        bias[role] = b
    pad_o = 64 * 1024
    outs = {role: guarded((L_R, n_recv, 8, 128), torch.bfloat16, pad_o) for role in ("k", "v")}
    kvx.translate(gcaches["k"], gcaches["v"], dev_i32(m_gpu), taps, maps["k"], maps["v"], bias["k"], bias["v"],
                  per_head=True, send_rope_base=5e5, recv_rope_base=1e6, k_recv=outs["k"][1], v_recv=outs["v"][1])
    torch.cuda.synchronize()
    rows = np.arange(n_recv)
    for role in ("k", "v"):
        rk = role == "k"
        assert bands_intact(outs[role][0], pad_o), f"{role}: guard band overwritten"
        want = O.translate_rows(caches[role], m_ref, taps, Maps(maps[role].cpu()), O.as_f64(bias[role]), rows,
                                per_head=True, recv_heads=8, recv_head_dim=128, send_rope_base=5e5 if rk else 0.0,
                                recv_rope_base=1e6 if rk else 0.0)
        err = O.rel_err(rows_of(outs[role][1], rows), want)
        say(f"  per-head {map_dtype} maps{' (clamped map)' if clamp else ''} {role}: max|err|/RMS = {err:.4e}")
        assert err <= TOL_BF16


def f32_setting(clamp, n_recv=96, seed=140):
    """fp32 caches (2 heads x 64), flattened over 3 taps with rotated keys."""
    send_end, recv_end = synth.token_ends(n_recv, seed)
    n_send = len(send_end)
    L_S, L_R, H, d = 5, 3, 2, 64
    shp = synth.CacheShape(L_S, n_send, H, d)
    taps = kvx.layer_map(L_S, L_R, 3, 1)
    tmap_o = O.token_align(send_end, recv_end)
    m_gpu = broken_map(tmap_o, n_send) if clamp else tmap_o
    m_ref = np.clip(m_gpu, 0, n_send - 1)
    pad_s = 256 * H * d
    caches, gcaches, maps, bias = {}, {}, {}, {}
    for r, role in enumerate(("k", "v")):
        caches[role] = synth.sender_cache(shp, seed * 10 + r, DEV, torch.float32)
        gcaches[role] = padded_sender(caches[role], pad_s)[1] if clamp else caches[role]
        wt, _, _, b = synth.flat_maps(L_R, 3 * H * d, H * d, seed * 10 + 5 + r, DEV, 2)
        maps[role], bias[role] = wt, b
    pad_o = 16 * H * d
    outs = {role: guarded((L_R, n_recv, H, d), torch.float32, pad_o) for role in ("k", "v")}
    kvx.translate(gcaches["k"], gcaches["v"], dev_i32(m_gpu), taps, maps["k"], maps["v"], bias["k"], bias["v"],
                  send_rope_base=1e4, recv_rope_base=1e4, k_recv=outs["k"][1], v_recv=outs["v"][1])
    torch.cuda.synchronize()
    rows = np.arange(n_recv)
    for role in ("k", "v"):
        rk = role == "k"
        assert bands_intact(outs[role][0], pad_o), f"{role}: guard band overwritten"
        want = O.translate_rows(caches[role], m_ref, taps, Maps(maps[role].cpu()), O.as_f64(bias[role]), rows,
                                per_head=False, recv_heads=H, recv_head_dim=d, send_rope_base=1e4 if rk else 0.0,
                                recv_rope_base=1e4 if rk else 0.0)
        err = O.rel_err(rows_of(outs[role][1], rows), want)
        say(f"  fp32 caches{' (clamped map)' if clamp else ''} {role}: max|err|/RMS = {err:.4e}")
        assert err <= TOL_F32


@pytest.mark.parametrize("map_kind", ["bf16", "f32", "fp8"])
def test_flat_guard_bands(map_kind):
    say(f"guard bands: flattened, {map_kind} maps, rotated keys")
    flat_setting(map_kind)


@pytest.mark.parametrize("map_dtype", [torch.bfloat16, torch.float32])
def test_perhead_guard_bands(map_dtype):
    say(f"guard bands: per-head, {map_dtype} maps, rotated keys")
    perhead_setting(map_dtype)


def test_f32_guard_bands():
    say("guard bands: fp32 caches")
    f32_setting(False)


@pytest.mark.parametrize("map_kind", ["bf16", "f32", "fp8"])
def test_flat_clamps_token_map(map_kind):
    say(f"out-of-range token map entries: flattened, {map_kind} maps")
    flat_setting(map_kind, clamp=True, seed=121)


@pytest.mark.parametrize("map_dtype", [torch.bfloat16, torch.float32])
def test_perhead_clamps_token_map(map_dtype):
    say(f"out-of-range token map entries: per-head, {map_dtype} maps")
    perhead_setting(map_dtype, clamp=True, seed=131)


def test_f32_clamps_token_map():
    say("out-of-range token map entries: fp32 caches")
    f32_setting(True, seed=141)


@pytest.mark.parametrize("map_kind", ["bf16", "f32"])
def test_flat_rotated_keys_large_values_small_maps(map_kind):
    """The fp16 operand path of rotated-back keys at the edges of its range:
    outlier channels of about 1e3 (fp16 holds up to 65504 with 11 significant
    bits) and map entries of about 1e-5 (below fp16's smallest normal,
    6.1e-5).  Every element of 300 receiver tokens is checked against a bound
    derived from the operand types: the map entries reach the products with
    an absolute error of at most 2^-25 (bf16 -> fp16; fp32 maps also lose
    2^-22 relative in the high/low split), the rotated keys with a relative
    error of 2^-11, the fp32 sums add at most 2^-16 of sum |x w|, the
    receiver rotation mixes the two members of a pair (bounds added), and
    the output is rounded to bf16 (half an ulp of the result).  max|err|/RMS
    is printed beside the bf16 floor: with outliers this large the rounding
    of the outputs alone reaches the 2e-2 of the bf16 bar, so the bar itself
    is not the check here."""
    say(f"rotated keys with outliers ~1e3, {map_kind} maps with entries ~1e-5")
    L_S, L_R, n_recv, seed = 10, 8, 300, 150
    send_end, recv_end = synth.token_ends(n_recv, seed)
    shp = synth.CacheShape(L_S, len(send_end), 8, 128)
    taps = kvx.layer_map(L_S, L_R, 3, 2)
    tmap_o = O.token_align(send_end, recv_end)
    k = synth.sender_cache(shp, seed * 10, DEV, outlier_frac=0.01, outlier_scale=1000.0, outlier_pairs=True)
    w32, _, _, b = synth.flat_maps(L_R, 3072, 1024, seed * 10 + 5, DEV, 4)
    w32 = w32 * 5e-4  # N(0,1)/sqrt(3072) * 5e-4: entries of about 1e-5
    b = b * 1e-2
    w = w32.to(torch.bfloat16) if map_kind == "bf16" else w32
    out, _ = kvx.translate(k, None, dev_i32(tmap_o), taps, w, None, b, None, send_rope_base=5e5,
                           recv_rope_base=1e6)
    torch.cuda.synchronize()
    rows = np.arange(n_recv)
    wm = Maps(w.cpu())
    want = O.translate_rows(k, tmap_o, taps, wm, O.as_f64(b), rows, per_head=False, recv_heads=8,
                            recv_head_dim=128, send_rope_base=5e5, recv_rope_base=1e6)
    got = rows_of(out, rows)
    assert np.all(np.isfinite(got))
    c_rel = 2.0 ** -11 + 2.0 ** -16 + (2.0 ** -22 if map_kind == "f32" else 0.0)
    worst = 0.0
    for l in range(L_R):
        x = O.features(k, tmap_o[rows], taps[l], 5e5)
        bound = 2.0 ** -25 * np.abs(x).sum(axis=1)[:, None] + c_rel * (np.abs(x) @ np.abs(wm[l]))
        bh = bound.reshape(n_recv, 8, 2, 64)
        pair = (bh[:, :, 0] + bh[:, :, 1])[:, :, None, :]          # the rotation mixes c and c + 64
        bound = np.broadcast_to(pair, bh.shape).reshape(n_recv, 1024)
        g = got[l]
        half_ulp = np.where(g != 0, 2.0 ** (np.floor(np.log2(np.abs(np.where(g != 0, g, 1.0)))) - 8), 0.0)
        excess = np.abs(g - want[l]) - (bound + half_ulp)
        worst = max(worst, float(np.max(np.abs(g - want[l]) / (bound + half_ulp))))
        assert np.all(excess <= 0), f"layer {l}: error above the operand bound"
    err = O.rel_err(got, want)
    say(f"  max|err|/RMS = {err:.4e} (bf16 floor {bf16_floor(want):.4e}); worst error / bound = {worst:.3f}")
