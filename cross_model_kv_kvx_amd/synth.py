"""Seeded synthetic inputs for the KV-cache translator.

This module only draws random numbers and lays them out in the shapes of the
workloads; it holds none of the translation arithmetic (no alignment, layer
matching, rotation, affine map, fold or fit).  Both the HIP path and the CPU
oracle take what it returns as plain inputs.

Workloads (sizes from the five translation settings the method is measured on):

* ``cfg1`` matched-KV single layer, fp32, 2 heads x 64 dims, 128 tokens,
  512 calibration tokens, identical tokenizations.
* ``cfg2`` matched-KV same family, bf16 caches, 32 -> 80 layers, 8 heads x 128,
  4096 tokens, fp32 per-head 128x128 maps, per-channel log-uniform scales.
* ``cfg3`` cross-family, 36 -> 32 layers, 8 heads x 128, three sender taps,
  flattened 3072 -> 1024 maps (dense + rank-16), 8192 receiver tokens over a
  shared synthetic string (sender token lengths 1..8 chars, receiver 1..6).
* ``cfg4`` as cfg3 at 32768 receiver tokens, keys stored rotated (base 5e5 at
  the sender, 1e6 at the receiver), 1% outlier channels scaled x20.
* ``cfg5`` ridge fit on 65536 calibration tokens, then translation of a fresh
  16384-token cache with the fitted maps.

Large tensors are drawn with ``torch`` on the requested device (a seeded
``torch.Generator``), token lengths with ``numpy.random.default_rng``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

__all__ = [
    "CacheShape", "CONFIGS", "token_ends", "identical_ends", "gaussian",
    "sender_cache", "flat_maps", "perhead_maps", "receiver_cache", "config",
]


@dataclass(frozen=True)
class CacheShape:
    layers: int
    tokens: int
    heads: int
    head_dim: int

    @property
    def row(self) -> int:
        return self.heads * self.head_dim

    def shape(self):
        return (self.layers, self.tokens, self.heads, self.head_dim)


# Per-workload constants.  Token counts of the sender side in cfg3-5 follow
# from the synthetic string and are filled in by ``config``.
CONFIGS = {
    1: dict(seed=1, send_layers=1, recv_layers=1, heads=2, head_dim=64,
            tokens=128, cal_tokens=512, per_head=True, n_taps=1, dtype="f32",
            lam=1e-2),
    2: dict(seed=2, send_layers=32, recv_layers=80, heads=8, head_dim=128,
            tokens=4096, per_head=True, n_taps=1, dtype="bf16"),
    3: dict(seed=3, send_layers=36, recv_layers=32, heads=8, head_dim=128,
            recv_tokens=8192, per_head=False, n_taps=3, tap_stride=4,
            dtype="bf16", rank=16),
    4: dict(seed=4, send_layers=36, recv_layers=32, heads=8, head_dim=128,
            recv_tokens=32768, per_head=False, n_taps=3, tap_stride=4,
            dtype="bf16", rank=16, send_rope=500000.0, recv_rope=1000000.0,
            outlier_frac=0.01, outlier_scale=20.0),
    5: dict(seed=5, fresh_seed=6, send_layers=36, recv_layers=32, heads=8,
            head_dim=128, cal_tokens=65536, recv_tokens=16384, per_head=False,
            n_taps=3, tap_stride=4, dtype="bf16", lam_rel=1e-3),
}


def token_ends(n_recv: int, seed: int, recv_len=(1, 6), send_len=(1, 8)):
    """Two tokenizations of one synthetic string of T characters.

    Receiver token lengths are drawn uniformly in ``recv_len`` (inclusive);
    T is their total.  Sender lengths are drawn uniformly in ``send_len``
    until they cover T; the last sender token is cut so it ends at T.
    Returns exclusive character-end offsets ``(send_end, recv_end)``, both
    int32 and strictly increasing.
    """
    rng = np.random.default_rng(seed)
    rl = rng.integers(recv_len[0], recv_len[1] + 1, size=n_recv, dtype=np.int64)
    recv_end = np.cumsum(rl)
    total = int(recv_end[-1]) if n_recv else 0
    mean_s = 0.5 * (send_len[0] + send_len[1])
    ends = []
    covered = 0
    while covered < total:
        k = max(16, int((total - covered) / mean_s * 1.1) + 16)
        sl = rng.integers(send_len[0], send_len[1] + 1, size=k, dtype=np.int64)
        e = covered + np.cumsum(sl)
        cut = np.searchsorted(e, total, side="left")
        if cut < k:
            e = e[: cut + 1]
            e[-1] = total
        ends.append(e)
        covered = int(e[-1])
    send_end = np.concatenate(ends) if ends else np.zeros(0, np.int64)
    return send_end.astype(np.int32), recv_end.astype(np.int32)


def identical_ends(n: int, seed: int, lens=(1, 6)):
    """One tokenization used by both sides (matched-KV settings)."""
    rng = np.random.default_rng(seed)
    e = np.cumsum(rng.integers(lens[0], lens[1] + 1, size=n, dtype=np.int64))
    return e.astype(np.int32), e.astype(np.int32).copy()


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian(shape, seed: int, device="cpu", std: float = 1.0) -> torch.Tensor:
    """fp32 N(0, std^2) of ``shape``, seeded."""
    g = _gen(device, seed)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def sender_cache(shape: CacheShape, seed: int, device="cpu", dtype=torch.bfloat16,
                 channel_scale=None, outlier_frac: float = 0.0,
                 outlier_scale: float = 1.0, outlier_pairs: bool = False):
    """One role's cache ``[layers][tokens][heads][head_dim]``, N(0,1) entries.

    ``channel_scale="loguniform"`` multiplies each (layer, head, channel) by a
    factor exp(U(ln 1/4, ln 4)), fixed over tokens.

    ``outlier_frac`` picks round(frac * heads * head_dim) channels per layer
    and multiplies them by ``outlier_scale``.  With ``outlier_pairs`` the picks
    are whole rotation pairs (channel c and c + head_dim/2 of one head), so a
    rotated cache drawn here has the same distribution as rotating a content
    cache whose outlier channels were drawn first: a pair of i.i.d. centred
    Gaussians scaled together is invariant in law under any planar rotation.
    """
    L, N, H, d = shape.shape()
    g = _gen(device, seed)
    x = torch.randn((L, N, H, d), generator=g, device=device, dtype=torch.float32)
    if channel_scale == "loguniform":
        u = torch.rand((L, 1, H, d), generator=g, device=device, dtype=torch.float32)
        s = torch.exp(math.log(0.25) + u * (math.log(4.0) - math.log(0.25)))
        x.mul_(s)
    elif channel_scale is not None:
        raise ValueError(channel_scale)
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * H * d))
        for layer in range(L):
            if outlier_pairs:
                n_pairs = max(1, n_out // 2)
                pick = torch.randperm(H * (d // 2), generator=g, device=device)[:n_pairs]
                h = pick // (d // 2)
                c = pick % (d // 2)
                x[layer, :, h, c] *= outlier_scale
                x[layer, :, h, c + d // 2] *= outlier_scale
            else:
                pick = torch.randperm(H * d, generator=g, device=device)[:n_out]
                x[layer, :, pick // d, pick % d] *= outlier_scale
    return x.to(dtype)


def receiver_cache(shape: CacheShape, seed: int, device="cpu", dtype=torch.bfloat16):
    """A stand-in for a receiver's own cache (ridge targets): N(0,1) entries."""
    return sender_cache(shape, seed, device=device, dtype=dtype)


def flat_maps(recv_layers: int, f_in: int, f_out: int, seed: int, device="cpu",
              rank: int = 16):
    """Flattened affine maps for one role, row-major (y = x W).

    Returns ``w`` fp32 ``[L][f_in][f_out]`` (w[f][o] multiplies feature f
    into output o), rank factors ``a`` fp32 ``[L][f_in][rank]`` and ``b_lr``
    fp32 ``[L][rank][f_out]`` (the correction is A B), and bias fp32
    ``[L][f_out]``.  w, a ~ N(0,1)/sqrt(f_in); b_lr ~ 0.1 N(0,1)/sqrt(rank);
    bias ~ N(0, 0.1^2).
    """
    g = _gen(device, seed)
    w = torch.randn((recv_layers, f_in, f_out), generator=g, device=device) / math.sqrt(f_in)
    a = torch.randn((recv_layers, f_in, rank), generator=g, device=device) / math.sqrt(f_in)
    b_lr = torch.randn((recv_layers, rank, f_out), generator=g, device=device) * (0.1 / math.sqrt(rank))
    b = torch.randn((recv_layers, f_out), generator=g, device=device) * 0.1
    return w.contiguous(), a.contiguous(), b_lr.contiguous(), b.contiguous()


def perhead_maps(recv_layers: int, heads: int, head_dim: int, seed: int, device="cpu",
                 std=None, bias_std: float = 0.1):
    """Per-head maps for one role: ``w`` fp32 ``[L][H][d_in][d_out]``
    (w[l][h][c][o]: input channel c to output channel o of head h) with
    N(0,1)/sqrt(d) entries (or ``std``), bias fp32 ``[L][H*d]``."""
    g = _gen(device, seed)
    s = (1.0 / math.sqrt(head_dim)) if std is None else std
    w = torch.randn((recv_layers, heads, head_dim, head_dim), generator=g, device=device) * s
    b = torch.randn((recv_layers, heads * head_dim), generator=g, device=device) * bias_std
    return w.contiguous(), b.contiguous()


def key_norm_weights(recv_layers: int, head_dim: int, seed: int, device="cpu"):
    """Weights of a receiver's key normalisation, fp32 [L][d], 1 + 0.1 N(0,1)
    (a trained norm's weights sit near one)."""
    g = _gen(device, seed)
    return (1.0 + 0.1 * torch.randn((recv_layers, head_dim), generator=g, device=device)).contiguous()


def config(k: int, device="cpu", small: bool = False):
    """Inputs of workload ``k`` as a dict of tensors / arrays.

    ``small=True`` shrinks token counts (same structure) for CPU tests.
    Keys depend on the workload; see the module docstring.
    """
    c = dict(CONFIGS[k])
    seed = c["seed"]
    out = dict(cfg=k, **c)
    if k == 1:
        n, ncal = c["tokens"], c["cal_tokens"]
        shp = CacheShape(1, n, c["heads"], c["head_dim"])
        cal = CacheShape(1, ncal, c["heads"], c["head_dim"])
        out["send_end"], out["recv_end"] = identical_ends(n, seed)
        for r, role in enumerate(("k", "v")):
            out[f"x_cal_{role}"] = sender_cache(cal, seed * 100 + r, device, torch.float32)
            out[f"x_{role}"] = sender_cache(shp, seed * 100 + 10 + r, device, torch.float32)
            w, b = perhead_maps(1, c["heads"], c["head_dim"], seed * 100 + 20 + r, device,
                                std=1.0 / math.sqrt(c["head_dim"]))
            out[f"w_true_{role}"], out[f"b_true_{role}"] = w, b
            out[f"noise_cal_{role}"] = gaussian(cal.shape(), seed * 100 + 30 + r, device, 0.01)
            out[f"noise_{role}"] = gaussian(shp.shape(), seed * 100 + 40 + r, device, 0.01)
        return out
    if k == 2:
        n = 256 if small else c["tokens"]
        ls, lr = c["send_layers"], c["recv_layers"]
        shp = CacheShape(ls, n, c["heads"], c["head_dim"])
        out["send_end"], out["recv_end"] = identical_ends(n, seed)
        out["send_shape"] = shp
        out["recv_shape"] = CacheShape(lr, n, c["heads"], c["head_dim"])
        for r, role in enumerate(("k", "v")):
            out[f"{role}_send"] = sender_cache(shp, seed * 100 + r, device,
                                               channel_scale="loguniform")
            w, b = perhead_maps(lr, c["heads"], c["head_dim"], seed * 100 + 20 + r, device)
            out[f"w_{role}"], out[f"b_{role}"] = w, b
        return out
    if k in (3, 4, 5):
        nr = c["cal_tokens"] if k == 5 else c["recv_tokens"]
        if small:
            nr = 512
        send_end, recv_end = token_ends(nr, seed)
        out["send_end"], out["recv_end"] = send_end, recv_end
        ls, lr, H, d = c["send_layers"], c["recv_layers"], c["heads"], c["head_dim"]
        shp = CacheShape(ls, len(send_end), H, d)
        out["send_shape"] = shp
        out["recv_shape"] = CacheShape(lr, nr, H, d)
        f_in, f_out = c["n_taps"] * H * d, H * d
        outl = c.get("outlier_frac", 0.0)
        for r, role in enumerate(("k", "v")):
            out[f"{role}_send"] = sender_cache(
                shp, seed * 100 + r, device, outlier_frac=outl,
                outlier_scale=c.get("outlier_scale", 1.0),
                outlier_pairs=(role == "k" and "send_rope" in c))
            if k == 5:
                out[f"{role}_recv_native"] = receiver_cache(out["recv_shape"], seed * 100 + 50 + r, device)
            else:
                w, a, b_lr, b = flat_maps(lr, f_in, f_out, seed * 100 + 20 + r, device, c["rank"])
                out[f"w_{role}"], out[f"a_{role}"], out[f"blr_{role}"], out[f"b_{role}"] = w, a, b_lr, b
        if k == 5:
            fs = c["fresh_seed"]
            nf = 256 if small else c["recv_tokens"]
            fe, fr = token_ends(nf, fs)
            out["fresh_send_end"], out["fresh_recv_end"] = fe, fr
            fshp = CacheShape(ls, len(fe), H, d)
            out["fresh_send_shape"] = fshp
            out["fresh_recv_shape"] = CacheShape(lr, nf, H, d)
            for r, role in enumerate(("k", "v")):
                out[f"{role}_fresh_send"] = sender_cache(fshp, fs * 100 + r, device)
        return out
    raise ValueError(k)
