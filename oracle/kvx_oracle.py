"""CPU oracle for cross-model KV-cache translation.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never does, and shares
no code with it.

Plain, slow, obviously-correct definitions in float64 (numpy), single pass,
per receiver token, no deduplication, no blocking or fusion.  Sources (the
reader has the pages; no line numbers):

* [HF]  "Prefill-Free Cross-Family KV Cache Transfer for Heterogeneous
  Multi-Agent LLMs" (ai.info summary), sections "Key Contributions" and
  "Methodology in Plain English" (token alignment, layer taps, flattened
  maps, rank-16 corrections folded into one affine map per layer and role).
* [LB]  "Cross-Model KV Cache Transfer in Production: Architecture,
  Closed-Form Ridge Projections, and Cascaded Serving Economics" (llms.blog),
  section "The Closed-Form Ridge Mapping Pipeline", stages 1-4 (RoPE strip,
  per-head ridge projection W = (X^T X + lambda I)^-1 X^T Y, layer alignment,
  RoPE re-application) and "Implementation Guidelines" (lambda range,
  precision).
* [UC]  "A Universal Context-Reuse Layer for Cross-Model KV Sharing"
  (review), section 2.2 (the interface KV_B = T_{A->B}(KV_A)).

Readings where the pages are silent are listed beside each function.
Parity pins: tests/test_oracle_*.py.  Nothing here is "parity unpinned".
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# ---------------------------------------------------------------------------
# number formats (not method arithmetic; the oracle keeps its own copy)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def as_f64(t) -> np.ndarray:
    """Any torch tensor (fp32/bf16/fp16) or numpy array -> float64 numpy."""
    if hasattr(t, "detach"):  # torch tensor
        import torch
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
        return t.to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


# ---------------------------------------------------------------------------
# A1  token alignment   [HF] "Key Contributions" 1, "Methodology" step 1


def token_align(send_end, recv_end) -> np.ndarray:
    """Receiver->sender token map from shared character-end boundaries.

    ``send_end``/``recv_end``: exclusive character-end offsets of each token,
    strictly increasing and > 0 (reading: a boundary is the end offset of a
    token; a *shared* boundary is an offset that ends both a sender and a
    receiver token).

    For receiver token i ending at e_i: take the latest shared boundary
    b <= e_i; map[i] is the sender token that ends at b.  If e_i itself is
    shared this is the sender token ending exactly there (many-to-one: the
    sender token at the matched boundary, no averaging); otherwise the
    receiver token reuses the state of the latest preceding shared boundary
    (forward fill).  Receiver tokens before the first shared boundary map to
    sender token 0 (reading: the pages do not say).
    """
    s = np.asarray(send_end, dtype=np.int64)
    r = np.asarray(recv_end, dtype=np.int64)
    for name, e in (("send_end", s), ("recv_end", r)):
        if e.size and (e[0] <= 0 or np.any(np.diff(e) <= 0)):
            raise ValueError(f"{name} must be positive and strictly increasing")
    out = np.zeros(r.size, dtype=np.int64)
    j = 0
    last_shared = -1
    for i in range(r.size):
        e = r[i]
        while j < s.size and s[j] < e:
            j += 1
        if j < s.size and s[j] == e:
            last_shared = j
        out[i] = last_shared if last_shared >= 0 else 0
    return out


# ---------------------------------------------------------------------------
# A2  layer matching   [HF] "Methodology" step 2; [LB] stage 3


def layer_match(l: int, send_layers: int, recv_layers: int) -> int:
    """Proportional depth match: round(l (L_S-1)/(L_R-1)), halves rounded up,
    in exact rational arithmetic; 0 when the receiver has one layer.

    Reading: the blog's round(L_t * L_src / L_tgt) runs past the last layer
    for 0-based indices, so the (L-1) ratio that maps first to first and last
    to last is used.
    """
    if recv_layers == 1:
        return 0
    q = Fraction(l * (send_layers - 1), recv_layers - 1)
    return int((q + Fraction(1, 2)).__floor__())


def layer_taps(send_layers: int, recv_layers: int, n_taps: int = 3, stride: int = 4) -> np.ndarray:
    """Sender layers read by each receiver layer: the matched layer m and its
    neighbours at offsets (t - (n_taps-1)/2) * stride, clamped into
    [0, L_S-1], duplicates kept, in offset order (-4, 0, +4 for 3 taps)."""
    if n_taps < 1 or n_taps % 2 == 0:
        raise ValueError("n_taps must be odd")
    taps = np.zeros((recv_layers, n_taps), dtype=np.int64)
    for l in range(recv_layers):
        m = layer_match(l, send_layers, recv_layers)
        for t in range(n_taps):
            off = (t - (n_taps - 1) // 2) * stride
            taps[l, t] = min(max(m + off, 0), send_layers - 1)
    return taps


# ---------------------------------------------------------------------------
# RoPE   [LB] stage 1 (strip R_-m) and stage 4 (re-apply R_m of the target)


def rope_angles(pos, head_dim: int, base: float) -> np.ndarray:
    """phi[p, j] = pos_p * base^(-2j/d), j < d/2, in float64.
    Reading: half-split pairs (c, c+d/2), no frequency scaling."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * j / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]


def rope_rotate(x, pos, base: float, sign: int) -> np.ndarray:
    """Rotate each head vector of ``x`` ([n, H, d]) at positions ``pos`` ([n])
    by angle sign*phi: pair (a, b) = (x_j, x_{j+d/2}) becomes
    (a cos - b sin, a sin + b cos).  sign=-1 is the inverse R_-m."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    phi = sign * rope_angles(pos, d, base)[:, None, :]  # [n, 1, d/2]
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


# ---------------------------------------------------------------------------
# A3  runs of equal map values (an exact restructuring of the reuse of one sender
#     token's state by every receiver token aligned to it)


def runs(token_map) -> tuple[np.ndarray, np.ndarray]:
    """Maximal runs of equal consecutive values of the map.
    Returns (uniq[U], run_begin[U+1]) with uniq[u] = map[run_begin[u]]."""
    m = np.asarray(token_map, dtype=np.int64)
    starts = [i for i in range(m.size) if i == 0 or m[i] != m[i - 1]]
    uniq = m[starts] if starts else np.zeros(0, np.int64)
    return uniq.astype(np.int64), np.array(starts + [m.size], dtype=np.int64)


# ---------------------------------------------------------------------------
# A4  features   [HF] "Methodology" step 2; [LB] stage 1


def features(cache, src_rows, taps_of_layer, derotate_base: float = 0.0) -> np.ndarray:
    """Flattened sender features of the receiver rows whose sender tokens are
    ``src_rows``: concatenate, over the taps in order, the whole cached row
    (all heads) of that sender layer; feature f = tap*H*d + h*d + c.
    With ``derotate_base`` > 0 each head vector is first rotated back by its
    own sender position (the sender token index src_rows[i]).

    ``cache``: [L_S][N_S][H][d] (torch or numpy)."""
    src_rows = np.asarray(src_rows, dtype=np.int64)
    parts = []
    for t in taps_of_layer:
        x = as_f64(cache[int(t)][src_rows]) if hasattr(cache, "detach") else \
            np.asarray(cache[int(t)], dtype=np.float64)[src_rows]
        if derotate_base:
            x = rope_rotate(x, src_rows, derotate_base, -1)
        parts.append(x.reshape(x.shape[0], -1))
    return np.concatenate(parts, axis=1)


# ---------------------------------------------------------------------------
# A5/A7 affine maps and A6 re-rotation   [LB] stages 2 and 4; [HF] step 2


def affine(x, w, b=None) -> np.ndarray:
    """y = x W + b, W row-major [F_in][F_out] (a row vector of features times
    the map, as the blog writes K_content W_K)."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64)
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)[None, :]
    return y


def key_norm(y, weight, eps: float) -> np.ndarray:
    """The receiver's own key normalisation, applied to mapped keys before
    its RoPE ([HF] "Methodology" step 2: keys are mapped before key
    normalisation and RoPE, then the receiver applies its own).  The pages
    do not give its form; reading: RMS normalisation of each head vector
    over head_dim with a per-channel weight shared by the heads of a layer,
    y / sqrt(mean(y^2) + eps) * weight.  ``y``: [n, H, d]; ``weight``: [d]."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    ms = np.mean(y * y, axis=-1, keepdims=True)
    return y / np.sqrt(ms + eps) * w


def translate_rows(send_cache, token_map, taps, w, bias, rows, *, per_head: bool,
                   recv_heads: int, recv_head_dim: int,
                   send_rope_base: float = 0.0, recv_rope_base: float = 0.0,
                   recv_key_norm=None, key_norm_eps: float = 1e-6) -> np.ndarray:
    """Translated receiver rows for one role (K or V), all receiver layers.

    ``rows``: receiver token indices to produce.  Returns float64
    [L_R][len(rows)][H_R*d_R], unrounded.

    Flattened: y = features(...) W_l + b_l, w [L_R][F_in][F_out].  Per head
    (single tap, H and d equal on both sides): y_h = x_h W_{l,h} + b_{l,h},
    w [L_R][H][d][d] with w[l][h][c][o] taking input channel c to output o.
    Keys: with ``send_rope_base`` the sender keys are de-rotated at the sender
    position; with ``recv_rope_base`` the mapped key of receiver row i is
    rotated at position i (bias added before the rotation; values are never
    rotated).  With ``recv_key_norm`` ([L_R][d_R]) the mapped keys are
    normalised by ``key_norm`` (after the bias, before the receiver rotation).
    """
    rows = np.asarray(rows, dtype=np.int64)
    tm = np.asarray(token_map, dtype=np.int64)
    src = tm[rows]
    L_R = len(taps)
    out = np.zeros((L_R, rows.size, recv_heads * recv_head_dim), dtype=np.float64)
    for l in range(L_R):
        x = features(send_cache, src, taps[l], send_rope_base)
        bl = None if bias is None else as_f64(bias[l])
        if per_head:
            d = recv_head_dim
            wl = as_f64(w[l])
            y = np.zeros((rows.size, recv_heads * d))
            for h in range(recv_heads):
                y[:, h * d:(h + 1) * d] = affine(x[:, h * d:(h + 1) * d], wl[h],
                                                 None if bl is None else bl[h * d:(h + 1) * d])
        else:
            y = affine(x, as_f64(w[l]), bl)
        if recv_key_norm is not None:
            y = key_norm(y.reshape(rows.size, recv_heads, recv_head_dim), as_f64(recv_key_norm[l]),
                         key_norm_eps).reshape(rows.size, -1)
        if recv_rope_base:
            y = rope_rotate(y.reshape(rows.size, recv_heads, recv_head_dim), rows,
                            recv_rope_base, +1).reshape(rows.size, -1)
        out[l] = y
    return out


# ---------------------------------------------------------------------------
# A8  rank-16 fold   [HF] "Key Contributions" 3, "Methodology" step 3


def fold_lowrank(w, a, b):
    """Fold a low-rank correction into a fixed map, in float32, then bf16.

    W_eff = W + A B with W [F_in][F_out], A [F_in][r], B [r][F_out]
    (row-major, y = x W): w_eff[f][o] = w[f][o] + sum_r a[f][r] b[r][o].
    Reading of a fold done in fp32 and cast to bf16: each product rounded to fp32, summed
    in rank order from r = 0 in fp32 (no fused multiply-add), added to w in
    fp32, then rounded to bf16 (nearest even).  Returns (fp32 sum, bf16
    bits)."""
    w = np.asarray(w, dtype=np.float32)
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    acc = None
    for r in range(a.shape[1]):
        p = (a[:, r][:, None] * b[r, :][None, :]).astype(np.float32)
        acc = p if acc is None else (acc + p).astype(np.float32)
    tot = w if acc is None else (w + acc).astype(np.float32)
    return tot, f32_to_bf16_bits(tot)


def fold_lowrank_f64(w, a, b) -> np.ndarray:
    """The same fold in float64, unrounded (for checking the fp32 order)."""
    return np.asarray(w, np.float64) + np.asarray(a, np.float64) @ np.asarray(b, np.float64)


# ---------------------------------------------------------------------------
# A9/A10  ridge fit   [LB] stage 2 and "Implementation Guidelines" 1


def gram(x, y):
    """G = X^T X, C = X^T Y, column sums; float64."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    return x.T @ x, x.T @ y, x.sum(axis=0), y.sum(axis=0)


def ridge_lambda(g, lam_abs: float, lam_rel: float) -> float:
    """lambda = lam_abs + lam_rel * trace(G) / F_in (reading: a relative
    penalty scales with the mean feature energy)."""
    return float(lam_abs + lam_rel * np.trace(g) / g.shape[0])


def ridge_fit(x, y, lam_abs: float = 0.0, lam_rel: float = 0.0, fit_intercept: bool = False):
    """W = (X^T X + lambda I)^-1 X^T Y.

    With ``fit_intercept`` the bias is unpenalised: X and Y are centred by
    their column means, W solves the centred system, b = mean_y - mean_x W.
    lambda is taken from the Gram that is regularised (centred if centring).
    Returns (W [F_in][F_out], b [F_out] or None, lambda)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if fit_intercept:
        mx, my = x.mean(axis=0), y.mean(axis=0)
        x, y = x - mx, y - my
    g, c, _, _ = gram(x, y)
    lam = ridge_lambda(g, lam_abs, lam_rel)
    w = np.linalg.solve(g + lam * np.eye(g.shape[0]), c)
    b = (my - mx @ w) if fit_intercept else None
    return w, b, lam


# ---------------------------------------------------------------------------
# Recolor: moment-matched affine map   [HF] Key Contributions 2, Methodology 3


def spd_power(s, p: float) -> np.ndarray:
    """S^p of a symmetric positive definite matrix from its eigendecomposition."""
    e, v = np.linalg.eigh(np.asarray(s, dtype=np.float64))
    if e.min() <= 0.0:
        raise np.linalg.LinAlgError("matrix is not positive definite")
    return (v * e ** p) @ v.T


def recolor_fit(x, y, rho_x: float = 0.0, rho_y: float = 0.0):
    """Recolor: both feature spaces are whitened, the whitened spaces are
    aligned by an orthogonal Procrustes solution, then the receiver's
    covariance and mean are put back.  Steps in the pages' order:

    1. moments of the calibration rows: means mu_x, mu_y and covariances
       S_xx, S_yy, S_xy of the centred rows (divided by n; the scale cancels);
    2. (reading) whitening needs S_xx and S_yy invertible, and duplicated
       layer taps make S_xx singular: rho * trace(S) / F is added to each
       diagonal, relative like the ridge penalty (rho_y = 0 keeps S_yy);
    3. whitening by the symmetric inverse square roots: a sender row x goes to
       (x - mu_x) S_xx^-1/2, a receiver row y to (y - mu_y) S_yy^-1/2;
    4. Procrustes: the map Q with orthonormal columns (rows when F_in < F_out)
       that best takes whitened x to whitened y maximises tr(Q^T M) for the
       whitened cross-covariance M = S_xx^-1/2 S_xy S_yy^-1/2, so Q = U V^T
       from the thin SVD M = U diag(s) V^T;
    5. recolouring: multiply by S_yy^1/2 and add mu_y, so
       W = S_xx^-1/2 Q S_yy^1/2 and b = mu_y - mu_x W.

    Returns (W [F_in][F_out], b [F_out]) in float64."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    n = x.shape[0]
    mx, my = x.mean(axis=0), y.mean(axis=0)
    xc, yc = x - mx, y - my
    sxx, syy, sxy = xc.T @ xc / n, yc.T @ yc / n, xc.T @ yc / n
    sxx = sxx + rho_x * np.trace(sxx) / sxx.shape[0] * np.eye(sxx.shape[0])
    syy = syy + rho_y * np.trace(syy) / syy.shape[0] * np.eye(syy.shape[0])
    wx = spd_power(sxx, -0.5)
    wy = spd_power(syy, -0.5)
    u, _, vt = np.linalg.svd(wx @ sxy @ wy, full_matrices=False)
    q = u @ vt
    w = wx @ q @ spd_power(syy, 0.5)
    return w, my - mx @ w


# ---------------------------------------------------------------------------
# FP8 map storage   [LB] "Implementation Guidelines" (weights may be stored
# quantised, e.g. FP8; the product keeps 16-bit precision)


def e4m3_values() -> np.ndarray:
    """Value of each of the 256 OCP FP8 E4M3 codes: sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent field 0 holds the subnormals
    m/8 * 2^-6; S.1111.111 is NaN and there are no infinities."""
    out = np.empty(256)
    for c in range(256):
        sgn = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 15 and m == 7:
            out[c] = np.nan
        elif e == 0:
            out[c] = sgn * (m / 8.0) * 2.0 ** -6
        else:
            out[c] = sgn * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each finite value by search over the 127
    non-negative finite values (codes 0..126, ascending); a tie goes to the
    even code (even mantissa); magnitudes past 448 saturate to 448; the sign
    bit follows the sign of x (also for zeros)."""
    x = np.asarray(x, dtype=np.float64)
    vals = e4m3_values()[:127]
    a = np.minimum(np.abs(x), vals[-1])
    hi = np.clip(np.searchsorted(vals, a), 1, 126)   # vals[hi - 1] < a <= vals[hi] inside the range
    lo = hi - 1
    dlo, dhi = a - vals[lo], vals[hi] - a
    code = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(a == 0.0, 0, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_fp8(w32):
    """Per-row FP8 storage of fp32 values [rows][cols]: scale = amax / 448
    and codes of w / scale, both quotients in fp32 (correctly rounded); a
    row whose scale is 0 gets scale 1.  Returns (codes uint8, scale float32).
    For a map W [F_in][F_out] the rows are its output channels: quantise W^T
    (one scale per output), so W = fp8_dequant(codes, scale)^T."""
    w32 = np.asarray(w32, dtype=np.float32)
    amax = np.max(np.abs(w32), axis=-1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = e4m3_encode((w32 / scale[..., None]).astype(np.float64))
    return q, scale


def fp8_dequant(q, scale) -> np.ndarray:
    """The map a row of codes stands for: scale * value(code), float64."""
    return e4m3_values()[np.asarray(q)] * np.asarray(scale, dtype=np.float64)[..., None]


# ---------------------------------------------------------------------------
# error metric used by the parity tests


def rel_err(got, ref) -> float:
    """max |got - ref| / RMS(ref) over all elements."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / (rms if rms > 0 else 1.0)
