"""The seeded generators: shapes, determinism and the token-length recipe."""
import os

import numpy as np
import torch

from cross_model_kv_kvx_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_token_ends_recipe():
    s, r = synth.token_ends(8192, 3)
    assert r.dtype == np.int32 and s.dtype == np.int32
    assert s[-1] == r[-1]
    rl = np.diff(np.concatenate([[0], r]))
    sl = np.diff(np.concatenate([[0], s]))
    assert rl.min() >= 1 and rl.max() <= 6
    assert sl.min() >= 1 and sl.max() <= 8
    # mean lengths 3.5 and 4.5 characters
    assert abs(rl.mean() - 3.5) < 0.1 and abs(sl[:-1].mean() - 4.5) < 0.1
    s2, r2 = synth.token_ends(8192, 3)
    assert np.array_equal(s, s2) and np.array_equal(r, r2)


def test_cache_shapes_and_outlier_pairs():
    shp = synth.CacheShape(2, 64, 8, 128)
    k = synth.sender_cache(shp, 4, outlier_frac=0.01, outlier_scale=20.0, outlier_pairs=True)
    assert k.shape == (2, 64, 8, 128) and k.dtype == torch.bfloat16
    big = (k.float().abs().amax(dim=1) > 20).reshape(2, 8, 2, 64)
    # picked channels come in rotation pairs (c, c + 64)
    assert torch.equal(big[:, :, 0], big[:, :, 1])
    v = synth.sender_cache(shp, 4)
    assert torch.equal(v, synth.sender_cache(shp, 4))


def test_configs_small():
    c = synth.config(3, small=True)
    assert c["k_send"].shape[0] == 36 and c["w_k"].shape == (32, 3072, 1024)
    c2 = synth.config(2, small=True)
    assert c2["w_v"].shape == (80, 8, 128, 128)
    c1 = synth.config(1)
    assert c1["x_cal_k"].shape == (1, 512, 2, 64) and c1["x_k"].dtype == torch.float32


def test_layer_bytes_golden():
    line = [l for l in open(os.path.join(GOLD, "kv_layer_bytes.txt")) if not l.startswith("#")][0]
    kv = dict(p.split("=") for p in line.split())
    shp = synth.CacheShape(1, int(kv["tokens"]), int(kv["heads"]), int(kv["head_dim"]))
    assert 2 * shp.tokens * shp.row * int(kv["elem_bytes"]) == int(kv["bytes"])
