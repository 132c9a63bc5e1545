"""The measurement probes through the C-ABI: the copy probe moves the bytes
(destination equals source), every probe reports a positive rate below the
chip's published peaks (8 TB/s HBM, 2.5 PFLOP/s dense bf16)."""
import pytest
import torch

from cross_model_kv_kvx_amd import kvx

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_hbm_probes():
    n = 64 << 20  # 256 MiB of int32
    a = torch.arange(n, dtype=torch.int32, device=DEV)
    b = torch.zeros_like(a)
    ms = kvx.probe_hbm("copy", a, b, iters=3)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    gbs = 2 * a.numel() * 4 / (ms * 1e-3) / 1e9
    print(f"copy {gbs:.0f} GB/s (read + write)")
    assert 0 < gbs < 8000 * 1.1
    ms_r = kvx.probe_hbm("read", a, iters=3)
    ms_f = kvx.probe_hbm("fill", b, iters=3)
    torch.cuda.synchronize()
    assert ms_r > 0 and ms_f > 0
    assert bool(torch.all(b.view(torch.int16) == 0x3c00))
    # a length that ends inside the last pass of the grid (every thread moves
    # eight 16-byte pieces per pass): the tail is copied and filled, nothing past it
    m = 4 * 300007
    c = torch.arange(m + 64, dtype=torch.int32, device=DEV)
    d = torch.full((m + 64,), -1, dtype=torch.int32, device=DEV)
    kvx.probe_hbm("copy", c[:m], d[:m], iters=1)
    torch.cuda.synchronize()
    assert torch.equal(d[:m], c[:m]) and bool(torch.all(d[m:] == -1))
    kvx.probe_hbm("fill", d[:m], iters=1)
    torch.cuda.synchronize()
    assert bool(torch.all(d[:m].view(torch.int16) == 0x3c00)) and bool(torch.all(d[m:] == -1))


def test_mfma_probe():
    ms, flops = kvx.probe_mfma(reps=2000, iters=2, device=DEV)
    tf = flops / (ms * 1e-3) / 1e12
    print(f"mfma {tf:.0f} TFLOP/s")
    assert 0 < tf < 2500 * 1.1
