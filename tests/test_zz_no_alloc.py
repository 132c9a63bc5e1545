"""The alignment entry that allocates nothing, through the C-ABI: its map and
validity flag equal those of kvx_align_tokens_async (the same kernels with a
caller workspace) on two calls in a row, the second with a smaller input,
and on a call with invalid offsets; sizes past its limit are refused before
anything runs."""
import sys

import numpy as np
import pytest
import torch

from cross_model_kv_kvx_amd import kvx, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=DEV)


def both(send_end, recv_end):
    n = recv_end.numel()
    ref = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    got = torch.full((n,), -9, dtype=torch.int32, device=DEV)
    inv_ref = torch.full((1,), 5, dtype=torch.int32, device=DEV)
    inv_got = torch.full((1,), 6, dtype=torch.int32, device=DEV)
    kvx.align_tokens(send_end, recv_end, out=ref, invalid=inv_ref)
    kvx.align_tokens_noalloc(send_end, recv_end, got, inv_got)
    torch.cuda.synchronize()
    return ref, got, int(inv_ref.item()), int(inv_got.item())


def test_noalloc_alignment_matches_async_entry():
    for n, seed in ((65536, 5), (777, 9)):  # second call smaller than the first
        say(f"no-allocation alignment, {n} receiver tokens")
        s, r = synth.token_ends(n, seed)
        ref, got, i_ref, i_got = both(dev_i32(s), dev_i32(r))
        assert i_ref == 0 and i_got == 0
        assert torch.equal(ref, got)
    say("no-allocation alignment, invalid receiver offsets")
    s, r = synth.token_ends(3000, 4)
    bad = r.copy()
    bad[1500] = bad[1499]
    ref, got, i_ref, i_got = both(dev_i32(s), dev_i32(bad))
    assert i_ref == 1 and i_got == 1


def test_noalloc_alignment_refuses_sizes_past_its_limit():
    L = kvx.lib()
    inv = torch.zeros(1, dtype=torch.int32, device=DEV)
    one = dev_i32([1])
    st = L.kvx_align_tokens_noalloc(one.data_ptr(), 1, one.data_ptr(), (1 << 24) + 1, one.data_ptr(),
                                    inv.data_ptr(), None)
    assert st == kvx.ERR_WORKSPACE
