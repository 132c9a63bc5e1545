"""The translation step captured as a HIP graph.

Token alignment (the asynchronous entry, which leaves its validity flag on
the device) and the flattened translation with prepared maps and rotated keys
("Cross-Model KV Cache Transfer in Production", stages 1-4 of the pipeline)
are captured once into a graph on torch's capture stream and replayed.  The
step synchronises nothing, allocates nothing and records no memset node (the
library clears its counters with fill kernels), so:
* each of several replays, with eager library work, output clearing and
  synchronisations between them, writes outputs bit-identical to the eager
  step's;
* a replay reads its inputs through the captured pointers: after the sender
  caches and the receiver's character-end offsets are overwritten in place, a
  replay gives the outputs of an eager step on the new inputs.
"""
import sys

import numpy as np
import pytest
import torch

from cross_model_kv_kvx_amd import kvx, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
L_S, L_R, H, D, N_TAPS = 10, 8, 8, 128, 3
SEND_ROPE, RECV_ROPE = 5e5, 1e6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=DEV)


class Step:
    """Inputs, prepared maps, workspaces and outputs of one translation step,
    every buffer allocated up front."""

    def __init__(self, n_recv, seed):
        send_end, recv_end = synth.token_ends(n_recv, seed)
        self.n_recv, self.n_send = n_recv, len(send_end)
        self.send_end, self.recv_end = dev_i32(send_end), dev_i32(recv_end)
        shp = synth.CacheShape(L_S, self.n_send, H, D)
        self.taps = kvx.layer_map(L_S, L_R, N_TAPS, 2)
        self.send_desc = kvx.cache_desc(torch.empty((L_S, self.n_send, H, D), dtype=torch.bfloat16), SEND_ROPE)
        self.recv_desc = kvx.CacheDesc(L_R, n_recv, H, D, kvx.BF16, RECV_ROPE)
        self.x, self.p, self.b = {}, {}, {}
        for r, role in enumerate(("k", "v")):
            self.x[role] = synth.sender_cache(shp, seed * 10 + r, DEV)
            w, _, _, b = synth.flat_maps(L_R, N_TAPS * H * D, H * D, seed * 10 + 5 + r, DEV, 2)
            self.p[role] = kvx.prepare_maps(w.to(torch.bfloat16), role, self.send_desc, self.recv_desc, N_TAPS)
            self.b[role] = b
        self.tmap = torch.empty(n_recv, dtype=torch.int32, device=DEV)
        self.invalid = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.align_ws = torch.empty(kvx.lib().kvx_align_workspace_size(n_recv), dtype=torch.uint8, device=DEV)
        self.ws = torch.empty(kvx.lib().kvx_translate_prepared_workspace_size(self.send_desc, self.recv_desc, N_TAPS,
                                                                             0, 0),
                              dtype=torch.uint8, device=DEV)

    def outputs(self):
        return {role: torch.zeros((L_R, self.n_recv, H, D), dtype=torch.bfloat16, device=DEV) for role in "kv"}

    def run(self, out):
        kvx.align_tokens(self.send_end, self.recv_end, out=self.tmap, workspace=self.align_ws,
                         invalid=self.invalid)
        kvx.translate(self.x["k"], self.x["v"], self.tmap, self.taps, self.p["k"], self.p["v"], self.b["k"],
                      self.b["v"], send_rope_base=SEND_ROPE, recv_rope_base=RECV_ROPE, k_recv=out["k"],
                      v_recv=out["v"], workspace=self.ws, prepared=True, w_dtype=kvx.BF16)


def test_translation_step_as_graph():
    st = Step(1536, 21)
    say(f"graph: {L_S} -> {L_R} layers, {st.n_recv} receiver / {st.n_send} sender tokens, rotated keys")
    ref = st.outputs()
    st.run(ref)                       # eager reference (also warms every lazy initialisation)
    torch.cuda.synchronize()
    assert int(st.invalid.item()) == 0
    out = st.outputs()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run(out)                   # one run on the capture's stream before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        st.run(out)
    torch.cuda.synchronize()
    other = st.outputs()
    for rep in range(3):
        for t in out.values():
            t.zero_()
        st.run(other)                 # eager library work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for role in "kv":
            assert torch.equal(out[role], ref[role]), f"replay {rep}, role {role}"
        assert torch.equal(other["k"], ref["k"]) and torch.equal(other["v"], ref["v"])
        say(f"  replay {rep}: outputs equal the eager step's")

    # new inputs in the same buffers: the receiver string cut into the same
    # number of tokens at other points, and new sender caches
    rng = np.random.default_rng(22)
    total = int(st.send_end[-1].item())
    cuts = np.sort(rng.choice(np.arange(1, total), size=st.n_recv - 1, replace=False))
    st.recv_end.copy_(dev_i32(np.append(cuts, total)))
    for r, role in enumerate(("k", "v")):
        st.x[role].copy_(synth.sender_cache(synth.CacheShape(L_S, st.n_send, H, D), 230 + r, DEV))
    ref2 = st.outputs()
    st.run(ref2)
    torch.cuda.synchronize()
    assert int(st.invalid.item()) == 0
    assert not torch.equal(ref2["k"], ref["k"])
    for t in out.values():
        t.zero_()
    g.replay()
    torch.cuda.synchronize()
    for role in "kv":
        assert torch.equal(out[role], ref2[role]), f"new inputs, role {role}"
    say("  replay on new inputs: outputs equal the eager step's")
    del g
