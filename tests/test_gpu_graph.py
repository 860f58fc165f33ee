"""The layer's forward step captured in a HIP graph (torch.cuda.CUDAGraph over
the library's launches) and replayed: every replay, with eager work and
synchronisations between replays, gives the same bits as the eager step.
The library records no memset into a graph: its buffers are cleared by
kernels."""
import numpy as np
import pytest
import torch

import synth
from halo_sharded_conv_amd.layer import ShardedConvGN
from helpers import bits_equal, say, small_cases

pytestmark = pytest.mark.gpu

CASES = small_cases()


@pytest.mark.parametrize("name", ["img64_small", "vol32_grid", "vol16k5", "grid256_small", "vol32_full"])
def test_graph_replays_match_eager(name):
    wl = CASES[name]
    say(f"graph replay == eager: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    gamma, beta = synth.make_affine(wl, seed=5)
    layer = ShardedConvGN(wl)
    layer.set_weight(w)
    layer.set_affine(gamma, beta)
    layer.load_input(x)
    layer.step()
    torch.cuda.synchronize()
    y0, z0 = layer.y_host(), layer.z_host()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step()
    for r in range(3):
        # eager work between replays: scribble over the outputs
        for t in layer.y_bufs + layer.z_bufs:
            t.fill_(float(r + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bits_equal(layer.y_host(), y0), f"replay {r}: y differs"
        assert bits_equal(layer.z_host(), z0), f"replay {r}: z differs"


def test_first_halo_call_under_capture_needs_an_uploaded_plan():
    """A plan whose descriptor table is not on the device yet cannot make its
    first upload inside a capture: the halo call fails and enqueues nothing.
    After st_plan_upload the whole step captures, with no eager call before
    it, and every replay gives the eager bits."""
    from halo_sharded_conv_amd import ShardConvError
    wl = CASES["vol32_grid"]
    say(f"capture before any eager halo call: {wl.name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    layer = ShardedConvGN(wl)
    layer.set_weight(w)
    layer.load_input(x)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(ShardConvError, match="st_plan_upload"):
        with torch.cuda.graph(g):
            layer.exchange_pack()
    layer.in_plan.upload()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        layer.step()
    for r in range(2):
        for t in layer.y_bufs + layer.z_bufs:
            t.fill_(float(r + 7))
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        y1, z1 = layer.y_host(), layer.z_host()
        if r == 0:
            ref = ShardedConvGN(wl)
            ref.set_weight(w)
            ref.load_input(x)
            ref.step()
            torch.cuda.synchronize()
            y0, z0 = ref.y_host(), ref.z_host()
        assert bits_equal(y1, y0), f"replay {r}: y differs"
        assert bits_equal(z1, z0), f"replay {r}: z differs"
