"""Input gradient of the sharded conv on the GPU against the oracle.

The input-gradient layer reads dy with the forward layer's shards and halo,
exchanges its halos like x, and runs the sharded conv with the transposed,
tap-flipped weights (st_conv_dgrad_weights, then st_conv_sharded).
Checks: the weight transform bit for bit; dx against the oracle's
conv_same_dgrad (the adjoint of conv_same, pinned on the CPU) within the
forward tolerance; sharded dx equal to unsharded dx bit for bit.
"""
import numpy as np
import pytest
import torch

import halo_sharded_conv_amd as hsc
import oracle
import synth
from halo_sharded_conv_amd.layer import ShardedConvGN, dgrad_config
from helpers import TOL, bits_equal, direct_cases, rel_err, say, small_cases

pytestmark = pytest.mark.gpu

CASES = {**small_cases(), **direct_cases()}


def run_dgrad(wl, dy, w):
    layer = ShardedConvGN(dgrad_config(wl))
    layer.set_weight_dgrad(w)
    layer.load_input(dy)
    layer.exchange()
    layer.conv()
    torch.cuda.synchronize()
    return layer


@pytest.mark.parametrize("name", ["img64_small", "vol16k5", "img_c5to12_k3", "vol32_full"])
def test_dgrad_weights_bit_exact(name):
    wl = CASES[name]
    w = synth.make_weight(wl)
    dt = torch.float32 if wl.dtype == "f32" else torch.int16
    src = torch.from_numpy(w.view(np.int16) if w.dtype == np.uint16 else w).reshape(-1).cuda()
    out = torch.empty_like(src)
    hsc.st_conv_dgrad_weights(wl.ndim, wl.cin, wl.cout, wl.ksize, wl.dtype, src, out)
    torch.cuda.synchronize()
    want = np.swapaxes(w, 0, 1)
    want = np.flip(want, axis=tuple(range(2, want.ndim)))
    got = out.cpu().numpy().view(w.dtype).reshape(want.shape)
    assert out.dtype == dt and bits_equal(got, np.ascontiguousarray(want))


@pytest.mark.parametrize("name", list(CASES))
def test_dgrad_matches_oracle(name):
    wl = CASES[name]
    wd = dgrad_config(wl)
    say(f"dgrad vs oracle: {name} spatial={wl.spatial} shards={wl.shards} N={wl.batch}")
    dy, w = synth.make_input(wd), synth.make_weight(wl)
    layer = run_dgrad(wl, dy, w)
    want = oracle.conv_same_dgrad(oracle.widen(dy, wl.dtype), oracle.widen(w, wl.dtype))
    err = rel_err(layer.y_host(), want)
    say(f"  max|err|/rms(dx) = {err:.3e}  (tolerance {TOL[wl.dtype]:.0e})")
    assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("name", ["img64_small", "img64_b2", "vol32_grid", "vol16k5", "vol16k5_b2",
                                  "grid256_small", "vol32_b2", "img_c5to12_k3"])
def test_dgrad_sharded_equals_unsharded_bitwise(name):
    wl = CASES[name]
    say(f"dgrad sharded == unsharded: {name}")
    dy, w = synth.make_input(dgrad_config(wl)), synth.make_weight(wl)
    a = run_dgrad(wl, dy, w)
    b = run_dgrad(wl.unsharded(), dy, w)
    assert bits_equal(a.y_host(), b.y_host())
