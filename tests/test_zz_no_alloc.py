"""moe_decode_layer_static: the entry point that allocates nothing (its
workspace is the library's static device array). Its outputs must equal
moe_decode_layer's (same kernel) on calls in a row, each later one with a
smaller input, across both batch regimes; a shape beyond the array's size is
refused before any launch. Routing bit-exact, outputs bit-identical (which
meets the parity bar of the layer)."""
import numpy as np
import pytest
import torch

import moe_decode_02_amd as md
import synth
from helpers import to_f64
from synth.device import DeviceLayer, act_tensor, desc_of, to_device, to_host, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    md.lib()
    return torch.device("cuda:0")


def both(w, dl, x, B, dev):
    d = desc_of(w)
    xd = to_device(x, dev)
    y1, y2 = act_tensor(w, B, dev), act_tensor(w, B, dev)
    i1 = torch.full((B, w.k), -7, dtype=torch.int32, device=dev)
    i2 = i1.clone()
    w1 = torch.zeros((B, w.k), dtype=torch.float32, device=dev)
    w2 = w1.clone()
    ws = workspace(d, B, 1, dev)
    md.moe_decode_layer(d, dl.weights, xd, y1, B, i1, w1, ws)
    md.moe_decode_layer_static(d, dl.weights, xd, y2, B, i2, w2)
    torch.cuda.synchronize()
    assert md.moe_check_workspace(ws) == md.MOE_OK
    return (to_host(y1), i1.cpu().numpy(), w1.cpu().numpy()), (to_host(y2), i2.cpu().numpy(), w2.cpu().numpy())


@pytest.mark.parametrize("name,batches", [("k3_b8", (8, 2, 1)), ("tiny_f32", (9, 3, 1)), ("k3_b1", (26, 5))])
def test_static_workspace_matches_caller_workspace(dev, name, batches):
    w = synth.WORKLOADS[name]
    dl = DeviceLayer(w, device=dev)
    for B in batches:  # each call after the first has a smaller input
        x = synth.x_tokens(w, B)
        (ya, ia, wa), (yb, ib, wb) = both(w, dl, x, B, dev)
        print(f"static workspace {name} B={B}: routing equal {np.array_equal(ia, ib)}, "
              f"outputs bit-identical {np.array_equal(ya, yb)}", flush=True)
        assert np.array_equal(ia, ib) and np.array_equal(wa, wb)
        assert np.array_equal(ya, yb)
        assert np.all(np.isfinite(to_f64(ya, w.act)))
    del dl
    torch.cuda.empty_cache()


def test_static_workspace_refuses_large_shapes(dev):
    w = synth.WORKLOADS["k3_b64_zipf"]
    d = desc_of(w)
    assert md.moe_workspace_bytes(d, 26, 1) <= 16 << 20 < md.moe_workspace_bytes(d, 27, 1)
    FAKE = 1 << 40
    wt = md.moe_layer_weights(FAKE, FAKE, None, FAKE, FAKE, None, None, FAKE, FAKE)
    st = md.moe_decode_layer_static(d, wt, FAKE + (1 << 30), FAKE + (2 << 30), 27, None, None, check=False)
    assert st == md.MOE_ERR_UNSUPPORTED and "static workspace" in md.moe_last_error()
