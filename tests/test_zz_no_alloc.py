"""moe_layer_forward_noalloc (the layer forward on the library's own scratch memory, for callers
that cannot allocate) gives moe_layer_forward's outputs bit for bit, through the C ABI, on two
calls in a row with the second on a smaller input; shapes beyond its scratch are refused before
any launch."""
import numpy as np
import pytest
import torch

from expert_ffn_layer_amd import native as N
from inputgen import layers as L

from _gpu import build, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _both(spec, lay, pl, T):
    """The same T first tokens through both entry points; returns their (y, idx, w)."""
    pl.set_tokens(T)
    x = (lay["x"] if spec.act == "f32" else lay["x"].view(torch.bfloat16))[:T]
    dt = torch.float32 if spec.act == "f32" else torch.bfloat16
    out = []
    for noalloc in (False, True):
        y = torch.full((T, spec.H), float("nan"), dtype=dt, device=DEV)
        idx = torch.full((T, spec.k), -5, dtype=torch.int32, device=DEV)
        w = torch.full((T, spec.k), -5.0, dtype=torch.float32, device=DEV)
        if noalloc:
            N.moe_layer_forward_noalloc(pl.shape, x, pl.Wr, lay["bias"], pl.routed, pl.shared, y, idx, w)
        else:
            N.moe_layer_forward(pl.shape, x, pl.Wr, lay["bias"], pl.routed, pl.shared, y, idx, w, pl.ws)
        torch.cuda.synchronize()
        out.append((y, idx, w))
    return out


SPECS = [
    # the Qwen3-shaped decode layer (fused routing, decode kernel), then 13 tokens
    ("qwen3-decode", L.CONFIGS["c2"], 64, 13),
    # a V3-shaped layer with a shared expert and Zipf routing on the decode kernel, then 5 tokens
    ("v3-width-decode", L.LayerSpec("na2", T=96, H=7168, E=16, k=8, I=2048, shared=True, router="zipf",
                                    zipf_alpha=1.0, calib_tokens=512, seed=91), 96, 5),
    # a prefill-path layer (fp8 weights, ragged groups), then a decode-sized batch of the same layer
    ("fp8-prefill", L.LayerSpec("na3", T=600, H=512, E=6, k=2, I=256, shared=True, w_routed="fp8", w_shared="fp8",
                                seed=92), 600, 40),
]


@pytest.mark.parametrize("name,spec,T1,T2", SPECS, ids=[s[0] for s in SPECS])
def test_noalloc_forward_equals_the_workspace_forward(name, spec, T1, T2):
    say("noalloc", name, spec, T1, T2)
    lay, pl = build(spec, DEV)
    for T in (T1, T2):
        (y, idx, w), (y2, idx2, w2) = _both(spec, lay, pl, T)
        assert torch.equal(idx, idx2) and torch.equal(w, w2)
        assert torch.equal(y, y2), "T=%d: max |dy| %g" % (T, (y.float() - y2.float()).abs().max().item())
        assert not torch.isnan(y2.float()).any()


def test_noalloc_refuses_shapes_beyond_its_scratch():
    spec = L.CONFIGS["c5"]  # a 16384-token prefill batch needs gigabytes of workspace
    shape = N.shape_from_spec(spec)
    assert N.moe_workspace_size(shape) > N.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((16,), dtype=torch.bfloat16, device=DEV)  # never read: refused first
    with pytest.raises(N.MoeError) as e:
        N.moe_layer_forward_noalloc(shape, x, x, None, {"gate": x, "up": x, "down": x, "gate_scale": x,
                                                          "up_scale": x, "down_scale": x},
                                    {"gate": x, "up": x, "down": x, "gate_scale": x, "up_scale": x,
                                     "down_scale": x}, x)
    assert e.value.status == 3 and "scratch" in str(e.value)
