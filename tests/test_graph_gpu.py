"""The library's calls under HIP graph capture: a decode step on the static scratch
(gdla_decode_noalloc, for callers that cannot allocate) and a prefill with a caller workspace,
each captured once and replayed several times, with the program's own eager calls and
synchronizations between the replays.  Every replay must equal the eager call bit for bit (the
same kernels on the same buffers), and the eager result matches the oracle."""

import pytest
import torch

import synth
import attention_gdla_prefill_decode_amd as gd
from tests import harness as H

pytestmark = pytest.mark.gpu


def _capture(fn):
    """fn() on a side stream once (warm-up), then captured into a graph on it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_noalloc_decode_replays_in_graph():
    assert torch.cuda.is_available(), "GPU test"
    cfg = H.BF80
    p0 = [(173 * b) % 2500 for b in range(16)]
    inp = synth.make_inputs(cfg, "cpu", seed=151, batch=len(p0), seq=1, p0=p0, random_gamma=True)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg)
    x = dev["x"][:, 0].contiguous()
    cache = dev["cache"].clone()
    out = torch.empty_like(x)
    gd.gdla_decode_noalloc(dims, dev["wstruct"], x, p0, cache, out)
    torch.cuda.synchronize()
    ref, ref_cache = out.clone(), cache.clone()
    r = H.decode_case(cfg, p0, seed=151)  # the same inputs through gdla_decode, and the oracle
    print(H.check(H.to_np(ref), r["exp_out"], "bf16", "eager no-alloc decode"), flush=True)

    g = _capture(lambda: gd.gdla_decode_noalloc(dims, dev["wstruct"], x, p0, cache, out))
    for rep in range(4):
        out.zero_()
        gd.gdla_decode(dims, dev["wstruct"], x, p0, dev["cache"].clone())  # other eager work
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager call"
        assert torch.equal(cache, ref_cache), f"replay {rep}: appended cache rows differ"


def test_prefill_replays_in_graph():
    assert torch.cuda.is_available(), "GPU test"
    cfg = H.BF80
    p0, T = [0, 37], 300
    inp = synth.make_inputs(cfg, "cpu", seed=152, batch=len(p0), seq=T, p0=p0, random_gamma=True)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg)
    cache = dev["cache"].clone()
    ws = torch.empty(gd.gdla_workspace_bytes(dims, gd.GDLA_OP_PREFILL, len(p0), T, p0, cache.shape[1]),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["x"])
    gd.gdla_prefill(dims, dev["wstruct"], dev["x"], p0, cache, out=out, ws=ws)
    torch.cuda.synchronize()
    ref = out.clone()
    g = _capture(lambda: gd.gdla_prefill(dims, dev["wstruct"], dev["x"], p0, cache, out=out, ws=ws))
    for rep in range(4):
        gd.gdla_prefill(dims, dev["wstruct"], dev["x"], p0, dev["cache"].clone())  # other eager work
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager call"
