"""gdla_decode_noalloc (the decode step on the library's static device scratch) against gdla_decode
with a caller-allocated workspace: two calls in a row through the C ABI, the second with fewer
sequences and a shorter context, each compared with gdla_decode on the same inputs and with the
oracle.  The kernels and the workspace layout are the same, so the outputs and the appended cache
rows must agree bit for bit."""

import numpy as np
import pytest
import torch

import synth
import attention_gdla_prefill_decode_amd as gd
from tests import harness as H

pytestmark = pytest.mark.gpu


def _one_call(cfg, p0, seed):
    inp = synth.make_inputs(cfg, "cpu", seed=seed, batch=len(p0), seq=1, p0=p0, random_gamma=True)
    dev = H.device_inputs(inp)
    dims = gd.make_dims(cfg)
    x = dev["x"][:, 0].contiguous()
    c_ref, c_na = dev["cache"].clone(), dev["cache"].clone()
    ref = gd.gdla_decode(dims, dev["wstruct"], x, p0, c_ref)
    out = torch.full_like(x, float("nan"))
    got = gd.gdla_decode_noalloc(dims, dev["wstruct"], x, p0, c_na, out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(out, ref), "no-alloc decode must equal gdla_decode bit for bit"
    assert torch.equal(c_na, c_ref), "appended cache rows must agree"
    r = H.decode_case(cfg, p0, seed=seed)  # the same inputs through gdla_decode, and the oracle
    print(H.check(H.to_np(out), r["exp_out"], "bf16", f"no-alloc decode B={len(p0)}"), flush=True)


def test_noalloc_decode_matches_decode_twice():
    assert torch.cuda.is_available(), "GPU test"
    cfg = H.BF80
    # first call: 24 sequences, contexts up to 3000 (several key splits each)
    _one_call(cfg, [(131 * b) % 3000 for b in range(24)], seed=141)
    # second call on the same scratch: fewer sequences, shorter contexts
    _one_call(cfg, [5, 700, 0], seed=142)
