"""Stream contract of the C ABI: every kernel of a call runs on the stream the
caller passes.  Each test queues, on a side stream, a spin of about 20 ms,
then the copy that produces the call's input, then the call itself, and
synchronises only that stream before comparing with a call made on the
default stream.  A kernel launched on any other stream would read the input
before the copy wrote it."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from tests import gpu_helpers as gh
from workloads import make_workload

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 50_000_000  # ~20 ms at 2.4 GHz


def _same_bits(a, b, what):
    np.testing.assert_array_equal(gh.raw_bits(a), gh.raw_bits(b), err_msg=what)


@pytest.mark.parametrize("key", ["mla_dec_t13", "mla_full_kvint8", 3])
def test_mla_runs_on_callers_stream(key):
    w = make_workload(key)
    gh.announce(f"mla {w.cfg.name} on a side stream behind a spin")
    ref = gh.run_mla_gpu(w, gh.upload(w))
    torch.cuda.synchronize()
    dev = gh.upload(w)
    x_src = dev["token_x"].clone()
    dev["token_x"].zero_()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN_CYCLES)
        dev["token_x"].copy_(x_src)
        out = gh.run_mla_gpu(w, dev)
    s.synchronize()
    for k in sorted(ref):
        if isinstance(ref[k], torch.Tensor):
            _same_bits(out[k], ref[k], k)
    gh.announce("  ok")


def test_qkv_runs_on_callers_stream():
    w = make_workload("qkv_ragged_asym")
    gh.announce(f"qkv {w.cfg.name} on a side stream behind a spin")
    ref = gh.run_qkv_gpu(w, gh.upload(w))
    torch.cuda.synchronize()
    dev = gh.upload(w)
    src = dev["qkv"].clone()
    dev["qkv"].zero_()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN_CYCLES)
        dev["qkv"].copy_(src)
        out = gh.run_qkv_gpu(w, dev)
    s.synchronize()
    for k in sorted(ref):
        _same_bits(out[k], ref[k], k)
    gh.announce("  ok")
