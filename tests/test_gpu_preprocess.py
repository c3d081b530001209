"""GPU parity of MlaPreprocessV2 (aclnnMlaPreprocessV2) against the float64
oracle, through the C ABI: a tiny shape, a ragged decode shape, the
DeepSeek-V3 dims with 32 heads at decode T = 32, and a T above the decode
plan's limit (tiled kernels), in both weight layouts; determinism.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import qkv_norm_rope_amd as qn
from tests import gpu_helpers as gh
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qn.load_library()


def _before(dev):
    return {k: gh.raw_bits(dev[k]).copy() for k in ("kv_cache", "kr_cache")}


# the ND layout (weights packed into the workspace on every call) runs on
# the smaller shapes
@pytest.mark.parametrize("key,layout", [
    ("pre_tiny", "packed"), ("pre_ragged", "packed"), ("pre_dsv3", "packed"),
    ("pre_large", "packed"), ("pre_tiny", "nd"), ("pre_ragged", "nd"),
    ("pre_large", "nd")])
def test_preprocess_parity(key, layout):
    w = make_workload(key)
    gh.announce(f"preprocess {w.cfg.name} T={w.cfg.T} {layout}")
    dev = gh.upload(w)
    before = _before(dev)
    out = gh.run_preprocess_gpu(w, dev, layout=layout,
                                bsh=w.cfg.layout == "BSH")
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_preprocess(w, out, before)}")


@pytest.mark.parametrize("key", ["pre_ragged", "pre_large"])
def test_preprocess_deterministic(key):
    w = make_workload(key)
    gh.announce(f"preprocess determinism {w.cfg.name}")
    dev = gh.upload(w)
    a = gh.run_preprocess_gpu(w, dict(dev, kv_cache=dev["kv_cache"].clone(),
                                      kr_cache=dev["kr_cache"].clone()))
    b = gh.run_preprocess_gpu(w, dict(dev, kv_cache=dev["kv_cache"].clone(),
                                      kr_cache=dev["kr_cache"].clone()))
    torch.cuda.synchronize()
    for k in a:
        np.testing.assert_array_equal(gh.raw_bits(a[k]), gh.raw_bits(b[k]),
                                      err_msg=k)
