"""Seeded random MLA prolog shapes on the GPU, each compared with the oracle.

The cases are drawn once from a fixed seed over the validator's accepted
space at small sizes (so the float64 oracle stays fast): every quantisation
mode; head dims 32, 64, 96 and 128 (and so the merged decode launch, the
fused and the unfused large-T paths); RoPE widths 16, 32 and 64; token
counts across the decode plan's one, two and four row blocks and the
large-T plan; both weight layouts; cache sizes with skipped and ragged
slots.  A failing case prints its configuration.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from tests import gpu_helpers as gh
from workloads import make_workload
from workloads.configs import MlaConfig, PreConfig

pytestmark = pytest.mark.gpu

MODES = ["none", "partial_kv_bf16", "partial_kv_int8", "full_kv_bf16",
         "full_kv_int8"]


def _draw_cases(n, seed=4242):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        mode = MODES[len(cases) % len(MODES)]
        quant = mode != "none"
        full = mode.startswith("full")
        D = int(rng.choice([32, 64, 96, 128]))
        Dr = int(rng.choice([16, 32, 64]))
        N = int(rng.integers(1, 9))
        if (N * D) % Dr:
            continue
        He = int(rng.choice([64, 128, 192, 256, 384]))
        if He % (64 if full else 32):
            continue
        Hcq = int(rng.choice([64, 128, 192, 256]))
        if quant and Hcq % 64:
            continue
        Hckv = int(16 * rng.integers(1, 17))
        T = int(rng.choice([1, 5, 17, 32, 33, 50, 64, 65, 100, 128, 129, 160, 257]))
        B = int(rng.choice([d for d in (1, 2, 3, 5) if T % d == 0]))
        bs = int(rng.choice([16, 32, 64]))
        bn = (T + 4 + bs - 1) // bs + int(rng.integers(0, 2))
        cases.append(MlaConfig(
            f"fuzz{len(cases)}_{mode}_T{T}_N{N}_D{D}_Dr{Dr}_Hckv{Hckv}",
            B=B, S=T // B, He=He, Hcq=Hcq, N=N, D=D, Hckv=Hckv, Dr=Dr,
            block_num=bn, block_size=bs, quant_mode=mode,
            n_skip=int(rng.integers(0, min(3, T) + 1)),
            seed=5000 + len(cases), layout="BSH" if B > 1 else "TND"))
    return cases


# the paths the random draw may miss: the fused large-T launch (D = 128,
# N*D a multiple of 256) in each family of modes, and the merged decode
# launch (bf16, T <= 32) at odd head counts
_FORCED = [
    ("none", 129, 2, 128, 64, 176), ("partial_kv_int8", 257, 4, 128, 32, 80),
    ("full_kv_bf16", 160, 6, 128, 16, 48), ("full_kv_int8", 200, 2, 128, 64, 64),
    ("none", 31, 5, 96, 32, 208), ("none", 1, 3, 128, 16, 16),
]
CASES = _draw_cases(30) + [
    MlaConfig(f"forced{i}_{m}_T{T}_N{N}_D{D}_Dr{Dr}_Hckv{H}", B=1, S=T,
              He=256 if m.startswith("full") else 192, Hcq=128, N=N, D=D,
              Hckv=H, Dr=Dr, block_num=(T + 40) // 32, block_size=32,
              quant_mode=m, n_skip=min(2, T - 1), seed=6000 + i)
    for i, (m, T, N, D, Dr, H) in enumerate(_FORCED)]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_mla_fuzzed_shapes_match_oracle(cfg):
    w = make_workload(cfg)
    layout = "nd" if cfg.seed % 3 == 0 else "packed"
    gh.announce(f"fuzz {cfg} layout={layout}")
    dev = gh.upload(w)
    before = {k: gh.raw_bits(dev[k]).copy() for k in ("kv_cache", "kr_cache")}
    out = gh.run_mla_gpu(w, dev, layout=layout, bsh=cfg.layout == "BSH")
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


def _draw_pre_cases(n, seed=4343):
    # MlaPreprocessV2 runs on the full-quantisation kernels: He and Hcq
    # multiples of 64
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        D = int(rng.choice([32, 64, 128]))
        Dr = int(rng.choice([16, 32, 64]))
        N = int(rng.integers(1, 7))
        if (N * D) % Dr:
            continue
        T = int(rng.choice([1, 7, 32, 40, 96, 130, 200]))
        cases.append(PreConfig(
            f"pfuzz{len(cases)}_T{T}_N{N}_D{D}_Dr{Dr}", B=1, S=T,
            He=int(rng.choice([64, 128, 256])), Hcq=int(rng.choice([64, 128, 192])),
            N=N, D=D, Hckv=int(16 * rng.integers(1, 13)), Dr=Dr,
            block_num=(T + 40) // 32, block_size=32,
            n_skip=int(rng.integers(0, min(2, T - 1) + 1)), seed=7000 + len(cases)))
    return cases


PRE_CASES = _draw_pre_cases(10)


@pytest.mark.parametrize("cfg", PRE_CASES, ids=[c.name for c in PRE_CASES])
def test_preprocess_fuzzed_shapes_match_oracle(cfg):
    w = make_workload(cfg)
    layout = "nd" if cfg.seed % 2 else "packed"
    gh.announce(f"preprocess fuzz {cfg} layout={layout}")
    dev = gh.upload(w)
    before = {k: gh.raw_bits(dev[k]).copy() for k in ("kv_cache", "kr_cache")}
    out = gh.run_preprocess_gpu(w, dev, layout=layout)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_preprocess(w, out, before)}")
