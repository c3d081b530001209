"""bench.py's algorithmic work counts, recomputed from the tensors of the
workloads it times: every input array a call reads once, every output it
writes, and one cache row per token whose index is not -1.  The byte counts
are the numerators of the reported HBM rates, so they are checked here
against the generator's own arrays rather than against the formulas."""

from __future__ import annotations

import numpy as np
import pytest

import bench
from workloads import get_config, make_workload

CACHES = ("kv_cache", "kr_cache", "k_cache", "v_cache")


def _slot_bytes(cache: np.ndarray) -> int:
    """Bytes of one paged-cache slot (all its heads)."""
    return cache.nbytes // (cache.shape[0] * cache.shape[1])


def _read_bytes(w) -> int:
    return sum(a.nbytes for k, a in w.arrays.items() if k not in CACHES)


def _mla_written(w, query_elem: int, query_scale: bool) -> int:
    c = w.cfg
    valid = int((w.arrays["cache_index"] >= 0).sum())
    rows = valid * (_slot_bytes(w.arrays["kv_cache"]) + _slot_bytes(w.arrays["kr_cache"]))
    out = c.T * c.N * c.Hckv * query_elem + c.T * c.N * c.Dr * 2
    if query_scale:
        out += c.T * c.N * 4  # dequant_scale_q_nope, fp32 per (token, head)
    return out + rows


def test_decode_bytes_match_the_workload_tensors():
    w = make_workload(1)
    assert (w.arrays["cache_index"] >= 0).all()  # every token writes its rows
    expect = _read_bytes(w) + _mla_written(w, 2, False)
    assert bench.mla_bytes(w.cfg) == expect == 127_779_072


def test_partial_quant_bytes_match_the_workload_tensors():
    w = make_workload(3)
    assert w.cfg.quant_mode == "partial_kv_int8"
    assert (w.arrays["cache_index"] >= 0).all()
    expect = _read_bytes(w) + _mla_written(w, 2, False)
    assert bench.mla_partial_bytes(w.cfg) == expect == 47_276_800


def test_full_quant_bytes_match_the_workload_tensors():
    cfg = get_config(1).replace(quant_mode="full_kv_int8", seed=1101)
    w = make_workload(cfg)
    assert (w.arrays["cache_index"] >= 0).all()
    expect = _read_bytes(w) + _mla_written(w, 1, True)
    assert bench.mla_full_bytes(w.cfg) == expect == 72_680_064


def test_qkv_bytes_match_the_workload_tensors():
    w = make_workload(4)
    c = w.cfg
    valid = int((w.arrays["index"] >= 0).sum())
    written = c.T * c.Nq * c.D * w.arrays["qkv"].itemsize + valid * (
        _slot_bytes(w.arrays["k_cache"]) + _slot_bytes(w.arrays["v_cache"]))
    assert bench.qkv_bytes(c, valid) == _read_bytes(w) + written == 187_978_240


@pytest.mark.parametrize("key", [0, 1])
def test_flops_match_the_gemm_shapes(key):
    # 2 * T * (K * N) summed over the four products, K and N read off the
    # weight arrays: x.W^DQ, x.W^DKV_KR, c^Q.W^UQ_QR, and q^C.W^UK per head
    w = make_workload(key)
    a = w.arrays
    kn = (a["weight_dq"].size + a["weight_dkv_kr"].size + a["weight_uq_qr"].size
          + a["weight_uk"].size)
    assert bench.mla_flops(w.cfg) == 2 * w.cfg.T * kn
    assert bench.uqqr_flops(w.cfg) + bench.uk_flops(w.cfg) == 2 * w.cfg.T * (
        a["weight_uq_qr"].size + a["weight_uk"].size)
    # the prefill workload has the decode weights and T = 4096 tokens
    if key == 1:
        assert bench.mla_flops(get_config(2)) == 2 * 4096 * kn == 501_974_302_720


def test_up_projection_bytes_match_the_workload_tensors():
    # the decode up projection's algorithmic bytes: W^UQ_QR and the cos/sin
    # rows it reads, the q^R rows it writes; the bf16 c^Q it reads and q^C
    # it writes (T x Hcq and T x N*D intermediates in the workspace) are
    # counted apart
    w = make_workload(1)
    c, a = w.cfg, w.arrays
    expect = (a["weight_uq_qr"].nbytes + a["rope_cos"].nbytes + a["rope_sin"].nbytes
              + c.T * c.N * c.Dr * 2)
    assert bench.uqqr_bytes(c) == expect == 76_029_952
    assert bench.uqqr_workspace_bytes(c) == c.T * c.Hcq * 2 + c.T * c.N * c.D * 2
    # the W^UK product in the same launch adds W^UK and the query, and
    # reads q^C back once per 128-column tile of each head's Hckv
    assert bench.uk_bytes(c) == a["weight_uk"].nbytes + c.T * c.N * c.Hckv * 2 \
        == 20_971_520
    assert bench.uqqr_workspace_bytes(c, merged=True) == \
        bench.uqqr_workspace_bytes(c) + 4 * c.T * c.N * c.D * 2


def test_preprocess_bytes_match_the_workload_tensors():
    # every input read once (weights, parameters, x, cos/sin, index), the
    # outputs written once, one bf16 cache row pair per token (all valid)
    w = make_workload("pre_dsv3")
    c, a = w.cfg, w.arrays
    read = sum(a[k].nbytes for k in a if k not in ("kv_cache", "kr_cache"))
    written = c.T * (c.N * c.Hckv * 2 + c.N * c.Dr * 2 + (c.Hckv + c.Dr) * 2)
    assert (a["cache_index"] >= 0).all()
    assert bench.preprocess_bytes(c) == read + written
