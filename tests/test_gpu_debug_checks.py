"""GPU tests of the opt-in debug input checks (both operators' index
restriction, and the qkv op's non-zero scales): a violating call returns
its status before anything is launched, so outputs and caches stay as they
were; a valid call runs as usual and matches the oracle.
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


def _mla_call(w, d, query, query_rope):
    cfg = w.cfg
    return qn.mla_prolog_v2(
        d["token_x"], qn.mla_pack_weight(d["weight_dq"]),
        qn.mla_pack_weight_uq_qr(d["weight_uq_qr"], cfg.N, cfg.D, cfg.Dr),
        qn.mla_pack_weight_uk(d["weight_uk"]),
        qn.mla_pack_weight(d["weight_dkv_kr"]), d["rmsnorm_gamma_cq"],
        d["rmsnorm_gamma_ckv"], d["rope_sin"], d["rope_cos"],
        d["cache_index"], d["kv_cache"], d["kr_cache"],
        rmsnorm_epsilon_cq=cfg.eps_cq, rmsnorm_epsilon_ckv=cfg.eps_ckv,
        query=query, query_rope=query_rope, debug_check_index=True)


@pytest.mark.parametrize("bad", ["repeat", "past_end", "below_minus_one"])
def test_mla_debug_index_check_refuses(bad):
    w = make_workload(0)
    gh.announce(f"mla debug index check: {bad}")
    d = gh.upload(w)
    idx = w.arrays["cache_index"].reshape(-1).copy()
    valid = np.nonzero(idx >= 0)[0]
    if bad == "repeat":
        idx[valid[1]] = idx[valid[0]]
    elif bad == "past_end":
        idx[valid[0]] = w.cfg.slots
    else:
        idx[valid[0]] = -2
    d["cache_index"] = torch.from_numpy(idx).cuda()
    q = torch.full((w.cfg.T, w.cfg.N, w.cfg.Hckv), 7.0, dtype=torch.bfloat16,
                   device="cuda")
    qr = torch.full((w.cfg.T, w.cfg.N, w.cfg.Dr), 7.0, dtype=torch.bfloat16,
                    device="cuda")
    before = {k: gh.raw_bits(d[k]).copy() for k in ("kv_cache", "kr_cache")}
    with pytest.raises(qn.QkvnrError) as e:
        _mla_call(w, d, q, qr)
    assert e.value.status == -11
    torch.cuda.synchronize()
    for k in ("kv_cache", "kr_cache"):
        np.testing.assert_array_equal(gh.raw_bits(d[k]), before[k])
    assert bool((q.float() == 7.0).all()) and bool((qr.float() == 7.0).all())


def test_mla_debug_index_check_passes_valid_call():
    w = make_workload(0)
    gh.announce("mla debug index check: valid call")
    d = gh.upload(w)
    before = {k: gh.raw_bits(d[k]).copy() for k in ("kv_cache", "kr_cache")}
    q = torch.empty((w.cfg.T, w.cfg.N, w.cfg.Hckv), dtype=torch.bfloat16,
                    device="cuda")
    qr = torch.empty((w.cfg.T, w.cfg.N, w.cfg.Dr), dtype=torch.bfloat16,
                     device="cuda")
    _mla_call(w, d, q, qr)
    torch.cuda.synchronize()
    out = {"query": q, "query_rope": qr, "kv_cache": d["kv_cache"],
           "kr_cache": d["kr_cache"]}
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


@pytest.mark.parametrize("bad", ["repeat", "past_end", "zero_k_scale",
                                 "zero_v_scale", None])
def test_qkv_debug_input_check(bad):
    w = make_workload("qkv_ragged")
    cfg = w.cfg
    gh.announce(f"qkv debug input check: {bad}")
    d = gh.upload(w)
    idx = w.arrays["index"].reshape(-1).copy()
    valid = np.nonzero(idx >= 0)[0]
    if bad == "repeat":
        idx[valid[2]] = idx[valid[1]]
    elif bad == "past_end":
        idx[valid[0]] = cfg.block_num * cfg.block_size
    d["index"] = torch.from_numpy(idx).cuda()
    if bad == "zero_k_scale":
        d["k_scale"][5] = 0.0
    if bad == "zero_v_scale":
        d["v_scale"][-1] = 0.0
    before = {k: gh.raw_bits(d[k]).copy() for k in ("k_cache", "v_cache")}

    def call():
        return qn.qkv_rmsnorm_rope_cache(
            d["qkv"], d["gamma_q"], d["gamma_k"], d["cos"], d["sin"],
            d["index"], d["k_cache"], d["v_cache"], Nq=cfg.Nq, Nk=cfg.Nk,
            Nv=cfg.Nv, quant_mode=cfg.quant_mode, epsilon=cfg.eps,
            k_scale=d.get("k_scale"), v_scale=d.get("v_scale"),
            k_offset=d.get("k_offset"), v_offset=d.get("v_offset"),
            B=cfg.B, S=cfg.S, debug_check_inputs=True)
    if bad is None:
        q_out = call()
        torch.cuda.synchronize()
        gh.announce(f"  ok {gh.check_qkv(w, {'q_out': q_out, 'k_cache': d['k_cache'], 'v_cache': d['v_cache']}, before)}")
        return
    with pytest.raises(qn.QkvnrError) as e:
        call()
    assert e.value.status == (-12 if "scale" in bad else -11)
    torch.cuda.synchronize()
    for k in ("k_cache", "v_cache"):
        np.testing.assert_array_equal(gh.raw_bits(d[k]), before[k])
