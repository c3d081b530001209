"""GPU tests of mla_prolog_v2_no_alloc, the entry point whose workspace is
the library's fixed per-device scratch array: its outputs and caches must
equal mla_prolog_v2's bit for bit (the same kernels on the same inputs) and
match the oracle, on consecutive calls of different sizes sharing the
array (the second smaller than the first, then the first again).
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


def _run(w, dev, no_alloc):
    """One call on copies of the caches; returns (outputs, cache copies)."""
    cfg = w.cfg
    d = dict(dev)
    d["kv_cache"] = dev["kv_cache"].clone()
    d["kr_cache"] = dev["kr_cache"].clone()
    fn = qn.mla_prolog_v2_no_alloc if no_alloc else qn.mla_prolog_v2
    res = fn(d["token_x"], d["w_dq"], d["w_uqqr"], d["w_uk"], d["w_dkvkr"],
             d["rmsnorm_gamma_cq"], d["rmsnorm_gamma_ckv"], d["rope_sin"],
             d["rope_cos"], d["cache_index"], d["kv_cache"], d["kr_cache"],
             quant_mode=cfg.quant_mode, rmsnorm_epsilon_cq=cfg.eps_cq,
             rmsnorm_epsilon_ckv=cfg.eps_ckv,
             dequant_scale_w_uq_qr=d.get("dequant_scale_w_uq_qr"),
             quant_scale_ckv=d.get("quant_scale_ckv"),
             quant_scale_ckr=d.get("quant_scale_ckr"),
             smooth_scales_cq=d.get("smooth_scales_cq"),
             dequant_scale_x=d.get("dequant_scale_x"),
             dequant_scale_w_dq=d.get("dequant_scale_w_dq"),
             dequant_scale_w_dkv_kr=d.get("dequant_scale_w_dkv_kr"),
             return_cq_quant=cfg.quant_mode != "none")
    out = {"query": res[0], "query_rope": res[1], "kv_cache": d["kv_cache"],
           "kr_cache": d["kr_cache"]}
    if cfg.quant_mode == "full_kv_int8":
        out["dequant_scale_q_nope"] = res[2]
    if cfg.quant_mode != "none":
        out["cq_int8"], out["cq_scale"] = res[-2], res[-1]
    return out


def _prepare(key):
    w = make_workload(key)
    cfg = w.cfg
    dev = gh.upload(w)
    dev["w_dq"] = qn.mla_pack_weight(dev["weight_dq"])
    dev["w_dkvkr"] = qn.mla_pack_weight(dev["weight_dkv_kr"])
    dev["w_uqqr"] = qn.mla_pack_weight_uq_qr(dev["weight_uq_qr"], cfg.N, cfg.D,
                                             cfg.Dr)
    dev["w_uk"] = qn.mla_pack_weight_uk(dev["weight_uk"])
    return w, dev


def _same(a, b, what):
    for k in a:
        np.testing.assert_array_equal(gh.raw_bits(a[k]), gh.raw_bits(b[k]),
                                      err_msg=f"{what}: {k}")


@pytest.mark.parametrize("keys", [(1, "mla_dec_t13"),
                                  ("mla_full_kvint8", "mla_ragged_qb")])
def test_no_alloc_matches_workspace_entry_point(keys):
    big, small = keys
    wb, db = _prepare(big)
    ws_, ds = _prepare(small)
    gh.announce(f"no-alloc: {wb.cfg.name} then {ws_.cfg.name} then "
                f"{wb.cfg.name} again")
    before_b = {k: gh.raw_bits(db[k]).copy() for k in ("kv_cache", "kr_cache")}
    before_s = {k: gh.raw_bits(ds[k]).copy() for k in ("kv_cache", "kr_cache")}
    ref_b = _run(wb, db, no_alloc=False)
    ref_s = _run(ws_, ds, no_alloc=False)
    got_b = _run(wb, db, no_alloc=True)   # first call on the scratch array
    got_s = _run(ws_, ds, no_alloc=True)  # smaller call reusing it
    got_b2 = _run(wb, db, no_alloc=True)  # and the larger one again
    torch.cuda.synchronize()
    _same(ref_b, got_b, wb.cfg.name)
    _same(ref_s, got_s, ws_.cfg.name)
    _same(ref_b, got_b2, wb.cfg.name + " (again)")
    gh.announce(f"  oracle {wb.cfg.name}: {gh.check_mla(wb, got_b, before_b)}")
    gh.announce(f"  oracle {ws_.cfg.name}: {gh.check_mla(ws_, got_s, before_s)}")


def test_no_alloc_refuses_calls_beyond_its_scratch():
    # T = 4096 at the DeepSeek-V3 dims needs far more than the fixed array:
    # refused on the host before any launch, outputs and caches untouched
    w, dev = _prepare(2)
    gh.announce("no-alloc: prefill T=4096 must be refused")
    q = torch.zeros((w.cfg.T, w.cfg.N, w.cfg.Hckv), dtype=torch.bfloat16,
                    device="cuda")
    before = gh.raw_bits(dev["kv_cache"]).copy()
    with pytest.raises(qn.QkvnrError) as e:
        qn.mla_prolog_v2_no_alloc(
            dev["token_x"], dev["w_dq"], dev["w_uqqr"], dev["w_uk"],
            dev["w_dkvkr"], dev["rmsnorm_gamma_cq"], dev["rmsnorm_gamma_ckv"],
            dev["rope_sin"], dev["rope_cos"], dev["cache_index"],
            dev["kv_cache"], dev["kr_cache"], query=q)
    assert e.value.status == -13
    torch.cuda.synchronize()
    assert not bool(q.float().abs().sum())
    np.testing.assert_array_equal(gh.raw_bits(dev["kv_cache"]), before)
