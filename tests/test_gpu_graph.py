"""HIP-graph capture of the library calls: every replay must reproduce the
eager result bit for bit, with eager work (output clearing, cache restore,
another eager call) between replays."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import qkv_norm_rope_amd as qn
from tests import gpu_helpers as gh
from workloads import get_config, make_workload

pytestmark = pytest.mark.gpu

NAMES = ("token_x", "weight_dq", "weight_uq_qr", "weight_uk", "weight_dkv_kr",
         "rmsnorm_gamma_cq", "rmsnorm_gamma_ckv", "rope_sin", "rope_cos",
         "cache_index", "kv_cache", "kr_cache")


def _prepared(w, d):
    cfg = w.cfg
    for k in ("weight_dq", "weight_dkv_kr"):
        d[k] = qn.mla_pack_weight(d[k])
    d["weight_uk"] = qn.mla_pack_weight_uk(d["weight_uk"])
    d["weight_uq_qr"] = qn.mla_pack_weight_uq_qr(d["weight_uq_qr"], cfg.N,
                                                 cfg.D, cfg.Dr)
    q8 = cfg.quant_mode == "full_kv_int8"
    q = torch.empty((cfg.T, cfg.N, cfg.Hckv),
                    dtype=torch.int8 if q8 else torch.bfloat16, device="cuda")
    qr = torch.empty((cfg.T, cfg.N, cfg.Dr), dtype=torch.bfloat16,
                     device="cuda")
    kw = {}
    if cfg.quant_mode != "none":
        kw = dict(dequant_scale_w_uq_qr=d["dequant_scale_w_uq_qr"],
                  smooth_scales_cq=d["smooth_scales_cq"])
    if cfg.quant_mode == "partial_kv_int8":
        kw.update(quant_scale_ckv=d["quant_scale_ckv"],
                  quant_scale_ckr=d["quant_scale_ckr"])
    if cfg.quant_mode.startswith("full"):
        kw.update(dequant_scale_x=d["dequant_scale_x"],
                  dequant_scale_w_dq=d["dequant_scale_w_dq"],
                  dequant_scale_w_dkv_kr=d["dequant_scale_w_dkv_kr"])
    if q8:
        d["dequant_scale_q_nope"] = torch.empty((cfg.T, cfg.N, 1),
                                                dtype=torch.float32,
                                                device="cuda")
        kw.update(quant_scale_ckv=d["quant_scale_ckv"],
                  dequant_scale_q_nope=d["dequant_scale_q_nope"])
    return qn.PreparedMlaPrologV2(*[d[k] for k in NAMES], q, qr,
                                  quant_mode=cfg.quant_mode,
                                  rmsnorm_epsilon_cq=cfg.eps_cq,
                                  rmsnorm_epsilon_ckv=cfg.eps_ckv, **kw)


@pytest.mark.parametrize("key", [1, 3, "mla_mid_dsv3", "mla_full_kvint8",
                                 "mla_full_kvint8_small_t", "mla_fused_ragged",
                                 "mla_fused_q"])
def test_mla_graph_replays_match_eager(key):
    if key == "mla_full_kvint8_small_t":  # the query quantised in A8's epilogue
        w = make_workload(get_config("mla_full_kvint8").replace(B=21, n_skip=2))
    else:
        w = make_workload(key)
    gh.announce(f"graph replay {w.cfg.name}")
    d = gh.upload(w)
    kv0, kr0 = d["kv_cache"].clone(), d["kr_cache"].clone()
    call = _prepared(w, d)
    q, qr = call()
    torch.cuda.synchronize()
    ref = {"q": gh.raw_bits(q), "qr": gh.raw_bits(qr),
           "kv": gh.raw_bits(d["kv_cache"]), "kr": gh.raw_bits(d["kr_cache"])}
    qs = d.get("dequant_scale_q_nope")  # full quantisation with an int8 query
    if qs is not None:
        ref["qs"] = gh.raw_bits(qs)
    # a second, independent eager call used as eager work between replays
    d2 = gh.upload(w)
    other = _prepared(w, d2)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        q.zero_()
        qr.zero_()
        if qs is not None:
            qs.zero_()
        d["kv_cache"].copy_(kv0)
        d["kr_cache"].copy_(kr0)
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(gh.raw_bits(q), ref["q"], err_msg=f"rep {rep}")
        np.testing.assert_array_equal(gh.raw_bits(qr), ref["qr"], err_msg=f"rep {rep}")
        np.testing.assert_array_equal(gh.raw_bits(d["kv_cache"]), ref["kv"])
        np.testing.assert_array_equal(gh.raw_bits(d["kr_cache"]), ref["kr"])
        if qs is not None:
            np.testing.assert_array_equal(gh.raw_bits(qs), ref["qs"])
    del g


@pytest.mark.parametrize("key", [4, "qkv_ragged_asym"])
def test_qkv_graph_replays_match_eager(key):
    w = make_workload(key)
    cfg = w.cfg
    gh.announce(f"graph replay {cfg.name}")
    d = gh.upload(w)
    kc0, vc0 = d["k_cache"].clone(), d["v_cache"].clone()
    q = torch.empty((cfg.T, cfg.Nq, cfg.D), dtype=d["qkv"].dtype, device="cuda")

    def call(dd, out):
        qn.qkv_rmsnorm_rope_cache(
            dd["qkv"], dd["gamma_q"], dd["gamma_k"], dd["cos"], dd["sin"],
            dd["index"], dd["k_cache"], dd["v_cache"], Nq=cfg.Nq, Nk=cfg.Nk,
            Nv=cfg.Nv, quant_mode=cfg.quant_mode, epsilon=cfg.eps,
            k_scale=dd.get("k_scale"), v_scale=dd.get("v_scale"),
            k_offset=dd.get("k_offset"), v_offset=dd.get("v_offset"),
            q_out=out, B=cfg.B, S=cfg.S)

    call(d, q)
    torch.cuda.synchronize()
    ref = {"q": gh.raw_bits(q), "k": gh.raw_bits(d["k_cache"]),
           "v": gh.raw_bits(d["v_cache"])}
    d2 = gh.upload(w)
    q2 = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(d, q)
    for rep in range(3):
        q.zero_()
        d["k_cache"].copy_(kc0)
        d["v_cache"].copy_(vc0)
        call(d2, q2)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(gh.raw_bits(q), ref["q"], err_msg=f"rep {rep}")
        np.testing.assert_array_equal(gh.raw_bits(d["k_cache"]), ref["k"])
        np.testing.assert_array_equal(gh.raw_bits(d["v_cache"]), ref["v"])
    del g
