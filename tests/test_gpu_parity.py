"""GPU parity: the HIP library against the float64 oracle, element by
element, on seeded workloads (all calls go through the C ABI via the
binding).  Needs an MI355X and the built library; a missing library fails
these tests rather than skipping them.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import qkv_norm_rope_amd as qn
from tests import gpu_helpers as gh
from workloads import get_config, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qn.load_library()  # raises if the HIP library is not built
    torch.cuda.init()


def _before(dev, names):
    return {k: gh.raw_bits(dev[k]).copy() for k in names}


# ---- weight packing: pure index work, bit-exact ----------------------------

@pytest.mark.parametrize("shape,dtype", [((64, 48), "bf16"), ((3, 32, 40), "bf16"),
                                         ((96, 80), "int8"), ((7168, 64), "bf16"),
                                         ((32, 576), "bf16")])
def test_pack_weight_bit_exact(shape, dtype):
    gh.announce(f"pack {shape} {dtype}")
    rng = np.random.default_rng(5)
    if dtype == "bf16":
        bits = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        G = 8
    else:
        bits = rng.integers(-128, 128, size=shape).astype(np.int8)
        t = torch.from_numpy(bits).cuda()
        G = 16
    p = qn.mla_pack_weight(t)
    torch.cuda.synchronize()
    got = gh.raw_bits(p).reshape(-1)
    src = bits.reshape((-1,) + shape[-2:])
    B, K, N = src.shape
    Np = (N + 31) // 32 * 32
    assert p.shape == tuple(shape[:-1]) + (Np,)
    # expected: element (k, n) at ((n//32 * K/G + k//G) * 32 + n%32) * G + k%G
    pad = np.zeros((B, K, Np), dtype=src.dtype)
    pad[:, :, :N] = src
    want = pad.reshape(B, K // G, G, Np // 32, 32).transpose(0, 3, 1, 4, 2).reshape(-1)
    np.testing.assert_array_equal(got.view(want.dtype), want)


def _rope_pair_order(N, D, Dr):
    """Source column of each packed column of weight_uq_qr: W^UQ in place;
    for Dr = 64 each head's packed 32-column block b holds rope columns
    [16b, 16b+16) then [32+16b, 32+16b+16)."""
    cols = list(range(N * D))
    for n in range(N):
        base = N * D + n * Dr
        if Dr <= 32:
            cols += [base + j for j in range(Dr)]
        else:
            for b in range(Dr // 32):
                cols += [base + 16 * b + j for j in range(16)]
                cols += [base + Dr // 2 + 16 * b + j for j in range(16)]
    return np.array(cols)


@pytest.mark.parametrize("N,D,Dr,dtype", [(3, 32, 64, "bf16"), (5, 64, 32, "bf16"),
                                          (4, 32, 16, "bf16"), (2, 32, 64, "int8")])
def test_pack_weight_uq_qr_bit_exact(N, D, Dr, dtype):
    gh.announce(f"pack uq_qr N={N} D={D} Dr={Dr} {dtype}")
    rng = np.random.default_rng(6)
    Hcq = 64
    shape = (Hcq, N * (D + Dr))
    if dtype == "bf16":
        bits = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        G = 8
    else:
        bits = rng.integers(-128, 128, size=shape).astype(np.int8)
        t = torch.from_numpy(bits).cuda()
        G = 16
    p = qn.mla_pack_weight_uq_qr(t, N, D, Dr)
    torch.cuda.synchronize()
    got = gh.raw_bits(p).reshape(-1)
    src = bits[:, _rope_pair_order(N, D, Dr)]
    K, Nc = src.shape
    Np = (Nc + 31) // 32 * 32
    pad = np.zeros((K, Np), dtype=src.dtype)
    pad[:, :Nc] = src
    want = pad.reshape(K // G, G, Np // 32, 32).transpose(2, 0, 3, 1).reshape(-1)
    np.testing.assert_array_equal(got.view(want.dtype), want)


@pytest.mark.parametrize("N,D,H", [(3, 32, 40), (2, 128, 512), (1, 16, 32)])
def test_pack_weight_uk_bit_exact(N, D, H):
    gh.announce(f"pack uk N={N} D={D} Hckv={H}")
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=(N, D, H), dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    p = qn.mla_pack_weight_uk(t)
    torch.cuda.synchronize()
    got = gh.raw_bits(p).reshape(-1)
    # k order inside each 16-k step: {0-3, 8-11, 4-7, 12-15}
    perm = np.concatenate([16 * s + np.array([0, 1, 2, 3, 8, 9, 10, 11,
                                              4, 5, 6, 7, 12, 13, 14, 15])
                           for s in range(D // 16)])
    src = bits[:, perm, :]
    Hp = (H + 31) // 32 * 32
    pad = np.zeros((N, D, Hp), dtype=np.uint16)
    pad[:, :, :H] = src
    want = pad.reshape(N, D // 8, 8, Hp // 32, 32).transpose(0, 3, 1, 4, 2).reshape(-1)
    np.testing.assert_array_equal(got.view(np.uint16), want)


# ---- MLA prolog --------------------------------------------------------------

MLA_SMALL = [0, "mla_ragged", "mla_ragged_q", "mla_ragged_qb", "mla_mid_dsv3",
             "mla_prefill_ragged", "mla_fused_ragged", "mla_full_kvbf16",
             "mla_full_kvint8", "mla_full_kvint8_large"]


@pytest.mark.parametrize("key", MLA_SMALL)
@pytest.mark.parametrize("layout", ["packed", "nd"])
def test_mla_parity_small(key, layout):
    w = make_workload(key)
    gh.announce(f"mla {w.cfg.name} T={w.cfg.T} quant={w.cfg.quant_mode} {layout}")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev, layout=layout)
    torch.cuda.synchronize()
    stats = gh.check_mla(w, out, before)
    gh.announce(f"  ok {stats}")


def test_mla_parity_decode_T32():
    w = make_workload(1)
    gh.announce(f"mla {w.cfg.name} full size")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev, bsh=True)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


def test_mla_parity_partial_quant_T64():
    w = make_workload(3)
    gh.announce(f"mla {w.cfg.name} full size")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


def test_mla_parity_prefill_T4096():
    # Full-size run; every one of the 4096 tokens is compared with the
    # oracle (run on 512-token pieces), and the whole cache for placement.
    w = make_workload(2)
    gh.announce(f"mla {w.cfg.name} full size")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev, bsh=True)
    torch.cuda.synchronize()
    gh.announce(f"  checking all {w.cfg.T} tokens in 512-token pieces")
    gh.announce(f"  ok (worst err/tol) {gh.check_mla(w, out, before, chunk=512)}")


def test_mla_prefill_partial_quant_large_t_path():
    # T > 128 takes the large-T GEMMs in the partial-quant scenario too
    # (D = 64: the unfused int8 up projection and hi | lo W^UK product).
    cfg = get_config("mla_ragged_q").replace(B=3, S=67, block_num=8,
                                            block_size=32, n_skip=9,
                                            seed=2010, layout="BSH")
    w = make_workload(cfg)
    gh.announce(f"mla large-T quant T={cfg.T}")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev, bsh=True)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


@pytest.mark.parametrize("mode", ["partial_kv_int8", "partial_kv_bf16",
                                  "full_kv_bf16", "full_kv_int8"])
def test_mla_large_t_quant_fused(mode):
    # D = 128 with N*D a multiple of 256: the int8 q^C tiles carry the W^UK
    # product in their epilogue (q^C as bf16 hi + lo in registers), except
    # FULL_KV_INT8, whose query quant takes the unfused path.
    w = make_workload(get_config("mla_fused_q").replace(quant_mode=mode))
    gh.announce(f"mla fused quant {mode} T={w.cfg.T}")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev, bsh=True)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


# config 2 (prefill T = 4096): every GEMM tile shape at full occupancy,
# where a stage-buffer race shows up as run-to-run differences
@pytest.mark.parametrize("key", [0, "mla_mid_dsv3", 3, "mla_dec_t13", 2,
                                 "mla_full_kvint8"])
def test_mla_deterministic(key):
    w = make_workload(key)
    gh.announce(f"mla determinism {w.cfg.name}")
    outs = []
    for _ in range(2):
        dev = gh.upload(w)
        o = gh.run_mla_gpu(w, dev)
        torch.cuda.synchronize()
        outs.append({k: gh.raw_bits(v) for k, v in o.items()})
    for k in outs[0]:
        np.testing.assert_array_equal(outs[0][k], outs[1][k], err_msg=k)


@pytest.mark.parametrize("Hckv,T", [(96, 21), (256, 9), (64, 1), (1024, 8)])
def test_mla_full_quant_query_in_epilogue(Hckv, T):
    """FULL_KV_INT8 with one row block: the W^UK product quantises the query
    per (token, head) in its epilogue, one workgroup per head of 4, 8 or 16
    waves (Hckv up to 128, 256, 512); a wider head (Hckv = 1024) takes the
    fp32 q^N + k_quant_query path."""
    cfg = get_config("mla_full_kvint8").replace(B=T, Hckv=Hckv,
                                                n_skip=min(2, T - 1),
                                                seed=2018 + Hckv)
    w = make_workload(cfg)
    gh.announce(f"mla {w.cfg.name} Hckv={Hckv} T={T}")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


@pytest.mark.parametrize("mode,D,Dr,T", [("partial_kv_int8", 64, 32, 33),
                                         ("partial_kv_bf16", 96, 64, 64),
                                         ("full_kv_bf16", 32, 16, 1),
                                         ("partial_kv_int8", 128, 64, 17)])
def test_mla_quant_merged_decode_launch(mode, D, Dr, T):
    """The quantised decode plans with a bf16 query and few heads run the up
    projection and the W^UK product as one launch (fp32 q^C handed over per
    head): one and two 32-row blocks, ragged T, D = 32 to 128."""
    cfg = get_config(3).replace(He=512, Hcq=256, N=8, D=D, Dr=Dr, Hckv=256, B=T,
                                quant_mode=mode, seed=2060 + D + T)
    w = make_workload(cfg)
    gh.announce(f"mla {w.cfg.name} {mode} D={D} Dr={Dr} T={T}")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


@pytest.mark.parametrize("mode,T", [("full_kv_int8", 32), ("full_kv_bf16", 64),
                                    ("full_kv_bf16", 32), ("full_kv_int8", 64),
                                    ("partial_kv_bf16", 64),
                                    ("partial_kv_bf16", 32)])
def test_mla_full_quant_dsv3_dims(mode, T):
    """The quantised scenarios at the DeepSeek-V3 dims with 32 heads (the
    partially quantised workload's shape), on the one- and two-block decode
    plans: both full-quantisation rows and the partial one with bf16
    caches."""
    w = make_workload(get_config(3).replace(B=T, quant_mode=mode, seed=2017))
    gh.announce(f"mla {w.cfg.name} {mode} T={T}")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


@pytest.mark.parametrize("key", ["mla_ragged_q", "mla_full_kvbf16",
                                 "mla_full_kvint8", "mla_dec_t13"])
def test_mla_zero_tokens(key):
    """All-zero tokens: c^Q = 0, so the dynamic quantisation's scale is 0
    with zero codes, the int8 query's per-head scale is 0, and the norms see
    a zero row (their epsilon keeps them finite).  The tokens around them
    are ordinary."""
    w = make_workload(key)
    x = w.arrays["token_x"].reshape(w.cfg.T, -1)
    x[[0, w.cfg.T // 2]] = 0
    gh.announce(f"mla zero tokens {w.cfg.name} {w.cfg.quant_mode}")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")
    if w.cfg.quant_mode != "none":
        s = out["cq_scale"].cpu().numpy()
        assert s[0] == 0 and s[w.cfg.T // 2] == 0
        assert not out["cq_int8"][0].any()


def test_mla_T0_and_no_slots():
    w = make_workload(0)
    cfg = w.cfg
    gh.announce("mla T=0 and BlockNum=0")
    dev = gh.upload(w)
    # T = 0: nothing happens, caches untouched
    before = _before(dev, ["kv_cache", "kr_cache"])
    e = {k: v[:0] for k, v in dev.items()
         if k in ("token_x", "rope_cos", "rope_sin", "cache_index")}
    d0 = dict(dev, **e)
    q, qr = qn.mla_prolog_v2(
        d0["token_x"], dev["weight_dq"], dev["weight_uq_qr"], dev["weight_uk"],
        dev["weight_dkv_kr"], dev["rmsnorm_gamma_cq"], dev["rmsnorm_gamma_ckv"],
        d0["rope_sin"], d0["rope_cos"], d0["cache_index"], dev["kv_cache"],
        dev["kr_cache"], weight_layout=qn.MLA_WEIGHT_ND)
    torch.cuda.synchronize()
    assert q.shape == (0, cfg.N, cfg.Hckv) and qr.shape == (0, cfg.N, cfg.Dr)
    np.testing.assert_array_equal(gh.raw_bits(dev["kv_cache"]), before["kv_cache"])
    # BlockNum = 0: queries as usual
    empty_kv = dev["kv_cache"][:0]
    empty_kr = dev["kr_cache"][:0]
    q1, qr1 = qn.mla_prolog_v2(
        dev["token_x"], dev["weight_dq"], dev["weight_uq_qr"], dev["weight_uk"],
        dev["weight_dkv_kr"], dev["rmsnorm_gamma_cq"], dev["rmsnorm_gamma_ckv"],
        dev["rope_sin"], dev["rope_cos"], dev["cache_index"], empty_kv, empty_kr,
        weight_layout=qn.MLA_WEIGHT_ND)
    full = gh.run_mla_gpu(w, gh.upload(w), layout="nd")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gh.raw_bits(q1), gh.raw_bits(full["query"]))
    np.testing.assert_array_equal(gh.raw_bits(qr1), gh.raw_bits(full["query_rope"]))


# decode-sized shapes beyond the small list: a ragged T = 21 (one partial
# 32-row block), wider N / Hckv than one pass of 256 workgroups covers, and
# two head-dim-128 shapes with partial tiles and batches
DECODE_CASES = ["mla_ragged_t21", "mla_wide", "mla_dec_t13", "mla_dec_hckv96",
                "mla_dec_d96"]


def _decode_case(key):
    if key == "mla_ragged_t21":
        return make_workload(get_config("mla_ragged").replace(B=21, n_skip=2,
                                                             seed=2011))
    return make_workload(key)


# token counts at each plan boundary: one token, the skinny plan with one,
# two and four 32-row blocks, and the first large-T shapes (ragged tile)
TOKEN_CASES = [("mla_ragged", 1), ("mla_ragged", 33), ("mla_ragged", 64),
               ("mla_ragged", 100), ("mla_ragged", 129), ("mla_mid_dsv3", 1),
               ("mla_mid_dsv3", 128), ("mla_mid_dsv3", 257),
               ("mla_fused_ragged", 150)]


@pytest.mark.parametrize("key,T", TOKEN_CASES)
def test_mla_token_counts(key, T):
    cfg = get_config(key)
    blocks = max(cfg.block_num, -(-(T + 8) // cfg.block_size))
    w = make_workload(cfg.replace(B=T, S=1, block_num=blocks,
                                  n_skip=min(cfg.n_skip, max(0, T - 1)),
                                  seed=3000 + T))
    gh.announce(f"mla {w.cfg.name} T={w.cfg.T}")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


@pytest.mark.parametrize("key", DECODE_CASES)
def test_mla_decode_shapes(key):
    w = _decode_case(key)
    gh.announce(f"mla decode {w.cfg.name} T={w.cfg.T}")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


# the largest row the validator accepts ((Hcq + Hckv + Dr) * 4 = 64 KB) on
# the decode and large-T plans, unquantised, partially and fully quantised
@pytest.mark.parametrize("mode,T", [("none", 13), ("none", 130),
                                    ("partial_kv_int8", 13),
                                    ("partial_kv_int8", 130),
                                    ("full_kv_int8", 13),
                                    ("full_kv_bf16", 130)])
def test_mla_max_row_width(mode, T):
    cfg = get_config("mla_max_row")
    blocks = max(cfg.block_num, -(-(T + 8) // cfg.block_size))
    w = make_workload(cfg.replace(B=T, quant_mode=mode, block_num=blocks,
                                  seed=cfg.seed + T))
    gh.announce(f"mla max row {mode} T={T}")
    dev = gh.upload(w)
    before = _before(dev, ["kv_cache", "kr_cache"])
    out = gh.run_mla_gpu(w, dev)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_mla(w, out, before)}")


def test_mla_packed_equals_nd():
    w = make_workload("mla_ragged")
    gh.announce("mla packed vs ND layouts")
    a = gh.run_mla_gpu(w, gh.upload(w), layout="packed")
    b = gh.run_mla_gpu(w, gh.upload(w), layout="nd")
    torch.cuda.synchronize()
    for k in a:
        np.testing.assert_array_equal(gh.raw_bits(a[k]), gh.raw_bits(b[k]), err_msg=k)


# ---- QkvRmsNormRopeCache -----------------------------------------------------

@pytest.mark.parametrize("key", ["qkv_ragged", "qkv_ragged_none", "qkv_ragged_asym", 4])
def test_qkv_parity(key):
    w = make_workload(key)
    gh.announce(f"qkv {w.cfg.name} T={w.cfg.T} quant={w.cfg.quant_mode}")
    dev = gh.upload(w)
    before = _before(dev, ["k_cache", "v_cache"])
    out = gh.run_qkv_gpu(w, dev)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_qkv(w, out, before)}")


@pytest.mark.parametrize("key,T", [("qkv_ragged", 1), ("qkv_ragged_none", 1),
                                   ("qkv_ragged_asym", 7), ("qkv_ragged", 191)])
def test_qkv_token_counts(key, T):
    cfg = get_config(key)
    w = make_workload(cfg.replace(B=1, S=T, seed=3100 + T))
    gh.announce(f"qkv {w.cfg.name} T={w.cfg.T} quant={w.cfg.quant_mode}")
    dev = gh.upload(w)
    before = _before(dev, ["k_cache", "v_cache"])
    out = gh.run_qkv_gpu(w, dev)
    torch.cuda.synchronize()
    gh.announce(f"  ok {gh.check_qkv(w, out, before)}")


def test_qkv_deterministic_and_bf16_input():
    w = make_workload("qkv_ragged")
    gh.announce("qkv determinism")
    outs = []
    for _ in range(2):
        o = gh.run_qkv_gpu(w, gh.upload(w))
        torch.cuda.synchronize()
        outs.append({k: gh.raw_bits(v) for k, v in o.items()})
    for k in outs[0]:
        np.testing.assert_array_equal(outs[0][k], outs[1][k], err_msg=k)
    # bf16 inputs: same op on bf16-rounded copies of the fp16 inputs
    import oracle
    from workloads.gen import bf16_bits_from_f64
    wb = make_workload("qkv_ragged")
    for k in ("qkv", "gamma_q", "gamma_k", "cos", "sin"):
        wb.arrays[k] = bf16_bits_from_f64(w.arrays[k].astype(np.float64))
        wb.dtypes[k] = "bf16"
    dev = gh.upload(wb)
    before = _before(dev, ["k_cache", "v_cache"])
    out = gh.run_qkv_gpu(wb, dev)
    torch.cuda.synchronize()
    assert out["q_out"].dtype == torch.bfloat16
    gh.announce(f"  bf16 ok {gh.check_qkv(wb, out, before)}")
    del oracle


def test_qkv_empty():
    w = make_workload("qkv_ragged")
    dev = gh.upload(w)
    gh.announce("qkv T=0")
    cfg = w.cfg
    before = _before(dev, ["k_cache", "v_cache"])
    q = qn.qkv_rmsnorm_rope_cache(
        dev["qkv"][:0], dev["gamma_q"], dev["gamma_k"], dev["cos"][:0],
        dev["sin"][:0], dev["index"][:0], dev["k_cache"], dev["v_cache"],
        Nq=cfg.Nq, Nk=cfg.Nk, Nv=cfg.Nv, k_scale=dev["k_scale"],
        v_scale=dev["v_scale"], B=0, S=cfg.S)
    torch.cuda.synchronize()
    assert q.shape[0] == 0
    np.testing.assert_array_equal(gh.raw_bits(dev["k_cache"]), before["k_cache"])
