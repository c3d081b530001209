"""Workload shapes.

Numbered cases 0-4 are the five headline workloads:

* 0: tiny MLA prolog, bf16, T=4 (the parity case the oracle runs instantly);
* 1: DeepSeek-V3-shaped decode, T=32, bf16;
* 2: prefill, T=4096, same dims as 1;
* 3: partially quantised MLA prolog (int8 W^UQ_QR, dynamic int8 c^Q, int8
  KV/KR caches), T=64, N=32;
* 4: fused qkv RmsNorm-RoPE-quant-cache on fp16 qkv, B=64, S=128,
  Nq/Nk/Nv = 32/8/8, D=128, int8 caches.

Named cases ("mla_ragged", ...) are extra parity shapes: small enough for the
float64 oracle, large enough to span several kernel tiles with ragged tails.

MLA dimension names follow the MlaPrologV2 page's shape table: He (hidden),
Hcq (query latent), N (heads), D (no-rope head dim), Hckv (kv latent), Dr (rope
head dim), Nkv (kv heads, 1), BlockNum and BlockSize of the paged caches.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class MlaConfig:
    name: str
    B: int
    S: int
    He: int
    Hcq: int
    N: int
    D: int
    Hckv: int
    Dr: int
    block_num: int
    block_size: int
    # "none" | "partial_kv_bf16" | "partial_kv_int8"
    quant_mode: str = "none"
    Nkv: int = 1
    eps_cq: float = 1e-5
    eps_ckv: float = 1e-5
    # number of tokens whose cache_index is -1 (skip)
    n_skip: int = 0
    seed: int = 0
    layout: str = "TND"  # or "BSH": same memory, (B,S,...) view

    kind = "mla"

    @property
    def T(self) -> int:
        return self.B * self.S

    @property
    def slots(self) -> int:
        return self.block_num * self.block_size

    @property
    def n_uqqr(self) -> int:
        return self.N * (self.D + self.Dr)

    def replace(self, **kw) -> "MlaConfig":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class QkvConfig:
    name: str
    B: int
    S: int
    Nq: int
    Nk: int
    Nv: int
    D: int
    block_num: int
    block_size: int
    # "none" (fp16 caches) | "symmetric" | "asymmetric" (int8 caches)
    quant_mode: str = "symmetric"
    eps: float = 1e-6
    # fraction of tokens whose index is -1
    skip_frac: float = 0.05
    seed: int = 0
    # also return the optional pre-quant copies of q, k and v
    before_quant: bool = False

    kind = "qkv"

    @property
    def T(self) -> int:
        return self.B * self.S

    @property
    def slots(self) -> int:
        return self.block_num * self.block_size

    def replace(self, **kw) -> "QkvConfig":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class PreConfig:
    """An MlaPreprocessV2 workload (aclnnMlaPreprocessV2): the same latent
    dimensions as the MLA prolog, int8 W^DQKV and W^UQ_QR, and one RmsNorm
    epsilon for its three norms."""
    name: str
    B: int
    S: int
    He: int
    Hcq: int
    N: int
    D: int
    Hckv: int
    Dr: int
    block_num: int
    block_size: int
    eps: float = 1e-6
    n_skip: int = 0
    seed: int = 0
    layout: str = "TND"

    kind = "pre"

    @property
    def T(self) -> int:
        return self.B * self.S

    @property
    def slots(self) -> int:
        return self.block_num * self.block_size

    def replace(self, **kw) -> "PreConfig":
        return dataclasses.replace(self, **kw)


_DSV3 = dict(He=7168, Hcq=1536, N=128, D=128, Hckv=512, Dr=64)

CONFIGS = {
    0: MlaConfig("mla_tiny_T4", B=4, S=1, He=256, Hcq=128, N=4, D=32, Hckv=64,
                 Dr=16, block_num=4, block_size=16, n_skip=1, seed=1000),
    1: MlaConfig("mla_decode_T32_dsv3", B=32, S=1, block_num=192,
                 block_size=128, seed=1001, layout="BSH", **_DSV3),
    2: MlaConfig("mla_prefill_T4096_dsv3", B=4, S=1024, block_num=192,
                 block_size=128, seed=1002, layout="BSH", **_DSV3),
    3: MlaConfig("mla_partial_quant_kvint8_T64_N32", B=64, S=1,
                 block_num=192, block_size=128, quant_mode="partial_kv_int8",
                 seed=1003, **{**_DSV3, "N": 32}),
    4: QkvConfig("qkv_rmsnorm_rope_cache_B64_S128_fp16", B=64, S=128, Nq=32,
                 Nk=8, Nv=8, D=128, block_num=64, block_size=128,
                 quant_mode="symmetric", eps=1e-6, skip_frac=0.05, seed=1004),
    # ---- extra parity shapes (not bench lines) ----
    "mla_ragged": MlaConfig("mla_ragged_T37", B=37, S=1, He=320, Hcq=192, N=6,
                            D=64, Hckv=128, Dr=32, block_num=5,
                            block_size=16, n_skip=3, seed=2001),
    "mla_ragged_q": MlaConfig("mla_ragged_q_T45", B=45, S=1, He=384, Hcq=256,
                              N=5, D=64, Hckv=128, Dr=32, block_num=4,
                              block_size=32, n_skip=4,
                              quant_mode="partial_kv_int8", seed=2002),
    "mla_ragged_qb": MlaConfig("mla_ragged_qb_T19", B=19, S=1, He=256,
                               Hcq=128, N=3, D=32, Hckv=64, Dr=16,
                               block_num=2, block_size=16, n_skip=2,
                               quant_mode="partial_kv_bf16", seed=2003),
    "mla_mid_dsv3": MlaConfig("mla_mid_T200_dsv3dims", B=2, S=100,
                              block_num=8, block_size=128, n_skip=5,
                              seed=2004, layout="BSH",
                              **{**_DSV3, "N": 16}),
    # more heads and a wider kv latent than the headline decode shape
    "mla_wide": MlaConfig("mla_wide_T8", B=8, S=1, He=1024,
                                Hcq=512, N=160, D=128, Hckv=1024, Dr=64,
                                block_num=2, block_size=64, n_skip=1,
                                seed=2005),
    # decode shapes with head dim 128: a partial row block, 2 W^UK column
    # blocks per wave and half a 64-column q^R tile
    "mla_dec_t13": MlaConfig("mla_dec_T13", B=13, S=1, He=512, Hcq=384,
                             N=7, D=128, Hckv=256, Dr=32, block_num=3,
                             block_size=16, n_skip=2, seed=2012),
    # Hcq of 10 k-steps (a partial register batch) and Hckv of 3 column
    # blocks
    "mla_dec_hckv96": MlaConfig("mla_dec_hckv96_T32", B=32, S=1, He=256,
                                Hcq=160, N=3, D=128, Hckv=96, Dr=64,
                                block_num=2, block_size=32, n_skip=1,
                                seed=2013),
    # head dim 96 (six 16-k steps per W^UK slice): each head's q^C is one
    # whole 96-column up-projection tile, and Hckv is 1.25 W^UK column tiles
    "mla_dec_d96": MlaConfig("mla_dec_d96_T17", B=17, S=1, He=256, Hcq=192,
                             N=5, D=96, Hckv=160, Dr=32, block_num=2,
                             block_size=16, n_skip=2, seed=2019),
    # full quantisation (int8 x and down-projection weights): a one-block
    # decode shape with bf16 caches, a two-block one with the int8 kv_cache
    # and int8 query, and a large-T shape on the tiled plan
    "mla_full_kvbf16": MlaConfig("mla_full_kvbf16_T21", B=21, S=1, He=512,
                                 Hcq=256, N=5, D=64, Hckv=128, Dr=32,
                                 block_num=4, block_size=16, n_skip=2,
                                 quant_mode="full_kv_bf16", seed=2014),
    "mla_full_kvint8": MlaConfig("mla_full_kvint8_T37", B=37, S=1, He=384,
                                 Hcq=192, N=6, D=128, Hckv=96, Dr=64,
                                 block_num=3, block_size=32, n_skip=3,
                                 quant_mode="full_kv_int8", seed=2015),
    "mla_full_kvint8_large": MlaConfig("mla_full_kvint8_T150", B=3, S=50,
                                       He=256, Hcq=128, N=3, D=32, Hckv=64,
                                       Dr=16, block_num=2, block_size=128,
                                       n_skip=4, quant_mode="full_kv_int8",
                                       seed=2016, layout="BSH"),
    # the widest down-projection row the kernels accept: Hcq + Hckv + Dr =
    # 16384 fp32 values (64 KB, the finish kernel's staged row), with a
    # kv row (4032) that is no multiple of 32 columns
    "mla_max_row": MlaConfig("mla_max_row_T13", B=13, S=1, He=64, Hcq=12288,
                             N=2, D=32, Hckv=4032, Dr=64, block_num=2,
                             block_size=16, n_skip=1, seed=2017),
    # the fused q^C + W^UK prefill path (D = 128, N*D a multiple of 256)
    # with a W^UK width (224) that ends in half a 64-column pass and a
    # ragged second row tile
    "mla_fused_ragged": MlaConfig("mla_fused_ragged_T300", B=3, S=100,
                                  He=256, Hcq=160, N=4, D=128, Hckv=224,
                                  Dr=64, block_num=4, block_size=128,
                                  n_skip=5, seed=2018, layout="BSH"),
    # the same fused path in the quantised modes (int8 q^C tiles, q^C as
    # bf16 hi + lo into W^UK): Hcq a multiple of 64, two heads per tile
    "mla_fused_q": MlaConfig("mla_fused_q_T300", B=3, S=100, He=256, Hcq=192,
                             N=4, D=128, Hckv=224, Dr=64, block_num=4,
                             block_size=128, n_skip=5, seed=2020, layout="BSH",
                             quant_mode="partial_kv_int8"),
    # prefill-sized T with no dimension a multiple of the 256x256 GEMM tile
    "mla_prefill_ragged": MlaConfig("mla_prefill_ragged_T300", B=3, S=100,
                                    He=512, Hcq=320, N=5, D=64, Hckv=96,
                                    Dr=32, block_num=4, block_size=128,
                                    n_skip=7, seed=2006, layout="BSH"),
    # MlaPreprocessV2: tiny, ragged decode, DeepSeek-V3 dims with 32 heads
    # (decode), and a T above the decode plan's limit (tiled kernels)
    "pre_tiny": PreConfig("pre_tiny_T4", B=4, S=1, He=256, Hcq=128, N=4, D=32,
                          Hckv=64, Dr=16, block_num=4, block_size=16,
                          n_skip=1, seed=3001),
    "pre_ragged": PreConfig("pre_ragged_T37", B=37, S=1, He=384, Hcq=192,
                            N=6, D=64, Hckv=128, Dr=32, block_num=5,
                            block_size=16, n_skip=3, seed=3002),
    "pre_dsv3": PreConfig("pre_decode_T32_dsv3_N32", B=32, S=1,
                          block_num=192, block_size=128, seed=3003,
                          **{**_DSV3, "N": 32}),
    "pre_large": PreConfig("pre_large_T300", B=3, S=100, He=512, Hcq=256,
                           N=5, D=64, Hckv=96, Dr=32, block_num=4,
                           block_size=128, n_skip=7, seed=3004,
                           layout="BSH"),
    "qkv_ragged": QkvConfig("qkv_ragged_B3_S50", B=3, S=50, Nq=4, Nk=2, Nv=2,
                            D=128, block_num=3, block_size=64,
                            quant_mode="symmetric", seed=2101),
    "qkv_ragged_none": QkvConfig("qkv_ragged_none_B2_S33", B=2, S=33, Nq=3,
                                 Nk=1, Nv=1, D=128, block_num=2,
                                 block_size=64, quant_mode="none",
                                 seed=2102, before_quant=True),
    "qkv_ragged_asym": QkvConfig("qkv_ragged_asym_B2_S41", B=2, S=41, Nq=2,
                                 Nk=2, Nv=2, D=128, block_num=2,
                                 block_size=64, quant_mode="asymmetric",
                                 seed=2103, before_quant=True),
}


def get_config(key):
    """Look up a workload by number (0-4) or by the name of a parity case."""
    if key in CONFIGS:
        return CONFIGS[key]
    if isinstance(key, str) and key.isdigit() and int(key) in CONFIGS:
        return CONFIGS[int(key)]
    for cfg in CONFIGS.values():
        if cfg.name == key:
            return cfg
    raise KeyError(f"unknown workload {key!r}")
