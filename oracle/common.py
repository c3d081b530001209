"""Building blocks of the oracle, each in float64 (test infrastructure only).

Every function is the plain definition of one step, with no blocking, fusion
or reordering.
"""

from __future__ import annotations

import numpy as np


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact value of a stored tensor as float64 (int8/int64 stay integers).

    bf16 arrives as raw 16-bit patterns: they are the upper half of a float32
    with the same sign, exponent and leading mantissa bits, so shifting them
    into place gives the exact value.  fp16 and fp32 widen exactly.
    """
    if dtype == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("fp16", "fp32", "fp64"):
        return np.asarray(arr).astype(np.float64)
    if dtype in ("int8", "int32", "int64"):
        return np.asarray(arr).astype(np.int64)
    raise ValueError(f"unknown dtype {dtype!r}")


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RmsNorm over the last axis.

    MlaPrologV2 README, formulas: RMS(x) is the square root of the mean of
    x_i^2 over the normalised axis plus epsilon, and the output is
    gamma * x_i / RMS(x).  aclnnQkvRmsNormRopeCache formula (2) states the
    same rule (square, mean over the last dim, add epsilon, square root,
    divide, scale by gamma).
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + float(eps))) * np.asarray(gamma, np.float64)


def rope_half(y: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Half-and-half rotary embedding over the last axis.

    aclnnQkvRmsNormRopeCache formula (3): split y into its first half y1 and
    second half y2, form the rotated vector cat(-y2, y1), and return
    y * cos + rotated * sin, elementwise with full-width cos and sin.  The
    MLA prolog applies the same form to q^R and k^R (its page names RoPE but
    does not spell it out).
    """
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even last dimension")
    h = d // 2
    rotated = np.concatenate([-y[..., h:], y[..., :h]], axis=-1)
    return y * cos + rotated * sin


def quant_int8(v: np.ndarray, scale: np.ndarray, offset=None) -> np.ndarray:
    """Static int8 quantisation: round(v / scale [+ offset]), saturated.

    aclnnQkvRmsNormRopeCache formula (4): symmetric quantisation divides by
    the scale; asymmetric adds the offset after dividing.  The pages do not
    fix rounding or saturation; the reading used is round half to even, then
    clamp to the int8 range [-128, 127].
    """
    q = np.asarray(v, dtype=np.float64) / np.asarray(scale, dtype=np.float64)
    if offset is not None:
        q = q + np.asarray(offset, dtype=np.float64)
    return np.clip(np.rint(q), -128, 127).astype(np.int64)


def dynamic_quant_int8(cq: np.ndarray, smooth: np.ndarray):
    """Per-token dynamic int8 quantisation of c^Q with a smooth scale.

    MlaPrologV2 README, parameter table: smooth_scales_cq is the dynamic
    quantisation parameter of the RmsNormCq output, shape (1, Hcq).  Reading:
    u = c^Q * smooth per channel; the token's scale s = max|u| / 127; codes
    are round-half-even(u / s) in [-127, 127].  An all-zero row gets s = 0 and
    zero codes.
    """
    u = np.asarray(cq, np.float64) * np.asarray(smooth, np.float64)
    amax = np.max(np.abs(u), axis=-1, keepdims=True)
    s = amax / 127.0
    safe = np.where(s > 0, s, 1.0)
    codes = np.where(s > 0, np.clip(np.rint(u / safe), -127, 127), 0.0)
    return codes.astype(np.int64), s[..., 0]


def int_matmul_exact(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Integer product in int64: exact for int8 operands and any sane K."""
    return np.matmul(np.asarray(a, np.int64), np.asarray(b, np.int64))


def check_index(index: np.ndarray, slots: int) -> None:
    """Preconditions on a cache index.

    aclnnQkvRmsNormRopeCache, other restrictions: each index lies in
    [-1, BlockNum*BlockSize), values do not repeat, and -1 means the update is
    skipped.  Repeats of -1 are allowed (they write nothing).
    """
    idx = np.asarray(index, np.int64).reshape(-1)
    bad = (idx < -1) | (idx >= slots)
    if np.any(bad):
        raise ValueError(f"cache index out of [-1, {slots}): {idx[bad][:8]}")
    valid = idx[idx >= 0]
    if np.unique(valid).size != valid.size:
        raise ValueError("cache index repeats a slot")


def scatter_slots(cache: np.ndarray, index: np.ndarray, rows: np.ndarray):
    """Return a copy of a paged cache with token rows written at their slots.

    cache has shape (BlockNum, BlockSize, H, W); slot s is
    cache[s // BlockSize, s % BlockSize].  rows has shape (T, H, W).  Tokens
    whose index is -1 write nothing.  With no slots at all (BlockNum *
    BlockSize == 0) nothing is written (MlaPrologV2 README, shape constraints:
    an empty Skv leaves the caches unchanged).
    """
    out = np.array(cache, copy=True)
    bn, bs = out.shape[0], out.shape[1]
    if bn * bs == 0:
        return out
    idx = np.asarray(index, np.int64).reshape(-1)
    check_index(idx, bn * bs)
    for t, s in enumerate(idx):
        if s >= 0:
            out[s // bs, s % bs] = rows[t]
    return out
