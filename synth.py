"""Seeded synthetic inputs for the q4_K x q8_1 MMQ path.

This module only *generates inputs*: f32 activations of the prefill workloads and
q4_K and q6_K weight blocks in the GGUF byte layouts. It holds none of the arithmetic of the
quantized multiply itself (no q8_1 quantization, no block dot product, no rescale);
both the HIP path and the CPU oracle consume what it produces.

Workloads (LLaMA-7B-shaped prefill, synthetic stand-ins for trained weights):
  tiny      M=128,  K=512,   N=256    x ~ N(0,1); random q4_K fields
  qproj     M=2048, K=4096,  N=4096   x ~ N(0,1) with 0.1% outliers x20; q4_K fit of N(0,0.02)
  gateup    M=2048, K=4096,  N=11008  same distributions as qproj
  down      M=2048, K=11008, N=4096   x = SiLU(g)*u with g,u ~ N(0,1); q4_K fit of N(0,0.02)
  sweep     M in {1,16,128,512,8192}, K=N=4096, distributions of qproj
  *_share8  one GPU's share of an 8-way split of the output features (column parallel):
            qproj and down with N=512, gateup with N=1376; distributions of their full shapes
"""
from __future__ import annotations

import numpy as np

QK_K = 256            # q4_K super-block length
Q4K_BLOCK_BYTES = 144  # 2 f16 + 12 packed scale bytes + 128 nibble bytes

SWEEP_M = (1, 16, 128, 512, 8192)

# name -> (M, K, N, activation kind, x seed, w kind, w seed)
WORKLOADS = {
    "tiny":   (128, 512, 256, "normal", 1000, "random_fields", 2000),
    "qproj":  (2048, 4096, 4096, "normal_outliers", 1001, "fit", 2001),
    "gateup": (2048, 4096, 11008, "normal_outliers", 1002, "fit", 2002),
    "down":   (2048, 11008, 4096, "swiglu", 1003, "fit", 2003),
}
for _i, _m in enumerate(SWEEP_M):
    WORKLOADS[f"sweep_m{_m}"] = (_m, 4096, 4096, "normal_outliers", 1400 + _i, "fit", 2004)
SHARE8 = ("qproj_share8", "gateup_share8", "down_share8")
WORKLOADS["qproj_share8"] = (2048, 4096, 512, "normal_outliers", 1001, "fit", 2011)
WORKLOADS["gateup_share8"] = (2048, 4096, 1376, "normal_outliers", 1002, "fit", 2012)
WORKLOADS["down_share8"] = (2048, 11008, 512, "swiglu", 1003, "fit", 2013)

# the seven projection shapes of one LLaMA-7B layer at 2K tokens: (name, N, K)
PREFILL_SHAPES = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                  ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008))


# ----------------------------------------------------------------------------- activations
def activations(kind: str, M: int, K: int, seed: int) -> np.ndarray:
    """f32 [M, K] activations of the given distribution, fully determined by seed."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal((M, K), dtype=np.float32)
    if kind == "normal_outliers":
        x = rng.standard_normal((M, K), dtype=np.float32)
        mask = rng.random((M, K)) < 0.001          # independent Bernoulli(0.001) per element
        x[mask] *= np.float32(20.0)
        return x
    if kind == "swiglu":
        g = rng.standard_normal((M, K), dtype=np.float32)
        u = rng.standard_normal((M, K), dtype=np.float32)
        one = np.float32(1.0)
        return (g / (one + np.exp(-g)) * u).astype(np.float32)
    raise ValueError(f"unknown activation kind {kind!r}")


# ----------------------------------------------------------------------------- q4_K fields
def _f16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _f16_val(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def q4k_random_fields(N: int, K: int, seed: int) -> dict:
    """Independent uniform q4_K fields: d, dmin = f16(U[1e-3, 2e-2]); sc, m ~ U{0..63}; v ~ U{0..15}."""
    assert K % QK_K == 0
    rng = np.random.default_rng(seed)
    nsb = K // QK_K
    return {
        "d_bits": _f16_bits(rng.uniform(1e-3, 2e-2, (N, nsb))),
        "dmin_bits": _f16_bits(rng.uniform(1e-3, 2e-2, (N, nsb))),
        "sc": rng.integers(0, 64, (N, K // 32), dtype=np.uint8),
        "m": rng.integers(0, 64, (N, K // 32), dtype=np.uint8),
        "v": rng.integers(0, 16, (N, K), dtype=np.uint8),
    }


def q4k_fit(w: np.ndarray) -> dict:
    """Fit q4_K fields to f32 weights [N, K] with a simple per-32 min/scale search.

    Per 32-element sub-block: lo = min(0, min x), sc_f = (max x - lo)/15. Per super-block:
    d = f16(max sc_f / 63), dmin = f16(max(-lo) / 63); sc = clamp(rint(sc_f/d), 0, 63),
    m = clamp(rint(-lo/dmin), 0, 63), v = clamp(rint((x + dmin*m)/(d*sc)), 0, 15);
    a zero denominator gives 0. Only the distribution of the resulting fields matters.
    """
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    assert K % QK_K == 0
    nsb = K // QK_K
    xs = w.reshape(N, nsb, 8, 32)
    lo = np.minimum(0.0, xs.min(axis=3))                     # [N, nsb, 8]
    sc_f = (xs.max(axis=3) - lo) / 15.0
    d_bits = _f16_bits(sc_f.max(axis=2) / 63.0)
    dmin_bits = _f16_bits((-lo).max(axis=2) / 63.0)
    d = _f16_val(d_bits)[..., None]
    dmin = _f16_val(dmin_bits)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d > 0, np.rint(sc_f / d), 0.0)
        m = np.where(dmin > 0, np.rint(-lo / dmin), 0.0)
        sc = np.clip(sc, 0, 63)
        m = np.clip(m, 0, 63)
        scale = (d * sc)[..., None]
        v = np.where(scale > 0, np.rint((xs + (dmin * m)[..., None]) / scale), 0.0)
    v = np.clip(v, 0, 15)
    return {
        "d_bits": d_bits, "dmin_bits": dmin_bits,
        "sc": sc.astype(np.uint8).reshape(N, K // 32),
        "m": m.astype(np.uint8).reshape(N, K // 32),
        "v": v.astype(np.uint8).reshape(N, K),
    }


def q4k_pack(f: dict) -> np.ndarray:
    """Pack q4_K fields into GGUF-layout blocks, u8 [N, K/256, 144].

    Byte layout of one 144-byte super-block:
      0..1   d    (f16, little endian)        2..3  dmin (f16)
      4..7   low 6 bits: sc of sub-blocks 0..3; top 2 bits: bits 4..5 of sc of sub-blocks 4..7
      8..11  low 6 bits: m  of sub-blocks 0..3; top 2 bits: bits 4..5 of m  of sub-blocks 4..7
      12..15 low nibble: bits 0..3 of sc of sub-blocks 4..7; high nibble: bits 0..3 of m of 4..7
      16..143 four 32-byte groups; group g byte t: low nibble = sub-block 2g element t,
              high nibble = sub-block 2g+1 element t
    """
    N, K = f["v"].shape
    nsb = K // QK_K
    sc = f["sc"].reshape(N, nsb, 8).astype(np.uint8)
    m = f["m"].reshape(N, nsb, 8).astype(np.uint8)
    v = f["v"].reshape(N, nsb, 4, 2, 32).astype(np.uint8)
    assert sc.max(initial=0) < 64 and m.max(initial=0) < 64 and v.max(initial=0) < 16
    out = np.zeros((N, nsb, Q4K_BLOCK_BYTES), dtype=np.uint8)
    out[..., 0:2] = np.asarray(f["d_bits"], np.uint16).reshape(N, nsb, 1).view(np.uint8)
    out[..., 2:4] = np.asarray(f["dmin_bits"], np.uint16).reshape(N, nsb, 1).view(np.uint8)
    out[..., 4:8] = (sc[..., 0:4] & 63) | ((sc[..., 4:8] >> 4) << 6)
    out[..., 8:12] = (m[..., 0:4] & 63) | ((m[..., 4:8] >> 4) << 6)
    out[..., 12:16] = (sc[..., 4:8] & 15) | ((m[..., 4:8] & 15) << 4)
    out[..., 16:144] = (v[:, :, :, 0, :] | (v[:, :, :, 1, :] << 4)).reshape(N, nsb, 128)
    return out


def q4k_weights(kind: str, N: int, K: int, seed: int) -> tuple[np.ndarray, dict]:
    """(packed q4_K blocks u8 [N, K/256, 144], the fields they encode)."""
    if kind == "random_fields":
        f = q4k_random_fields(N, K, seed)
    elif kind == "fit":
        rng = np.random.default_rng(seed)
        w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        f = q4k_fit(w)
    else:
        raise ValueError(f"unknown weight kind {kind!r}")
    return q4k_pack(f), f


# ----------------------------------------------------------------------------- q6_K fields
Q6K_BLOCK_BYTES = 210  # 128 bytes low nibbles + 64 bytes high 2-bit pairs + 16 int8 scales + f16 d


def q6k_random_fields(N: int, K: int, seed: int) -> dict:
    """Independent uniform q6_K fields: d = f16(U[1e-4, 2e-3]); 16-element group scales
    sc ~ U{-127..127} (int8); 6-bit values u ~ U{0..63}."""
    assert K % QK_K == 0
    rng = np.random.default_rng(seed)
    return {
        "d_bits": _f16_bits(rng.uniform(1e-4, 2e-3, (N, K // QK_K))),
        "sc": rng.integers(-127, 128, (N, K // 16), dtype=np.int8),
        "u": rng.integers(0, 64, (N, K), dtype=np.uint8),
    }


def q6k_fit(w: np.ndarray) -> dict:
    """Fit q6_K fields to f32 weights [N, K]: per 16-element group the scale sc_f = max|x|/31;
    per super-block d = f16(max |sc_f| / 127); sc = clamp(rint(sc_f/d), -127, 127) (int8),
    u = clamp(rint(x/(d*sc)) + 32, 0, 63); a zero denominator gives sc = 0 or u = 32. Only
    the distribution of the resulting fields matters."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    assert K % QK_K == 0
    xs = w.reshape(N, K // QK_K, 16, 16)
    sc_f = np.abs(xs).max(axis=3) / 31.0                          # [N, nsb, 16]
    d_bits = _f16_bits(sc_f.max(axis=2) / 127.0)
    d = _f16_val(d_bits)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d > 0, np.rint(sc_f / d), 0.0)
        sc = np.clip(sc, -127, 127)
        scale = (d * sc)[..., None]
        u = np.where(scale != 0, np.rint(xs / scale) + 32, 32.0)
    u = np.clip(u, 0, 63)
    return {"d_bits": d_bits, "sc": sc.astype(np.int8).reshape(N, K // 16),
            "u": u.astype(np.uint8).reshape(N, K)}


def q6k_pack(f: dict) -> np.ndarray:
    """Pack q6_K fields into GGUF-layout blocks, u8 [N, K/256, 210].

    Byte layout of one 210-byte super-block of 256 values (6-bit u, stored value u - 32):
      0..127    ql: the low 4 bits. The block is two halves of 128 values; half h owns bytes
                64h..64h+63. Value 128h + 32q + l (q = 0..3, l = 0..31) keeps its low 4 bits in
                byte 64h + l + 32*(q & 1), in the low nibble for q < 2 and the high nibble for
                q >= 2.
      128..191  qh: the high 2 bits. Half h owns bytes 128 + 32h .. +31; value 128h + 32q + l
                keeps them in bits 2q..2q+1 of byte 128 + 32h + l.
      192..207  the 16 int8 scales, one per 16 consecutive values (value v uses scale v // 16).
      208..209  d (f16, little endian).
    """
    N, K = f["u"].shape
    nsb = K // QK_K
    u = f["u"].reshape(N, nsb, 2, 4, 32).astype(np.uint8)        # [n, s, half, q, l]
    assert u.max(initial=0) < 64
    out = np.zeros((N, nsb, Q6K_BLOCK_BYTES), dtype=np.uint8)
    lo = u & 15
    hi = u >> 4
    ql = np.zeros((N, nsb, 2, 64), dtype=np.uint8)
    ql[..., 0:32] = lo[:, :, :, 0, :] | (lo[:, :, :, 2, :] << 4)
    ql[..., 32:64] = lo[:, :, :, 1, :] | (lo[:, :, :, 3, :] << 4)
    qh = hi[:, :, :, 0, :] | (hi[:, :, :, 1, :] << 2) | (hi[:, :, :, 2, :] << 4) \
        | (hi[:, :, :, 3, :] << 6)
    out[..., 0:128] = ql.reshape(N, nsb, 128)
    out[..., 128:192] = qh.reshape(N, nsb, 64)
    out[..., 192:208] = np.asarray(f["sc"], np.int8).reshape(N, nsb, 16).view(np.uint8)
    out[..., 208:210] = np.asarray(f["d_bits"], np.uint16).reshape(N, nsb, 1).view(np.uint8)
    return out


def q6k_weights(kind: str, N: int, K: int, seed: int) -> tuple[np.ndarray, dict]:
    """(packed q6_K blocks u8 [N, K/256, 210], the fields they encode)."""
    if kind == "random_fields":
        f = q6k_random_fields(N, K, seed)
    elif kind == "fit":
        rng = np.random.default_rng(seed)
        w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        f = q6k_fit(w)
    else:
        raise ValueError(f"unknown weight kind {kind!r}")
    return q6k_pack(f), f


def workload(name: str, need_fields: bool = False) -> dict:
    """Inputs of a named workload: dict(M, K, N, x [M,K] f32, w [N,K/256,144] u8[, fields])."""
    M, K, N, xkind, xseed, wkind, wseed = WORKLOADS[name]
    x = activations(xkind, M, K, xseed)
    w, f = q4k_weights(wkind, N, K, wseed)
    out = {"name": name, "M": M, "K": K, "N": N, "x": x, "w": w}
    if need_fields:
        out["fields"] = f
    return out
