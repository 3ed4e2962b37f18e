"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds data generation only -- none of the attention arithmetic.
Each (config, tensor, batch) slice has its own generator seed
``10000*config + 1000*tensor + batch`` (tensor ids: q=0, k=1, v=2, lens=3),
so a slice can be regenerated on its own.  Values are float32 standard
normals times a multiplier, rounded to bfloat16 (round-to-nearest-even) for
the bf16 configs.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import torch

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_LENS, TENSOR_DOUT = 0, 1, 2, 3, 4

# The five workloads.  "N" is both Nq and Nk for prefill; decode has Nq = 1.
CONFIGS = {
    1: dict(name="tiny_fp32", kind="prefill", B=1, Hq=1, Hkv=1, Nq=128, Nk=128, d=64,
            dtype="f32", mult=1.0, causal=(False,), padded=False),
    2: dict(name="bf16_selfattn_n2048_d64", kind="prefill", B=2, Hq=16, Hkv=16, Nq=2048,
            Nk=2048, d=64, dtype="bf16", mult=1.0, causal=(False, True), padded=False),
    3: dict(name="long_causal_n8192_d128", kind="prefill", B=1, Hq=32, Hkv=32, Nq=8192,
            Nk=8192, d=128, dtype="bf16", mult=0.5, causal=(True,), padded=False),
    4: dict(name="gqa_padded_n4096_d128", kind="prefill", B=4, Hq=32, Hkv=8, Nq=4096,
            Nk=4096, d=128, dtype="bf16", mult=1.0, causal=(True,), padded=True,
            len_lo=2048, len_hi=4096),
    5: dict(name="splitkv_decode_b64_nk32768", kind="decode", B=64, Hq=32, Hkv=8, Nq=1,
            Nk=32768, d=128, dtype="bf16", mult=1.0, causal=(False,), padded=False,
            num_splits=16),
}

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def slice_seed(config_id, tensor_id, batch):
    return 10000 * config_id + 1000 * tensor_id + batch


def _slice(config_id, tensor_id, b, shape, mult, dtype):
    g = torch.Generator("cpu").manual_seed(slice_seed(config_id, tensor_id, b))
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if mult != 1.0:
        x.mul_(mult)
    return x.to(dtype)


def randn_tensor(config_id, tensor_id, B, H, N, d, mult=1.0, dtype="bf16", threads=None):
    """[B, H, N, d] tensor whose batch slice b comes from its own seeded generator."""
    tdt = _TORCH_DTYPE[dtype]
    out = torch.empty((B, H, N, d), dtype=tdt)

    def fill(b):
        out[b] = _slice(config_id, tensor_id, b, (H, N, d), mult, tdt)

    big = B * H * N * d >= (1 << 26)
    workers = threads or (min(16, os.cpu_count() or 1) if big else 1)
    if workers > 1 and B > 1:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(B)))
    else:
        for b in range(B):
            fill(b)
    return out


def lengths(config_id, B, lo, hi):
    """Per-sequence valid KV lengths, integer-uniform on [lo, hi] inclusive."""
    g = torch.Generator("cpu").manual_seed(slice_seed(config_id, TENSOR_LENS, 0))
    return torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def make_inputs(config_id, *, B=None, Hq=None, Hkv=None, Nq=None, Nk=None, d=None,
                dtype=None, mult=None, len_lo=None, len_hi=None, padded=None):
    """CPU tensors (q, k, v, kv_seqlens-or-None) for a config.

    Keyword overrides shrink or reshape a config (for parity tests at sizes the
    oracle finishes quickly) while keeping its seeds and value distribution.
    """
    c = dict(CONFIGS[config_id])
    for key, val in dict(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d, dtype=dtype, mult=mult,
                         len_lo=len_lo, len_hi=len_hi, padded=padded).items():
        if val is not None:
            c[key] = val
    q = randn_tensor(config_id, TENSOR_Q, c["B"], c["Hq"], c["Nq"], c["d"], c["mult"], c["dtype"])
    k = randn_tensor(config_id, TENSOR_K, c["B"], c["Hkv"], c["Nk"], c["d"], c["mult"], c["dtype"])
    v = randn_tensor(config_id, TENSOR_V, c["B"], c["Hkv"], c["Nk"], c["d"], c["mult"], c["dtype"])
    lens = None
    if c.get("padded"):
        lo = c.get("len_lo", c["Nk"] // 2)
        hi = c.get("len_hi", c["Nk"])
        lens = lengths(config_id, c["B"], lo, hi)
    return q, k, v, lens


TENSOR_PACKED = 100  # packed-layout tensors use tensor ids 100 + (q, k, v)


def cumulative(lens):
    """int32 offsets [0, l0, l0 + l1, ...] of packed sequences."""
    out = torch.zeros(len(lens) + 1, dtype=torch.int32)
    if len(lens):
        out[1:] = torch.cumsum(torch.as_tensor(list(lens), dtype=torch.int64), 0).to(torch.int32)
    return out


def make_packed(config_id, lens_q, lens_k, Hq, Hkv, d, mult=1.0, dtype="bf16"):
    """Packed variable-length inputs: q [Hq, total_q, d], k, v [Hkv, total_k, d]
    (sequence b's rows drawn from their own seeded generator, then concatenated
    along the token axis) and the int32 offsets cu_q, cu_k [B + 1]."""
    tdt = _TORCH_DTYPE[dtype]

    def cat(tensor_id, H, lens):
        parts = [_slice(config_id, TENSOR_PACKED + tensor_id, b, (H, int(L), d), mult, tdt)
                 for b, L in enumerate(lens)]
        return torch.cat(parts, dim=1) if parts else torch.empty((H, 0, d), dtype=tdt)

    q = cat(TENSOR_Q, Hq, lens_q)
    k = cat(TENSOR_K, Hkv, lens_k)
    v = cat(TENSOR_V, Hkv, lens_k)
    return q, k, v, cumulative(lens_q), cumulative(lens_k)


FP8_DTYPES = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


def quantize_fp8(x, fmt):
    """Per-tensor FP8 quantisation of a float tensor: descale = amax / (largest
    finite code), codes = x / descale rounded to nearest-even in the format.
    Returns (codes as a torch float8 tensor, descale as a Python float holding
    a float32 value); the real input the codes stand for is descale * codes."""
    x = x.to(torch.float32)
    amax = float(x.abs().max()) if x.numel() else 0.0
    descale = float(torch.tensor(amax / FP8_MAX[fmt] if amax > 0 else 1.0, dtype=torch.float32))
    return (x / descale).to(FP8_DTYPES[fmt]), descale


def make_fp8_inputs(config_id, fmt, **overrides):
    """FP8 versions of a config's q, k, v: the config's float32 draws (before
    any bf16 rounding), each quantised per tensor.  Returns
    (q, k, v, kv_seqlens, (q_descale, k_descale, v_descale))."""
    q, k, v, lens = make_inputs(config_id, dtype="f32", **overrides)
    (qc, qs), (kc, ks), (vc, vs) = (quantize_fp8(t, fmt) for t in (q, k, v))
    return qc, kc, vc, lens, (qs, ks, vs)


def make_dout(config_id, **overrides):
    """Seeded upstream gradient dL/dO shaped like a config's q (same value
    distribution as q), for the backward pass."""
    c = dict(CONFIGS[config_id])
    c.update({k: v for k, v in overrides.items() if v is not None})
    return randn_tensor(config_id, TENSOR_DOUT, c["B"], c["Hq"], c["Nq"], c["d"], c["mult"], c["dtype"])
