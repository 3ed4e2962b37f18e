"""FP8 inputs for the fp64 oracle -- TEST INFRASTRUCTURE, not product code.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module; it shares no code with the GPU path.

The pages mention FP8 attention (FlashAttention-3 on H100) only for its
throughput (2026 explainer, section "二代和三代"); they fix neither the
formats nor the scaling.  The plainest reading, used here: Q, K and V arrive as
8-bit floating-point codes in one of the two OCP FP8 formats, each tensor
with one float32 "descale" factor, so the real input is descale * value(code).
What the attention then computes is unchanged: the oracle decodes the codes
exactly to fp64, multiplies by the descale, and applies the definition
(attention_ref).

Code layouts (OCP 8-bit floating point, sign | exponent | mantissa):
  E4M3 ("fn"): 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
      is subnormal (value m/8 * 2^-6); no infinities; S.1111.111 is NaN, so
      the largest finite value is 1.75 * 2^8 = 448.
  E5M2: 5 exponent bits (bias 15), 2 mantissa bits; exponent field 0 is
      subnormal (m/4 * 2^-14); exponent field 31 holds +-inf (m = 0) and NaN.
"""
import numpy as np

from .attention import attention_ref, to_f64

E4M3, E5M2 = "e4m3", "e5m2"
_FIELDS = {E4M3: (4, 3, 7), E5M2: (5, 2, 15)}  # exponent bits, mantissa bits, bias


def decode_fp8(codes, fmt):
    """Exact fp64 values of 8-bit codes (any integer array holding 0..255)."""
    if fmt not in _FIELDS:
        raise ValueError(f"unknown FP8 format {fmt!r}")
    ebits, mbits, bias = _FIELDS[fmt]
    c = np.asarray(to_f64(codes), dtype=np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = (c & ((1 << mbits) - 1)).astype(np.float64)
    frac = m / (1 << mbits)
    normal = sign * (1.0 + frac) * np.exp2(e.astype(np.float64) - bias)
    sub = sign * frac * np.exp2(1.0 - bias)
    out = np.where(e == 0, sub, normal)
    emax = (1 << ebits) - 1
    if fmt == E4M3:
        out = np.where((e == emax) & (m == (1 << mbits) - 1), np.nan, out)
    else:
        out = np.where(e == emax, np.where(m == 0, sign * np.inf, np.nan), out)
    return out


def attention_fp8_ref(q, k, v, fmt, q_descale, k_descale, v_descale, causal=False, kv_seqlens=None,
                      scale=None):
    """Exact attention on dequantised FP8 inputs, fp64.

    q [B, Hq, Nq, d], k, v [B, Hkv, Nk, d] hold FP8 codes of format `fmt`; the
    inputs are x = descale * value(code) with the descales as float32 numbers.
    Returns (O, LSE) of attention_ref on those inputs.
    """
    deq = lambda x, s: decode_fp8(x, fmt) * float(np.float32(s))  # noqa: E731
    return attention_ref(deq(q, q_descale), deq(k, k_descale), deq(v, v_descale), causal=causal,
                         kv_seqlens=kv_seqlens, scale=scale)
