"""GPU parity of fa_fwd_fp8 (FP8 prefill forward, d = 128).

Q, K and V are per-tensor-quantised OCP FP8 codes (E4M3 or E5M2) with float32
descales; the oracle decodes the codes exactly, applies the descales and runs
the fp64 definition.  The GPU path keeps V exact in bf16 and rounds P to bf16
before P.V, as the bf16 path does; S comes from the FP8 matrix cores, whose
internal sums carry an error of up to ~2^-15 of sum_d |q_d k_d| (measured),
i.e. at most ~2e-4 in a scaled score for these workloads' magnitudes.  The
bf16 bars therefore apply unchanged: max|dO| <= 1e-2, max|dLSE| <= 1e-3,
-inf rows exact.  (Scores of magnitude ~1e4 would move the LSE by ~1e-1: the
bar holds for inputs whose real values have the workloads' magnitudes, which
per-tensor scaling preserves.)
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
from exact_tiled_attention_08_amd import inputs
from fa_testutil import compare, dev, log

FMT = {"e4m3": oracle.E4M3, "e5m2": oracle.E5M2}


def run_fp8(q, k, v, ds, causal, lens, scale=None):
    log(f"  fa_fwd_fp8 q{tuple(q.shape)} k{tuple(k.shape)} {q.dtype} causal={causal} descales={ds} "
        f"lens={'none' if lens is None else lens.tolist()[:8]}")
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    ld = None if lens is None else lens.to(dev())
    o, lse = fa.fa_fwd_fp8(qd, kd, vd, *ds, causal=causal, kv_seqlens=ld, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def codes(t):
    return t.view(torch.uint8)


CASES = [  # B, Hq, Hkv, Nq, Nk, causal, lens, fmt
    (1, 2, 2, 300, 300, True, None, "e4m3"),
    (2, 4, 2, 257, 513, True, [513, 100], "e4m3"),
    (1, 4, 1, 130, 77, False, None, "e5m2"),
    (2, 2, 2, 64, 64, False, [0, 64], "e4m3"),
    (1, 2, 2, 100, 40, True, None, "e5m2"),          # rows with no visible key
    (1, 1, 1, 1, 1, False, None, "e4m3"),
    (1, 8, 2, 600, 600, True, [555], "e5m2"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_H{}x{}_{}x{}_{}_{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full", "pad" if c[6] else "nopad", c[7]))
def test_fp8_parity(case):
    B, Hq, Hkv, Nq, Nk, causal, lens, fmt = case
    q, k, v, _, ds = inputs.make_fp8_inputs(4, fmt, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, padded=False)
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32)
    o, lse = run_fp8(q, k, v, ds, causal, lt)
    O_ref, L_ref = oracle.attention_fp8_ref(codes(q), codes(k), codes(v), FMT[fmt], *ds, causal=causal,
                                            kv_seqlens=lt)
    compare(o, lse, O_ref, L_ref, torch.bfloat16, f"fp8 {case}")


@pytest.mark.gpu
def test_fp8_descales_and_scale():
    """Descales far from 1 (2^-6, 4, 2^-5) with a non-default softmax scale: the
    real inputs keep the workload's magnitudes and the codes absorb the
    descales, so each descale must be applied where it belongs."""
    x = inputs.make_inputs(3, B=1, Hq=2, Hkv=2, Nq=200, Nk=333, dtype="f32", padded=False)[:3]
    ds = (2.0 ** -6, 4.0, 2.0 ** -5)
    q, k, v = ((t / d).to(torch.float8_e4m3fn) for t, d in zip(x, ds))
    o, lse = run_fp8(q, k, v, ds, True, None, scale=0.7)
    O_ref, L_ref = oracle.attention_fp8_ref(codes(q), codes(k), codes(v), oracle.E4M3, *ds, causal=True, scale=0.7)
    compare(o, lse, O_ref, L_ref, torch.bfloat16, "fp8 descales")


@pytest.mark.gpu
def test_fp8_nan_past_length_is_never_read():
    """NaN codes planted in K and V rows past each sequence's length must not
    reach the output."""
    q, k, v, _, ds = inputs.make_fp8_inputs(4, "e4m3", B=2, Hq=4, Hkv=2, Nq=150, Nk=300, padded=False)
    lens = torch.tensor([131, 300], dtype=torch.int32)
    kc, vc = codes(k).clone(), codes(v).clone()
    kc[0, :, 131:] = 0x7F
    vc[0, :, 131:] = 0x7F  # NaN in E4M3
    kn, vn = kc.view(torch.float8_e4m3fn), vc.view(torch.float8_e4m3fn)
    o, lse = run_fp8(q, kn, vn, ds, True, lens)
    # the oracle sees the clean codes: keys past a length take no part by definition
    O_ref, L_ref = oracle.attention_fp8_ref(codes(q), codes(k), codes(v), oracle.E4M3, *ds, causal=True,
                                            kv_seqlens=lens)
    compare(o, lse, O_ref, L_ref, torch.bfloat16, "fp8 NaN past length")


@pytest.mark.gpu
@pytest.mark.slow
def test_fp8_full_size_sampled():
    """The long-context shape (B=1, H=32, N=8192, d=128, causal) in E4M3, run in
    full; rows of heads 0 and 31 sampled across the sequence."""
    q, k, v, _, ds = inputs.make_fp8_inputs(3, "e4m3")
    o, lse = run_fp8(q, k, v, ds, True, None)
    rows = np.unique(np.concatenate([np.arange(0, 8192, 97), [0, 1, 255, 256, 4095, 8190, 8191]]))
    deq = [oracle.decode_fp8(codes(t).numpy(), oracle.E4M3) * np.float32(s) for t, s in zip((q, k, v), ds)]
    O_ref, L_ref = oracle.attention_ref(*deq, causal=True, heads=[(0, 0), (0, 31)], rows=rows)
    compare(o, lse, O_ref, L_ref, torch.bfloat16, "fp8 N=8192 sampled")
