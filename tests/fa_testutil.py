"""Shared helpers for the GPU parity tests: run the HIP path, run the oracle,
compare element by element at the stated tolerances."""
import sys

import numpy as np
import torch

import exact_tiled_attention_08_amd as fa
import oracle

# Tolerances on max |O - O_ref| and max |LSE - LSE_ref|.
TOL = {torch.bfloat16: (1e-2, 1e-3), torch.float32: (1e-5, 1e-5)}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(*ts):
    return [None if t is None else t.to(dev()).contiguous() for t in ts]


def run_fwd(q, k, v, causal=False, lens=None, scale=None):
    log(f"  fa_fwd q{tuple(q.shape)} k{tuple(k.shape)} {q.dtype} causal={causal} "
        f"lens={'none' if lens is None else lens.tolist()[:8]}")
    qd, kd, vd, ld = to_dev(q, k, v, lens)
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, kv_seqlens=ld, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def compare(o, lse, O_ref, L_ref, dtype, what="", o_tol=None, l_tol=None):
    """Element-wise check of GPU (o, lse) against oracle (O_ref, L_ref)."""
    to, tl = TOL[dtype]
    to = o_tol or to
    tl = l_tol or tl
    o64 = o.to(torch.float64).numpy()
    l64 = lse.to(torch.float64).numpy()
    sel = ~np.isnan(L_ref)  # rows the oracle computed
    assert not np.isnan(o64[sel]).any() and not np.isnan(l64[sel]).any(), f"{what}: NaN in output"
    ninf_ref = np.isneginf(L_ref) & sel
    assert np.array_equal(np.isneginf(l64) & sel, ninf_ref), f"{what}: -inf LSE pattern differs"
    assert np.all(o64[ninf_ref] == 0.0), f"{what}: rows without keys must be 0"
    fin = sel & ~ninf_ref
    do = np.abs(o64 - O_ref)
    do[~fin] = 0.0
    with np.errstate(invalid="ignore"):  # -inf - -inf on rows outside `fin`
        dl = np.abs(np.where(fin, l64 - L_ref, 0.0))
    eo, el = float(do.max(initial=0.0)), float(dl.max(initial=0.0))
    if eo > 0:
        idx = np.unravel_index(int(np.argmax(do)), do.shape)
        ref = O_ref[idx]
        irr = abs(float(torch.tensor(ref).to(dtype).double()) - ref)
        log(f"  {what}: max|dO|={eo:.3e} at {idx} (ref {ref:+.4f}, output rounding {irr:.1e}); "
            f"max|dLSE|={el:.3e}")
    assert eo <= to, f"{what}: max|O-O_ref| = {eo:.3e} > {to}"
    assert el <= tl, f"{what}: max|LSE-LSE_ref| = {el:.3e} > {tl}"
    return eo, el


def check_fwd(q, k, v, causal=False, lens=None, scale=None, rows=None, heads=None, what=""):
    o, lse = run_fwd(q, k, v, causal, lens, scale)
    O_ref, L_ref = oracle.attention_ref(q, k, v, causal=causal, kv_seqlens=lens, scale=scale,
                                        rows=rows, heads=heads)
    return compare(o, lse, O_ref, L_ref, q.dtype, what or f"fwd causal={causal}")
