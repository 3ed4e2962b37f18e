"""GPU parity of fa_bwd (dQ, dK, dV) against the fp64 oracle.

Bar: for each of dQ, dK and dV, max |GPU - oracle| <= 1 % of that tensor's
largest oracle magnitude (at least 0.1 % of the largest of the three).  The
GPU path rounds P and dS to bf16 before their matrix-core products (relative
error <= 2^-9 each), sums in float32 and rounds
the outputs to bf16 (another 2^-9); the forward's O enters through
D = rowsum(dO * O) already rounded to bf16.  Gradients that are zero by
structure (dQ of a row that sees no key; dK, dV of a key that no query sees)
must be exactly zero.
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
from fa_testutil import dev, log

REL_TOL = 1e-2


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * scale).to(torch.bfloat16)


def run_bwd(q, k, v, do, causal, lens, scale=None):
    qd, kd, vd, dod = (t.to(dev()).contiguous() for t in (q, k, v, do))
    ld = None if lens is None else lens.to(dev())
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, kv_seqlens=ld, scale=scale)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=causal, kv_seqlens=ld, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def structural_zeros(q, k, v, causal, lens, scale=None):
    """Masks of gradients that are zero by structure: dQ rows of queries that see
    no key, dK / dV rows of keys that no query of their group sees."""
    P = oracle.attention_probs_ref(q, k, v, causal=causal, kv_seqlens=lens, scale=scale)
    B, Hq, Nq, Nk = P.shape
    Hkv = k.shape[1]
    row_empty = (P.sum(axis=-1) == 0.0)[..., None]
    key_unused = (P.reshape(B, Hkv, Hq // Hkv, Nq, Nk).sum(axis=(2, 3)) == 0.0)[..., None]
    d = q.shape[-1]
    return (np.broadcast_to(row_empty, (B, Hq, Nq, d)), np.broadcast_to(key_unused, (B, Hkv, Nk, d)),
            np.broadcast_to(key_unused, (B, Hkv, Nk, d)))


def compare_grads(got, ref, what, zeros):
    # A gradient that vanishes analytically (dQ, dK with a single key) is only
    # rounding noise in the oracle too, so each tensor's bar has a floor of
    # 0.1 % of the largest of the three gradients.
    floor = 0.1 * max(float(np.abs(r).max(initial=0.0)) for r in ref)
    for name, g, r, zero in zip(("dQ", "dK", "dV"), got, ref, zeros):
        g64 = g.to(torch.float64).numpy()
        assert np.isfinite(g64).all(), f"{what} {name}: non-finite values"
        if not np.all(g64[zero] == 0.0):
            bad = np.argwhere(zero & (g64 != 0.0))
            raise AssertionError(f"{what} {name}: {len(bad)} structurally zero entries are not, e.g. "
                                 f"{bad[:4].tolist()} = {[float(g64[tuple(i)]) for i in bad[:4]]}")
        scale = max(float(np.abs(r).max(initial=0.0)), floor)
        err = float(np.abs(g64 - r).max(initial=0.0))
        log(f"  {what} {name}: max|d|={err:.3e}  bar {REL_TOL} x {scale:.3e}  ({int(zero.sum())} structural zeros)")
        assert err <= REL_TOL * scale, f"{what} {name}: {err:.3e} > {REL_TOL} x {scale:.3e}"


CASES = [  # B, Hq, Hkv, Nq, Nk, d, causal, lens
    (1, 2, 2, 64, 64, 128, False, None),
    (1, 2, 2, 100, 100, 128, True, None),
    (2, 4, 2, 130, 77, 128, True, [77, 40]),
    (1, 2, 1, 77, 300, 64, True, None),
    (2, 2, 2, 257, 200, 64, False, [200, 1]),
    (1, 2, 2, 100, 40, 128, True, None),       # rows with no visible key (Nq > Nk, causal)
    (2, 2, 1, 33, 129, 128, False, [0, 129]),   # a sequence of length 0
    (1, 1, 1, 1, 1, 128, False, None),
    (1, 4, 1, 300, 300, 128, True, None),      # GQA group of 4, several key blocks
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_H{}x{}_{}x{}_d{}_{}_{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full", "pad" if c[7] else "nopad"))
def test_bwd_parity(case):
    B, Hq, Hkv, Nq, Nk, d, causal, lens = case
    seed = 7 * Nq + Nk + d
    q, k, v, do = rnd((B, Hq, Nq, d), seed), rnd((B, Hkv, Nk, d), seed + 1), rnd((B, Hkv, Nk, d), seed + 2), \
        rnd((B, Hq, Nq, d), seed + 3)
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32)
    got = run_bwd(q, k, v, do, causal, lt)
    ref = oracle.attention_bwd_ref(q, k, v, do, causal=causal, kv_seqlens=lt)
    compare_grads(got, ref, f"bwd {case}", structural_zeros(q, k, v, causal, lt))


@pytest.mark.gpu
def test_bwd_scale_argument():
    q, k, v, do = rnd((1, 2, 90, 64), 1), rnd((1, 2, 70, 64), 2), rnd((1, 2, 70, 64), 3), rnd((1, 2, 90, 64), 4)
    got = run_bwd(q, k, v, do, True, None, scale=0.3)
    ref = oracle.attention_bwd_ref(q, k, v, do, causal=True, scale=0.3)
    compare_grads(got, ref, "bwd scale=0.3", structural_zeros(q, k, v, True, None, 0.3))


@pytest.mark.gpu
@pytest.mark.slow
def test_bwd_full_size_sampled_heads():
    """N=8192 causal d=128 with 32 heads (the long-context workload), run in
    full; heads 0 and 31 checked against the oracle, every element."""
    B, H, N, d = 1, 32, 8192, 128
    q, k, v, do = (rnd((B, H, N, d), 100 + i, 0.5) for i in range(4))
    got = run_bwd(q, k, v, do, True, None)
    for h in (0, 31):
        sl = slice(h, h + 1)
        ref = oracle.attention_bwd_ref(q[:, sl], k[:, sl], v[:, sl], do[:, sl], causal=True)
        zeros = [np.zeros(r.shape, dtype=bool) for r in ref]  # every row and key is used
        compare_grads([g[:, sl] for g in got], ref, f"bwd N=8192 head {h}", zeros)
