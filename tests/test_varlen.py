"""GPU parity of fa_fwd_varlen (packed variable-length and chunked prefill).

Sequences are packed along the token axis of every head, q [Hq, total_q, d],
k/v [Hkv, total_k, d], delimited by int32 cumulative offsets; each sequence
attends to its own keys with the causal mask aligned bottom-right per
sequence.  Checks:
  * element-wise parity with the oracle at the forward bar (bf16: max|dO| <=
    1e-2, max|dLSE| <= 1e-3; f32: 1e-5 for both), including empty sequences,
    sequences with no keys, chunks shorter and longer than their key range and
    lengths that are not multiples of any tile;
  * bit-identity with fa_fwd on the [B, H, N, d] layout when every sequence has
    the same lengths (the same rows meet the same tiles);
  * chunked prefill: query chunks that start on a multiple of the 256-row work
    tile, each against the keys up to its end, reproduce the rows of one
    causal call bit for bit;
  * rows outside every sequence are never written.
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
from exact_tiled_attention_08_amd import inputs
from fa_testutil import compare, dev, log

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def run_varlen(q, k, v, cu_q, cu_k, causal, max_q=None, scale=None, fill=None):
    lq = (cu_q[1:] - cu_q[:-1]).tolist()
    max_q = max(lq, default=0) if max_q is None else max_q
    log(f"  fa_fwd_varlen q{tuple(q.shape)} k{tuple(k.shape)} {q.dtype} causal={causal} "
        f"lq={lq[:8]} lk={(cu_k[1:] - cu_k[:-1]).tolist()[:8]} max_q={max_q}")
    qd, kd, vd, cqd, ckd = (t.to(dev()).contiguous() for t in (q, k, v, cu_q, cu_k))
    out = lse = None
    if fill is not None:
        out = torch.full(q.shape, fill, dtype=q.dtype, device=dev())
        lse = torch.full(q.shape[:2], fill, dtype=torch.float32, device=dev())
    o, l = fa.fa_fwd_varlen(qd, kd, vd, cqd, ckd, max_q, causal=causal, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), l.cpu()


CASES = [  # Hq, Hkv, d, dtype, causal, lens_q, lens_k
    (4, 4, 128, "bf16", True, [300, 1, 0, 257, 64, 129], [300, 1, 0, 257, 64, 129]),        # self-attention
    (4, 2, 128, "bf16", True, [64, 100, 1, 256, 300], [1000, 100, 513, 300, 300]),          # chunks vs cache
    (2, 2, 128, "bf16", True, [200, 33, 5], [50, 0, 77]),                                   # Lq > Lk, no keys
    (8, 2, 128, "bf16", False, [77, 513, 3], [129, 64, 1000]),                              # GQA 4:1
    (4, 1, 64, "bf16", True, [130, 1, 250, 0, 77], [130, 700, 250, 5, 40]),
    (2, 2, 64, "bf16", False, [33, 128], [1, 300]),
    (2, 1, 64, "f32", True, [130, 7, 300], [200, 7, 100]),
    (2, 2, 128, "f32", False, [40, 129], [333, 64]),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: "H{}x{}_d{}_{}_{}_B{}".format(
    c[0], c[1], c[2], c[3], "causal" if c[4] else "full", len(c[5])))
def test_varlen_parity(case):
    Hq, Hkv, d, dt, causal, lq, lk = case
    q, k, v, cu_q, cu_k = inputs.make_packed(4, lq, lk, Hq, Hkv, d, dtype=dt)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, causal)
    O_ref, L_ref = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, causal=causal)
    compare(o, lse, O_ref, L_ref, DT[dt], f"varlen {case}")


@pytest.mark.gpu
def test_varlen_scale_and_oversized_grid():
    """A non-default scale, and max_seqlen_q above the longest sequence (the
    extra work-groups find no rows and exit)."""
    lq, lk = [90, 300], [90, 310]
    q, k, v, cu_q, cu_k = inputs.make_packed(4, lq, lk, 4, 2, 128)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, True, max_q=2000, scale=0.3)
    O_ref, L_ref = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, causal=True, scale=0.3)
    compare(o, lse, O_ref, L_ref, torch.bfloat16, "varlen scale=0.3 max_q=2000")


@pytest.mark.gpu
def test_varlen_rows_outside_sequences_untouched():
    """Offsets that leave gaps (rows 0..9 and 60..69 belong to no sequence):
    those rows keep what the caller put there."""
    Hq, d = 2, 128
    q = inputs.make_packed(4, [70], [80], Hq, 2, d)[0]
    _, k, v, _, _ = inputs.make_packed(4, [1], [80], Hq, 2, d)
    cu_q = torch.tensor([10, 35, 60], dtype=torch.int32)
    cu_k = torch.tensor([0, 30, 80], dtype=torch.int32)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, True, max_q=25, fill=7.0)
    for r in list(range(10)) + list(range(60, 70)):
        assert torch.all(o[:, r] == 7.0) and torch.all(lse[:, r] == 7.0), f"row {r} was written"
    O_ref, L_ref = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, causal=True)
    compare(o, lse, O_ref, L_ref, torch.bfloat16, "varlen with gaps")


@pytest.mark.gpu
@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, True)])
def test_varlen_equals_batched_layout_bitwise(d, causal):
    B, Hq, Hkv, nq, nk = 3, 4, 2, 300, 420
    qb, kb, vb, _ = inputs.make_inputs(2, B=B, Hq=Hq, Hkv=Hkv, Nq=nq, Nk=nk, d=d, padded=False)
    ob, lb = fa.fa_fwd(qb.to(dev()), kb.to(dev()), vb.to(dev()), causal=causal)
    pack = lambda x: torch.cat(list(x), dim=1).contiguous()  # noqa: E731  [B,H,N,d] -> [H,B*N,d]
    cu_q = torch.arange(B + 1, dtype=torch.int32) * nq
    cu_k = torch.arange(B + 1, dtype=torch.int32) * nk
    o, lse = run_varlen(pack(qb), pack(kb), pack(vb), cu_q, cu_k, causal)
    assert torch.equal(o, pack(ob.cpu())), "packed output differs from the batched layout"
    assert torch.equal(lse, torch.cat(list(lb.cpu()), dim=1)), "packed LSE differs from the batched layout"


@pytest.mark.gpu
@pytest.mark.parametrize("d", [128, 64])
def test_chunked_prefill_matches_one_shot(d):
    """One causal sequence of 1300 tokens, queried in chunks [0,512), [512,768),
    [768,1300), each chunk against the keys up to its end (the KV cache plus
    the chunk itself), equals the one-shot causal call row for row, bit for bit."""
    H, L = 4, 1300
    q1, k1, v1, _ = inputs.make_inputs(2, B=1, Hq=H, Hkv=H, Nq=L, Nk=L, d=d, padded=False)
    o_full, l_full = fa.fa_fwd(q1.to(dev()), k1.to(dev()), v1.to(dev()), causal=True)
    ends = [512, 768, 1300]
    kp = torch.cat([k1[0, :, :e] for e in ends], dim=1)
    vp = torch.cat([v1[0, :, :e] for e in ends], dim=1)
    cu_q = torch.tensor([0] + ends, dtype=torch.int32)
    cu_k = inputs.cumulative(ends)
    o, lse = run_varlen(q1[0].contiguous(), kp, vp, cu_q, cu_k, True)
    assert torch.equal(o, o_full[0].cpu()), "chunked prefill output differs from the one-shot call"
    assert torch.equal(lse, l_full[0].cpu()), "chunked prefill LSE differs from the one-shot call"


@pytest.mark.gpu
@pytest.mark.slow
def test_varlen_full_size_sampled():
    """The packed GQA workload: 4 sequences with the padded workload's lengths
    (U{2048..4096}), Hq=32, Hkv=8, d=128, causal self-attention; heads 0 and 31
    of every sequence checked against the oracle, every row."""
    lens = inputs.lengths(4, 4, 2048, 4096).tolist()
    q, k, v, cu_q, cu_k = inputs.make_packed(4, lens, lens, 32, 8, 128)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, True)
    for h in (0, 31):
        hk = h // 4
        O_ref, L_ref = oracle.attention_varlen_ref(q[h:h + 1], k[hk:hk + 1], v[hk:hk + 1], cu_q, cu_k, causal=True)
        compare(o[h:h + 1], lse[h:h + 1], O_ref, L_ref, torch.bfloat16, f"varlen full size head {h}")


@pytest.mark.gpu
@pytest.mark.slow
@pytest.mark.parametrize("chunked", [False, True])
def test_varlen_d64_causal_on_a_large_grid(chunked):
    """d = 64 under a causal mask with enough heads that the packed grid has
    two 256-row work-groups per CU (the ping-pong kernel; the small d = 64
    cases above take the 128-row kernel): Hq=64, Hkv=16, four sequences,
    self-attention or 300-query chunks against their keys; four heads compared
    with the oracle, every row."""
    lens_k = [1500, 2048, 901, 1777]
    lens_q = [300, 300, 300, 300] if chunked else lens_k
    q, k, v, cu_q, cu_k = inputs.make_packed(2, lens_q, lens_k, 64, 16, 64)
    o, lse = run_varlen(q, k, v, cu_q, cu_k, True)
    for h in (0, 17, 42, 63):
        hk = h // 4
        O_ref, L_ref = oracle.attention_varlen_ref(q[h:h + 1], k[hk:hk + 1], v[hk:hk + 1], cu_q, cu_k, causal=True)
        compare(o[h:h + 1], lse[h:h + 1], O_ref, L_ref, torch.bfloat16, f"varlen d=64 large grid head {h}")
