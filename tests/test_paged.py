"""GPU parity of fa_decode_paged (split-KV decode over a paged KV cache).

A contiguous cache is scattered into a shuffled page pool; the paged decode
must then (1) agree with the oracle on the gathered keys at the decode bar
(bf16: max|dO| <= 1e-2, max|dLSE| <= 1e-3) and (2) be bit-identical to
fa_decode on the contiguous cache, since the same keys arrive in the same
order and tiles.
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
from fa_testutil import compare, dev, log


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * scale).to(torch.bfloat16)


def make_paged(k, v, page_size, seed, spare=3):
    """Scatter contiguous k, v [B, Hkv, Nk, d] (Nk a multiple of page_size) into a
    shuffled pool with `spare` unused pages filled with NaN."""
    B, Hkv, Nk, d = k.shape
    max_pages = Nk // page_size
    n_pages = B * max_pages + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g)[:B * max_pages].reshape(B, max_pages).to(torch.int32)
    kp = torch.full((n_pages, Hkv, page_size, d), float("nan"), dtype=torch.bfloat16)
    vp = kp.clone()
    src_k = k.reshape(B, Hkv, max_pages, page_size, d).permute(0, 2, 1, 3, 4)
    src_v = v.reshape(B, Hkv, max_pages, page_size, d).permute(0, 2, 1, 3, 4)
    kp[perm.long().reshape(-1)] = src_k.reshape(-1, Hkv, page_size, d)
    vp[perm.long().reshape(-1)] = src_v.reshape(-1, Hkv, page_size, d)
    return kp, vp, perm


CASES = [  # B, Hq, Hkv, Nk, d, page_size, lens, splits
    (3, 8, 2, 2048, 128, 16, [2048, 1000, 0], 16),
    (2, 4, 4, 1024, 128, 128, [1024, 129], 4),
    (2, 32, 8, 768, 128, 256, [700, 768], 3),
    (3, 8, 1, 512, 64, 64, [512, 1, 257], 16),
    (1, 2, 2, 96, 128, 1, [95], 1),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_H{c[1]}x{c[2]}_Nk{c[3]}_d{c[4]}_page{c[5]}_S{c[7]}")
def test_paged_decode(case):
    B, Hq, Hkv, Nk, d, page, lens, S = case
    seed = Nk + page + d
    q, k, v = rnd((B, Hq, 1, d), seed), rnd((B, Hkv, Nk, d), seed + 1), rnd((B, Hkv, Nk, d), seed + 2)
    kp, vp, table = make_paged(k, v, page, seed + 3)
    # entries past a sequence's length are never read: poison them
    for b, L in enumerate(lens):
        first_unused = (L + page - 1) // page
        table[b, first_unused:] = -12345
    lt = torch.tensor(lens, dtype=torch.int32)
    log(f"  fa_decode_paged B={B} Hq={Hq} Hkv={Hkv} Nk={Nk} d={d} page={page} lens={lens} S={S}")
    qd = q.to(dev())
    o, lse = fa.fa_decode_paged(qd, kp.to(dev()), vp.to(dev()), table.to(dev()), lt.to(dev()), num_splits=S)
    o_c, lse_c = fa.fa_decode(qd, k.to(dev()), v.to(dev()), kv_seqlens=lt.to(dev()), num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), o_c.cpu()) and torch.equal(lse.cpu(), lse_c.cpu()), "paged != contiguous"
    kc = oracle.paged_to_contiguous(kp, table.clamp(min=0), lt, page)
    vc = oracle.paged_to_contiguous(vp, table.clamp(min=0), lt, page)
    O_ref, L_ref = oracle.attention_ref(q, np.nan_to_num(kc), np.nan_to_num(vc), kv_seqlens=lt)
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, torch.bfloat16, f"paged page={page}")


@pytest.mark.gpu
@pytest.mark.slow
def test_paged_decode_full_size():
    """The split-KV decode workload (B=64, Hq=32, Hkv=8, Nk=32768, d=128, 16
    splits) with 16-key pages: bit-identical to the contiguous decode."""
    from exact_tiled_attention_08_amd import inputs
    q, k, v, _ = inputs.make_inputs(5)
    kp, vp, table = make_paged(k, v, 16, 99, spare=0)
    lt = torch.full((64,), 32768, dtype=torch.int32)
    qd = q.to(dev())
    o, lse = fa.fa_decode_paged(qd, kp.to(dev()), vp.to(dev()), table.to(dev()), lt.to(dev()), num_splits=16)
    del kp, vp
    o_c, lse_c = fa.fa_decode(qd, k.to(dev()), v.to(dev()), num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), o_c.cpu()) and torch.equal(lse.cpu(), lse_c.cpu())
    log("  full-size paged decode bit-identical to contiguous")
