"""Large-size edge cases: tensors with more than 2^31 elements (row offsets
need 64-bit arithmetic) and a decode over millions of keys with the largest
split count.  The work is kept small with padding lengths; the oracle sees
slices of the inputs that reproduce the same visible keys."""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle

from fa_testutil import compare, log

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def test_prefill_offsets_past_2_31_elements():
    """B=1, Hq=24, Hkv=8, N=2^20, d=128 causal: Q and O hold 3.2e9 elements
    each (a row offset (head * N + row) * d passes 2^31 from head 16 on); K
    and V 1.1e9.  Keys are limited to the first 1000 by kv_seqlens."""
    dev = torch.device("cuda:0")
    B, Hq, Hkv, N, d, L = 1, 24, 8, 1 << 20, 128, 1000
    assert B * Hq * N * d > 2 ** 31
    g = torch.Generator(device=dev).manual_seed(2031)
    q = torch.randn(B, Hq, N, d, device=dev, dtype=torch.bfloat16, generator=g)
    k = torch.randn(B, Hkv, N, d, device=dev, dtype=torch.bfloat16, generator=g)
    v = torch.randn(B, Hkv, N, d, device=dev, dtype=torch.bfloat16, generator=g)
    lens = torch.tensor([L], dtype=torch.int32, device=dev)
    log(f"  fa_fwd q{tuple(q.shape)} k{tuple(k.shape)} causal, kv_seqlens=[{L}]")
    o, lse = fa.fa_fwd(q, k, v, causal=True, kv_seqlens=lens)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    far = np.unique(np.concatenate([[L, L + 1, 4095, 4096, N // 2, N - 2, N - 1], rng.integers(L, N, 24)]))
    for hq in (0, 5, 16, Hq - 1):
        hk = hq // (Hq // Hkv)
        kh = k[:, hk:hk + 1, :L].cpu()
        vh = v[:, hk:hk + 1, :L].cpu()
        # rows 0 .. L-1: the same causal problem as a self-attention over L keys
        qh = q[:, hq:hq + 1, :L].cpu()
        O_ref, L_ref = oracle.attention_ref(qh, kh, vh, causal=True)
        compare(o[:, hq:hq + 1, :L].cpu(), lse[:, hq:hq + 1, :L].cpu(), O_ref, L_ref, torch.bfloat16,
                f"rows 0..{L - 1}, head {hq}")
        # rows past L see every valid key
        idx = torch.as_tensor(far, device=dev)
        qf = q[:, hq:hq + 1].index_select(2, idx).cpu()
        O_ref, L_ref = oracle.attention_ref(qf, kh, vh, causal=False)
        compare(o[:, hq:hq + 1].index_select(2, idx).cpu(), lse[:, hq:hq + 1].index_select(2, idx).cpu(),
                O_ref, L_ref, torch.bfloat16, f"{len(far)} rows past {L}, head {hq}")
    del q, k, v, o, lse


@pytest.mark.parametrize("S", [256, 7])
def test_decode_four_million_keys(S):
    """B=1, Hq=8, Hkv=1, Nk=2^22 - 77 valid keys of 2^22, d=128, bf16, with
    the largest split count and an odd one."""
    dev = torch.device("cuda:0")
    B, Hq, Hkv, Nk, d = 1, 8, 1, 1 << 22, 128
    g = torch.Generator(device=dev).manual_seed(4194 + S)
    q = torch.randn(B, Hq, 1, d, device=dev, dtype=torch.bfloat16, generator=g)
    k = torch.randn(B, Hkv, Nk, d, device=dev, dtype=torch.bfloat16, generator=g)
    v = torch.randn(B, Hkv, Nk, d, device=dev, dtype=torch.bfloat16, generator=g)
    lens = torch.tensor([Nk - 77], dtype=torch.int32)
    log(f"  fa_decode k{tuple(k.shape)} S={S} kv_seqlens={lens.tolist()}")
    o, lse = fa.fa_decode(q, k, v, kv_seqlens=lens.to(dev), num_splits=S)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_ref(q.cpu(), k.cpu(), v.cpu(), kv_seqlens=lens)
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, torch.bfloat16, f"decode Nk=2^22 S={S}")
