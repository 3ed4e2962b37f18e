"""attention(): the autograd wrapper over fa_fwd and fa_bwd.

The wrapper only marshals arguments, so its forward output must equal fa_fwd's
and the gradients autograd delivers must equal fa_bwd's, bit for bit, for
causal and padded GQA inputs; gradients of an upstream expression must chain
through it.  Numerical parity of fa_fwd and fa_bwd with the oracle is tested
on their own (test_parity.py, test_bwd.py).  On the CPU the wrapper must
refuse CPU tensors and non-bf16 inputs rather than fall back to anything.
"""
import pytest
import torch

import exact_tiled_attention_08_amd as fa
from fa_testutil import dev, log


def rnd(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * 0.5).to(torch.bfloat16)


def test_attention_refuses_cpu_and_non_bf16():
    x = rnd((1, 2, 8, 64), 0)
    with pytest.raises(ValueError):
        fa.attention(x, x, x)
    with pytest.raises(ValueError):
        fa.attention(x.float(), x.float(), x.float())


@pytest.mark.gpu
@pytest.mark.parametrize("causal,padded", [(True, False), (False, True), (True, True)])
def test_attention_autograd_matches_direct_calls(causal, padded):
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 300, 333, 128
    q, k, v, do = (rnd(s, i).to(dev()) for i, s in enumerate(
        [(B, Hq, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d), (B, Hq, Nq, d)]))
    lens = torch.tensor([333, 150], dtype=torch.int32, device=dev()) if padded else None
    log(f"  attention causal={causal} padded={padded}")
    qa, ka, va = (t.clone().requires_grad_() for t in (q, k, v))
    o = fa.attention(qa, ka, va, causal=causal, kv_seqlens=lens)
    o.backward(do)
    o_ref, lse_ref = fa.fa_fwd(q, k, v, causal=causal, kv_seqlens=lens)
    dq, dk, dv = fa.fa_bwd(q, k, v, o_ref, lse_ref, do, causal=causal, kv_seqlens=lens)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    assert torch.equal(qa.grad, dq) and torch.equal(ka.grad, dk) and torch.equal(va.grad, dv)


@pytest.mark.gpu
def test_attention_chains_with_upstream_ops():
    """loss = sum(attention(2 q, k, v) * w): dq must be 2 * fa_bwd's dq for dO = w
    (the factor 2 is exact in bf16), and dk, dv fa_bwd's."""
    B, H, N, d = 1, 4, 200, 64
    q, k, v, w = (rnd((B, H, N, d), 10 + i).to(dev()) for i in range(4))
    qa, ka, va = (t.clone().requires_grad_() for t in (q, k, v))
    o = fa.attention(qa * 2, ka, va, causal=True)
    (o.float() * w.float()).sum().backward()
    o_ref, lse_ref = fa.fa_fwd(q * 2, k, v, causal=True)
    dq, dk, dv = fa.fa_bwd(q * 2, k, v, o_ref, lse_ref, w, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(qa.grad, dq * 2)
    assert torch.equal(ka.grad, dk) and torch.equal(va.grad, dv)
