"""fa_decode_noalloc (partials in the library's static per-GPU scratch) against
fa_decode (partials in a caller workspace): two calls in a row through the C
ABI, the second with a smaller input, each bit-identical to fa_decode (the two
share their kernels) and within the decode tolerances of the oracle."""
import ctypes

import pytest
import torch

import exact_tiled_attention_08_amd as fa
from exact_tiled_attention_08_amd import _lib, inputs
import oracle

from fa_testutil import compare, log

pytestmark = pytest.mark.gpu


def _noalloc_via_cabi(q, k, v, lens, S):
    B, Hq, _, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, 1), float("nan"), dtype=torch.float32, device=q.device)
    lib = _lib.load()
    st = lib.fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                               Nk, d, ctypes.c_float(fa.default_scale(d)),
                               None if lens is None else lens.data_ptr(), S, _lib.FA_BF16,
                               torch.cuda.current_stream().cuda_stream)
    _lib.check(st)
    return o, lse


@pytest.mark.parametrize("seed", [0])
def test_noalloc_matches_workspace_decode_twice(seed):
    dev = torch.device("cuda:0")
    cases = [  # (B, Hq, Hkv, Nk, lens, S): the second call is smaller
        (8, 32, 8, 20000, [20000, 1, 0, 129, 4096, 19999, 7777, 128], 16),
        (3, 8, 2, 700, [700, 5, 300], 4),
    ]
    for B, Hq, Hkv, Nk, lens, S in cases:
        log(f"  noalloc decode B={B} Hq={Hq} Hkv={Hkv} Nk={Nk} S={S}")
        q, k, v, _ = inputs.make_inputs(5, B=B, Hq=Hq, Hkv=Hkv, Nk=Nk)
        lt = torch.tensor(lens, dtype=torch.int32)
        qd, kd, vd, ld = q.to(dev), k.to(dev), v.to(dev), lt.to(dev)
        o_ref, l_ref = fa.fa_decode(qd, kd, vd, kv_seqlens=ld, num_splits=S)
        o, l = _noalloc_via_cabi(qd, kd, vd, ld, S)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "O differs from fa_decode"
        assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32)), "LSE differs from fa_decode"
        O, L = oracle.attention_ref(q, k, v, kv_seqlens=lt)
        compare(o.cpu(), l.cpu(), O, L, torch.bfloat16, f"noalloc B={B} Nk={Nk}")
