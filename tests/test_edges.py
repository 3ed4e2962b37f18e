"""Edge cases of the GPU path against the oracle and closed forms: ragged and
tiny sizes, Nq != Nk under the causal mask, padding lengths at tile
boundaries, MHA / GQA / MQA, empty inputs, rows without keys, decode splits
that are empty, and cache rows past a sequence's length never being read."""
import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle

from fa_testutil import check_fwd, compare, log, to_dev

pytestmark = pytest.mark.gpu


def rnd(shape, dtype, seed, mult=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * mult).to(dtype)


def qkv(B, Hq, Hkv, Nq, Nk, d, dtype, seed=0):
    return (rnd((B, Hq, Nq, d), dtype, seed), rnd((B, Hkv, Nk, d), dtype, seed + 1),
            rnd((B, Hkv, Nk, d), dtype, seed + 2))


SIZES = [(1, 1), (17, 17), (63, 63), (64, 64), (65, 65), (127, 129), (129, 127), (300, 300),
         (1, 300), (300, 1), (5, 200), (200, 5)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk", SIZES)
def test_sizes_causal_and_not(nq, nk, d, dtype):
    q, k, v = qkv(2, 4, 2, nq, nk, d, dtype, seed=nq * 1000 + nk)
    for causal in (False, True):
        check_fwd(q, k, v, causal=causal, what=f"nq={nq} nk={nk} d={d} causal={causal}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2), (8, 1)], ids=["mha", "gqa", "mqa"])
def test_head_mappings(heads, dtype):
    q, k, v = qkv(2, heads[0], heads[1], 150, 150, 128, dtype, seed=11)
    check_fwd(q, k, v, causal=True, what=f"heads={heads}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_padding_lengths_at_tile_edges(dtype):
    Nk = 200
    lens = torch.tensor([0, 1, 63, 64, 65, 127, 128, 129, 200], dtype=torch.int32)
    q, k, v = qkv(len(lens), 4, 2, 160, Nk, 128, dtype, seed=5)
    for causal in (False, True):
        check_fwd(q, k, v, causal=causal, lens=lens, what=f"padding causal={causal}")


def test_lengths_are_clamped():
    lens = torch.tensor([-5, 10_000], dtype=torch.int32)
    q, k, v = qkv(2, 2, 2, 70, 90, 64, torch.bfloat16, seed=9)
    o, lse = fa.fa_fwd(*to_dev(q, k, v), kv_seqlens=lens.cuda())
    O_ref, L_ref = oracle.attention_ref(q, k, v, kv_seqlens=lens)
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, torch.bfloat16, "clamped lengths")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_rows_past_length_never_read(dtype):
    """NaN planted in K/V rows at or past each length must not reach O."""
    q, k, v = qkv(2, 4, 2, 100, 260, 128, dtype, seed=21)
    lens = torch.tensor([70, 200], dtype=torch.int32)
    kn, vn = k.clone(), v.clone()
    for b, L in enumerate(lens.tolist()):
        kn[b, :, L:] = float("nan")
        vn[b, :, L:] = float("nan")
    o, lse = fa.fa_fwd(*to_dev(q, kn, vn), causal=False, kv_seqlens=lens.cuda())
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_ref(q, k, v, kv_seqlens=lens)
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, dtype, "NaN past length")
    # decode reads the same way
    qd = q[:, :, :1].contiguous()
    od, ld = fa.fa_decode(*to_dev(qd, kn, vn), kv_seqlens=lens.cuda(), num_splits=3)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_ref(qd, k, v, kv_seqlens=lens)
    compare(od.cpu(), ld.cpu(), O_ref, L_ref, dtype, "decode NaN past length")


def test_rows_without_keys():
    # causal with Nq > Nk: the first Nq - Nk rows see no key
    q, k, v = qkv(1, 2, 2, 90, 30, 64, torch.bfloat16, seed=2)
    o, lse = fa.fa_fwd(*to_dev(q, k, v), causal=True)
    torch.cuda.synchronize()
    assert torch.all(o[:, :, :60].cpu() == 0) and torch.all(torch.isneginf(lse[:, :, :60].cpu()))
    # Nk == 0: every row is empty
    k0 = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16)
    o, lse = fa.fa_fwd(*to_dev(q, k0, k0))
    torch.cuda.synchronize()
    assert torch.all(o.cpu() == 0) and torch.all(torch.isneginf(lse.cpu()))


def test_empty_inputs_are_noops():
    q = torch.empty((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fa_fwd(q, k, k)
    assert o.shape == q.shape and lse.shape == (0, 2, 16)
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 5, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fa_fwd(q, k, k, causal=True)
    assert o.numel() == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_zero_q_closed_form_on_gpu(dtype):
    """Q = 0: O_i = mean of visible V rows, LSE_i = ln(#visible)."""
    B, Hq, Hkv, Nq, Nk, d = 3, 4, 1, 150, 180, 128
    q = torch.zeros((B, Hq, Nq, d), dtype=dtype)
    _, k, v = qkv(B, Hq, Hkv, Nq, Nk, d, dtype, seed=31)
    lens = torch.tensor([180, 77, 0], dtype=torch.int32)
    o, lse = fa.fa_fwd(*to_dev(q, k, v), causal=True, kv_seqlens=lens.cuda())
    torch.cuda.synchronize()
    o, lse = o.cpu().double(), lse.cpu().double()
    v64 = v.double()
    tol_o = 1e-2 if dtype == torch.bfloat16 else 1e-5
    for b in range(B):
        for i in range(Nq):
            n = min(int(lens[b]), max(0, i + Nk - Nq + 1))
            if n == 0:
                assert torch.all(o[b, :, i] == 0) and torch.all(torch.isneginf(lse[b, :, i]))
                continue
            mean = v64[b, 0, :n].mean(0)
            assert float((o[b, :, i] - mean).abs().max()) <= tol_o
            assert float((lse[b, :, i] - math.log(n)).abs().max()) <= 1e-5


def test_constant_v_on_gpu():
    q, k, _ = qkv(2, 4, 2, 200, 200, 64, torch.bfloat16, seed=41)
    c = torch.linspace(-3, 3, 64).to(torch.bfloat16)
    v = c.expand(2, 2, 200, 64).contiguous()
    o, _ = fa.fa_fwd(*to_dev(q, k, v), causal=True)
    torch.cuda.synchronize()
    assert float((o.cpu().double() - c.double()).abs().max()) <= 1e-2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("S", [1, 2, 3, 16, 64])
def test_decode_splits(S, dtype):
    B, Hq, Hkv, Nk, d = 4, 8, 2, 1000, 128
    q, k, v = qkv(B, Hq, Hkv, 1, Nk, d, dtype, seed=51 + S)
    lens = torch.tensor([1000, 1, 129, 0], dtype=torch.int32)   # many splits are empty
    qd, kd, vd, ld = to_dev(q, k, v, lens)
    o, lse = fa.fa_decode(qd, kd, vd, kv_seqlens=ld, num_splits=S)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_ref(q, k, v, kv_seqlens=lens)
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, dtype, f"decode S={S}")
    op, lp = fa.fa_decode_splitkv(qd, kd, vd, num_splits=S, kv_seqlens=ld)
    torch.cuda.synchronize()
    Op, Lp = oracle.decode_partials_ref(q, k, v, lens, oracle.attention.default_scale(d), S,
                                        fa.FA_DECODE_SPLIT_ALIGN)
    tol = (1e-2, 1e-3) if dtype == torch.bfloat16 else (1e-5, 1e-5)
    compare(op.cpu(), lp.cpu(), Op, Lp, torch.float32, f"partials S={S}", *tol)


@pytest.mark.parametrize("g", [1, 4, 32, 40])
def test_decode_group_sizes(g):
    B, Hkv, Nk, d = 2, 2, 700, 64
    q, k, v = qkv(B, Hkv * g, Hkv, 1, Nk, d, torch.bfloat16, seed=60 + g)
    o, lse = fa.fa_decode(*to_dev(q, k, v), num_splits=5)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_ref(q, k, v)
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, torch.bfloat16, f"decode g={g}")


def test_decode_matches_fwd_and_is_split_independent():
    q, k, v = qkv(3, 8, 2, 1, 2000, 128, torch.bfloat16, seed=71)
    qd, kd, vd = to_dev(q, k, v)
    o_f, l_f = fa.fa_fwd(qd, kd, vd, causal=True)  # bottom-right: the one query sees every key
    outs = [fa.fa_decode(qd, kd, vd, num_splits=S) for S in (1, 4, 16, 256)]
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_ref(q, k, v)
    compare(o_f.cpu(), l_f.cpu(), O_ref, L_ref, torch.bfloat16, "fwd Nq=1")
    for o, lse in outs:
        compare(o.cpu(), lse.cpu(), O_ref, L_ref, torch.bfloat16, "decode vs oracle")
        assert float((o.float() - o_f.float()).abs().max()) <= 1.6e-2
        assert float((lse - l_f).abs().max()) <= 1e-3


def test_scale_argument():
    q, k, v = qkv(1, 2, 2, 130, 130, 64, torch.bfloat16, seed=81)
    for s in (0.03125, 0.5, 1.0):
        check_fwd(q, k, v, causal=True, scale=s, what=f"scale={s}")


def test_non_default_stream():
    q, k, v = qkv(2, 4, 4, 256, 256, 128, torch.bfloat16, seed=91)
    qd, kd, vd = to_dev(q, k, v)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.fa_fwd(qd, kd, vd, causal=True)
    s.synchronize()
    O_ref, L_ref = oracle.attention_ref(q, k, v, causal=True)
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, torch.bfloat16, "side stream")


def test_large_values_stay_finite():
    # scores of several hundred: the running max must prevent overflow
    q, k, v = qkv(1, 2, 2, 200, 200, 128, torch.bfloat16, seed=101)
    q = (q.float() * 8).to(torch.bfloat16)
    k = (k.float() * 8).to(torch.bfloat16)
    check_fwd(q, k, v, causal=True, what="large scores")


def test_decode_rejects_wrong_output_shapes():
    """The merge writes B*Hq rows: a wrong-shaped out or lse is refused in the
    binding before any kernel is launched (the C ABI cannot see sizes)."""
    q, k, v = (t.cuda() for t in qkv(2, 4, 2, 1, 100, 128, torch.bfloat16, seed=21))
    lens = torch.tensor([100, 37], dtype=torch.int32, device="cuda")
    table = torch.arange(2 * 7, dtype=torch.int32, device="cuda").reshape(2, 7)
    kp = torch.zeros((14, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    good_o = torch.empty((2, 4, 1, 128), dtype=torch.bfloat16, device="cuda")
    good_l = torch.empty((2, 4, 1), dtype=torch.float32, device="cuda")
    bad = [(torch.empty((2, 2, 1, 128), dtype=torch.bfloat16, device="cuda"), good_l),
           (torch.empty((1, 4, 1, 128), dtype=torch.bfloat16, device="cuda"), good_l),
           (good_o, torch.empty((2, 3, 1), dtype=torch.float32, device="cuda")),
           (good_o, torch.empty((2, 4, 2), dtype=torch.float32, device="cuda"))]
    for o, l in bad:
        with pytest.raises(ValueError):
            fa.fa_decode(q, k, v, kv_seqlens=lens, out=o, lse=l)
        with pytest.raises(ValueError):
            fa.fa_decode_paged(q, kp, kp, table, lens, out=o, lse=l)
    torch.cuda.synchronize()
