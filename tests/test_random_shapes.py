"""Seeded random sweep over shapes, masks and head layouts for every entry
point, each case checked element by element against the oracle at the bars
of its own parity tests (forward / decode / packed / FP8: bf16 max|dO| <= 1e-2,
max|dLSE| <= 1e-3, f32 1e-5; backward: 1 % of each gradient's largest
magnitude).  The draws are fixed by the seed, so a failure names a
reproducible case; sizes stay small enough for the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import exact_tiled_attention_08_amd as fa
import oracle
from exact_tiled_attention_08_amd import inputs
from fa_testutil import compare, dev, log

N_CASES = 12


def draw(seed):
    r = np.random.default_rng(seed)
    hkv = int(r.choice([1, 2, 4]))
    group = int(r.choice([1, 2, 4]))
    return dict(
        B=int(r.integers(1, 4)), Hkv=hkv, Hq=hkv * group, d=int(r.choice([64, 128])),
        Nq=int(r.integers(1, 400)), Nk=int(r.integers(1, 400)), causal=bool(r.integers(0, 2)),
        padded=bool(r.integers(0, 2)), rng=r)


def rnd(shape, gen, dtype=torch.bfloat16, scale=1.0):
    return (torch.randn(shape, generator=gen) * scale).to(dtype)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_random_fwd(seed, dtype):
    c = draw(1000 + seed)
    g = torch.Generator().manual_seed(seed)
    q = rnd((c["B"], c["Hq"], c["Nq"], c["d"]), g, dtype)
    k = rnd((c["B"], c["Hkv"], c["Nk"], c["d"]), g, dtype)
    v = rnd((c["B"], c["Hkv"], c["Nk"], c["d"]), g, dtype)
    lens = torch.from_numpy(c["rng"].integers(0, c["Nk"] + 1, c["B"]).astype(np.int32)) if c["padded"] else None
    log(f"  case {seed}: {dict((k_, v_) for k_, v_ in c.items() if k_ != 'rng')} lens={lens}")
    o, lse = fa.fa_fwd(q.to(dev()), k.to(dev()), v.to(dev()), causal=c["causal"],
                       kv_seqlens=None if lens is None else lens.to(dev()))
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_ref(q, k, v, causal=c["causal"], kv_seqlens=lens)
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, dtype, f"random fwd {seed}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_decode(seed):
    c = draw(2000 + seed)
    r = c["rng"]
    S = int(r.choice([1, 3, 7, 16, 33]))
    g = torch.Generator().manual_seed(seed)
    nk = int(r.integers(1, 3000))
    q = rnd((c["B"], c["Hq"], 1, c["d"]), g)
    k = rnd((c["B"], c["Hkv"], nk, c["d"]), g)
    v = rnd((c["B"], c["Hkv"], nk, c["d"]), g)
    lens = torch.from_numpy(r.integers(0, nk + 1, c["B"]).astype(np.int32))
    log(f"  case {seed}: B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} d={c['d']} Nk={nk} S={S} lens={lens.tolist()}")
    o, lse = fa.fa_decode(q.to(dev()), k.to(dev()), v.to(dev()), kv_seqlens=lens.to(dev()), num_splits=S)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_ref(q, k, v, kv_seqlens=lens)
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, torch.bfloat16, f"random decode {seed}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_varlen(seed):
    c = draw(3000 + seed)
    r = c["rng"]
    nseq = int(r.integers(1, 6))
    lq = r.integers(0, 300, nseq).tolist()
    # a mix of self-attention (Lk = Lq) and chunks against a longer cache
    lk = [int(a + r.integers(0, 200)) if r.integers(0, 2) else int(a) for a in lq]
    dt = "f32" if r.integers(0, 4) == 0 else "bf16"
    q, k, v, cu_q, cu_k = inputs.make_packed(4, lq, lk, c["Hq"], c["Hkv"], c["d"], dtype=dt)
    log(f"  case {seed}: Hq={c['Hq']} Hkv={c['Hkv']} d={c['d']} {dt} causal={c['causal']} lq={lq} lk={lk}")
    o, lse = fa.fa_fwd_varlen(q.to(dev()), k.to(dev()), v.to(dev()), cu_q.to(dev()), cu_k.to(dev()),
                              max(lq, default=0), causal=c["causal"])
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_varlen_ref(q, k, v, cu_q, cu_k, causal=c["causal"])
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, q.dtype, f"random varlen {seed}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_fp8(seed):
    c = draw(4000 + seed)
    fmt = "e5m2" if c["rng"].integers(0, 2) else "e4m3"
    q, k, v, _, ds = inputs.make_fp8_inputs(4, fmt, B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], Nq=c["Nq"], Nk=c["Nk"],
                                            padded=False)
    lens = torch.from_numpy(c["rng"].integers(0, c["Nk"] + 1, c["B"]).astype(np.int32)) if c["padded"] else None
    log(f"  case {seed}: B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} Nq={c['Nq']} Nk={c['Nk']} {fmt} "
        f"causal={c['causal']} lens={lens}")
    o, lse = fa.fa_fwd_fp8(q.to(dev()), k.to(dev()), v.to(dev()), *ds, causal=c["causal"],
                           kv_seqlens=None if lens is None else lens.to(dev()))
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_fp8_ref(q.view(torch.uint8), k.view(torch.uint8), v.view(torch.uint8),
                                            {"e4m3": oracle.E4M3, "e5m2": oracle.E5M2}[fmt], *ds,
                                            causal=c["causal"], kv_seqlens=lens)
    compare(o.cpu(), lse.cpu(), O_ref, L_ref, torch.bfloat16, f"random fp8 {seed}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_bwd(seed):
    from test_bwd import compare_grads, structural_zeros
    c = draw(5000 + seed)
    g = torch.Generator().manual_seed(seed)
    q = rnd((c["B"], c["Hq"], c["Nq"], c["d"]), g)
    k = rnd((c["B"], c["Hkv"], c["Nk"], c["d"]), g)
    v = rnd((c["B"], c["Hkv"], c["Nk"], c["d"]), g)
    do = rnd((c["B"], c["Hq"], c["Nq"], c["d"]), g)
    lens = torch.from_numpy(c["rng"].integers(0, c["Nk"] + 1, c["B"]).astype(np.int32)) if c["padded"] else None
    log(f"  case {seed}: {dict((k_, v_) for k_, v_ in c.items() if k_ != 'rng')} lens={lens}")
    ld = None if lens is None else lens.to(dev())
    qd, kd, vd, dod = (t.to(dev()) for t in (q, k, v, do))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=c["causal"], kv_seqlens=ld)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, lse, dod, causal=c["causal"], kv_seqlens=ld)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd_ref(q, k, v, do, causal=c["causal"], kv_seqlens=lens)
    compare_grads([dq.cpu(), dk.cpu(), dv.cpu()], ref, f"random bwd {seed}",
                  structural_zeros(q, k, v, c["causal"], lens))
