"""The C ABI loads, exports what include/fa.h declares, and rejects bad
arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from exact_tiled_attention_08_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "fa_ceilings.h")]

BAD, UNSUP, WS = _lib.FA_ERR_INVALID_ARG, _lib.FA_ERR_UNSUPPORTED, _lib.FA_ERR_WORKSPACE
P = 0x10000  # a 256-byte-aligned fake device address; never dereferenced by these calls


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(fa_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_exports_match_header(lib):
    names = declared_functions()
    assert set(names) == set(_lib.PROTOTYPES), names
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define FA_DECODE_SPLIT_ALIGN (\d+)", text).group(1)) == _lib.FA_DECODE_SPLIT_ALIGN
    assert int(re.search(r"#define FA_MAX_SPLITS (\d+)", text).group(1)) == _lib.FA_MAX_SPLITS
    assert int(re.search(r"#define FA_NOALLOC_SCRATCH_BYTES (\d+)", text).group(1)) == _lib.FA_NOALLOC_SCRATCH_BYTES
    for name, val in [("FA_OK", 0), ("FA_ERR_INVALID_ARG", -1), ("FA_ERR_UNSUPPORTED", -2),
                      ("FA_ERR_WORKSPACE", -3), ("FA_ERR_HIP", -4), ("FA_F32", 0), ("FA_BF16", 1),
                      ("FA_FP8_E4M3", 2), ("FA_FP8_E5M2", 3)]:
        assert re.search(rf"\b{name} = {val}\b", text), name


def test_status_strings(lib):
    assert lib.fa_status_string(0) == b"FA_OK"
    assert lib.fa_status_string(-3) == b"FA_ERR_WORKSPACE"
    assert lib.fa_status_string(7) == b"FA_UNKNOWN_STATUS"
    assert lib.fa_version() >= 100


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Nq=16, Nk=16, d=64, scale=0.125, causal=0,
        lens=None, dtype=1):
    return lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, lens, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(q=None), BAD), (dict(k=None), BAD), (dict(v=None), BAD), (dict(o=None), BAD),
    (dict(lse=None), BAD), (dict(q=P + 8), BAD), (dict(o=P + 4), BAD), (dict(lse=P + 2), BAD),
    (dict(lens=P + 1), BAD), (dict(d=96), UNSUP), (dict(d=256), UNSUP), (dict(Hq=3), UNSUP),
    (dict(Hkv=0), UNSUP), (dict(B=-1), BAD), (dict(Nk=-5), BAD), (dict(scale=0.0), BAD),
    (dict(scale=-1.0), BAD), (dict(scale=float("nan")), BAD), (dict(scale=float("inf")), BAD),
    (dict(causal=2), BAD), (dict(dtype=2), UNSUP),
    (dict(B=65536, Hq=65536, Hkv=1, Nq=128, Nk=128), UNSUP),  # 2^32 work-groups: more than one launch holds
])
def test_fwd_rejects(lib, kwargs, status):
    assert fwd(lib, **kwargs) == status
    assert lib.fa_last_error() != b""


@pytest.mark.parametrize("kwargs", [dict(B=0), dict(Hq=0), dict(Nq=0), dict(B=0, q=None, o=None, lse=None)])
def test_fwd_empty_is_noop(lib, kwargs):
    assert fwd(lib, **kwargs) == _lib.FA_OK


def test_workspace_bytes(lib):
    rows = 64 * 32 * 16
    need = lib.fa_decode_workspace_bytes(64, 32, 128, 16)
    assert need == (rows * 128 * 4 + 255) // 256 * 256 + rows * 4
    assert lib.fa_decode_workspace_bytes(1, 1, 96, 16) == 0
    assert lib.fa_decode_workspace_bytes(1, 1, 64, 0) == 0
    assert lib.fa_decode_workspace_bytes(1, 1, 64, 257) == 0


def decode(lib, q=P, k=P, v=P, o=P, lse=P, B=2, Hq=8, Hkv=2, Nk=100, d=128, scale=0.1, lens=None, S=16,
           ws=P, ws_bytes=None, dtype=1):
    if ws_bytes is None:
        ws_bytes = lib.fa_decode_workspace_bytes(B, Hq, d, S) if S >= 1 else 0
    return lib.fa_decode(q, k, v, o, lse, B, Hq, Hkv, Nk, d, scale, lens, S, ws, ws_bytes, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(S=0), UNSUP), (dict(S=257), UNSUP), (dict(ws=None), WS), (dict(ws_bytes=1000), WS),
    (dict(ws=P + 16), BAD), (dict(q=None), BAD), (dict(k=None), BAD), (dict(o=None), BAD),
    (dict(d=32), UNSUP), (dict(Hq=6, Hkv=4), UNSUP), (dict(scale=-0.5), BAD), (dict(dtype=5), UNSUP),
    (dict(B=70000), UNSUP),
])
def test_decode_rejects(lib, kwargs, status):
    assert decode(lib, **kwargs) == status


def test_splitkv_and_merge_reject(lib):
    assert lib.fa_decode_splitkv(P, P, P, None, P, 1, 4, 1, 64, 128, 0.1, None, 4, 1, None) == BAD
    assert lib.fa_decode_splitkv(P, P, P, P, P, 1, 4, 1, 64, 128, 0.1, None, 0, 1, None) == UNSUP
    assert lib.fa_lse_merge(P, P, P, P, -1, 128, 4, 1, None) == BAD
    assert lib.fa_lse_merge(P, P, P, P, 10, 100, 4, 1, None) == UNSUP
    assert lib.fa_lse_merge(P, P, None, P, 10, 128, 4, 1, None) == BAD
    assert lib.fa_lse_merge(P, P, P, P, 0, 128, 4, 1, None) == _lib.FA_OK


def test_python_binding_requires_gpu_tensors():
    import torch
    import exact_tiled_attention_08_amd as fa
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)


def bwd(lib, q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, Hq=4, Hkv=2, Nq=16, Nk=16, d=128,
        scale=0.1, causal=1, lens=None, ws=P, ws_bytes=None, dtype=1):
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(max(B, 0), max(Hq, 0), max(Nq, 0), d) if d in (64, 128) else 0
    return lib.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, causal, lens, ws, ws_bytes,
                      dtype, None)


def test_bwd_workspace_bytes(lib):
    assert lib.fa_bwd_workspace_bytes(1, 32, 8192, 128) == 32 * 8192 * 4
    assert lib.fa_bwd_workspace_bytes(1, 1, 3, 64) == 256
    assert lib.fa_bwd_workspace_bytes(1, 1, 4, 96) == 0
    assert lib.fa_bwd_workspace_bytes(-1, 1, 4, 64) == 0


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=0), UNSUP), (dict(dtype=3), UNSUP), (dict(d=96), UNSUP), (dict(Hq=3), UNSUP),
    (dict(q=None), BAD), (dict(o=None), BAD), (dict(do=None), BAD), (dict(lse=None), BAD),
    (dict(dq=None), BAD), (dict(dk=None), BAD), (dict(dv=None), BAD), (dict(k=P + 8), BAD),
    (dict(ws=None), WS), (dict(ws_bytes=100), WS), (dict(ws=P + 64), BAD), (dict(causal=5), BAD),
    (dict(scale=0.0), BAD), (dict(lens=P + 2), BAD), (dict(Nk=-1), BAD),
])
def test_bwd_rejects(lib, kwargs, status):
    assert bwd(lib, **kwargs) == status
    assert lib.fa_last_error() != b""


def test_bwd_empty_is_noop(lib):
    # nothing to write at all
    assert bwd(lib, B=0, q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None,
               ws=None) == _lib.FA_OK
    assert bwd(lib, Hq=0, Hkv=0, q=None, k=None, v=None, o=None, do=None, lse=None, dq=None, dk=None, dv=None,
               ws=None) == _lib.FA_OK


def paged(lib, q=P, kp=P, vp=P, table=P, o=P, lse=P, B=2, Hq=8, Hkv=2, num_pages=10, page=16, max_pages=4,
          d=128, scale=0.1, lens=P, S=4, ws=P, ws_bytes=None, dtype=1):
    if ws_bytes is None:
        ws_bytes = lib.fa_decode_workspace_bytes(B, Hq, d, S) if S >= 1 else 0
    return lib.fa_decode_paged(q, kp, vp, table, o, lse, B, Hq, Hkv, num_pages, page, max_pages, d, scale, lens,
                               S, ws, ws_bytes, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(page=0), BAD), (dict(max_pages=0), BAD), (dict(num_pages=0), BAD), (dict(table=None), BAD),
    (dict(lens=None), BAD), (dict(table=P + 2), BAD), (dict(dtype=0), UNSUP), (dict(ws=None), WS),
    (dict(d=96), UNSUP), (dict(S=0), UNSUP), (dict(kp=None), BAD), (dict(o=None), BAD),
    (dict(page=1 << 20, max_pages=1 << 12), UNSUP),
])
def test_paged_rejects(lib, kwargs, status):
    assert paged(lib, **kwargs) == status


def varlen(lib, q=P, k=P, v=P, o=P, lse=P, cu_q=P, cu_k=P, B=2, Hq=4, Hkv=2, total_q=40, total_k=50, max_q=30,
           d=128, scale=0.125, causal=1, dtype=1):
    return lib.fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, B, Hq, Hkv, total_q, total_k, max_q, d, scale, causal,
                             dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(cu_q=None), BAD), (dict(cu_k=None), BAD), (dict(cu_q=P + 2), BAD), (dict(max_q=-1), BAD),
    (dict(total_q=-1), BAD), (dict(total_k=-1), BAD), (dict(B=-1), BAD), (dict(q=None), BAD),
    (dict(o=P + 8), BAD), (dict(lse=None), BAD), (dict(k=None), BAD), (dict(v=P + 4), BAD),
    (dict(causal=2), BAD), (dict(scale=0.0), BAD), (dict(d=96), UNSUP), (dict(dtype=5), UNSUP),
    (dict(Hq=3), UNSUP)])
def test_varlen_rejects(lib, kwargs, status):
    assert varlen(lib, **kwargs) == status, lib.fa_last_error()
    assert lib.fa_last_error() != b""


@pytest.mark.parametrize("kwargs", [dict(total_q=0, q=None, o=None, lse=None), dict(max_q=0), dict(B=0),
                                    dict(Hq=0, Hkv=0)])
def test_varlen_empty_is_noop(lib, kwargs):
    assert varlen(lib, **kwargs) == 0, lib.fa_last_error()


def fwd_fp8(lib, q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Nq=16, Nk=16, d=128, scale=0.125, causal=0,
            lens=None, qd=0.5, kd=0.5, vd=0.5, dtype=2):
    return lib.fa_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, lens, qd, kd, vd, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=1), UNSUP), (dict(dtype=0), UNSUP), (dict(dtype=4), UNSUP), (dict(d=64), UNSUP),
    (dict(Hq=3), UNSUP), (dict(qd=0.0), BAD), (dict(kd=-1.0), BAD), (dict(vd=float("nan")), BAD),
    (dict(vd=float("inf")), BAD), (dict(scale=0.0), BAD), (dict(causal=2), BAD), (dict(q=None), BAD),
    (dict(k=P + 8), BAD), (dict(o=None), BAD), (dict(lse=P + 2), BAD), (dict(lens=P + 1), BAD),
    (dict(B=-1), BAD)])
def test_fp8_rejects(lib, kwargs, status):
    assert fwd_fp8(lib, **kwargs) == status, lib.fa_last_error()
    assert lib.fa_last_error() != b""


@pytest.mark.parametrize("kwargs", [dict(B=0), dict(Nq=0, q=None, o=None, lse=None), dict(dtype=3, Hq=0)])
def test_fp8_empty_is_noop(lib, kwargs):
    assert fwd_fp8(lib, **kwargs) == _lib.FA_OK, lib.fa_last_error()


def decode_noalloc(lib, q=P, k=P, v=P, o=P, lse=P, B=2, Hq=8, Hkv=2, Nk=100, d=128, scale=0.1, lens=None,
                   S=16, dtype=1):
    return lib.fa_decode_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nk, d, scale, lens, S, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(q=None), BAD), (dict(o=None), BAD), (dict(lse=None), BAD), (dict(o=P + 8), BAD), (dict(lens=P + 2), BAD),
    (dict(d=96), UNSUP), (dict(S=0), UNSUP), (dict(S=257), UNSUP), (dict(Hq=7), UNSUP), (dict(scale=0.0), BAD),
    # partials beyond the static scratch: refused before any HIP call
    (dict(B=64, Hq=32, S=64), WS), (dict(B=4096, Hq=64, S=1), WS),
])
def test_decode_noalloc_rejects(lib, kwargs, status):
    assert decode_noalloc(lib, **kwargs) == status
    assert lib.fa_last_error() != b""


def test_decode_noalloc_limit_matches_workspace_size(lib):
    # the long decode workload (B=64, Hq=32, d=128, 16 splits) fits the scratch,
    # four times its splits do not
    assert lib.fa_decode_workspace_bytes(64, 32, 128, 16) <= _lib.FA_NOALLOC_SCRATCH_BYTES
    assert lib.fa_decode_workspace_bytes(64, 32, 128, 64) > _lib.FA_NOALLOC_SCRATCH_BYTES
    assert decode_noalloc(lib, B=0) == _lib.FA_OK and decode_noalloc(lib, Hq=0) == _lib.FA_OK


def test_ceiling_aids_reject_bad_arguments(lib):
    assert lib.fa_ceiling_mfma(None, None, 4, 10, None) == -1
    assert lib.fa_ceiling_mfma(None, P, 0, 10, None) == -1
    assert lib.fa_ceiling_mfma(None, P, 4, 0, None) == -1
    assert lib.fa_ceiling_mfma(P + 8, P, 4, 10, None) == -1
    assert lib.fa_ceiling_read(P, 17, P, 4, None) == -1
    assert lib.fa_ceiling_read(P + 4, 32, P, 4, None) == -1
    assert lib.fa_ceiling_read(None, 32, P, 4, None) == -1
