"""The C ABI seen from the host (CPU only: nothing here launches a kernel).

Every call below fails an argument check, which the library performs before
it touches the HIP runtime, or is an empty call that returns at once.
"""
import os
import re

import pytest

import io_aware_tiled_09_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

A = 0x7F0000000000  # a fake, 16-byte aligned device address (never dereferenced)
MB = 1 << 20


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = fa.load()
    names = _declared_functions()
    assert set(names) == set(fa.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    assert fa.fa_status_string(0) == "ok"
    for code in range(1, 12):
        s = fa.fa_status_string(code)
        assert s and s != "unknown status"
    assert fa.fa_status_string(99) == "unknown status"


def test_tile_shape():
    assert fa.fa_tile_rows() == 256 and fa.fa_tile_cols() == 64


@pytest.mark.parametrize("B,H,N,causal,expect", [
    # (workgroups, rows per block, paired)
    (4, 12, 512, 0, (192, 128, False)),     # BERT shape: 96 blocks of 256 rows -> key split
    (8, 12, 1024, 1, (240, 256, True)),     # GPT-2 shape: balanced groups (key split: 768, 3 rounds)
    (1, 40, 2000, 1, (180, 256, True)),     # balanced, nqb = 8: 40 x 4 + 20 middle pairs
    (3, 9, 1300, 1, (95, 256, True)),       # balanced, 27 heads: one middle block alone
    (1, 33, 2300, 1, (165, 256, True)),     # balanced, nqb = 9 odd: no middles
    (2, 32, 8192, 1, (1024, 256, True)),    # long document: paired
    (1, 32, 32768, 1, (4096, 256, False)),  # very long context: one block per workgroup
    (1, 2, 65, 1, (2, 256, False)),         # one block either way: 256 rows
    (1, 2, 200, 0, (4, 128, False)),
    (1, 4, 8000, 1, (252, 128, False)),
    (1, 16, 8000, 1, (256, 256, True)),
    (2, 16, 1000, 0, (256, 128, False)),
    (2, 16, 1100, 0, (160, 256, False)),   # 128-row grid (288) would not fit one round
    (1, 1, 0, 0, (0, 256, False)),
])
def test_forward_grid(B, H, N, causal, expect):
    assert fa.fa_fwd_grid(B, H, N, causal) == expect


def test_forward_grid_errors():
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_grid(-1, 2, 3, 0)
    assert e.value.status == 2
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_grid(1 << 16, 1 << 14, 1 << 20, 0)
    assert e.value.status == 8


def _call(fn=fa.fa_fwd, q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB,
          B=1, H=2, N=100, d=64, scale=0.125, causal=0):
    return fn(q, k, v, o, lse, B, H, N, d, scale, causal, 0)


@pytest.mark.parametrize("fn", [fa.fa_fwd, fa.fa_fwd_f32])
def test_argument_errors(fn):
    assert _call(fn, q=0) == 1
    assert _call(fn, lse=0) == 1
    assert _call(fn, B=-1) == 2
    assert _call(fn, N=-5) == 2
    assert _call(fn, d=96) == 3
    assert _call(fn, d=256) == 3
    assert _call(fn, scale=float("nan")) == 4
    assert _call(fn, scale=float("inf")) == 4
    assert _call(fn, scale=-0.5) == 4
    assert _call(fn, q=A + 8) == 5
    assert _call(fn, o=A + 192 * MB + 4) == 5
    assert _call(fn, lse=A + 256 * MB + 2) == 5
    assert _call(fn, o=A) == 6                       # o is q
    assert _call(fn, lse=A + 64 * MB + 1024) == 6    # lse inside k
    assert _call(fn, lse=A + 192 * MB + 128) == 6    # lse inside o
    assert _call(fn, B=65536, H=65536, N=128) == 8   # 2^32 workgroups


@pytest.mark.parametrize("fn", [fa.fa_fwd, fa.fa_fwd_f32])
def test_empty_calls_return_ok_without_pointers(fn):
    for B, H, N in ((0, 4, 100), (2, 0, 100), (2, 4, 0)):
        assert fn(None, None, None, None, None, B, H, N, 64, 0.125, 1, None) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from io_aware_tiled_09_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "libfa.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _binding.fa_fwd(A, A, A, A, A, 1, 1, 1, 64, 1.0, 0)


def _fp8(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB, B=1, H=2, N=100,
         d=128, scale=0.1, qs=0.01, ks=0.01, vs=0.01, causal=1):
    return fa.fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, qs, ks, vs, causal, 0)


def test_fp8_argument_errors():
    assert _fp8(v=0) == 1
    assert _fp8(H=-2) == 2
    assert _fp8(d=64) == 3
    assert _fp8(scale=float("inf")) == 4
    assert _fp8(qs=0.0) == 4
    assert _fp8(vs=float("nan")) == 4
    assert _fp8(ks=-1.0) == 4
    assert _fp8(k=A + 64 * MB + 4) == 5
    assert _fp8(o=A + 64 * MB) == 6                 # o over k
    assert _fp8(lse=A + 192 * MB + 1024) == 6       # lse inside o
    assert _fp8(B=65536, H=65536, N=128) == 8
    for B, H, N in ((0, 4, 100), (2, 0, 100), (2, 4, 0)):
        assert fa.fa_fwd_fp8(None, None, None, None, None, B, H, N, 128, 0.1, 1, 1, 1, 1, None) == 0


def _dec(q=A, kc=A + 64 * MB, vc=A + 128 * MB, pt=A + 192 * MB, sl=A + 193 * MB, o=A + 194 * MB,
         lse=A + 195 * MB, ws=A + 196 * MB, ws_bytes=None, B=3, H=8, H_kv=2, d=128,
         num_pages=40, page_size=16, max_pages=10, scale=0.1):
    if ws_bytes is None:
        ws_bytes = fa.fa_decode_workspace_bytes(B, H, d, page_size, max_pages)
    return fa.fa_decode_paged(q, kc, vc, pt, sl, o, lse, ws, ws_bytes, B, H, H_kv, d, num_pages,
                              page_size, max_pages, scale, 0)


def test_decode_workspace_bytes():
    # B * H * ceil(max_pages * page_size / 512) slots of (d + 2) floats
    assert fa.fa_decode_workspace_bytes(3, 8, 128, 16, 10) == 3 * 8 * 1 * 130 * 4
    assert fa.fa_decode_workspace_bytes(50, 32, 128, 16, 512) == 50 * 32 * 16 * 130 * 4
    assert fa.fa_decode_workspace_bytes(0, 8, 128, 16, 10) == 0


def test_decode_argument_errors():
    assert _dec(pt=0) == 1
    assert _dec(H=8, H_kv=3) == 2           # H not a multiple of H_kv
    assert _dec(H=32, H_kv=2) == 2          # 16 query heads per KV head: not built
    assert _dec(page_size=24) == 2          # not a multiple of 16
    assert _dec(num_pages=0) == 2
    assert _dec(d=96) == 3
    assert _dec(scale=-1.0) == 4
    assert _dec(kc=A + 64 * MB + 8) == 5
    assert _dec(sl=A + 193 * MB + 2) == 5
    assert _dec(ws_bytes=100) == 9
    assert _dec(ws=0) == 9
    assert _dec(o=A + 64 * MB) == 6         # o over the K cache
    assert _dec(ws=A + 128 * MB) == 6       # workspace over the V cache
    assert _dec(B=70000) == 8
    assert fa.fa_decode_paged(*([None] * 8), 0, 0, 8, 2, 128, 4, 16, 4, 0.1, None) == 0


def _bwd(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB,
         dout=A + 320 * MB, dq=A + 384 * MB, dk=A + 448 * MB, dv=A + 512 * MB, ws=A + 576 * MB,
         B=1, H=2, N=100, d=64, scale=0.125, causal=0):
    return fa.fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, N, d, scale, causal, 0)


def test_bwd_argument_errors():
    assert _bwd(dout=0) == 1
    assert _bwd(ws=0) == 1
    assert _bwd(N=-1) == 2
    assert _bwd(d=32) == 3
    assert _bwd(scale=float("nan")) == 4
    assert _bwd(dq=A + 384 * MB + 8) == 5
    assert _bwd(ws=A + 576 * MB + 2) == 5
    assert _bwd(dq=A) == 6                        # dq is q
    assert _bwd(dk=A + 320 * MB + 256) == 6       # dk inside dout
    assert _bwd(ws=A + 256 * MB) == 6             # workspace is lse
    assert _bwd(dv=A + 448 * MB) == 6             # dv is dk
    assert _bwd(B=65536, H=65536, N=128) == 8
    for B, H, N in ((0, 4, 100), (2, 0, 100), (2, 4, 0)):
        assert fa.fa_bwd(*([None] * 10), B, H, N, 64, 0.125, 1, None) == 0


def _bwd_na(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB,
            dout=A + 320 * MB, dq=A + 384 * MB, dk=A + 448 * MB, dv=A + 512 * MB,
            B=1, H=2, N=100, d=64, scale=0.125, causal=0):
    return fa.fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, 0)


def test_bwd_noalloc_argument_errors():
    # every check runs before the static scratch is looked up or anything is
    # launched
    assert fa.fa_bwd_noalloc_max_rows() == 4194304
    assert _bwd_na(dout=0) == 1
    assert _bwd_na(N=-1) == 2
    assert _bwd_na(d=32) == 3
    assert _bwd_na(scale=float("inf")) == 4
    assert _bwd_na(dq=A + 384 * MB + 8) == 5
    assert _bwd_na(lse=A + 256 * MB + 2) == 5
    assert _bwd_na(dq=A) == 6
    assert _bwd_na(dv=A + 448 * MB) == 6
    # one row past the static scratch: 4194305 rows of d = 64 (512 MiB per
    # tensor, addresses 1 GiB apart)
    G = 1024 * MB
    big = dict(q=A, k=A + G, v=A + 2 * G, o=A + 3 * G, lse=A + 4 * G, dout=A + 5 * G,
               dq=A + 6 * G, dk=A + 7 * G, dv=A + 8 * G)
    assert _bwd_na(B=1, H=1, N=4194305, **big) == 11
    assert _bwd_na(B=2, H=1, N=2097153, **big) == 11
    assert "static scratch" in fa.fa_status_string(11)
    for B, H, N in ((0, 4, 100), (2, 0, 100), (2, 4, 0)):
        assert fa.fa_bwd_noalloc(*([None] * 9), B, H, N, 64, 0.125, 1, None) == 0


# ---------------------------------------------------------------- libfa_std.so
from io_aware_tiled_09_amd import standard as std  # noqa: E402

STD_HEADER = os.path.join(ROOT, "include", "fa_std.h")


def test_std_library_exports_every_declared_symbol():
    lib = std.load_std()
    text = re.sub(r"/\*.*?\*/", "", open(STD_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(fa_std_[a-z0-9_]+)\s*\(", text)))
    assert set(names) == set(std.STD_EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_std_workspace_bytes():
    nn = 2 * 3 * 100 * 100
    r = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert std.fa_std_workspace_bytes(2, 3, 100) == r(nn * 4) + r(nn * 2) + (32 << 20)
    assert std.fa_std_workspace_bytes(0, 3, 100) == 0
    assert std.fa_std_workspace_bytes(-1, 3, 100) == 0
    assert std.fa_std_workspace_bytes(2, 32, 8192) == 2 * 32 * 8192 * 8192 * 6 + (32 << 20)


def _std(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB,
         ws=A + 512 * MB, ws_bytes=None, B=1, H=2, N=100, d=64, scale=0.125, causal=0):
    if ws_bytes is None:
        ws_bytes = std.fa_std_workspace_bytes(B, H, N)
    return std.fa_std_fwd(q, k, v, o, lse, ws, ws_bytes, B, H, N, d, scale, causal, 0)


def test_std_argument_errors():
    assert _std(q=0) == 1
    assert _std(N=-1) == 2
    assert _std(d=96) == 3
    assert _std(scale=float("nan")) == 4
    assert _std(o=A + 192 * MB + 8) == 5
    assert _std(ws=0) == 9
    assert _std(ws=A + 512 * MB + 16) == 9                 # not 256-byte aligned
    assert _std(ws_bytes=1000) == 9                        # too small
    assert _std(o=A) == 6                                  # o is q
    assert _std(ws=A + 64 * MB) == 6                       # workspace over k
    assert _std(B=65536, H=65536, N=2) == 8
    for B, H, N in ((0, 4, 100), (2, 0, 100), (2, 4, 0)):
        assert std.fa_std_fwd(*([None] * 6), 0, B, H, N, 64, 0.125, 1, None) == 0
    # the three steps check their own arguments
    assert std.fa_std_scores(A, A + 64 * MB, 0, A + 512 * MB, 1, 2, 100, 64, 0.1) == 1
    assert std.fa_std_scores(A, A + 64 * MB, A + 128 * MB, 0, 1, 2, 100, 64, 0.1) == 9
    assert std.fa_std_scores(A, A + 64 * MB, A, A + 512 * MB, 1, 2, 100, 64, 0.1) == 6
    assert std.fa_std_softmax(A, A, A + 256 * MB, 1, 2, 100, 1) == 6
    assert std.fa_std_softmax(A, A + 64 * MB + 2, A + 256 * MB, 1, 2, 100, 1) == 5
    assert std.fa_std_output(A, A + 64 * MB, A + 64 * MB, A + 512 * MB, 1, 2, 100, 64) == 6
    assert std.fa_std_output(A, A + 64 * MB, A + 128 * MB, A + 512 * MB, 1, 2, 100, 32) == 3


def test_python_face_rejects_mismatched_outputs():
    # The C ABI sees raw pointers only, so the Python face must refuse an
    # out or lse buffer that does not have exactly the extent the kernels
    # write: checked here on CPU tensors, before any launch could happen.
    import torch
    from io_aware_tiled_09_amd._binding import check_outputs
    q = torch.zeros((2, 3, 40, 64), dtype=torch.float32)
    good_o = torch.empty_like(q)
    good_l = torch.empty((2, 3, 40), dtype=torch.float32)
    check_outputs(q, good_o, good_l)
    bad = [
        (torch.empty_like(q, dtype=torch.bfloat16), good_l),          # fp32 q, bf16 out
        (torch.empty((2, 3, 41, 64)), good_l),                         # wrong shape
        (torch.empty((2, 3, 64, 40)).transpose(2, 3), good_l),         # not contiguous
        (torch.empty_like(q, device="meta"), good_l),                  # other device
        (good_o, torch.empty((2, 3, 40), dtype=torch.float64)),        # lse not fp32
        (good_o, torch.empty((2, 3, 39), dtype=torch.float32)),        # lse too short
        (good_o, torch.empty((2, 3, 40), dtype=torch.float32, device="meta")),
        (good_o, torch.empty((3, 40, 2), dtype=torch.float32).permute(2, 0, 1)),
    ]
    for o, l in bad:
        with pytest.raises(ValueError):
            check_outputs(q, o, l)
