"""The C ABI of libfa.so on the host (CPU only, no kernel launches).

Checks that the library loads, exports every function include/fa.h declares, and rejects
bad requests with the documented status codes. Validation runs before any HIP call, so none
of these calls touches a device.
"""

import ctypes
import os
import re
import subprocess

import pytest

import exact_tiled_attention_24_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.LIB_PATH),
                                reason="libfa.so not built (run the package build first)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fa_fwd", "fa_decode_splitk", "fa_merge", "fa_status_string",
              "fa_decode_workspace_bytes", "fa_decode_plan_splits", "fa_fwd_paged",
              "fa_fwd_block_sparse", "fa_bwd", "fa_bwd_workspace_bytes", "fa_fwd_fp8"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in fa.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    assert set(declared_functions()) <= exported
    # C linkage: no mangled names for the entry points
    assert not any(s.startswith("_Z") and "fa_fwd" in s for s in out.split())


def test_status_strings():
    for code in range(5):
        assert fa.fa_status_string(code).startswith("FA_")
    assert "unknown" in fa.fa_status_string(99)


NULL = None
DEV = ctypes.c_void_p(0x1000)  # an aligned, never dereferenced fake pointer
MIS = ctypes.c_void_p(0x1002)  # misaligned


def fwd(lib, dt=1, q=DEV, k=DEV, v=DEV, o=DEV, B=1, Hq=2, Hkv=1, N=8, d=64, scale=0.125, causal=1):
    return lib.fa_fwd(dt, q, k, v, o, None, None, B, Hq, Hkv, N, d, scale, causal, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dt=7), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(dt=2), fa.FA_ERR_UNSUPPORTED),            # e4m3 goes through fa_fwd_fp8
    (dict(B=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(N=-5), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(q=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(o=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(k=MIS), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(N=1 << 24, d=128), fa.FA_ERR_UNSUPPORTED),
    # bf16: a head's K or V rows may span at most 2^30 bytes (N d <= 2^29)
    (dict(N=(1 << 22) + 1, d=128), fa.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 23, d=128), fa.FA_ERR_UNSUPPORTED),
    (dict(N=(1 << 23) + 1, d=64), fa.FA_ERR_UNSUPPORTED),
    # empty problems are valid no-ops, even with NULL pointers
    (dict(B=0, q=NULL, k=NULL, v=NULL, o=NULL), fa.FA_OK),
    (dict(N=0, q=NULL), fa.FA_OK),
    (dict(Hq=0, Hkv=0), fa.FA_OK),
])
def test_fwd_validation(kwargs, code):
    assert fwd(fa.load_library(), **kwargs) == code


def decode(lib, dt=1, q=DEV, kc=DEV, vc=DEV, table=DEV, lens=DEV, o=DEV, B=2, Hq=8, Hkv=2, d=128,
           page=16, num_pages=10, max_pages=5, max_len=80, scale=0.08, splits=0, ws=DEV,
           ws_bytes=1 << 30):
    return lib.fa_decode_splitk(dt, q, kc, vc, table, lens, o, B, Hq, Hkv, d, page, num_pages,
                                max_pages, max_len, scale, splits, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dt=5), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(dt=0), fa.FA_ERR_UNSUPPORTED),
    (dict(d=64), fa.FA_ERR_UNSUPPORTED),
    (dict(page=32), fa.FA_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=2), fa.FA_ERR_UNSUPPORTED),   # group of 3 query heads per KV head
    (dict(Hq=7, Hkv=2), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(Hq=32, Hkv=2), fa.FA_ERR_UNSUPPORTED),  # group of 16
    (dict(B=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(num_pages=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(splits=-2), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(max_len=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(table=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(lens=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(ws=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(kc=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(q=MIS), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=16), fa.FA_ERR_WORKSPACE_TOO_SMALL),
    (dict(B=0, q=NULL, o=NULL), fa.FA_OK),
])
def test_decode_validation(kwargs, code):
    assert decode(fa.load_library(), **kwargs) == code


def test_decode_workspace_and_plan():
    # the auto plan fills the chip with (sequence, KV head, chunk) workgroups
    s = fa.fa_decode_plan_splits(8, 8, 16, 32768)
    assert 1 <= s <= 2048
    assert fa.fa_decode_plan_splits(1, 1, 16, 16) == 1  # never more chunks than pages
    assert fa.fa_decode_plan_splits(8, 8, 32, 100) == 0  # unsupported page size
    need = fa.fa_decode_workspace_bytes(8, 32, 128, 16, 32768, 0)
    assert need >= s * 8 * 32 * 130 * 4
    # completion words (8 bytes per query head) and the float32 partials of 5 chunks
    assert fa.fa_decode_workspace_bytes(8, 32, 128, 16, 32768, 5) == 8 * 8 * 32 + 5 * 8 * 32 * 130 * 4
    assert fa.fa_decode_workspace_bytes(8, 32, 128, 16, 32768, -1) == 0
    # the exact workspace is accepted by validation (rejected by nothing but a bad argument)
    lib = fa.load_library()
    exact = fa.fa_decode_workspace_bytes(2, 8, 128, 16, 80, 3)
    assert decode(lib, splits=3, ws_bytes=exact - 1) == fa.FA_ERR_WORKSPACE_TOO_SMALL


def paged(lib, dt=1, q=DEV, kc=DEV, vc=DEV, table=DEV, lens=DEV, o=DEV, B=2, Hq=8, Hkv=2, Nq=64,
          d=128, page=16, num_pages=10, max_pages=8, scale=0.1, causal=1):
    return lib.fa_fwd_paged(dt, q, kc, vc, table, lens, None, o, None, None, B, Hq, Hkv, Nq, d, page,
                            num_pages, max_pages, scale, causal, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dt=7), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(dt=0), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(page=32), fa.FA_ERR_UNSUPPORTED),
    (dict(page=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(Hq=7, Hkv=2), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(Hkv=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(B=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(Nq=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(num_pages=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(max_pages=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(table=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(lens=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(q=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(kc=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(o=MIS), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(max_pages=1 << 28), fa.FA_ERR_UNSUPPORTED),
    (dict(num_pages=1 << 16, Hkv=8, Hq=8), fa.FA_ERR_UNSUPPORTED),   # a 2 GiB cache
    (dict(Nq=(1 << 22) + 1), fa.FA_ERR_UNSUPPORTED),                 # Nq d > 2^29
    (dict(Nq=0, q=NULL, o=NULL), fa.FA_OK),
    (dict(B=0, q=NULL, o=NULL), fa.FA_OK),
])
def test_fwd_paged_validation(kwargs, code):
    assert paged(fa.load_library(), **kwargs) == code


def sparse(lib, dt=1, q=DEV, k=DEV, v=DEV, o=DEV, offs=DEV, idx=DEV, nnz=4, B=1, Hq=4, Hkv=2,
           N=512, d=128, scale=0.1, causal=0):
    return lib.fa_fwd_block_sparse(dt, q, k, v, o, None, None, offs, idx, nnz, B, Hq, Hkv, N, d,
                                   scale, causal, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dt=3), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(dt=0), fa.FA_ERR_UNSUPPORTED),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(nnz=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(N=-5), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(offs=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(idx=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(v=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(k=MIS), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(N=1 << 25), fa.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 23), fa.FA_ERR_UNSUPPORTED),         # N d = 2^30: past 2^30 bytes per head
    (dict(N=(1 << 22) + 1), fa.FA_ERR_UNSUPPORTED),
    (dict(N=(1 << 23) + 1, d=64), fa.FA_ERR_UNSUPPORTED),
    (dict(N=0, q=NULL), fa.FA_OK),
])
def test_fwd_block_sparse_validation(kwargs, code):
    assert sparse(fa.load_library(), **kwargs) == code


def fp8(lib, vdt=1, q=DEV, k=DEV, v=DEV, o=DEV, B=1, Hq=4, Hkv=2, N=300, d=128, scale=0.1, causal=1):
    return lib.fa_fwd_fp8(vdt, q, k, v, o, None, None, B, Hq, Hkv, N, d, scale, causal, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(vdt=0), fa.FA_ERR_INVALID_ARGUMENT),      # float32 V: no such variant
    (dict(vdt=9), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(vdt=2, d=64), fa.FA_ERR_UNSUPPORTED),
    (dict(vdt=2, N=(1 << 22) + 1), fa.FA_ERR_UNSUPPORTED),
    (dict(vdt=2, k=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(vdt=2, N=0, q=NULL), fa.FA_OK),
    (dict(d=64), fa.FA_ERR_UNSUPPORTED),
    (dict(Hq=3, Hkv=2), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(B=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(k=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(v=MIS), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(N=1 << 23), fa.FA_ERR_UNSUPPORTED),
    (dict(N=(1 << 22) + 1), fa.FA_ERR_UNSUPPORTED),
    (dict(N=0, q=NULL), fa.FA_OK),
])
def test_fwd_fp8_validation(kwargs, code):
    assert fp8(fa.load_library(), **kwargs) == code


def bwd(lib, dt=1, q=DEV, k=DEV, v=DEV, o=DEV, do=DEV, m=DEV, l=DEV, dq=DEV, dk=DEV, dv=DEV,
        B=1, Hq=4, Hkv=2, N=300, d=128, scale=0.1, causal=1, ws=DEV, ws_bytes=1 << 20):
    return lib.fa_bwd(dt, q, k, v, o, do, m, l, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal, ws,
                      ws_bytes, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dt=4), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(dt=0), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Hq=5, Hkv=2), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(N=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(do=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(l=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(dk=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(ws=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(dq=MIS), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=2 * 4 * 300 * 4 - 1), fa.FA_ERR_WORKSPACE_TOO_SMALL),
    (dict(N=1 << 23), fa.FA_ERR_UNSUPPORTED),            # N d = 2^30
    (dict(N=1 << 23, d=64), fa.FA_ERR_WORKSPACE_TOO_SMALL),  # N d = 2^29 passes the size check
    (dict(B=0, q=NULL), fa.FA_OK),
])
def test_bwd_validation(kwargs, code):
    assert bwd(fa.load_library(), **kwargs) == code


def test_bwd_workspace_bytes():
    assert fa.fa_bwd_workspace_bytes(2, 8, 1000) == 2 * 2 * 8 * 1024 * 4  # rows padded to 32
    assert fa.fa_bwd_workspace_bytes(1, 1, 32) == 2 * 32 * 4
    assert fa.fa_bwd_workspace_bytes(-1, 8, 10) == 0


def merge(lib, dt=0, op=DEV, mp=DEV, lp=DEV, o=DEV, S=4, R=8, d=128):
    return lib.fa_merge(dt, op, mp, lp, o, None, None, S, R, d, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(dt=9), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(S=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(R=-1), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(d=0), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(d=2048), fa.FA_ERR_UNSUPPORTED),
    (dict(op=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(o=NULL), fa.FA_ERR_INVALID_ARGUMENT),
    (dict(R=0, op=NULL, o=NULL), fa.FA_OK),
])
def test_merge_validation(kwargs, code):
    assert merge(fa.load_library(), **kwargs) == code


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, q, q)


@pytest.mark.parametrize("which", ["k", "v", "o", "dout"])
def test_bwd_binding_rejects_mixed_dtypes(which):
    """fa_bwd reads every tensor as q's dtype (bf16): another dtype is refused on the host."""
    import torch

    t = {n: torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16) for n in ("q", "k", "v", "o", "dout")}
    t[which] = t[which].to(torch.float16)
    m = torch.zeros(1, 2, 8, dtype=torch.float32)
    with pytest.raises(TypeError, match=which):
        fa.fa_bwd(t["q"], t["k"], t["v"], t["o"], t["dout"], m, m.clone())
    t[which] = t[which].to(torch.uint8)
    with pytest.raises(TypeError):
        fa.fa_bwd(t["q"], t["k"], t["v"], t["o"], t["dout"], m, m.clone())


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        fa.load_library(str(tmp_path / "libfa.so"))


def test_decode_noalloc_limits():
    """The allocation-free decode rejects, before any HIP call, a request whose partials would
    not fit its static scratch, and validates like fa_decode_splitk."""
    lib = fa.load_library()
    cap = fa.fa_decode_noalloc_max_bytes()
    assert cap == 16 << 20

    def noalloc(**kw):
        a = dict(dt=1, q=DEV, kc=DEV, vc=DEV, table=DEV, lens=DEV, o=DEV, B=2, Hq=8, Hkv=2, d=128,
                 page=16, num_pages=10, max_pages=5, max_len=80, scale=0.08, splits=0)
        a.update(kw)
        return lib.fa_decode_splitk_noalloc(a["dt"], a["q"], a["kc"], a["vc"], a["table"],
                                            a["lens"], a["o"], a["B"], a["Hq"], a["Hkv"], a["d"],
                                            a["page"], a["num_pages"], a["max_pages"],
                                            a["max_len"], a["scale"], a["splits"], None)

    # 64 sequences x 64 query heads x 64 chunks of 130 floats: 136 MB of partials
    big = dict(B=64, Hq=64, Hkv=8, max_pages=4096, max_len=65536, splits=64)
    assert fa.fa_decode_workspace_bytes(64, 64, 128, 16, 65536, 64) > cap
    assert noalloc(**big) == fa.FA_ERR_WORKSPACE_TOO_SMALL
    assert noalloc(dt=0) == fa.FA_ERR_UNSUPPORTED
    assert noalloc(Hq=7) == fa.FA_ERR_INVALID_ARGUMENT
    assert noalloc(q=NULL) == fa.FA_ERR_INVALID_ARGUMENT
    assert noalloc(kc=MIS) == fa.FA_ERR_INVALID_ARGUMENT
    assert noalloc(B=0, q=NULL, o=NULL) == fa.FA_OK
