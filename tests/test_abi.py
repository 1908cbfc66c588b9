"""The C-ABI library: loads, exports every symbol include/*.h declares, sizes workspaces and
rejects bad arguments with status codes (CPU only: no call here reaches a GPU)."""
from __future__ import annotations

import ctypes
import glob
import os
import re

import pytest

import chunked_kimi_delta_amd as kda
from chunked_kimi_delta_amd import _lib
from chunked_kimi_delta_amd._lib import KdaFwdArgs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.library_path()):
        from chunked_kimi_delta_amd.build import build
        build()
    return kda.load()


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(kda_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    assert declared_functions() == ["kda_bwd", "kda_bwd_workspace_bytes", "kda_fwd",
                                    "kda_fwd_noalloc", "kda_fwd_prepare", "kda_fwd_state",
                                    "kda_fwd_workspace_bytes", "kda_strerror", "kda_version"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def args(**kw):
    a = KdaFwdArgs()
    d = dict(B=1, T=4096, N=1, H=16, HV=16, K=128, V=128, io=0, chunk=16)
    d.update(kw)
    for key, val in d.items():
        setattr(a, key, val)
    return a


def split_bytes(records, units, K, T, a_permille=580):
    """Workspace of the two-segment 32-token state pass: the chunk records, then (each
    256-aligned) the state after segment A and segment B's K x K transition (fp16 operand
    fragments), segment B's end state from zero (fp32), segment B's output fragments and the
    transition's output fragments (both fp16)."""
    al = lambda x: (x + 255) // 256 * 256
    nc = (T + 31) // 32
    c0 = min(max((nc * a_permille + 500) // 1000, 1), nc - 1)
    nb = nc - c0
    return (al(records) + al(units * K * K * 2) + al(units * K * K * 2) +
            al(units * K * K * 4) + al(units * nb * 32 * K * 2) + al(units * nb * 32 * K * 2))


def test_two_segment_plan_boundaries(lib):
    # the two-segment state pass (and its scratch) applies exactly to bf16 io, 32-token chunks,
    # dense sequences of at least 512 tokens, K == V, and at most CUs / 2 (without a device the
    # library assumes 256 CUs) sixteen-column slices N * HV * V / 16
    f = lambda **kw: lib.kda_fwd_workspace_bytes(ctypes.byref(args(**kw)))
    # 32-token record bytes: W, QD, KR (64 K each), -U (64 V), the two Mqk blocks (1,536)
    # and e^gam (4 K), rounded up to 256
    rb = lambda K, V: (192 * K + 64 * V + 1536 + 4 * K + 255) // 256 * 256
    rec = lambda T, HV, K=128, V=128, N=1: ((N * T) // 32 + N) * HV * rb(K, V)
    assert rb(128, 128) == 34816
    assert f(chunk=32, T=512) == split_bytes(rec(512, 16), 16, 128, 512)
    assert f(chunk=32, T=511) == rec(511, 16)                      # fewer than 16 chunks
    assert f(chunk=32, H=16, HV=16) > rec(4096, 16)                 # 256 slices: split
    assert f(chunk=32, H=17, HV=17) == rec(4096, 17)                # 272 slices: one segment
    assert f(chunk=32, H=8, HV=32, K=64, V=64) == split_bytes(rec(4096, 32, 64, 64), 32, 64,
                                                              4096)  # 32 x 4 slices x 2
    assert f(chunk=32, K=64, V=128, H=4, HV=4) == rec(4096, 4, 64, 128)   # K != V
    assert f(chunk=32, B=2, N=2, H=8, HV=8) == split_bytes(rec(4096, 8, N=2), 16, 128, 4096)
    assert f(chunk=16) == (4096 // 16 + 1) * 16 * 17408            # other chunks: no split
    assert f(chunk=64) == (4096 // 64 + 1) * 16 * 2 * 36864
    assert f(io=1, chunk=16) == (4096 // 16 + 1) * 16 * 34304


def test_workspace_bytes(lib):
    f = lambda a: lib.kda_fwd_workspace_bytes(ctypes.byref(a))
    assert f(args()) == (4096 // 16 + 1) * 16 * 17408
    assert f(args(K=64, V=64)) == (4096 // 16 + 1) * 16 * 8960
    assert f(args(io=1)) == (4096 // 16 + 1) * 16 * 34304
    assert f(args(B=4, T=8192, N=4, H=16, HV=32)) == (4 * 8192 // 16 + 4) * 32 * 17408
    assert f(args(T=45, N=1)) == (45 // 16 + 1) * 16 * 17408
    # 16 x 4096 at chunk 32 fills at most half of the (fallback, without a device: 256) compute
    # units, so the state pass runs as two segments whose scratch follows the records
    assert f(args(chunk=32)) == split_bytes((4096 // 32 + 1) * 16 * 34816, 16, 128, 4096)
    assert f(args(chunk=0)) == f(args(chunk=32))          # bf16 default: 32-token chunks
    assert f(args(io=1, chunk=0)) == f(args(io=1, chunk=16))
    assert f(args(chunk=32, T=45)) == (45 // 32 + 1) * 16 * 34816
    assert f(args(io=1, chunk=32)) == 0                   # fp32 io: 16-token chunks only
    assert f(args(chunk=1)) == 0 and f(args(io=1, chunk=1)) == 0   # recurrent: no workspace
    assert f(args(T=16, chunk=0)) == 0 and f(args(T=17, chunk=0)) > 0   # default, short batch
    assert f(args(chunk=64)) == (4096 // 64 + 1) * 16 * 2 * 36864   # pairs of 32-token records
    assert f(args(io=1, chunk=64)) == 0                   # fp32 io: 16-token chunks only
    assert f(args(chunk=128)) == 0
    assert f(args(K=96)) == 0          # unsupported head dim
    assert f(args(HV=24, H=16)) == 0   # HV % H != 0
    assert f(args(N=2)) == 0           # dense batch needs N == B
    assert f(args(B=0)) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(K=96), _lib.KDA_ERR_UNSUPPORTED),
    (dict(V=32), _lib.KDA_ERR_UNSUPPORTED),
    (dict(io=7), _lib.KDA_ERR_UNSUPPORTED),
    (dict(chunk=8), _lib.KDA_ERR_UNSUPPORTED),
    (dict(io=1, chunk=32), _lib.KDA_ERR_UNSUPPORTED),
    (dict(chunk=1, K=96), _lib.KDA_ERR_UNSUPPORTED),
    (dict(chunk=1, HV=24), _lib.KDA_ERR_INVALID_ARG),
    (dict(chunk=1), _lib.KDA_ERR_INVALID_ARG),     # null tensor pointers, no workspace needed
    (dict(HV=24), _lib.KDA_ERR_INVALID_ARG),
    (dict(N=3), _lib.KDA_ERR_INVALID_ARG),
    (dict(T=-1), _lib.KDA_ERR_INVALID_ARG),
    (dict(), _lib.KDA_ERR_INVALID_ARG),            # null tensor pointers
])
def test_kda_fwd_rejects_bad_arguments(lib, kw, status):
    a = args(**kw)
    for fn in (lib.kda_fwd, lib.kda_fwd_prepare, lib.kda_fwd_state):
        assert fn(ctypes.byref(a), None, 0, None) == status


def test_kda_fwd_checks_alignment_and_workspace(lib):
    a = args(T=32)
    fake = 1 << 40                                # never dereferenced: rejected before launch
    for name in ("q", "k", "v", "g", "beta", "o"):
        setattr(a, name, fake)
    assert lib.kda_fwd(ctypes.byref(a), None, 0, None) == _lib.KDA_ERR_WORKSPACE
    need = lib.kda_fwd_workspace_bytes(ctypes.byref(a))
    assert lib.kda_fwd(ctypes.byref(a), ctypes.c_void_p(fake), need - 1, None) == \
        _lib.KDA_ERR_WORKSPACE
    assert lib.kda_fwd(ctypes.byref(a), ctypes.c_void_p(fake + 16), need, None) == \
        _lib.KDA_ERR_WORKSPACE                   # workspace must be 256-byte aligned
    a.q = fake + 8                                # 16-byte alignment of tensors
    assert lib.kda_fwd(ctypes.byref(a), ctypes.c_void_p(fake), need, None) == \
        _lib.KDA_ERR_INVALID_ARG
    b = args(T=32, B=2, N=1)
    b.cu_seqlens = fake                           # varlen requires B == 1
    assert lib.kda_fwd(ctypes.byref(b), None, 0, None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_fwd(None, None, 0, None) == _lib.KDA_ERR_INVALID_ARG


def test_strerror_and_version(lib):
    for st in range(5):
        assert kda._lib.strerror(st)
    assert "unknown" in kda._lib.strerror(99)
    assert lib.kda_version() == 105


def test_product_path_has_no_fallback(monkeypatch, tmp_path):
    # with the library missing, the binding raises instead of computing anything itself
    monkeypatch.setenv("KDA_FWD_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        kda.load()


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "chunked_kimi_delta_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if os.path.isfile(path) and path.endswith((".py", ".hip", ".h", ".cpp")):
            src = open(path, encoding="utf-8").read()
            assert not re.search(r"^\s*(from|import)\s+oracle", src, flags=re.M), path
            assert "kda_oracle" not in src, path


def test_prestage_arguments_are_checked(lib):
    # gate validation comes before the workspace check (fake, never dereferenced pointers)
    fake = 1 << 40
    def mk(**kw):
        a = args(T=32, **kw)
        for name in ("q", "k", "v", "g", "beta", "o"):
            setattr(a, name, fake)
        return a
    call = lambda a: lib.kda_fwd(ctypes.byref(a), None, 0, None)
    assert call(mk(gate=3)) == _lib.KDA_ERR_UNSUPPORTED
    assert call(mk(gate=1)) == _lib.KDA_ERR_INVALID_ARG                 # no A_log
    assert call(mk(gate=2, A_log=fake, gate_lower_bound=0.5)) == _lib.KDA_ERR_INVALID_ARG
    assert call(mk(gate=2, A_log=fake, gate_lower_bound=float("nan"))) == \
        _lib.KDA_ERR_INVALID_ARG
    assert call(mk(gate=1, A_log=fake, dt_bias=fake + 4)) == _lib.KDA_ERR_INVALID_ARG
    # valid pre-stage arguments reach the workspace check
    assert call(mk(gate=2, A_log=fake, gate_lower_bound=-5.0, dt_bias=fake, qk_l2norm=1,
                   beta_sigmoid=1)) == _lib.KDA_ERR_WORKSPACE
    assert call(mk(gate=1, A_log=fake + 4)) == _lib.KDA_ERR_WORKSPACE
    # the workspace size does not depend on the pre-stage
    f = lambda a: lib.kda_fwd_workspace_bytes(ctypes.byref(a))
    assert f(mk(gate=1, A_log=fake, qk_l2norm=1)) == f(mk())


def test_bwd_workspace_bytes(lib):
    f = lambda a: lib.kda_bwd_workspace_bytes(ctypes.byref(a))
    up = lambda x: (x + 255) // 256 * 256
    for kw in (dict(), dict(K=64, V=128), dict(B=2, N=2, T=45, H=4, HV=8, K=64, V=64),
               dict(io=1, chunk=0)):
        a = args(**kw)
        B, T, N, H, HV, K, V = (getattr(a, n) for n in ("B", "T", "N", "H", "HV", "K", "V"))
        slots = B * T // 16 + N
        # the forward's fp32 record plus the inverse and the Gram (two 16 x 16 fp32 blocks)
        # and the chunk's dO (16 x V fp32)
        rec = lib.kda_fwd_workspace_bytes(ctypes.byref(args(**dict(kw, io=1, chunk=16))))
        rec += slots * HV * (2048 + 16 * V * 4)
        part = B * T * HV * K * 4 if HV > H else 0
        assert f(a) == up(rec) + 2 * up(slots * HV * K * V * 4) + 2 * up(part), kw
    base = f(args())
    slots = 4096 // 16 + 1
    assert f(args(qk_l2norm=1)) == base + 2 * up(4096 * 16 * 128 * 4)     # dq, dk partials
    assert f(args(gate=1)) == base + up(slots * 16 * 4) + up(slots * 16 * 128 * 4)
    assert f(args(beta_sigmoid=1)) == base
    assert f(args(chunk=32)) == 0 and f(args(chunk=1)) == 0     # 16-token chunks only
    assert f(args(K=96)) == 0 and f(args(HV=24)) == 0


def test_kda_bwd_rejects_bad_arguments(lib):
    fake = 1 << 40                                 # never dereferenced: rejected before launch
    call = lambda a, **kw: lib.kda_bwd(
        ctypes.byref(a), kw.get("do"), kw.get("dht"), kw.get("ws"), kw.get("nbytes", 0),
        *[kw.get(n, fake) for n in ("dq", "dk", "dv", "dg", "dbeta")], kw.get("dh0"),
        kw.get("dA"), kw.get("ddt"), None)
    a = args(T=32)
    assert call(a, do=fake) == _lib.KDA_ERR_INVALID_ARG          # null q, k, v, g, beta
    for name in ("q", "k", "v", "g", "beta"):
        setattr(a, name, fake)
    assert call(a) == _lib.KDA_ERR_INVALID_ARG                   # null d_o
    assert call(a, do=fake, dq=None) == _lib.KDA_ERR_INVALID_ARG  # null output
    assert call(a, do=fake, dh0=fake + 4) == _lib.KDA_ERR_INVALID_ARG
    assert call(a, do=fake) == _lib.KDA_ERR_WORKSPACE
    need = lib.kda_bwd_workspace_bytes(ctypes.byref(a))
    assert call(a, do=fake, ws=fake, nbytes=need - 1) == _lib.KDA_ERR_WORKSPACE
    assert call(a, do=fake, ws=fake + 16, nbytes=need) == _lib.KDA_ERR_WORKSPACE
    assert call(args(T=32, chunk=32), do=fake) == _lib.KDA_ERR_UNSUPPORTED
    pre = args(T=32, gate=1, A_log=fake)
    for name in ("q", "k", "v", "g", "beta"):
        setattr(pre, name, fake)
    assert call(pre, do=fake) == _lib.KDA_ERR_INVALID_ARG          # a gate needs dA_log
    assert call(pre, do=fake, dA=fake + 2) == _lib.KDA_ERR_INVALID_ARG
    assert call(pre, do=fake, dA=fake, ddt=fake + 4) == _lib.KDA_ERR_INVALID_ARG
    assert call(pre, do=fake, dA=fake) == _lib.KDA_ERR_WORKSPACE
    pre.gate = 3
    assert call(pre, do=fake, dA=fake) == _lib.KDA_ERR_UNSUPPORTED
    assert call(args(T=32, K=96), do=fake) == _lib.KDA_ERR_UNSUPPORTED
    assert call(args(T=32, N=2), do=fake) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_bwd(None, None, None, None, 0, *([None] * 8), None) == \
        _lib.KDA_ERR_INVALID_ARG


def test_noalloc_rejects_before_any_device_work(lib):
    # both rejections return before the entry point touches a device
    assert lib.kda_fwd_noalloc(None, None) == _lib.KDA_ERR_INVALID_ARG
    big = args(B=1, T=131072, N=1, H=32, HV=32, chunk=32)
    assert lib.kda_fwd_workspace_bytes(ctypes.byref(big)) > _lib.KDA_NOALLOC_WORKSPACE_BYTES
    assert lib.kda_fwd_noalloc(ctypes.byref(big), None) == _lib.KDA_ERR_NOALLOC_TOO_LARGE
    assert "static device array" in lib.kda_strerror(_lib.KDA_ERR_NOALLOC_TOO_LARGE).decode()
    # the array holds the throughput workload's records (16 heads x 4096 tokens, chunk 32)
    assert lib.kda_fwd_workspace_bytes(ctypes.byref(args(chunk=32))) <= \
        _lib.KDA_NOALLOC_WORKSPACE_BYTES
