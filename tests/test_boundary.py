"""CPU tests of the C-ABI boundary: the library loads, exports every entry
point include/kda.h declares, and rejects invalid arguments with the
documented status codes before making any HIP call (no compute, no GPU)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import kimi_delta_attention_04_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
FAKE = 0x100000          # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.library_path):
        from kimi_delta_attention_04_amd import _build
        _build.build()
    return kda.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "kda_fwd" in names and "kda_status_string" in names
    out = subprocess.run(["nm", "-D", "--defined-only", kda.library_path],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kda_\w+)", out))
    for n in names:
        assert n in exported, f"{n} declared in kda.h but not exported"
        assert hasattr(lib, n)


def test_status_strings(lib):
    for code, name in ((0, "KDA_OK"), (1, "KDA_ERR_INVALID_ARG"), (2, "KDA_ERR_UNSUPPORTED"),
                       (3, "KDA_ERR_LAUNCH"), (4, "KDA_ERR_OUT_OF_MEMORY")):
        assert kda.status_string(code) == name
    assert kda.status_string(99) == "KDA_ERR_UNKNOWN"


def test_constants(lib):
    assert kda.chunk_size() == 16
    lb = kda.lower_bound_min()
    # 16 tokens at the bound keep 2^(+-G) inside the fp32 normal range
    assert -5.5 < lb <= -5.0
    assert 16 * abs(lb) * 1.4426950408889634 < 126


def test_workspace_size(lib):
    # 16-token chunks with 13 KB records at K = 128
    assert kda.workspace_size(1, 8192, 96, 1) == (8192 // 16 + 1) * 96 * 13312
    assert kda.workspace_size(1, 8192, 96, 12) == (8192 // 16 + 12) * 96 * 13312
    assert kda.workspace_size(3, 37, 2, 3) == (111 // 16 + 3) * 2 * 13312
    assert kda.workspace_size(0, 16, 1, 1) == 0
    assert kda.workspace_size(1, 16, 1, 0) == 0
    # head dimension 64 takes 7 KB records, 256 26 KB ones
    assert kda.workspace_size(1, 8192, 96, 1, K=64) == (8192 // 16 + 1) * 96 * 7168
    assert kda.workspace_size(1, 8192, 96, 1, K=256) == (8192 // 16 + 1) * 96 * 26624
    assert kda.workspace_size(1, 8192, 96, 1, K=96) == 0
    assert lib.kda_workspace_size(1, 100, 3, 1) == kda.workspace_size(1, 100, 3, 1, K=128)


def call_fwd(lib, entry="kda_fwd", **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.088, A_log=FAKE, dt_bias=None,
             lb=-5.0, cu=None, N=1, init=None, init_dt=0, fin=None, fin_dt=1, out=FAKE,
             B=1, T=32, H=2, K=128, V=128)
    a.update(over)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return getattr(lib, entry)(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]), a["scale"],
                       P(a["A_log"]), P(a["dt_bias"]), a["lb"], P(a["cu"]), a["N"],
                       P(a["init"]), a["init_dt"], P(a["fin"]), a["fin_dt"], P(a["out"]),
                       a["B"], a["T"], a["H"], a["K"], a["V"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(g=None), INVALID), (dict(beta=None), INVALID), (dict(A_log=None), INVALID),
    (dict(out=None), INVALID),
    (dict(q=FAKE + 8), INVALID), (dict(out=FAKE + 2), INVALID), (dict(beta=FAKE + 1), INVALID),
    (dict(A_log=FAKE + 2), INVALID), (dict(init=FAKE + 4), INVALID),
    (dict(K=64), UNSUPPORTED), (dict(V=256), UNSUPPORTED), (dict(K=256, V=128), UNSUPPORTED),
    (dict(K=64, V=128), UNSUPPORTED), (dict(K=32, V=32), UNSUPPORTED),
    (dict(K=512, V=512), UNSUPPORTED), (dict(K=192, V=192), UNSUPPORTED),
    (dict(B=0), INVALID), (dict(T=-1), INVALID), (dict(H=0), INVALID),
    (dict(N=2), INVALID),                              # fixed length needs N == B
    (dict(cu=FAKE, B=2, N=2), INVALID),                # cu_seqlens needs B == 1
    (dict(cu=FAKE, N=0), INVALID),
    (dict(init_dt=7), INVALID), (dict(fin_dt=-1), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(lb=float("nan")), INVALID), (dict(lb=float("-inf")), INVALID),
    (dict(lb=0.5), INVALID), (dict(lb=-6.0), UNSUPPORTED), (dict(lb=-100.0), UNSUPPORTED),
    (dict(B=2, N=2, T=2 ** 30 + 1), UNSUPPORTED),       # token rows overflow int32
    (dict(H=2 ** 26), UNSUPPORTED),                     # (sequence, head) units overflow the grid
    (dict(H=2 ** 19), UNSUPPORTED),                     # 16-row byte offsets overflow int32
    (dict(T=2 ** 26, H=1024), UNSUPPORTED),             # (chunk slot, head) pairs overflow the grid
])
def test_fwd_rejects_before_any_hip_call(lib, over, code):
    assert call_fwd(lib, **over) == code
    # the allocation-free entry point validates the same way
    assert call_fwd(lib, entry="kda_fwd_noalloc", **over) == code


@pytest.mark.parametrize("over", [dict(T=8192, H=96), dict(T=8192, H=10), dict(B=4, N=4, T=4096, H=5)])
def test_noalloc_rejects_workspace_beyond_its_array(lib, over):
    """kda_fwd_noalloc rejects, before any HIP call, calls whose workspace
    exceeds KDA_NOALLOC_WORKSPACE_BYTES (64 MiB)."""
    a = dict(B=1, N=1, K=128)
    a.update(over)
    assert kda.workspace_size(a["B"], a["T"], a["H"], a["N"]) > 64 << 20
    assert call_fwd(lib, entry="kda_fwd_noalloc", **over) == UNSUPPORTED


@pytest.mark.parametrize("over,code", [
    (dict(g=None), INVALID), (dict(g=FAKE + 1), INVALID), (dict(K=64), UNSUPPORTED),
    (dict(lb=-6.0), UNSUPPORTED), (dict(cu=FAKE, B=2), INVALID),
])
def test_scalar_gate_rejects_before_any_hip_call(lib, over, code):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE + 2, beta=FAKE, scale=0.088, A_log=FAKE, dt_bias=None,
             lb=-5.0, cu=None, N=1, init=None, init_dt=0, fin=None, fin_dt=1, out=FAKE,
             B=1, T=32, H=2, K=128, V=128)
    a.update(over)
    if "cu" in over:
        a["N"] = 1
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    rc = lib.kda_fwd_scalar_gate(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]), a["scale"],
                                 P(a["A_log"]), P(a["dt_bias"]), a["lb"], P(a["cu"]), a["N"],
                                 P(a["init"]), a["init_dt"], P(a["fin"]), a["fin_dt"], P(a["out"]),
                                 a["B"], a["T"], a["H"], a["K"], a["V"], None)
    assert rc == code


def call_decode(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.088, A_log=FAKE, dt_bias=None,
             lb=-5.0, state=FAKE, st_dt=1, out=FAKE, N=4, H=2, K=128, V=128)
    a.update(over)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.kda_decode(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]), a["scale"],
                          P(a["A_log"]), P(a["dt_bias"]), a["lb"], P(a["state"]), a["st_dt"],
                          P(a["out"]), a["N"], a["H"], a["K"], a["V"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), INVALID), (dict(state=None), INVALID), (dict(out=None), INVALID),
    (dict(A_log=None), INVALID), (dict(beta=FAKE + 1), INVALID), (dict(state=FAKE + 8), INVALID),
    (dict(st_dt=2), INVALID), (dict(scale=float("nan")), INVALID), (dict(lb=0.5), INVALID),
    (dict(lb=float("-inf")), INVALID), (dict(N=0), INVALID), (dict(H=0), INVALID),
    (dict(K=64), UNSUPPORTED), (dict(V=256), UNSUPPORTED), (dict(K=96, V=96), UNSUPPORTED),
    (dict(K=512, V=512), UNSUPPORTED), (dict(N=2 ** 20, H=2 ** 12), UNSUPPORTED),
])
def test_decode_rejects_before_any_hip_call(lib, over, code):
    assert call_decode(lib, **over) == code


def test_debug_intra_validates(lib):
    P = ctypes.c_void_p
    f = lambda **o: lib.kda_debug_intra(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None,
                                        o.get("lb", -5.0), None, 1, 1, 16, 1, o.get("K", 128),
                                        o.get("ws", P(FAKE)), None)
    assert f(K=512) == UNSUPPORTED and f(K=32) == UNSUPPORTED
    assert f(lb=-7.0) == UNSUPPORTED
    assert f(ws=None) == INVALID


def test_debug_gate_validates(lib):
    P = ctypes.c_void_p
    f = lambda **o: lib.kda_debug_gate(P(FAKE), P(FAKE), P(FAKE), None, o.get("lb", -5.0), None,
                                       1, o.get("G", P(FAKE)), P(FAKE), 1, o.get("T", 16), 1,
                                       o.get("K", 128), None)
    assert f(K=512) == UNSUPPORTED and f(K=32) == UNSUPPORTED
    assert f(lb=-7.0) == UNSUPPORTED
    assert f(lb=0.5) == INVALID and f(lb=float("nan")) == INVALID
    assert f(G=None) == INVALID
    assert f(G=P(FAKE + 4)) == INVALID                      # G must be 16-byte aligned
    assert f(T=0, G=None) == OK                             # no tokens: nothing to write or launch


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import kimi_delta_attention_04_amd as mod
    monkeypatch.setattr(mod, "_lib", None)
    monkeypatch.setattr(mod, "library_path", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        mod.load()


def call_bwd(lib, scalar_gate=False, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=0.088, A_log=FAKE, dt_bias=None,
             lb=-5.0, cu=None, N=1, init=None, init_dt=0, dout=FAKE, dfin=None,
             dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, dbeta=FAKE, dA_log=FAKE, ddtb=None, dinit=None,
             B=1, T=32, H=2, K=128, V=128)
    a.update(over)
    P = lambda x: None if x is None else ctypes.c_void_p(x)
    fn = lib.kda_bwd_scalar_gate if scalar_gate else lib.kda_bwd
    return fn(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]), a["scale"],
              P(a["A_log"]), P(a["dt_bias"]), a["lb"], P(a["cu"]), a["N"],
              P(a["init"]), a["init_dt"], P(a["dout"]), P(a["dfin"]),
              P(a["dq"]), P(a["dk"]), P(a["dv"]), P(a["dg"]), P(a["dbeta"]),
              P(a["dA_log"]), P(a["ddtb"]), P(a["dinit"]),
              a["B"], a["T"], a["H"], a["K"], a["V"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), INVALID), (dict(dout=None), INVALID), (dict(dq=None), INVALID),
    (dict(dbeta=None), INVALID), (dict(dA_log=None), INVALID), (dict(A_log=None), INVALID),
    (dict(dk=FAKE + 8), INVALID), (dict(dinit=FAKE + 4), INVALID), (dict(dfin=FAKE + 4), INVALID),
    (dict(ddtb=FAKE + 2), INVALID), (dict(init_dt=5), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(lb=0.5), INVALID), (dict(lb=-6.0), UNSUPPORTED),
    (dict(K=96, V=96), UNSUPPORTED), (dict(K=512, V=512), UNSUPPORTED), (dict(V=64), UNSUPPORTED),
    (dict(K=256, V=128), UNSUPPORTED),
    (dict(N=2), INVALID), (dict(cu=FAKE, B=2, N=2), INVALID), (dict(H=0), INVALID),
    (dict(T=2 ** 26, H=1024), UNSUPPORTED),
])
def test_bwd_rejects_before_any_hip_call(lib, over, code):
    assert call_bwd(lib, **over) == code
    # the scalar-gate backward validates the same arguments the same way
    # (its g and dg need only 2-byte alignment)
    assert call_bwd(lib, scalar_gate=True, **over) == code


def test_bwd_scalar_gate_alignment(lib):
    assert call_bwd(lib, scalar_gate=True, g=FAKE + 1) == INVALID
    assert call_bwd(lib, scalar_gate=True, dg=FAKE + 1) == INVALID
    assert call_bwd(lib, g=FAKE + 2) == INVALID
