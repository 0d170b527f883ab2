"""Python binding of libkda (Kimi Delta Attention forward on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C-ABI declared in include/kda.h.  PyTorch supplies device
memory and the current HIP stream.  If the built library is missing the
binding raises; there is no fallback implementation.

    fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
        initial_state=None, final_state=None, cu_seqlens=None)

mirrors the flash_kda.fwd argument list described in "Moonshot AI Rilis
FlashKDA" (API paragraphs);

    fwd_scalar_gate(...)   the same with one gate value per token and head
                           (the Gated DeltaNet case): g [B, T, H], dt_bias [H]
    decode(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, state)

applies one new token per sequence to the recurrent state in place;

    bwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, d_out, ...)

computes the gradients of the forward (training).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["attention", "fwd", "fwd_noalloc", "fwd_scalar_gate", "decode", "bwd", "bwd_scalar_gate", "debug_gate", "debug_intra", "debug_scan_step", "set_stage_events", "set_bwd_stage_events", "workspace_size", "lower_bound_min", "chunk_size",
           "status_string", "KDAError", "library_path", "load", "HEAD_DIM"]

HEAD_DIM = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libkda.so")

KDA_DTYPE_BF16 = 0
KDA_DTYPE_FP32 = 1
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED",
           3: "KDA_ERR_LAUNCH", 4: "KDA_ERR_OUT_OF_MEMORY"}

_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def load():
    """Load libkda.so (built by __graft_entry__.build / _build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(f"libkda.so is not built ({library_path}); run "
                          "python -c 'import __graft_entry__ as g; g.build()'")
    # torch ships its own HIP runtime under the same soname; loading torch
    # first makes libkda bind to that one copy instead of a second runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(library_path)
    P, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.kda_fwd.restype = ctypes.c_int
    lib.kda_fwd.argtypes = [P, P, P, P, P, f32, P, P, f32, P, i32, P, ctypes.c_int, P,
                            ctypes.c_int, P, i32, i32, i32, i32, i32, P]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_lower_bound_min.restype = f32
    lib.kda_lower_bound_min.argtypes = []
    lib.kda_chunk_size.restype = i32
    lib.kda_chunk_size.argtypes = []
    lib.kda_workspace_size.restype = ctypes.c_size_t
    lib.kda_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.kda_workspace_size_hd.restype = ctypes.c_size_t
    lib.kda_workspace_size_hd.argtypes = [i32, i32, i32, i32, i32]
    lib.kda_set_stage_events.restype = ctypes.c_int
    lib.kda_set_stage_events.argtypes = [P, P, P]
    lib.kda_fwd_scalar_gate.restype = ctypes.c_int
    lib.kda_fwd_scalar_gate.argtypes = lib.kda_fwd.argtypes
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode.argtypes = [P, P, P, P, P, f32, P, P, f32, P, ctypes.c_int, P, i32, i32, i32, i32, P]
    lib.kda_set_bwd_stage_events.restype = ctypes.c_int
    lib.kda_set_bwd_stage_events.argtypes = [P]
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_bwd.argtypes = [P, P, P, P, P, f32, P, P, f32, P, i32, P, ctypes.c_int, P, P,
                            P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, P]
    lib.kda_bwd_scalar_gate.restype = ctypes.c_int
    lib.kda_bwd_scalar_gate.argtypes = lib.kda_bwd.argtypes
    lib.kda_debug_gate.restype = ctypes.c_int
    lib.kda_debug_gate.argtypes = [P, P, P, P, f32, P, i32, P, P, i32, i32, i32, i32, P]
    lib.kda_debug_intra.restype = ctypes.c_int
    lib.kda_debug_intra.argtypes = [P, P, P, P, P, P, f32, P, i32, i32, i32, i32, i32, P, P]
    lib.kda_debug_scan_step.restype = ctypes.c_int
    lib.kda_debug_scan_step.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, f32, P, ctypes.c_int,
                                        P, ctypes.c_int, P, i32, P]
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_fwd_noalloc.argtypes = lib.kda_fwd.argtypes
    lib.kda_record_workspace_size.restype = ctypes.c_size_t
    lib.kda_record_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.kda_trim_workspace.restype = ctypes.c_int
    lib.kda_trim_workspace.argtypes = [ctypes.c_size_t]
    lib.kda_workspace_reserved.restype = ctypes.c_size_t
    lib.kda_workspace_reserved.argtypes = []
    _lib = lib
    return lib


# The sources the forward kernels (intra stage and scan) are compiled from,
# and those of the backward kernels.
FORWARD_KERNEL_SOURCES = ("kda_device.h", "kda_intra_dev.h", "kda_intra.hip", "kda_scan_dev.h", "kda_scan.hip")
BACKWARD_KERNEL_SOURCES = ("kda_device.h", "kda_intra_dev.h", "kda_bwd_dev.h", "kda_bwd.hip",
                           "kda_scan_dev.h", "kda_bwd_scan.hip")


def source_digest(sources=FORWARD_KERNEL_SOURCES) -> str:
    """sha256 over the code of the given kernel sources (the forward's by
    default), comments and whitespace removed: identifies the kernels a
    stored profile was taken on."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(_HERE, "csrc")
    for name in sources:
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)     # block comments
        text = re.sub(r"//[^\n]*", " ", text)                   # line comments
        text = " ".join(text.split())
        h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()


def status_string(status: int) -> str:
    if _lib is not None:
        return _lib.kda_status_string(int(status)).decode()
    return _STATUS.get(int(status), "KDA_ERR_UNKNOWN")


def lower_bound_min() -> float:
    return float(load().kda_lower_bound_min())


def chunk_size() -> int:
    return int(load().kda_chunk_size())


def workspace_size(B: int, T: int, H: int, num_seqs: int, K: int = 128) -> int:
    """Bytes of the hand-off records of one forward call (head dimension K)."""
    return int(load().kda_workspace_size_hd(B, T, H, num_seqs, K))


def trim_workspace(keep_bytes: int = 0) -> None:
    """Return the library pool's unused reserved memory on the current
    device until at most keep_bytes stay reserved (kda_trim_workspace)."""
    st = load().kda_trim_workspace(int(keep_bytes))
    if st != 0:
        raise KDAError(st, "kda_trim_workspace")


def workspace_reserved() -> int:
    """Bytes the library pool holds reserved on the current device."""
    return int(load().kda_workspace_reserved())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, dtype, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _state_dtype(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t.dtype == torch.float32:
        return KDA_DTYPE_FP32
    raise TypeError(f"state tensors must be bf16 or fp32, got {t.dtype}")


def fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
        initial_state=None, final_state=None, cu_seqlens=None):
    """KDA forward into `out` (and `final_state` when given); returns out.

    q, k, g: bf16 [B, T, H, K]; v, out: bf16 [B, T, H, V]; beta: bf16
    [B, T, H] logits; A_log: fp32 [H]; dt_bias: fp32 [H*K] or None;
    initial_state / final_state: bf16 or fp32 [N, H, K, V] or None;
    cu_seqlens: int32 [N+1] (B == 1) or None.  Enqueued on the current stream.
    """
    return _fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                initial_state, final_state, cu_seqlens, scalar_gate=False)


def fwd_noalloc(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                initial_state=None, final_state=None, cu_seqlens=None):
    """As fwd, through kda_fwd_noalloc: the library allocates nothing (its
    workspace is a fixed device array of NOALLOC_WORKSPACE_BYTES); calls
    needing more workspace raise KDAError (KDA_ERR_UNSUPPORTED)."""
    return _fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                initial_state, final_state, cu_seqlens, scalar_gate=False, noalloc=True)


# kda.h: KDA_NOALLOC_WORKSPACE_BYTES
NOALLOC_WORKSPACE_BYTES = 64 << 20


def fwd_scalar_gate(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                    initial_state=None, final_state=None, cu_seqlens=None):
    """The Gated DeltaNet case: as fwd, but g is bf16 [B, T, H] (one gate
    value per token and head, shared by all channels) and dt_bias fp32 [H]
    or None."""
    return _fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                initial_state, final_state, cu_seqlens, scalar_gate=True)


def _fwd(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
         initial_state, final_state, cu_seqlens, scalar_gate, noalloc=False):
    import torch
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    bf = torch.bfloat16
    _check(q, "q", bf)
    _check(k, "k", bf, q.shape)
    _check(g, "g", bf, (B, T, H) if scalar_gate else q.shape)
    _check(v, "v", bf, (B, T, H, V))
    _check(out, "out", bf, (B, T, H, V))
    _check(beta, "beta", bf, (B, T, H))
    _check(A_log, "A_log", torch.float32, (H,))
    if dt_bias is not None:
        _check(dt_bias, "dt_bias", torch.float32, (H,) if scalar_gate else (H * K,))
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    init_dt = fin_dt = KDA_DTYPE_FP32
    if initial_state is not None:
        init_dt = _state_dtype(initial_state)
        _check(initial_state, "initial_state", initial_state.dtype, (N, H, K, V))
    if final_state is not None:
        fin_dt = _state_dtype(final_state)
        _check(final_state, "final_state", final_state.dtype, (N, H, K, V))
    name = "kda_fwd_scalar_gate" if scalar_gate else ("kda_fwd_noalloc" if noalloc else "kda_fwd")
    entry = getattr(lib, name)
    rc = entry(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
               _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(cu_seqlens), int(N),
               _ptr(initial_state), init_dt, _ptr(final_state), fin_dt, _ptr(out),
               int(B), int(T), int(H), int(K), int(V), _stream(q.device))
    if rc != 0:
        raise KDAError(rc, name)
    return out


def decode(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, state):
    """One decode step: the new token of each sequence applied to `state`
    (bf16 or fp32 [N, H, K, V]) in place; the output into `out`.

    q, k, g: bf16 [N, H, K]; v, out: bf16 [N, H, V]; beta: bf16 [N, H]
    logits; A_log: fp32 [H]; dt_bias: fp32 [H*K] or None.  Enqueued on the
    current stream; returns out.
    """
    import torch
    lib = load()
    if q.dim() != 3:
        raise ValueError("q must be [N, H, K]")
    N, H, K = q.shape
    V = v.shape[-1]
    bf = torch.bfloat16
    _check(q, "q", bf)
    _check(k, "k", bf, q.shape)
    _check(g, "g", bf, q.shape)
    _check(v, "v", bf, (N, H, V))
    _check(out, "out", bf, (N, H, V))
    _check(beta, "beta", bf, (N, H))
    _check(A_log, "A_log", torch.float32, (H,))
    if dt_bias is not None:
        _check(dt_bias, "dt_bias", torch.float32, (H * K,))
    st_dt = _state_dtype(state)
    _check(state, "state", state.dtype, (N, H, K, V))
    rc = lib.kda_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                        _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(state), st_dt,
                        _ptr(out), int(N), int(H), int(K), int(V), _stream(q.device))
    if rc != 0:
        raise KDAError(rc, "kda_decode")
    return out


def bwd_scalar_gate(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, d_out, dq, dk, dv,
                    dg, dbeta, dA_log, ddt_bias=None, initial_state=None, d_final_state=None,
                    d_initial_state=None, cu_seqlens=None):
    """The backward of fwd_scalar_gate: as bwd, but g and dg are bf16
    [B, T, H] (one gate value per token and head) and dt_bias, ddt_bias fp32
    [H] or None."""
    _bwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, d_out, dq, dk, dv, dg, dbeta,
         dA_log, ddt_bias, initial_state, d_final_state, d_initial_state, cu_seqlens,
         scalar_gate=True)


def bwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, d_out, dq, dk, dv, dg, dbeta,
        dA_log, ddt_bias=None, initial_state=None, d_final_state=None, d_initial_state=None,
        cu_seqlens=None):
    """Gradients of L = <d_out, o> + <d_final_state, final_state> of the
    forward with these inputs, written into the caller's tensors.

    Inputs as fwd (K = V = 64, 128 or 256); d_out: bf16 [B, T, H, V]; d_final_state:
    fp32 [N, H, K, V] or None.  Outputs: dq, dk, dg bf16 [B, T, H, K]; dv
    bf16 [B, T, H, V]; dbeta bf16 [B, T, H]; dA_log fp32 [H]; ddt_bias fp32
    [H*K] or None; d_initial_state fp32 [N, H, K, V] or None.  Enqueued on
    the current stream.
    """
    _bwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, d_out, dq, dk, dv, dg, dbeta,
         dA_log, ddt_bias, initial_state, d_final_state, d_initial_state, cu_seqlens,
         scalar_gate=False)


def _bwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, d_out, dq, dk, dv, dg, dbeta,
         dA_log, ddt_bias, initial_state, d_final_state, d_initial_state, cu_seqlens,
         scalar_gate):
    import torch
    lib = load()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    bf, f32 = torch.bfloat16, torch.float32
    gshape = (B, T, H) if scalar_gate else q.shape
    for t, name, shape in ((q, "q", None), (k, "k", q.shape), (g, "g", gshape),
                           (v, "v", (B, T, H, V)), (beta, "beta", (B, T, H)),
                           (d_out, "d_out", (B, T, H, V)), (dq, "dq", q.shape),
                           (dk, "dk", q.shape), (dg, "dg", gshape), (dv, "dv", (B, T, H, V)),
                           (dbeta, "dbeta", (B, T, H))):
        _check(t, name, bf, shape)
    _check(A_log, "A_log", f32, (H,))
    _check(dA_log, "dA_log", f32, (H,))
    for t, name in ((dt_bias, "dt_bias"), (ddt_bias, "ddt_bias")):
        if t is not None:
            _check(t, name, f32, (H,) if scalar_gate else (H * K,))
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    init_dt = KDA_DTYPE_FP32
    if initial_state is not None:
        init_dt = _state_dtype(initial_state)
        _check(initial_state, "initial_state", initial_state.dtype, (N, H, K, V))
    for t, name in ((d_final_state, "d_final_state"), (d_initial_state, "d_initial_state")):
        if t is not None:
            _check(t, name, f32, (N, H, K, V))
    fn = lib.kda_bwd_scalar_gate if scalar_gate else lib.kda_bwd
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(A_log),
                     _ptr(dt_bias), float(lower_bound), _ptr(cu_seqlens), int(N),
                     _ptr(initial_state), init_dt, _ptr(d_out), _ptr(d_final_state),
                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dA_log),
                     _ptr(ddt_bias), _ptr(d_initial_state), int(B), int(T), int(H), int(K),
                     int(V), _stream(q.device))
    if rc != 0:
        raise KDAError(rc, "kda_bwd_scalar_gate" if scalar_gate else "kda_bwd")


_attention_fn = None


def _attention_function():
    """The torch.autograd.Function behind attention(), made on first use
    (the module itself imports torch only when a call needs it)."""
    global _attention_fn
    if _attention_fn is not None:
        return _attention_fn
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens, scale,
                    lower_bound, output_final_state):
            scalar = g.dim() == 3                           # Gated DeltaNet form
            B, T, H, K = q.shape
            V = v.shape[-1]
            N = B if cu_seqlens is None else cu_seqlens.numel() - 1
            o = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=q.device)
            fs = None
            if output_final_state:
                fs = torch.empty((N, H, K, V), dtype=torch.float32, device=q.device)
            (fwd_scalar_gate if scalar else fwd)(
                q, k, v, g, beta, scale, o, A_log, dt_bias, lower_bound,
                initial_state=initial_state, final_state=fs, cu_seqlens=cu_seqlens)
            ctx.save_for_backward(q, k, v, g, beta, A_log, dt_bias, initial_state, cu_seqlens)
            ctx.scale, ctx.lower_bound, ctx.scalar = scale, lower_bound, scalar
            return o, fs

        @staticmethod
        def backward(ctx, d_o, d_fs):
            q, k, v, g, beta, A_log, dt_bias, init, cu = ctx.saved_tensors
            d_o = d_o.to(torch.bfloat16).contiguous()        # autograd passes zeros if unused
            d_fs = None if d_fs is None else d_fs.to(torch.float32).contiguous()
            dq, dk, dg = torch.empty_like(q), torch.empty_like(k), torch.empty_like(g)
            dv, dbeta, dA = torch.empty_like(v), torch.empty_like(beta), torch.empty_like(A_log)
            ddt = torch.empty_like(dt_bias) if dt_bias is not None else None
            dinit = None
            if init is not None and ctx.needs_input_grad[7]:
                dinit = torch.empty(init.shape, dtype=torch.float32, device=q.device)
            (bwd_scalar_gate if ctx.scalar else bwd)(
                q, k, v, g, beta, ctx.scale, A_log, dt_bias, ctx.lower_bound, d_o, dq, dk, dv,
                dg, dbeta, dA, ddt_bias=ddt, initial_state=init, d_final_state=d_fs,
                d_initial_state=dinit, cu_seqlens=cu)
            if dinit is not None:
                dinit = dinit.to(init.dtype)
            return dq, dk, dv, dg, dbeta, dA, ddt, dinit, None, None, None, None

    _attention_fn = _Attention
    return _attention_fn


def attention(q, k, v, g, beta, A_log, dt_bias, lower_bound, scale=None, initial_state=None,
              output_final_state=False, cu_seqlens=None):
    """Differentiable KDA: returns (o, final_state), o bf16 [B, T, H, V] and
    final_state fp32 [N, H, K, V] (None unless output_final_state), with
    gradients through kda_bwd for q, k, v, g, beta, A_log, dt_bias and
    initial_state.  Arguments as fwd; scale defaults to K^-1/2.  A gate g of
    shape [B, T, H] (dt_bias [H] or None) selects the Gated DeltaNet form
    (fwd_scalar_gate, bwd_scalar_gate)."""
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return _attention_function().apply(q, k, v, g, beta, A_log, dt_bias, initial_state,
                                       cu_seqlens, float(scale), float(lower_bound),
                                       bool(output_final_state))


def set_bwd_stage_events(events=None):
    """Six raw hipEvent_t handles (ints) recorded around the five backward
    kernels by the next kda_bwd calls from this thread; None to stop."""
    lib = load()
    if events is None:
        lib.kda_set_bwd_stage_events(None)
        return
    arr = (ctypes.c_void_p * 6)(*[int(e) for e in events])
    lib.kda_set_bwd_stage_events(ctypes.cast(arr, ctypes.c_void_p))


def set_stage_events(before_intra=None, before_scan=None, after_scan=None):
    """Raw hipEvent_t handles (ints) recorded around the two kernels by the
    next kda_fwd calls from this thread; all None to stop."""
    P = ctypes.c_void_p
    load().kda_set_stage_events(P(before_intra), P(before_scan), P(after_scan))


def debug_scan_step(v, records, scale, out, initial_state=None, final_state=None,
                    cu_seqlens=None, part_cols=0):
    """Run only the inter-chunk scan (K = V = 64, 128 or 256) over `records` (as
    debug_intra returns them) from initial_state, writing out and
    final_state; part_cols fixes the columns per scan workgroup (0: the
    forward's choice)."""
    import torch
    lib = load()
    if v.dim() != 4:
        raise ValueError("v must be [B, T, H, V]")
    B, T, H, V = v.shape
    bf = torch.bfloat16
    _check(v, "v", bf)
    _check(out, "out", bf, (B, T, H, V))
    _check(records, "records", torch.uint8)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    need = int(lib.kda_record_workspace_size(B, T, H, N, V))
    if records.numel() < need:
        raise ValueError(f"records holds {records.numel()} bytes, the scan reads {need}")
    init_dt = fin_dt = KDA_DTYPE_FP32
    if initial_state is not None:
        init_dt = _state_dtype(initial_state)
        _check(initial_state, "initial_state", initial_state.dtype, (N, H, V, V))
    if final_state is not None:
        fin_dt = _state_dtype(final_state)
        _check(final_state, "final_state", final_state.dtype, (N, H, V, V))
    rc = lib.kda_debug_scan_step(_ptr(v), _ptr(records), _ptr(cu_seqlens), int(N), int(B), int(T),
                                 int(H), int(V), int(V), float(scale), _ptr(initial_state),
                                 int(init_dt), _ptr(final_state), int(fin_dt), _ptr(out),
                                 int(part_cols), _stream(v.device))
    if rc != 0:
        raise KDAError(rc, "kda_debug_scan_step")


def debug_gate(g, beta, A_log, dt_bias, lower_bound, cu_seqlens=None):
    """Run only the gate and the in-chunk cumulative decay; returns (G, beta)
    as fp32 device tensors [B, T, H, K] and [B, T, H]: G is the inclusive
    cumulative base-2 log-decay of each token within its 16-token chunk,
    beta the sigmoid of the logits."""
    import torch
    lib = load()
    B, T, H, K = g.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    G = torch.empty((B, T, H, K), dtype=torch.float32, device=g.device)
    b = torch.empty((B, T, H), dtype=torch.float32, device=g.device)
    rc = lib.kda_debug_gate(_ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias), float(lower_bound),
                            _ptr(cu_seqlens), int(N), _ptr(G), _ptr(b), int(B), int(T), int(H),
                            int(K), _stream(g.device))
    if rc != 0:
        raise KDAError(rc, "kda_debug_gate")
    return G, b


def debug_intra(q, k, g, beta, A_log, dt_bias, lower_bound, cu_seqlens=None):
    """Run only the intra-chunk stage; returns its hand-off records as a
    uint8 device tensor of kda_record_workspace_size(B, T, H, N, K) bytes."""
    import torch
    lib = load()
    B, T, H, K = q.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    ws = torch.zeros(int(lib.kda_record_workspace_size(B, T, H, N, K)), dtype=torch.uint8,
                     device=q.device)
    rc = lib.kda_debug_intra(_ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias),
                             float(lower_bound), _ptr(cu_seqlens), int(N), int(B), int(T),
                             int(H), int(K), _ptr(ws), _stream(q.device))
    if rc != 0:
        raise KDAError(rc, "kda_debug_intra")
    return ws
