"""Thin Python binding of libattn.so (argument marshalling only).

The functions named like the C ABI (``attn_fwd``, ``attn_fwd_ex``, ``attn_bwd``,
``attn_prefill``, ``attn_decode``, the ``*_workspace_bytes`` queries, ``attn_yarn_tau``,
``attn_strerror``) take exactly the C arguments, with device pointers as Python
ints.  ``fwd``, ``bwd``, ``prefill`` and ``decode`` accept torch tensors, check
their shapes/dtypes, allocate the output and workspace with torch, pass the
current torch stream, and raise ``AttnError`` on a non-zero status.  Every step
of the computation runs in the library's HIP kernels; nothing here computes.

The library must have been built (``transformer_attention_causal_amd.build``);
there is no fallback: a missing library raises at first use.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# ATTN_LIB names another build of the same library (the host-sanitized one
# the CPU-side ABI tests can run against); by default the in-tree libattn.so.
LIB_PATH = os.environ.get("ATTN_LIB") or os.path.join(PKG, "libattn.so")

ATTN_OK, ATTN_EINVAL, ATTN_ENOTSUP, ATTN_EWORKSPACE, ATTN_EHIP, ATTN_ESCRATCH = 0, -1, -2, -3, -4, -5
ATTN_NOALLOC_SCRATCH_BYTES = 128 << 20
ATTN_TEMPERED, ATTN_DILUTION = 0, 1
ATTN_F32, ATTN_BF16 = 0, 1

EXPORTED = ("attn_fwd", "attn_fwd_ex", "attn_fwd_workspace_bytes", "attn_fwd_noalloc",
            "attn_dilution_lse",
            "attn_dilution_committed", "attn_dilution_shares", "attn_bwd",
            "attn_bwd_ex", "attn_bwd_workspace_bytes", "attn_prefill", "attn_prefill_workspace_bytes",
            "attn_prefill_rope", "attn_prefill_rope_workspace_bytes",
            "attn_decode", "attn_decode_ex", "attn_decode_workspace_bytes",
            "attn_yarn_tau", "attn_strerror")


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {attn_strerror(status)} (status {status})")


_lib = None


def load() -> ctypes.CDLL:
    """Open libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m transformer_attention_causal_amd.build` (no fallback path exists)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.attn_fwd.restype = i
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, f, i, f, i, vp, sz, vp]
        lib.attn_fwd_ex.restype = i
        lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, f, i, f, i, vp, sz, vp, vp, vp,
                                    vp]
        lib.attn_fwd_noalloc.restype = i
        lib.attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, f, i, f, i, vp]
        lib.attn_bwd.restype = i
        lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, f, i,
                                 vp, sz, vp]
        lib.attn_bwd_ex.restype = i
        lib.attn_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, vp, i,
                                    f, i, vp, vp, sz, vp, sz, vp]
        lib.attn_bwd_workspace_bytes.restype = sz
        lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
        lib.attn_prefill.restype = i
        lib.attn_prefill.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i, f, i, vp, vp,
                                     vp, vp, vp, sz, vp]
        lib.attn_prefill_rope.restype = i
        lib.attn_prefill_rope.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i, f, i, vp, i,
                                          vp, vp, vp, vp, vp, sz, vp]
        lib.attn_prefill_rope_workspace_bytes.restype = sz
        lib.attn_prefill_rope_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
        lib.attn_prefill_workspace_bytes.restype = sz
        lib.attn_prefill_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        lib.attn_dilution_lse.restype = i
        lib.attn_dilution_lse.argtypes = [vp, vp, i, i, i, i, f, i, vp, sz, vp, vp]
        lib.attn_dilution_committed.restype = i
        lib.attn_dilution_committed.argtypes = [vp, vp, i, i, i, i, f, f, i, vp, sz, vp, vp]
        lib.attn_dilution_shares.restype = i
        lib.attn_dilution_shares.argtypes = [vp, vp, vp, vp, i, i, i, i, f, f, i, vp, sz, vp]
        lib.attn_fwd_workspace_bytes.restype = sz
        lib.attn_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
        lib.attn_decode.restype = i
        lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp, i, f, f, i, vp, sz, vp]
        lib.attn_decode_ex.restype = i
        lib.attn_decode_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, vp, i, f, vp, f, i, vp, sz,
                                       vp]
        lib.attn_decode_workspace_bytes.restype = sz
        lib.attn_decode_workspace_bytes.argtypes = [i, i, i, i]
        lib.attn_yarn_tau.restype = ctypes.c_double
        lib.attn_yarn_tau.argtypes = [ctypes.c_double]
        lib.attn_strerror.restype = ctypes.c_char_p
        lib.attn_strerror.argtypes = [i]
        _lib = lib
    return _lib


# ------------------------------------------------------------- raw C ABI names

def attn_fwd(q, k, v, out, B, H, T, d, tau, mode, eps, dtype, workspace, workspace_bytes,
             hip_stream) -> int:
    return load().attn_fwd(q, k, v, out, B, H, T, d, tau, mode, eps, dtype, workspace,
                           workspace_bytes, hip_stream)


def attn_fwd_ex(q, k, v, out, B, H, T, d, tau, mode, eps, dtype, workspace, workspace_bytes,
                lse_out, demand_out, rowsum_out, hip_stream) -> int:
    return load().attn_fwd_ex(q, k, v, out, B, H, T, d, tau, mode, eps, dtype, workspace,
                              workspace_bytes, lse_out, demand_out, rowsum_out, hip_stream)


def attn_fwd_noalloc(q, k, v, out, B, H, T, d, tau, mode, eps, dtype, hip_stream) -> int:
    return load().attn_fwd_noalloc(q, k, v, out, B, H, T, d, tau, mode, eps, dtype, hip_stream)


def attn_bwd(q, k, v, out, dout, lse, rowsum, dq, dk, dv, B, H, T, d, tau, mode, eps, dtype,
             workspace, workspace_bytes, hip_stream) -> int:
    return load().attn_bwd(q, k, v, out, dout, lse, rowsum, dq, dk, dv, B, H, T, d, tau, mode,
                           eps, dtype, workspace, workspace_bytes, hip_stream)


def attn_bwd_ex(q, k, v, out, dout, lse, rowsum, dq, dk, dv, B, H, T, d, tau, tau_bh, mode, eps,
                dtype, dtau_out, fwd_workspace, fwd_workspace_bytes, workspace, workspace_bytes,
                hip_stream) -> int:
    return load().attn_bwd_ex(q, k, v, out, dout, lse, rowsum, dq, dk, dv, B, H, T, d, tau,
                              tau_bh, mode, eps, dtype, dtau_out, fwd_workspace,
                              fwd_workspace_bytes, workspace, workspace_bytes, hip_stream)


def attn_bwd_workspace_bytes(B, H, T, d, mode, dtype) -> int:
    return int(load().attn_bwd_workspace_bytes(B, H, T, d, mode, dtype))


def attn_prefill(q, kcache, vcache, out, B, H, Tq, Tk, Lcap, d, tau, tau_bh, mode, eps, dtype,
                 demand_in, demand_out, lse_out, rowsum_out, workspace, workspace_bytes,
                 hip_stream) -> int:
    return load().attn_prefill(q, kcache, vcache, out, B, H, Tq, Tk, Lcap, d, tau, tau_bh, mode,
                               eps, dtype, demand_in, demand_out, lse_out, rowsum_out, workspace,
                               workspace_bytes, hip_stream)


def attn_prefill_rope(q, kcache, vcache, out, B, H, Tq, Tk, Lcap, d, tau, tau_bh, mode, eps,
                      dtype, rope_freq, pos0, demand_in, demand_out, lse_out, rowsum_out,
                      workspace, workspace_bytes, hip_stream) -> int:
    return load().attn_prefill_rope(q, kcache, vcache, out, B, H, Tq, Tk, Lcap, d, tau, tau_bh,
                                    mode, eps, dtype, rope_freq, pos0, demand_in, demand_out,
                                    lse_out, rowsum_out, workspace, workspace_bytes, hip_stream)


def attn_prefill_rope_workspace_bytes(B, H, Tq, Tk, Lcap, d, mode, dtype) -> int:
    return int(load().attn_prefill_rope_workspace_bytes(B, H, Tq, Tk, Lcap, d, mode, dtype))


def attn_prefill_workspace_bytes(B, H, Tq, Tk, d, mode, dtype) -> int:
    return int(load().attn_prefill_workspace_bytes(B, H, Tq, Tk, d, mode, dtype))


def attn_dilution_lse(q, k, B, H, T, d, tau, dtype, workspace, workspace_bytes, lse_out,
                      hip_stream) -> int:
    return load().attn_dilution_lse(q, k, B, H, T, d, tau, dtype, workspace, workspace_bytes,
                                    lse_out, hip_stream)


def attn_dilution_committed(q, k, B, H, T, d, tau, eps, dtype, workspace, workspace_bytes,
                            demand_out, hip_stream) -> int:
    return load().attn_dilution_committed(q, k, B, H, T, d, tau, eps, dtype, workspace,
                                          workspace_bytes, demand_out, hip_stream)


def attn_dilution_shares(q, k, v, out, B, H, T, d, tau, eps, dtype, workspace, workspace_bytes,
                         hip_stream) -> int:
    return load().attn_dilution_shares(q, k, v, out, B, H, T, d, tau, eps, dtype, workspace,
                                       workspace_bytes, hip_stream)


def attn_fwd_workspace_bytes(B, H, T, d, mode, dtype) -> int:
    return int(load().attn_fwd_workspace_bytes(B, H, T, d, mode, dtype))


def attn_decode(q, kcache, vcache, demand, out, S, H, Lcap, kv_len, d, tau, eps, dtype,
                workspace, workspace_bytes, hip_stream) -> int:
    return load().attn_decode(q, kcache, vcache, demand, out, S, H, Lcap, kv_len, d, tau, eps,
                              dtype, workspace, workspace_bytes, hip_stream)


def attn_decode_ex(q, kcache, vcache, demand, out, S, H, Lcap, kv_len, d, tau, tau_sh, eps,
                   dtype, workspace, workspace_bytes, hip_stream) -> int:
    return load().attn_decode_ex(q, kcache, vcache, demand, out, S, H, Lcap, kv_len, d, tau,
                                 tau_sh, eps, dtype, workspace, workspace_bytes, hip_stream)


def attn_decode_workspace_bytes(S, H, Lcap, d) -> int:
    return int(load().attn_decode_workspace_bytes(S, H, Lcap, d))


def attn_yarn_tau(s: float) -> float:
    return float(load().attn_yarn_tau(float(s)))


def attn_strerror(status: int) -> str:
    return load().attn_strerror(int(status)).decode()


# ------------------------------------------------------------ torch marshalling

def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    """The device address of an optional tensor (None passes through)."""
    return t.data_ptr() if t is not None else None


def _stream_handle(device):
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def _check_like(t, ref, name):
    """``t`` must be a contiguous tensor of ``ref``'s shape, dtype and device."""
    if t is None:
        return
    if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous() \
            or t.device != ref.device:
        raise ValueError(f"{name} must be a contiguous {ref.dtype} tensor of shape "
                         f"{tuple(ref.shape)} on {ref.device}")


def _check_gpu(t, name):
    """``t`` must be a tensor in GPU memory: the kernels dereference its pointer."""
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a tensor on a GPU device")


def _check_buf(t, device, name):
    """``t`` (optional: a workspace or another byte buffer) must be a contiguous
    tensor on ``device``."""
    if t is None:
        return
    if t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}")


def _check_small(t, shape, dtype, device, name):
    """``t`` (optional) must be a contiguous ``dtype`` tensor of ``shape`` on ``device``."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() \
            or t.device != device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}")


def _check_rows(t, shape, device, name):
    """``t`` (optional) must be a contiguous float32 tensor of ``shape`` on ``device``."""
    import torch

    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or not t.is_contiguous() \
            or t.device != device:
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)} "
                         f"on {device}")


def fwd_workspace(B, H, T, mode, dtype_code, device, d=64):
    import torch

    n = attn_fwd_workspace_bytes(B, H, T, d, mode, dtype_code)
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def fwd(q, k, v, tau: float = 1.0, mode: int = ATTN_TEMPERED, eps: float = 1e-6,
        out=None, workspace=None, lse_out=None, demand_out=None, rowsum_out=None):
    """Run attn_fwd_ex on [B,H,T,d] tensors (d = 64 or 128); returns ``out``."""
    import torch

    if q.dim() != 4:
        raise ValueError("q, k, v must share one [B,H,T,d] shape")
    code = _dtype_code(q)
    _check_gpu(q, "q")
    _check_like(q, q, "q")
    _check_like(k, q, "k")
    _check_like(v, q, "v")
    _check_like(out, q, "out")
    _check_buf(workspace, q.device, "workspace")
    B, H, T, d = q.shape
    for name, t in (("lse_out", lse_out), ("demand_out", demand_out), ("rowsum_out", rowsum_out)):
        _check_rows(t, (B, H, T), q.device, name)
    if out is None:
        out = torch.empty_like(q)
    ws_bytes = 0
    if workspace is None:
        workspace, ws_bytes = fwd_workspace(B, H, T, mode, code, q.device, d)
    else:
        ws_bytes = workspace.numel() * workspace.element_size()
    st = attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, T, d,
                     float(tau), int(mode), float(eps), code,
                     workspace.data_ptr() if workspace is not None else None, ws_bytes,
                     lse_out.data_ptr() if lse_out is not None else None,
                     demand_out.data_ptr() if demand_out is not None else None,
                     rowsum_out.data_ptr() if rowsum_out is not None else None,
                     _stream_handle(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_ex")
    return out


def fwd_noalloc(q, k, v, out, tau: float = 1.0, mode: int = ATTN_TEMPERED, eps: float = 1e-6):
    """Run attn_fwd_noalloc on [B,H,T,d] tensors into the caller's ``out``
    (nothing is allocated: the dilution workspace is the library's fixed
    scratch array); returns ``out``."""
    if q.dim() != 4 or out is None:
        raise ValueError("q, k, v, out must share one [B,H,T,d] shape")
    code = _dtype_code(q)
    _check_gpu(q, "q")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_like(t, q, name)
    B, H, T, d = q.shape
    st = attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, T, d,
                          float(tau), int(mode), float(eps), code, _stream_handle(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_noalloc")
    return out


def bwd_workspace(B, H, T, mode, dtype_code, device, d=64):
    import torch

    n = attn_bwd_workspace_bytes(B, H, T, d, mode, dtype_code)
    if n == 0:
        raise AttnError(ATTN_ENOTSUP, "attn_bwd_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device), n


def bwd(q, k, v, out, dout, lse, rowsum=None, tau: float = 1.0, mode: int = ATTN_TEMPERED,
        eps: float = 1e-6, dq=None, dk=None, dv=None, workspace=None, tau_bh=None,
        dtau_out=None, fwd_workspace=None):
    """Run attn_bwd_ex on [B,H,T,d] tensors, d = 64 or 128 (``lse``/``rowsum`` from the
    forward's ``lse_out``/``rowsum_out``); ``tau_bh`` an optional [B,H] fp32
    tensor of per-head multipliers (as given to ``prefill``), ``dtau_out`` an
    optional [B,H] fp32 tensor that receives dL/dtau per head, ``fwd_workspace``
    optionally the dilution forward's workspace tensor (its committed-demand
    table is then read instead of recomputed).  Returns (dq, dk, dv)."""
    import torch

    if q.dim() != 4:
        raise ValueError("q, k, v, out, dout must share one [B,H,T,d] shape")
    code = _dtype_code(q)
    _check_gpu(q, "q")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq),
                    ("dk", dk), ("dv", dv)):
        _check_like(t, q, name)
    _check_buf(workspace, q.device, "workspace")
    _check_buf(fwd_workspace, q.device, "fwd_workspace")
    B, H, T, d = q.shape
    if lse is None:
        raise ValueError("lse (the forward's lse_out) is required")
    _check_rows(lse, (B, H, T), q.device, "lse")
    _check_rows(rowsum, (B, H, T), q.device, "rowsum")
    if mode == ATTN_DILUTION and rowsum is None:
        raise ValueError("rowsum (the forward's rowsum_out) is required for dilution")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    if workspace is None:
        workspace, ws_bytes = bwd_workspace(B, H, T, mode, code, q.device, d)
    else:
        ws_bytes = workspace.numel() * workspace.element_size()
    for name, t in (("tau_bh", tau_bh), ("dtau_out", dtau_out)):
        _check_small(t, (B, H), torch.float32, q.device, name)
    st = attn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                     lse.data_ptr(), rowsum.data_ptr() if rowsum is not None else None,
                     dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, T, d, float(tau),
                     tau_bh.data_ptr() if tau_bh is not None else None, int(mode), float(eps),
                     code, dtau_out.data_ptr() if dtau_out is not None else None,
                     fwd_workspace.data_ptr() if fwd_workspace is not None else None,
                     (fwd_workspace.numel() * fwd_workspace.element_size()
                      if fwd_workspace is not None else 0),
                     _ptr(workspace), ws_bytes, _stream_handle(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_ex")
    return dq, dk, dv


def prefill(q, kcache, vcache, Tk: int, tau: float = 1.0, mode: int = ATTN_DILUTION,
            eps: float = 1e-6, demand_in=None, demand_out=None, lse_out=None, out=None,
            workspace=None, tau_bh=None, rowsum_out=None, rope_freq=None, pos0: int = 0):
    """Run attn_prefill: q [B,H,Tq,d] holds the rows at positions Tk-Tq..Tk-1,
    the caches [B,H,Lcap,d] keys/values 0..Tk-1; ``demand_in``/``demand_out``
    are [B,H,Lcap] fp32 (may be one tensor: updated in place); ``tau_bh`` an
    optional [B,H] fp32 tensor of per-head multipliers; ``lse_out`` and
    ``rowsum_out`` optional [B,H,Tq] fp32 (what ``bwd`` needs).  With
    ``rope_freq`` (a [d/2] fp32 tensor) it runs attn_prefill_rope instead: Q
    and the (unrotated) cached keys are rotated at positions pos0 + index
    first.  Returns ``out``."""
    import torch

    if q.dim() != 4 or kcache.dim() != 4 or vcache.shape != kcache.shape:
        raise ValueError("q must be [B,H,Tq,d] and the caches one [B,H,Lcap,d] shape")
    B, H, Tq, d = q.shape
    Lcap = kcache.shape[2]
    if kcache.shape[:2] != (B, H) or kcache.shape[3] != d:
        raise ValueError("q and the caches disagree on B, H or d")
    _check_gpu(q, "q")
    for t in (q, kcache, vcache):
        if not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q and the caches must be contiguous, on one device and share "
                             "one dtype")
    for name, t in (("demand_in", demand_in), ("demand_out", demand_out)):
        _check_small(t, (B, H, Lcap), torch.float32, q.device, name)
    _check_small(tau_bh, (B, H), torch.float32, q.device, "tau_bh")
    _check_buf(workspace, q.device, "workspace")
    code = _dtype_code(q)
    _check_like(out, q, "out")
    for name, t in (("lse_out", lse_out), ("rowsum_out", rowsum_out)):
        _check_rows(t, (B, H, Tq), q.device, name)
    if rope_freq is not None:
        _check_rows(rope_freq, (d // 2,), q.device, "rope_freq")
    if out is None:
        out = torch.empty_like(q)
    ws_bytes = 0
    if workspace is None:
        if rope_freq is not None:
            n = attn_prefill_rope_workspace_bytes(B, H, Tq, int(Tk), Lcap, d, mode, code)
        else:
            n = attn_prefill_workspace_bytes(B, H, Tq, int(Tk), d, mode, code)
        if n:
            workspace, ws_bytes = torch.empty(n, dtype=torch.uint8, device=q.device), n
    else:
        ws_bytes = workspace.numel() * workspace.element_size()
    if rope_freq is not None:
        st = attn_prefill_rope(
            q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), out.data_ptr(), B, H, Tq,
            int(Tk), Lcap, d, float(tau), tau_bh.data_ptr() if tau_bh is not None else None,
            int(mode), float(eps), code, rope_freq.data_ptr(), int(pos0),
            demand_in.data_ptr() if demand_in is not None else None,
            demand_out.data_ptr() if demand_out is not None else None,
            lse_out.data_ptr() if lse_out is not None else None,
            rowsum_out.data_ptr() if rowsum_out is not None else None,
            workspace.data_ptr() if workspace is not None else None, ws_bytes,
            _stream_handle(q.device))
        if st != ATTN_OK:
            raise AttnError(st, "attn_prefill_rope")
        return out
    st = attn_prefill(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), out.data_ptr(), B, H,
                      Tq, int(Tk), Lcap, d, float(tau),
                      tau_bh.data_ptr() if tau_bh is not None else None, int(mode), float(eps), code,
                      demand_in.data_ptr() if demand_in is not None else None,
                      demand_out.data_ptr() if demand_out is not None else None,
                      lse_out.data_ptr() if lse_out is not None else None,
                      rowsum_out.data_ptr() if rowsum_out is not None else None,
                      workspace.data_ptr() if workspace is not None else None, ws_bytes,
                      _stream_handle(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_prefill")
    return out


def dilution_stages(q, k, v, tau: float = 1.0, eps: float = 1e-6, out=None, workspace=None,
                    lse_out=None, demand_out=None):
    """Run the three dilution stages as separate calls; returns a list of
    three zero-argument callables (lse, committed, shares) that enqueue one
    stage each on the current stream, and the output tensor they fill.  The
    callables hold the workspace (allocated here when none is given), so it
    stays allocated for as long as they do."""
    import torch

    if q.dim() != 4:
        raise ValueError("q, k, v must share one [B,H,T,d] shape")
    code = _dtype_code(q)
    _check_gpu(q, "q")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _check_like(t, q, name)
    _check_buf(workspace, q.device, "workspace")
    B, H, T, d = q.shape
    for name, t in (("lse_out", lse_out), ("demand_out", demand_out)):
        _check_rows(t, (B, H, T), q.device, name)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace, ws_bytes = fwd_workspace(B, H, T, ATTN_DILUTION, code, q.device, d)
    else:
        ws_bytes = workspace.numel() * workspace.element_size()
    # The closures read every pointer from the tensors themselves, so each
    # tensor (the workspace included) lives as long as the closures: a raw
    # pointer alone would let the allocator hand its memory to a later tensor
    # before a stage writes there.

    def check(st, where):
        if st != ATTN_OK:
            raise AttnError(st, where)

    def lse():
        check(attn_dilution_lse(q.data_ptr(), k.data_ptr(), B, H, T, d, float(tau), code,
                                _ptr(workspace), ws_bytes, _ptr(lse_out),
                                _stream_handle(q.device)), "attn_dilution_lse")

    def committed():
        check(attn_dilution_committed(q.data_ptr(), k.data_ptr(), B, H, T, d, float(tau),
                                      float(eps), code, _ptr(workspace), ws_bytes,
                                      _ptr(demand_out), _stream_handle(q.device)),
              "attn_dilution_committed")

    def shares():
        check(attn_dilution_shares(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B,
                                   H, T, d, float(tau), float(eps), code, _ptr(workspace),
                                   ws_bytes, _stream_handle(q.device)), "attn_dilution_shares")

    return [lse, committed, shares], out


def decode_workspace(S, H, Lcap, device, d=64):
    import torch

    n = attn_decode_workspace_bytes(S, H, Lcap, d)
    return torch.empty(n, dtype=torch.uint8, device=device), n


def decode(q, kcache, vcache, demand, tau: float = 1.0, eps: float = 1e-6, kv_len=None,
           out=None, workspace=None, tau_sh=None):
    """Run one attn_decode_ex step; ``demand`` is updated in place; ``tau_sh`` an
    optional [S,H] fp32 tensor of per-(sequence, head) multipliers.  Returns ``out``."""
    import torch

    if kcache.dim() != 4:
        raise ValueError("decode shapes must be q [S,H,d], caches [S,H,L,d], demand [S,H,L]")
    S, H, Lcap, d = kcache.shape
    if vcache.shape != kcache.shape or q.shape != (S, H, d) or demand.shape != (S, H, Lcap):
        raise ValueError("decode shapes must be q [S,H,d], caches [S,H,L,d], demand [S,H,L]")
    if demand.dtype != torch.float32:
        raise TypeError("demand must be float32")
    _check_gpu(q, "q")
    for t in (q, kcache, vcache, demand):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError("decode tensors must be contiguous and on one device")
    if kcache.dtype != q.dtype or vcache.dtype != q.dtype:
        raise ValueError("q and the caches must share one dtype")
    _check_like(out, q, "out")
    _check_buf(workspace, q.device, "workspace")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace, ws_bytes = decode_workspace(S, H, Lcap, q.device, d)
    else:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check_small(kv_len, (S,), torch.int32, q.device, "kv_len")
    _check_small(tau_sh, (S, H), torch.float32, q.device, "tau_sh")
    st = attn_decode_ex(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), demand.data_ptr(),
                        out.data_ptr(), S, H, Lcap,
                        kv_len.data_ptr() if kv_len is not None else None, d, float(tau),
                        tau_sh.data_ptr() if tau_sh is not None else None, float(eps),
                        _dtype_code(q), _ptr(workspace), ws_bytes, _stream_handle(q.device))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_ex")
    return out
