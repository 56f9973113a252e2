"""fp64 CPU oracle for reshaped-softmax causal attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP product
path and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP); this
module only builds/loads that library and marshals numpy arrays.  Functions:

* ``tempered_fwd``  -- causal softmax attention with logits tau*<q,k>/sqrt(d)
  (Focal Attention sec. 2.1 eq. focal-const with tau = 1/t; YaRN "Attention
  Temperature Scaling", score multiplier sqrt(t)).
* ``dilution_fwd``  -- dilution attention (DilutionAttention v0.1.0, "The
  operator": bids, exclusive column cumsum, shares, renormalised A, A@v).
* ``dilution_decode_step`` -- its cached-decode step (same page: K/V cache
  plus one running demand total per key and head).
* ``prefill`` -- a later chunk of a prefill (queries at the last Tq
  positions over cached keys), either operator; dilution continues from the
  demand the earlier rows committed (the cached-decoding sentence's running
  demand per key and head).
* ``attn_bwd`` -- exact gradients (dq, dk, dv) of either operator by the
  chain rule through its definition (the dilution page ships training kernels
  with exact gradients), plus the dilution row sums of the shares.
* ``rope`` -- the rotary position embedding YaRN's code cell applies to Q and
  K before the scores, with caller-supplied per-pair frequencies.
* ``yarn_t`` / ``yarn_tau`` -- t = 0.1 ln s + 1 and sqrt(t) (YaRN page).

Inputs may be numpy float64/float32 arrays or ``Bf16`` wrappers around raw
bf16 bit patterns (uint16); the C code widens them exactly to double.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_F64, _F32, _BF16 = 0, 1, 2


@dataclass
class Bf16:
    """Raw bf16 bit patterns (numpy uint16) standing for exact fp64 values."""

    bits: np.ndarray

    @property
    def shape(self):
        return self.bits.shape

    def to_f64(self) -> np.ndarray:
        return (self.bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")

# Host sanitizers for the oracle (ORACLE_SANITIZE=1): AddressSanitizer and
# UndefinedBehaviorSanitizer, any report fatal.  The process must have the
# ASan runtime loaded first (oracle/sanitize.sh does that).
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def _sanitized() -> bool:
    return os.environ.get("ORACLE_SANITIZE", "") == "1"


def build(src: str = _SRC, out: str | None = None, sanitize: bool | None = None) -> str:
    """Compile oracle.c into liboracle.so (gcc, OpenMP, IEEE arithmetic); with
    ``sanitize`` (default: the ORACLE_SANITIZE environment variable) into an
    ASan + UBSan build, liboracle_san.so by default."""
    if sanitize is None:
        sanitize = _sanitized()
    if out is None:
        out = _LIB_SAN if sanitize else _LIB
    cmd = ["gcc", "-O3", "-mavx2", "-mfma", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wno-unknown-pragmas", *(SANITIZE_FLAGS if sanitize else []), src,
           "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def load_library(path: str):
    """Open a compiled oracle library (the default one, or a test build)."""
    lib = ctypes.CDLL(path)
    _declare(lib)
    return lib


def use_library(lib) -> None:
    """Route the module functions through ``lib`` (None: back to the default)."""
    global _lib
    _lib = lib


def _load():
    global _lib
    if _lib is None:
        path = _LIB_SAN if _sanitized() else _LIB
        if not os.path.exists(path):
            build()
        _lib = load_library(path)
    return _lib


def _declare(lib):
    """Give ctypes the C signatures of the oracle's entry points."""
    for _ in (0,):
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        vp = ctypes.c_void_p
        i = ctypes.c_int
        d = ctypes.c_double
        lib.oracle_yarn_t.restype = d
        lib.oracle_yarn_t.argtypes = [d]
        lib.oracle_yarn_tau.restype = d
        lib.oracle_yarn_tau.argtypes = [d]
        lib.oracle_num_threads.restype = i
        lib.oracle_tempered_fwd.restype = i
        lib.oracle_tempered_fwd.argtypes = [vp, vp, vp, i, dp, dp, i, i, i, i, d, ip, i]
        lib.oracle_dilution_fwd.restype = i
        lib.oracle_dilution_fwd.argtypes = [vp, vp, vp, i, dp, dp, dp, i, i, i, i, d, d,
                                            ip, i, ip, i]
        lib.oracle_dilution_decode_step.restype = i
        lib.oracle_dilution_decode_step.argtypes = [vp, vp, vp, i, dp, dp, i, i, i, i, ip,
                                                    d, d, ip, i]
        lib.oracle_prefill.restype = i
        lib.oracle_prefill.argtypes = [vp, vp, vp, i, dp, dp, dp, i, i, i, i, i, i, d, d, i]
        lib.oracle_rope.restype = i
        lib.oracle_rope.argtypes = [vp, i, dp, i, i, i, i, dp, ctypes.c_long, i]
        lib.oracle_attn_bwd.restype = i
        lib.oracle_attn_bwd.argtypes = [vp, vp, vp, vp, i, dp, dp, dp, dp, dp, i, i, i, i, d, dp,
                                        d, i]


def _as_input(x):
    """Return (contiguous array, dtype code) without changing any value."""
    if isinstance(x, Bf16):
        a = np.ascontiguousarray(x.bits, dtype=np.uint16)
        return a, _BF16
    a = np.asarray(x)
    if a.dtype == np.float32:
        return np.ascontiguousarray(a), _F32
    if a.dtype == np.float64:
        return np.ascontiguousarray(a), _F64
    raise TypeError(f"oracle input must be float64, float32 or Bf16, got {a.dtype}")


def _same_code(*codes):
    if len(set(codes)) != 1:
        raise TypeError("q, k and v must share one storage type")
    return codes[0]


def _ptr(a, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _int_array(xs):
    if xs is None:
        return None, 0
    a = np.ascontiguousarray(np.asarray(xs, dtype=np.int32))
    return a, int(a.size)


def yarn_t(s: float) -> float:
    return _load().oracle_yarn_t(float(s))


def yarn_tau(s: float) -> float:
    return _load().oracle_yarn_tau(float(s))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def tempered_fwd(q, k, v, tau: float, rows=None):
    """Tempered causal attention. q,k,v: [B,H,T,d]. Returns (out, lse) in fp64.

    With ``rows`` only those query rows are computed; the others are NaN.
    """
    lib = _load()
    qa, c1 = _as_input(q)
    ka, c2 = _as_input(k)
    va, c3 = _as_input(v)
    code = _same_code(c1, c2, c3)
    B, H, T, d = qa.shape
    out = np.full((B, H, T, d), np.nan)
    lse = np.full((B, H, T), np.nan)
    ra, nr = _int_array(rows)
    rc = lib.oracle_tempered_fwd(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, code,
                                 _ptr(out), _ptr(lse), B, H, T, d, float(tau),
                                 _ptr(ra, ctypes.c_int) if ra is not None else None, nr)
    if rc != 0:
        raise RuntimeError(f"oracle_tempered_fwd failed ({rc})")
    return out, lse


def dilution_fwd(q, k, v, tau: float = 1.0, eps: float = 1e-6, rows=None, heads=None):
    """Dilution attention. q,k,v: [B,H,T,d]. Returns (out, lse, demand) in fp64.

    ``demand[b,h,j]`` is the final column total sum_i p_ij.  ``rows`` limits
    which outputs are formed (all rows still add their bids to the demand);
    ``heads`` (flattened b*H+h) limits which heads are processed.  Entries not
    computed are NaN.
    """
    lib = _load()
    qa, c1 = _as_input(q)
    ka, c2 = _as_input(k)
    va, c3 = _as_input(v)
    code = _same_code(c1, c2, c3)
    B, H, T, d = qa.shape
    out = np.full((B, H, T, d), np.nan)
    lse = np.full((B, H, T), np.nan)
    dem = np.full((B, H, T), np.nan)
    ra, nr = _int_array(rows)
    ha, nh = _int_array(heads)
    rc = lib.oracle_dilution_fwd(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, code,
                                 _ptr(out), _ptr(lse), _ptr(dem), B, H, T, d, float(tau),
                                 float(eps),
                                 _ptr(ra, ctypes.c_int) if ra is not None else None, nr,
                                 _ptr(ha, ctypes.c_int) if ha is not None else None, nh)
    if rc != 0:
        raise RuntimeError(f"oracle_dilution_fwd failed ({rc})")
    return out, lse, dem


def dilution_decode_step(q, kcache, vcache, demand: np.ndarray, tau: float = 1.0,
                         eps: float = 1e-6, kv_len=None, pairs=None):
    """One cached-decode step. q: [S,H,d]; caches: [S,H,Lcap,d]; demand: [S,H,Lcap]
    float64, updated IN PLACE (D += p).  Returns out [S,H,d] fp64 (NaN for
    pairs not selected)."""
    lib = _load()
    qa, c1 = _as_input(q)
    ka, c2 = _as_input(kcache)
    va, c3 = _as_input(vcache)
    code = _same_code(c1, c2, c3)
    S, H, Lcap, d = ka.shape
    if demand.dtype != np.float64 or not demand.flags.c_contiguous:
        raise TypeError("demand must be a C-contiguous float64 array (updated in place)")
    if demand.shape != (S, H, Lcap):
        raise ValueError("demand shape mismatch")
    out = np.full((S, H, d), np.nan)
    la, _ = _int_array(kv_len)
    pa, npairs = _int_array(pairs)
    rc = lib.oracle_dilution_decode_step(
        qa.ctypes.data, ka.ctypes.data, va.ctypes.data, code, _ptr(demand), _ptr(out),
        S, H, Lcap, d, _ptr(la, ctypes.c_int) if la is not None else None,
        float(tau), float(eps), _ptr(pa, ctypes.c_int) if pa is not None else None, npairs)
    if rc != 0:
        raise RuntimeError(f"oracle_dilution_decode_step failed ({rc})")
    return out


def rope(x, freq, pos0: int = 0, round_to_bf16: bool = False) -> np.ndarray:
    """Rotary position embedding of x [B,H,T,d]: row t of every head is at
    position pos0 + t, and dimension pair (2m, 2m+1) turns by that position
    times freq[m] (freq: [d/2], the per-pair frequencies with YaRN's gamma
    applied; widened exactly from its float32 values when given as float32).
    Returns the rotated rows in fp64; with ``round_to_bf16`` each value is
    rounded to the nearest bf16 (ties to even), as a method that stores the
    rotated rows in bf16 would hold them."""
    lib = _load()
    xa, code = _as_input(x)
    B, H, T, d = xa.shape
    f = np.ascontiguousarray(np.asarray(freq), dtype=np.float64)
    if f.shape != (d // 2,):
        raise ValueError("freq must hold d/2 values")
    out = np.empty((B, H, T, d))
    rc = lib.oracle_rope(xa.ctypes.data, code, _ptr(out), B, H, T, d, _ptr(f), int(pos0),
                         1 if round_to_bf16 else 0)
    if rc != 0:
        raise RuntimeError(f"oracle_rope failed ({rc})")
    return out


def prefill(q, kcache, vcache, Tk: int, tau: float = 1.0, eps: float = 1e-6, mode: int = 1,
            demand=None):
    """A chunk of a prefill: q [B,H,Tq,d] holds the rows at positions Tk-Tq..Tk-1;
    the caches [B,H,Lcap,d] hold keys 0..Tk-1.  mode 0 tempered, 1 dilution.
    ``demand`` ([B,H,Lcap] float64, dilution) is the demand committed before the
    chunk and is updated IN PLACE to include the chunk's bids (None: zero start,
    nothing returned).  Returns (out [B,H,Tq,d], lse [B,H,Tq]) in fp64."""
    lib = _load()
    qa, c1 = _as_input(q)
    ka, c2 = _as_input(kcache)
    va, c3 = _as_input(vcache)
    code = _same_code(c1, c2, c3)
    B, H, Tq, d = qa.shape
    Lcap = ka.shape[2]
    if ka.shape != (B, H, Lcap, d) or va.shape != ka.shape:
        raise ValueError("cache shape mismatch")
    dp_ = None
    if demand is not None:
        if demand.dtype != np.float64 or not demand.flags.c_contiguous:
            raise TypeError("demand must be a C-contiguous float64 array (updated in place)")
        if demand.shape != (B, H, Lcap):
            raise ValueError("demand shape mismatch")
        dp_ = _ptr(demand)
    out = np.full((B, H, Tq, d), np.nan)
    lse = np.full((B, H, Tq), np.nan)
    rc = lib.oracle_prefill(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, code, _ptr(out),
                            _ptr(lse), dp_, B, H, Tq, int(Tk), Lcap, d, float(tau), float(eps),
                            int(mode))
    if rc != 0:
        raise RuntimeError(f"oracle_prefill failed ({rc})")
    return out, lse


def attn_bwd(q, k, v, dout, tau: float = 1.0, eps: float = 1e-6, mode: int = 1, tau_bh=None,
             want_dtau: bool = False):
    """Exact gradients of the scalar sum(out * dout).  q,k,v,dout: [B,H,T,d] in
    one storage type; mode 0 tempered, 1 dilution; ``tau_bh`` ([B,H]) replaces
    tau per head.  Returns (dq, dk, dv, rsum) in fp64 -- plus dtau [B,H], the
    gradient with respect to each head's multiplier, when ``want_dtau``; rsum
    [B,H,T] holds the dilution row sums of the shares (NaN for tempered)."""
    lib = _load()
    qa, c1 = _as_input(q)
    ka, c2 = _as_input(k)
    va, c3 = _as_input(v)
    ga, c4 = _as_input(dout)
    code = _same_code(c1, c2, c3, c4)
    B, H, T, d = qa.shape
    dq = np.zeros((B, H, T, d))
    dk = np.zeros((B, H, T, d))
    dv = np.zeros((B, H, T, d))
    rs = np.full((B, H, T), np.nan)
    dt = np.full((B, H), np.nan)
    tb = None
    if tau_bh is not None:
        tb = np.ascontiguousarray(np.asarray(tau_bh, dtype=np.float64).reshape(B, H))
    rc = lib.oracle_attn_bwd(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, ga.ctypes.data,
                             code, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(rs),
                             _ptr(dt) if want_dtau else None, B, H, T, d, float(tau),
                             _ptr(tb) if tb is not None else None, float(eps), int(mode))
    if rc != 0:
        raise RuntimeError(f"oracle_attn_bwd failed ({rc})")
    if want_dtau:
        return dq, dk, dv, rs, dt
    return dq, dk, dv, rs
