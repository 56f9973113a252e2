"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments before it touches the device."""
import ctypes
import math
import os
import re
import subprocess

import pytest

from transformer_attention_causal_amd import binding as ab

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def declared_functions(header=HEADER):
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)))


def test_header_declarations_are_exported():
    lib = ab.load()
    names = declared_functions()
    assert set(names) == set(ab.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ab.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_[a-z0-9_]+)\b", out))
    assert set(names) <= exported


def declared_signatures(header=HEADER):
    """{name: (return type, [parameter types])} of every prototype in the header."""
    src = open(header).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    sigs = {}
    for ret, name, params in re.findall(
            r"([A-Za-z_][\w\s\*]*?)\b(attn_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;", src):
        ps = [x.strip() for x in params.split(",") if x.strip() and x.strip() != "void"]
        # drop the parameter name: what is left is its type
        types = [re.sub(r"\b\w+$", "", x).strip() if not x.endswith("*") else x for x in ps]
        sigs[name] = (ret.strip(), types)
    return sigs


def _ctype_of(decl):
    import ctypes

    if "*" in decl:
        return ctypes.c_char_p if decl.replace(" ", "") == "constchar*" else ctypes.c_void_p
    words = decl.replace("const", "").split()
    kind = words[-1] if words else ""
    return {"int": ctypes.c_int, "int32_t": ctypes.c_int, "float": ctypes.c_float,
            "double": ctypes.c_double, "size_t": ctypes.c_size_t}[kind]


def test_binding_argtypes_match_the_header():
    """Every prototype's parameter count and types (pointer, int, float,
    double, size_t) agree with the ctypes binding, so a changed signature
    cannot be called with a stale argument list."""
    import ctypes

    lib = ab.load()
    sigs = declared_signatures()
    assert set(sigs) == set(ab.EXPORTED)
    for name, (ret, params) in sigs.items():
        fn = getattr(lib, name)
        want = [_ctype_of(t) for t in params]
        got = list(fn.argtypes or [])
        assert len(got) == len(want), (name, len(got), len(want))
        for i, (g, w) in enumerate(zip(got, want)):
            if w is ctypes.c_char_p:
                w = ctypes.c_void_p
            assert g is w or (g is ctypes.c_char_p and w is ctypes.c_void_p), (name, i, g, w)
        assert fn.restype is _ctype_of(ret) or (ret.endswith("*") and fn.restype in
                                                (ctypes.c_char_p, ctypes.c_void_p)), name


def test_peaks_library_exports_its_header():
    """The benchmark's measured-ceiling kernels: libattn_peaks.so exports what
    include/attn_peaks.h declares, and rejects bad arguments on the host."""
    path = os.path.join(os.path.dirname(ab.LIB_PATH), "libattn_peaks.so")
    names = declared_functions(os.path.join(ROOT, "include", "attn_peaks.h"))
    assert names == ["attn_peak_mfma_bf16", "attn_peak_mfma_bf16_flops", "attn_peak_stream_read"]
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    assert set(names) <= set(re.findall(r"\bT (attn_[a-z0-9_]+)\b", out))
    lib = ctypes.CDLL(path)
    lib.attn_peak_mfma_bf16_flops.restype = ctypes.c_double
    lib.attn_peak_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    assert lib.attn_peak_mfma_bf16_flops(10, 3) == 10 * 3 * 4 * 4 * 2 * 32 * 32 * 16
    lib.attn_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
    assert lib.attn_peak_mfma_bf16(0, 1, FAKE, None) == -1
    assert lib.attn_peak_mfma_bf16(1, 1, None, None) == -1
    assert lib.attn_peak_stream_read(FAKE + 4, 1 << 20, FAKE, 8, None) == -1   # misaligned
    assert lib.attn_peak_stream_read(FAKE, 8, FAKE, 8, None) == -1             # under 16 bytes


def test_yarn_tau_against_page_table():
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", "yarn_temperature_table.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                s, _, st = line.split()
                rows.append((float(s), float(st)))
    for s, st in rows:
        assert round(ab.attn_yarn_tau(s), 4) == st
    assert ab.attn_yarn_tau(1.0) == 1.0
    assert math.isnan(ab.attn_yarn_tau(0.5)) and math.isnan(ab.attn_yarn_tau(float("nan")))


def test_strerror_is_static_text():
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(ab.attn_strerror(st), str) and ab.attn_strerror(st)


def fwd(**kw):
    args = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, out=FAKE + 0x3000000, B=1, H=1,
                T=16, d=64, tau=1.0, mode=0, eps=1e-6, dtype=1, workspace=None,
                workspace_bytes=0, lse_out=None, demand_out=None, rowsum_out=None,
                hip_stream=None)
    args.update(kw)
    return ab.attn_fwd_ex(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ab.ATTN_EINVAL),
    (dict(out=None), ab.ATTN_EINVAL),
    (dict(q=FAKE + 2), ab.ATTN_EINVAL),              # misaligned
    (dict(B=0), ab.ATTN_EINVAL),
    (dict(T=-3), ab.ATTN_EINVAL),
    (dict(mode=2), ab.ATTN_EINVAL),
    (dict(dtype=5), ab.ATTN_EINVAL),
    (dict(tau=-1.0), ab.ATTN_EINVAL),
    (dict(tau=float("nan")), ab.ATTN_EINVAL),
    (dict(tau=float("inf")), ab.ATTN_EINVAL),
    (dict(eps=-1e-6), ab.ATTN_EINVAL),
    (dict(eps=float("nan")), ab.ATTN_EINVAL),
    (dict(out=FAKE), ab.ATTN_EINVAL),                # out aliases q
    (dict(demand_out=FAKE + 0x4000000), ab.ATTN_EINVAL),  # demand_out in tempered mode
    (dict(rowsum_out=FAKE + 0x4000000), ab.ATTN_EINVAL),  # rowsum_out in tempered mode
    (dict(mode=1, lse_out=FAKE + 0x4000000, rowsum_out=FAKE + 0x4000010,
          workspace=FAKE + 0x5000000, workspace_bytes=1 << 30), ab.ATTN_EINVAL),  # outputs overlap
    (dict(d=96), ab.ATTN_ENOTSUP),
    (dict(d=128, dtype=0, mode=1), ab.ATTN_EWORKSPACE),   # fp32 at d = 128 is supported
    (dict(d=128, mode=1), ab.ATTN_EWORKSPACE),       # bf16 at d = 128 is supported
    (dict(T=1 << 24), ab.ATTN_EINVAL),               # one head's rows need offsets >= 2^31
    (dict(mode=1, T=(1 << 24) - 1, k=FAKE + (1 << 32), v=FAKE + (2 << 32),
          out=FAKE + (3 << 32)), ab.ATTN_EWORKSPACE),   # largest T passes the shape check
    (dict(d=128, T=1 << 23), ab.ATTN_EINVAL),        # bf16 rows of 256 B: T < 2^23
    (dict(mode=1, d=128, T=(1 << 23) - 1, k=FAKE + (1 << 32), v=FAKE + (2 << 32),
          out=FAKE + (3 << 32)), ab.ATTN_EWORKSPACE),   # largest T at d = 128
    (dict(dtype=0, T=1 << 23), ab.ATTN_EINVAL),      # fp32 rows of 256 B: T < 2^23
    (dict(H=4097, T=1 << 20), ab.ATTN_EINVAL),       # more than 2^32 rows in all
    (dict(mode=1, H=4096, T=1 << 20, k=FAKE + (1 << 40), v=FAKE + (2 << 40),
          out=FAKE + (3 << 40)), ab.ATTN_EWORKSPACE),   # exactly 2^32 rows passes
    (dict(mode=1), ab.ATTN_EWORKSPACE),              # dilution without workspace
    (dict(mode=1, workspace=FAKE + 0x5000000, workspace_bytes=16), ab.ATTN_EWORKSPACE),
    # the workspace is written: on a tensor argument or an output it is refused
    (dict(mode=1, workspace=FAKE + 0x2000000 - 256, workspace_bytes=1 << 20),
     ab.ATTN_EINVAL),                                                  # runs into v
    (dict(mode=1, workspace=FAKE + 0x3000000, workspace_bytes=1 << 20), ab.ATTN_EINVAL),  # on out
    (dict(mode=1, lse_out=FAKE + 0x4000000, workspace=FAKE + 0x4000000 - 256,
          workspace_bytes=1 << 20), ab.ATTN_EINVAL),                   # runs into lse_out
    (dict(mode=1, workspace=FAKE + 0x5000000, workspace_bytes=1 << 20),
     ab.ATTN_EHIP),        # valid: validation passes and only the missing device is reported
])
def test_fwd_rejects_bad_arguments(kw, status):
    assert fwd(**kw) == status


def noalloc(**kw):
    args = dict(q=FAKE, k=FAKE + (1 << 32), v=FAKE + (2 << 32), out=FAKE + (3 << 32), B=1, H=16,
                T=16384, d=64, tau=1.0, mode=1, eps=1e-6, dtype=1, hip_stream=None)
    args.update(kw)
    return ab.attn_fwd_noalloc(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(), ab.ATTN_ESCRATCH),                      # 16 heads at T = 16384: ~270 MB
    (dict(T=8193 * 2), ab.ATTN_ESCRATCH),
    (dict(B=2, H=16, T=8192, d=128), ab.ATTN_ESCRATCH),
    (dict(q=None, T=64), ab.ATTN_EINVAL),
    (dict(q=None, mode=0), ab.ATTN_EINVAL),          # tempered: attn_fwd's checks
    (dict(mode=3), ab.ATTN_EINVAL),
    (dict(d=96, T=64), ab.ATTN_ENOTSUP),
])
def test_noalloc_rejects_before_the_device(kw, status):
    """attn_fwd_noalloc refuses shapes beyond its fixed scratch array (and bad
    arguments) on the host, before any device call."""
    assert noalloc(**kw) == status


def test_noalloc_limit_covers_16_heads_at_8k():
    need = ab.attn_fwd_workspace_bytes(1, 16, 8192, 128, 1, 1)
    assert 0 < need <= ab.ATTN_NOALLOC_SCRATCH_BYTES
    assert ab.attn_fwd_workspace_bytes(1, 16, 16384, 64, 1, 1) > ab.ATTN_NOALLOC_SCRATCH_BYTES


def test_workspace_sizes():
    # tempered needs none; dilution keeps lse (B*H*T) + committed demand
    assert ab.attn_fwd_workspace_bytes(1, 16, 16384, 64, 0, 1) == 0
    n = 16384 // 32
    want = 16 * 16384 * 4 + 16 * 16 * n * (n + 1) * 4
    got = ab.attn_fwd_workspace_bytes(1, 16, 16384, 64, 1, 1)
    assert want <= got <= want + 512
    assert ab.attn_fwd_workspace_bytes(1, 1, 16, 96, 1, 1) == 0
    # fp32 keeps no per-range partials: its workspace does not depend on d
    assert (ab.attn_fwd_workspace_bytes(1, 3, 1000, 128, 1, 0)
            == ab.attn_fwd_workspace_bytes(1, 3, 1000, 64, 1, 0) > 0)
    assert (ab.attn_fwd_workspace_bytes(1, 16, 16384, 128, 1, 1)
            == ab.attn_fwd_workspace_bytes(1, 16, 16384, 64, 1, 1))  # independent of d
    assert ab.attn_fwd_workspace_bytes(0, 1, 16, 64, 1, 1) == 0
    assert ab.attn_decode_workspace_bytes(64, 16, 32768, 64) >= 64 * 16 * 32768 * 4
    assert ab.attn_decode_workspace_bytes(64, 16, 32768, 32) == 0
    assert (ab.attn_decode_workspace_bytes(64, 16, 32768, 128)
            > ab.attn_decode_workspace_bytes(64, 16, 32768, 64))


def test_bwd_workspace_sizes():
    n = 16384 // 32
    rows = 16 * 16384 * 4
    # five per-row arrays: lse2, 1/r, delta/r, rho and the rows' dL/dtau terms;
    # bf16 dilution adds the fp32 partial key gradients and each 128-key
    # block's part of rho per row
    rho_parts = 16 * (16384 // 128) * 16384 * 4
    want = 5 * rows + 2 * 16 * 16 * n * (n + 1) * 4 + 16 * 16384 * 64 * 4 + rho_parts
    got = ab.attn_bwd_workspace_bytes(1, 16, 16384, 64, 1, 1)
    assert want <= got <= want + 9 * 256
    assert 5 * rows <= ab.attn_bwd_workspace_bytes(1, 16, 16384, 64, 0, 1) <= 5 * rows + 5 * 256
    # fp32 (d = 64): the fp32 softmax-weighted keys in place of the partial
    # key gradients, and no parts of rho
    assert (ab.attn_bwd_workspace_bytes(1, 16, 16384, 64, 1, 1)
            - ab.attn_bwd_workspace_bytes(1, 16, 16384, 64, 1, 0)) == rho_parts
    # fp32 at d = 128: the softmax-weighted keys are twice as wide
    assert (ab.attn_bwd_workspace_bytes(1, 16, 16384, 128, 1, 0)
            - ab.attn_bwd_workspace_bytes(1, 16, 16384, 64, 1, 0)) == 16 * 16384 * 64 * 4
    assert (ab.attn_bwd_workspace_bytes(1, 16, 16384, 128, 0, 0)
            == ab.attn_bwd_workspace_bytes(1, 16, 16384, 64, 0, 0))
    assert ab.attn_bwd_workspace_bytes(1, 16, 16384, 64, 1, 2) == 0    # unknown dtype
    assert ab.attn_bwd_workspace_bytes(1, 16, 16384, 96, 1, 1) == 0
    # d = 128: the partial key gradients are twice as wide
    assert (ab.attn_bwd_workspace_bytes(1, 16, 16384, 128, 1, 1)
            - ab.attn_bwd_workspace_bytes(1, 16, 16384, 64, 1, 1)) == 16 * 16384 * 64 * 4
    assert (ab.attn_bwd_workspace_bytes(1, 16, 16384, 128, 0, 1)
            == ab.attn_bwd_workspace_bytes(1, 16, 16384, 64, 0, 1))


def test_prefill_workspace_sizes():
    # a whole prefill needs what attn_fwd needs
    for T in (1, 100, 16384):
        assert (ab.attn_prefill_workspace_bytes(2, 3, T, T, 64, 1, 1)
                == ab.attn_fwd_workspace_bytes(2, 3, T, 64, 1, 1))
    # a 2048-row chunk after 30000 cached keys: blocks from position 29952
    Tq, Tk = 2048, 32048
    n, b0 = (Tk + 31) // 32, 29952 // 32
    # 17 query blocks x 16 heads is a small grid: the row stages split each
    # block's keys 4 ways and keep per-range partials (max, sum, share @ V)
    ks = 4
    want = (16 * Tq * 4 + 16 * 16 * (n * (n + 1) - b0 * (b0 + 1)) * 4
            + 16 * Tq * ks * (2 + 64) * 4)
    got = ab.attn_prefill_workspace_bytes(1, 16, Tq, Tk, 64, 1, 1)
    assert want <= got <= want + 512
    assert ab.attn_prefill_workspace_bytes(1, 16, Tq, Tk, 64, 0, 1) == 0   # tempered
    assert ab.attn_prefill_workspace_bytes(1, 16, 10, 9, 64, 1, 1) == 0    # Tq > Tk
    assert ab.attn_prefill_workspace_bytes(1, 16, 0, 9, 64, 1, 1) == 0
    assert ab.attn_prefill_workspace_bytes(1, 16, 8, 9, 96, 1, 1) == 0
    assert (ab.attn_prefill_workspace_bytes(1, 16, 8, 9, 128, 1, 0)
            == ab.attn_prefill_workspace_bytes(1, 16, 8, 9, 64, 1, 0) > 0)


def pre(**kw):
    args = dict(q=FAKE, kcache=FAKE + 0x1000000, vcache=FAKE + 0x2000000, out=FAKE + 0x3000000,
                B=1, H=2, Tq=16, Tk=40, Lcap=64, d=64, tau=1.0, tau_bh=None, mode=1, eps=1e-6,
                dtype=1,
                demand_in=FAKE + 0x4000000, demand_out=FAKE + 0x4000000, lse_out=None,
                rowsum_out=None, workspace=None, workspace_bytes=0, hip_stream=None)
    args.update(kw)
    return ab.attn_prefill(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ab.ATTN_EINVAL),
    (dict(vcache=None), ab.ATTN_EINVAL),
    (dict(out=FAKE + 0x3000004), ab.ATTN_EINVAL),       # misaligned
    (dict(demand_in=FAKE + 0x4000008), ab.ATTN_EINVAL),
    (dict(Tq=0), ab.ATTN_EINVAL),
    (dict(Tq=41), ab.ATTN_EINVAL),                      # more rows than keys
    (dict(Lcap=39), ab.ATTN_EINVAL),                    # keys beyond the cache
    (dict(Lcap=1 << 24), ab.ATTN_EINVAL),
    (dict(mode=0), ab.ATTN_EINVAL),                     # demand arrays in tempered mode
    (dict(mode=2), ab.ATTN_EINVAL),
    (dict(tau=float("nan")), ab.ATTN_EINVAL),
    (dict(eps=-1.0), ab.ATTN_EINVAL),
    (dict(out=FAKE + 0x1000000 + 64 * 64 * 2), ab.ATTN_EINVAL),    # out inside the K cache
    (dict(demand_out=FAKE + 0x4000010), ab.ATTN_EINVAL),   # partial overlap with demand_in
    (dict(lse_out=FAKE + 0x4000000 + 256), ab.ATTN_EINVAL),  # lse inside the demand
    (dict(lse_out=FAKE), ab.ATTN_EINVAL),               # lse aliases q
    (dict(demand_out=FAKE + 0x2000000), ab.ATTN_EINVAL),   # demand inside the V cache
    (dict(rowsum_out=FAKE + 0x6000004), ab.ATTN_EINVAL),   # misaligned
    (dict(rowsum_out=FAKE + 0x4000000 + 64), ab.ATTN_EINVAL),  # row sums inside the demand
    (dict(rowsum_out=FAKE + 0x6000000, lse_out=FAKE + 0x6000040), ab.ATTN_EINVAL),  # overlap
    (dict(rowsum_out=FAKE + 0x6000000, tau_bh=FAKE + 0x6000000), ab.ATTN_EINVAL),
    (dict(mode=0, demand_in=None, demand_out=None, rowsum_out=FAKE + 0x6000000),
     ab.ATTN_EINVAL),                                   # row sums in tempered mode
    (dict(rowsum_out=FAKE + 0x6000000, lse_out=FAKE + 0x6000100), ab.ATTN_EWORKSPACE),
    (dict(d=96), ab.ATTN_ENOTSUP),
    (dict(d=128, dtype=0), ab.ATTN_EWORKSPACE),         # fp32 at d = 128 is supported
    (dict(d=128), ab.ATTN_EWORKSPACE),                  # bf16 at d = 128 is supported
    (dict(tau_bh=FAKE + 0x6000004), ab.ATTN_EINVAL),    # misaligned tau array
    (dict(tau_bh=FAKE + 0x4000000 + 64), ab.ATTN_EINVAL),  # tau array inside the demand
    (dict(tau_bh=FAKE + 0x6000000), ab.ATTN_EWORKSPACE),
    (dict(), ab.ATTN_EWORKSPACE),                       # in-place demand is accepted
    (dict(demand_in=None, demand_out=None), ab.ATTN_EWORKSPACE),
    (dict(workspace=FAKE + 0x5000000, workspace_bytes=64), ab.ATTN_EWORKSPACE),
])
def test_prefill_rejects_bad_arguments(kw, status):
    assert pre(**kw) == status


def pre_rope(**kw):
    args = dict(q=FAKE, kcache=FAKE + 0x1000000, vcache=FAKE + 0x2000000, out=FAKE + 0x3000000,
                B=1, H=2, Tq=16, Tk=40, Lcap=64, d=64, tau=1.0, tau_bh=None, mode=1, eps=1e-6,
                dtype=1, rope_freq=FAKE + 0x7000000, pos0=0,
                demand_in=FAKE + 0x4000000, demand_out=FAKE + 0x4000000, lse_out=None,
                rowsum_out=None, workspace=None, workspace_bytes=0, hip_stream=None)
    args.update(kw)
    return ab.attn_prefill_rope(**args)


ROPE_WS = FAKE + 0x8000000


@pytest.mark.parametrize("kw,status", [
    (dict(rope_freq=None), ab.ATTN_EINVAL),
    (dict(rope_freq=FAKE + 0x7000002), ab.ATTN_EINVAL),    # misaligned frequencies
    (dict(rope_freq=FAKE + 0x1000000 + 128), ab.ATTN_EINVAL),  # inside the K cache
    (dict(pos0=-1), ab.ATTN_EINVAL),
    (dict(pos0=(1 << 31) - 40), ab.ATTN_EINVAL),           # last key past 2^31 - 1
    (dict(pos0=(1 << 31) - 41, workspace=ROPE_WS, workspace_bytes=1 << 20),
     ab.ATTN_EHIP),                                        # largest pos0 passes the checks
    (dict(q=None), ab.ATTN_EINVAL),
    (dict(d=96), ab.ATTN_ENOTSUP),
    (dict(mode=0, demand_in=None, demand_out=None), ab.ATTN_EWORKSPACE),  # tempered needs it too
    (dict(), ab.ATTN_EWORKSPACE),
    (dict(workspace=ROPE_WS, workspace_bytes=64), ab.ATTN_EWORKSPACE),
    (dict(workspace=FAKE + 0x2000000, workspace_bytes=1 << 20), ab.ATTN_EINVAL),  # on the V cache
    (dict(workspace=FAKE + 0x7000000 - 64, workspace_bytes=1 << 20), ab.ATTN_EINVAL),  # on freq
])
def test_prefill_rope_rejects_bad_arguments(kw, status):
    """Every status is decided on the host; the one call that passes every
    check reaches the device query, which fails without a GPU (ATTN_EHIP)."""
    import torch

    if status == ab.ATTN_EHIP and torch.cuda.is_available():
        pytest.skip("a GPU is present: the call would launch")
    assert pre_rope(**kw) == status


def test_prefill_rope_workspace_sizes():
    # rotated Q [B,H,Tq,d] and keys [B,H,Lcap,d], then the attention workspace
    for (B, H, Tq, Tk, Lcap, d, dt) in ((1, 2, 16, 40, 64, 64, 1), (2, 3, 100, 100, 100, 128, 0)):
        esz = 2 if dt == 1 else 4
        qk = B * H * Tq * d * esz + B * H * Lcap * d * esz
        t = ab.attn_prefill_rope_workspace_bytes(B, H, Tq, Tk, Lcap, d, 0, dt)
        assert qk <= t <= qk + 512
        dil = ab.attn_prefill_rope_workspace_bytes(B, H, Tq, Tk, Lcap, d, 1, dt)
        assert dil - t == ab.attn_prefill_workspace_bytes(B, H, Tq, Tk, d, 1, dt)
    assert ab.attn_prefill_rope_workspace_bytes(1, 2, 16, 40, 39, 64, 1, 1) == 0   # Tk > Lcap
    assert ab.attn_prefill_rope_workspace_bytes(1, 2, 16, 40, 64, 96, 1, 1) == 0
    assert ab.attn_prefill_rope_workspace_bytes(1, 2, 16, 40, 64, 64, 2, 1) == 0


BWD_WS = dict(workspace=FAKE + 0xc000000, workspace_bytes=1 << 24)


def bwd(**kw):
    base = FAKE
    args = dict(q=base, k=base + 0x1000000, v=base + 0x2000000, out=base + 0x3000000,
                dout=base + 0x4000000, lse=base + 0x5000000, rowsum=base + 0x6000000,
                dq=base + 0x7000000, dk=base + 0x8000000, dv=base + 0x9000000, B=1, H=1, T=16,
                d=64, tau=1.0, tau_bh=None, mode=1, eps=1e-6, dtype=1, dtau_out=None,
                fwd_workspace=None, fwd_workspace_bytes=0, workspace=None, workspace_bytes=0,
                hip_stream=None)
    args.update(kw)
    ex_only = ("tau_bh", "dtau_out", "fwd_workspace", "fwd_workspace_bytes")
    if not any(n in kw for n in ex_only):
        for n in ex_only:
            del args[n]
        return ab.attn_bwd(**args)
    return ab.attn_bwd_ex(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(dout=None), ab.ATTN_EINVAL),
    (dict(lse=None), ab.ATTN_EINVAL),
    (dict(rowsum=None), ab.ATTN_EINVAL),              # dilution needs the row sums
    (dict(dq=FAKE + 4), ab.ATTN_EINVAL),              # misaligned
    (dict(mode=3), ab.ATTN_EINVAL),
    (dict(T=0), ab.ATTN_EINVAL),
    (dict(tau=-1.0), ab.ATTN_EINVAL),
    (dict(eps=float("nan")), ab.ATTN_EINVAL),
    (dict(dtype=0), ab.ATTN_EWORKSPACE),              # fp32 backward is supported
    (dict(dtype=2), ab.ATTN_EINVAL),
    (dict(d=96), ab.ATTN_ENOTSUP),
    (dict(d=128), ab.ATTN_EWORKSPACE),                # d = 128 is supported
    (dict(d=128, dtype=0), ab.ATTN_EWORKSPACE),       # fp32 at d = 128 is supported
    (dict(dk=FAKE + 0x7000000), ab.ATTN_EINVAL),      # dk aliases dq
    (dict(dv=FAKE), ab.ATTN_EINVAL),                  # dv aliases q
    (dict(), ab.ATTN_EWORKSPACE),
    (dict(mode=0, rowsum=None), ab.ATTN_EWORKSPACE),  # tempered: row sums not needed
    (dict(tau_bh=FAKE + 0xa000004), ab.ATTN_EINVAL),  # misaligned tau array
    (dict(dtau_out=FAKE + 0xa000008), ab.ATTN_EINVAL),
    (dict(tau_bh=FAKE + 0x8000000), ab.ATTN_EINVAL),  # tau array inside dk
    (dict(dtau_out=FAKE + 0x5000000), ab.ATTN_EINVAL),  # dL/dtau inside lse
    (dict(dtau_out=FAKE + 0x9000040), ab.ATTN_EINVAL),  # dL/dtau inside dv
    (dict(tau_bh=FAKE + 0xa000000, dtau_out=FAKE + 0xa000000), ab.ATTN_EINVAL),
    (dict(tau_bh=FAKE + 0xa000000, dtau_out=FAKE + 0xb000000), ab.ATTN_EWORKSPACE),
    (dict(tau_bh=None, dtau_out=FAKE + 0xb000000), ab.ATTN_EWORKSPACE),
    # the forward's workspace (read only; its committed-demand table is reused)
    (dict(fwd_workspace=FAKE + 0xd000000, fwd_workspace_bytes=64, **BWD_WS), ab.ATTN_EWORKSPACE),
    (dict(fwd_workspace=FAKE + 0xd000004, fwd_workspace_bytes=1 << 20, **BWD_WS),
     ab.ATTN_EWORKSPACE),                                # misaligned
    (dict(fwd_workspace=FAKE + 0x6ffff00, fwd_workspace_bytes=1 << 20, **BWD_WS),
     ab.ATTN_EINVAL),                                    # runs into dq
    (dict(fwd_workspace=FAKE + 0xc000100, fwd_workspace_bytes=1 << 20, **BWD_WS),
     ab.ATTN_EINVAL),                                    # inside the backward's workspace
    (dict(fwd_workspace=FAKE + 0xd000000, fwd_workspace_bytes=1 << 20,
          dtau_out=FAKE + 0xd000100, **BWD_WS), ab.ATTN_EINVAL),
    # the backward's own workspace is written: on an argument it is refused
    (dict(workspace=FAKE + 0x7000000, workspace_bytes=1 << 24), ab.ATTN_EINVAL),   # on dq
    (dict(workspace=FAKE + 0x5000000 - 256, workspace_bytes=1 << 24),
     ab.ATTN_EINVAL),                                                    # runs into lse
    (dict(dtau_out=FAKE + 0xc000100, **BWD_WS), ab.ATTN_EINVAL),        # dtau_out inside it
    (dict(**BWD_WS), ab.ATTN_EHIP),       # valid: only the missing device is reported
])
def test_bwd_rejects_bad_arguments(kw, status):
    assert bwd(**kw) == status


def dec(**kw):
    args = dict(q=FAKE, kcache=FAKE + 0x1000000, vcache=FAKE + 0x20000000,
                demand=FAKE + 0x40000000, out=FAKE + 0x60000000, S=2, H=2, Lcap=100,
                kv_len=None, d=64, tau=1.0, tau_sh=None, eps=1e-6, dtype=1, workspace=None,
                workspace_bytes=0, hip_stream=None)
    args.update(kw)
    if args["tau_sh"] is None and "tau_sh" not in kw:
        del args["tau_sh"]
        return ab.attn_decode(**args)
    return ab.attn_decode_ex(**args)


@pytest.mark.parametrize("kw,status", [
    (dict(demand=None), ab.ATTN_EINVAL),
    (dict(kcache=FAKE + 8), ab.ATTN_EINVAL),
    (dict(S=0), ab.ATTN_EINVAL),
    (dict(Lcap=0), ab.ATTN_EINVAL),
    (dict(tau=-0.5), ab.ATTN_EINVAL),
    (dict(eps=float("inf")), ab.ATTN_EINVAL),
    (dict(dtype=0), ab.ATTN_ENOTSUP),                # fp32 decode
    (dict(d=96), ab.ATTN_ENOTSUP),
    (dict(d=128), ab.ATTN_EWORKSPACE),               # d = 128 is supported
    (dict(tau_sh=FAKE + 0x70000004), ab.ATTN_EINVAL),   # misaligned tau array
    (dict(tau_sh=FAKE + 0x40000000), ab.ATTN_EINVAL),   # tau array inside the demand
    (dict(tau_sh=FAKE + 0x70000000), ab.ATTN_EWORKSPACE),
    (dict(out=FAKE + 0x1000000), ab.ATTN_EINVAL),     # out inside the K cache
    (dict(), ab.ATTN_EWORKSPACE),
    (dict(workspace=FAKE + 0x40000000, workspace_bytes=1 << 20), ab.ATTN_EINVAL),  # on the demand
    (dict(workspace=FAKE + 0x20000000 - 256, workspace_bytes=1 << 20),
     ab.ATTN_EINVAL),                                                  # runs into the V cache
    (dict(workspace=FAKE + 0x70000000, workspace_bytes=1 << 20), ab.ATTN_EHIP),  # valid
])
def test_decode_rejects_bad_arguments(kw, status):
    assert dec(**kw) == status


def stage(name, **kw):
    args = dict(q=FAKE, k=FAKE + 0x1000000, B=1, H=2, T=40, d=64, tau=1.0, dtype=1,
                workspace=None, workspace_bytes=0, hip_stream=None)
    if name == "attn_dilution_lse":
        args.update(lse_out=None)
    elif name == "attn_dilution_committed":
        args.update(eps=1e-6, demand_out=None)
    else:
        args.update(v=FAKE + 0x2000000, out=FAKE + 0x3000000, eps=1e-6)
    args.update(kw)
    return getattr(ab, name)(**args)


@pytest.mark.parametrize("name", ["attn_dilution_lse", "attn_dilution_committed",
                                  "attn_dilution_shares"])
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ab.ATTN_EINVAL),
    (dict(k=FAKE + 0x1000004), ab.ATTN_EINVAL),       # misaligned
    (dict(T=0), ab.ATTN_EINVAL),
    (dict(tau=float("inf")), ab.ATTN_EINVAL),
    (dict(d=96), ab.ATTN_ENOTSUP),
    (dict(), ab.ATTN_EWORKSPACE),                     # every stage reads or writes the workspace
    (dict(workspace=FAKE + 0x5000000, workspace_bytes=64), ab.ATTN_EWORKSPACE),
    (dict(workspace=FAKE + 0x1000000 - 256, workspace_bytes=1 << 20),
     ab.ATTN_EINVAL),                                 # the written workspace runs into k
    (dict(workspace=FAKE + 0x5000000, workspace_bytes=1 << 20), ab.ATTN_EHIP),  # valid
])
def test_stage_calls_reject_bad_arguments(name, kw, status):
    assert stage(name, **kw) == status


@pytest.mark.parametrize("name", ["attn_dilution_committed", "attn_dilution_shares"])
def test_stage_calls_check_eps(name):
    # the committed stage stores committed + eps, so it validates eps too
    assert stage(name, eps=-1.0) == ab.ATTN_EINVAL
    assert stage(name, eps=float("nan")) == ab.ATTN_EINVAL


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(ab, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(ab, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        ab.load()


def _host_calls():
    import torch

    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    rows = torch.zeros(1, 2, 8, dtype=torch.float32)
    dq = torch.zeros(2, 2, 64, dtype=torch.bfloat16)
    cache = torch.zeros(2, 2, 16, 64, dtype=torch.bfloat16)
    dem = torch.zeros(2, 2, 16, dtype=torch.float32)
    return {
        "fwd": lambda: ab.fwd(q, q, q),
        "fwd_noalloc": lambda: ab.fwd_noalloc(q, q, q, q.clone()),
        "bwd": lambda: ab.bwd(q, q, q, q, q, rows, rows, mode=ab.ATTN_DILUTION),
        "prefill": lambda: ab.prefill(q, q, q, 8),
        "dilution_stages": lambda: ab.dilution_stages(q, q, q),
        "decode": lambda: ab.decode(dq, cache, cache, dem),
    }


@pytest.mark.parametrize("name", ["fwd", "fwd_noalloc", "bwd", "prefill", "dilution_stages",
                                  "decode"])
def test_wrappers_refuse_host_tensors(name):
    """The kernels dereference every pointer they are given, so the torch
    wrappers refuse tensors in host memory before anything reaches the
    library."""
    with pytest.raises(ValueError, match="GPU"):
        _host_calls()[name]()
