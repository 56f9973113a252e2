"""Helpers for the GPU parity tests: move seeded host inputs to the device,
hand the same values to the oracle, and measure the error."""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from transformer_attention_causal_amd.workloads import HostInputs

BF16_MAX_ABS = 2e-2   # bf16 I/O with fp32 accumulation
BF16_REL_RMS = 1e-2
F32_MAX_ABS = 1e-5    # fp32 path
DEMAND_TOTAL_REL = 1e-4

# pytest's config, set by conftest: lets say() write past output capture
PYTEST_CONFIG = None


def say(*args, **_kw):
    """Print a figure or a progress line straight to the terminal, past
    pytest's output capture, so that a long comparison shows each finished
    step as it happens rather than only when its test ends."""
    import sys

    msg = " ".join(str(a) for a in args)
    capman = PYTEST_CONFIG.pluginmanager.getplugin("capturemanager") if PYTEST_CONFIG else None
    if capman is None:
        say(msg, flush=True)
        return
    with capman.global_and_fixture_disabled():
        sys.stderr.write(msg + "\n")
        sys.stderr.flush()


def to_device(x: np.ndarray, dtype: str):
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def oracle_view(x: np.ndarray, dtype: str):
    return oracle.Bf16(x) if dtype == "bf16" else x


def device_qkv(inp: HostInputs):
    return tuple(to_device(a, inp.dtype) for a in (inp.q, inp.k, inp.v))


def oracle_qkv(inp: HostInputs):
    return tuple(oracle_view(a, inp.dtype) for a in (inp.q, inp.k, inp.v))


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite output"
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.sqrt(np.sum(ref * ref)))
    rel_rms = float(np.sqrt(np.sum(diff * diff)) / denom) if denom > 0 else 0.0
    return max_abs, rel_rms


def assert_close(got, ref, dtype: str, what: str = ""):
    max_abs, rel_rms = errors(got, ref)
    say(f"{what}: max-abs {max_abs:.3e} rel-RMS {rel_rms:.3e}")
    if dtype == "bf16":
        assert max_abs <= BF16_MAX_ABS and rel_rms <= BF16_REL_RMS, \
            f"{what}: max-abs {max_abs:.3e} rel-RMS {rel_rms:.3e}"
    else:
        assert max_abs <= F32_MAX_ABS, f"{what}: max-abs {max_abs:.3e}"
    return max_abs, rel_rms


def worst_element(got, ref):
    """Index, reference value and device value of the largest absolute error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    w = np.unravel_index(int(np.argmax(np.abs(got - ref))), ref.shape)
    return tuple(int(i) for i in w), float(ref[w]), float(got[w])


def record(name: str, **fields):
    """Append one parity figure to the JSON-lines file named by the
    ATTN_PARITY_RECORD environment variable (nothing when it is unset)."""
    path = os.environ.get("ATTN_PARITY_RECORD")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps({"name": name, **fields}) + "\n")


def assert_workload(got, ref, what: str):
    """The bf16 bars, absolute, on a whole workload's compared elements; the
    figures and the worst element are printed and recorded."""
    max_abs, rel_rms = errors(got, ref)
    where, r, g = worst_element(got, ref)
    say(f"{what}: max-abs {max_abs:.3e} rel-RMS {rel_rms:.3e} "
          f"(worst at {where}: ref {r:.5f}, got {g:.5f})", flush=True)
    record(what, max_abs=max_abs, rel_rms=rel_rms, worst_at=list(where), worst_ref=r,
           worst_got=g, elements=int(np.asarray(ref).size))
    assert max_abs <= BF16_MAX_ABS and rel_rms <= BF16_REL_RMS, \
        f"{what}: max-abs {max_abs:.3e} rel-RMS {rel_rms:.3e}"
    return max_abs, rel_rms


def sample_rows(T: int, n: int, seed: int = 0):
    """Rows spread over [0, T): both ends, tile edges and random interior rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, T // 2, T - 2, T - 1]
    rows = set(r for r in fixed if 0 <= r < T)
    rows.update(int(r) for r in rng.integers(0, T, size=max(0, n - len(rows))))
    return np.array(sorted(rows), dtype=np.int32)
