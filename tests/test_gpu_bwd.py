"""GPU parity of the backward pass (exact gradients of both operators)
against the fp64 oracle, through the C ABI.  The device forward supplies the
saved tensors (out, lse, row sums) as a training step would; the oracle
differentiates the operator from q, k, v and dO alone."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import errors, to_device
from transformer_attention_causal_amd import binding as ab
from transformer_attention_causal_amd.workloads import PREFILL, draw_grad, draw_qkv, prefill_inputs

pytestmark = pytest.mark.gpu

TAU4 = math.sqrt(0.1 * math.log(4.0) + 1.0)

# The forward's bf16 bar (rel-RMS 1e-2, max-abs 2e-2 on O(1) outputs) applied
# to the gradients, with max-abs taken relative to each gradient's largest
# magnitude (gradients are not O(1)).  Sources of error: bf16 storage of q, k,
# v, dO and the three gradients, and bf16 matrix-core operands (bids, shares,
# gradient terms) with fp32 accumulation, each ~2^-9 relative.
GRAD_REL_RMS = 1e-2
GRAD_MAX_REL = 2e-2   # max-abs error over the largest reference magnitude


def run_bwd(inp, dout_bits, tau, mode, eps=1e-6):
    import torch

    q, k, v = (to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    dout = to_device(dout_bits, "bf16")
    B, H, T, _ = q.shape
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    rs = torch.empty((B, H, T), dtype=torch.float32, device="cuda") if mode == 1 else None
    out = ab.fwd(q, k, v, tau=tau, mode=mode, eps=eps, lse_out=lse, rowsum_out=rs)
    dq, dk, dv = ab.bwd(q, k, v, out, dout, lse, rs, tau=tau, mode=mode, eps=eps)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() for t in (dq, dk, dv)] + ([rs.cpu().numpy()] if rs is not None else [])


def check_grads(got, ref, what):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        max_abs, rel_rms = errors(g, r)
        scale = max(1e-30, float(np.max(np.abs(r))))
        print(f"{what} {name}: max-abs {max_abs:.3e} (scale {scale:.3e}) rel-RMS {rel_rms:.3e}")
        assert rel_rms <= GRAD_REL_RMS and max_abs <= GRAD_MAX_REL * scale, (what, name)


def oracle_grads(inp, dout_bits, tau, mode, eps=1e-6):
    return oracle.attn_bwd(oracle.Bf16(inp.q), oracle.Bf16(inp.k), oracle.Bf16(inp.v),
                           oracle.Bf16(dout_bits), tau, eps, mode)


@pytest.mark.parametrize("mode", [0, 1], ids=["tempered", "dilution"])
@pytest.mark.parametrize("T", [1, 7, 32, 33, 64, 100, 129, 257, 300])
def test_bwd_ragged_lengths(mode, T):
    inp = draw_qkv(1, 2, T, 64, "bf16", seed=900 + T)
    g = draw_grad(1, 2, T, 64, seed=900 + T)
    got = run_bwd(inp, g, 1.0, mode)
    ref = oracle_grads(inp, g, 1.0, mode)
    check_grads(got[:3], ref[:3], f"mode={mode} T={T}")
    if mode == 1:   # the forward's saved row sums are the oracle's
        assert np.max(np.abs(got[3] - ref[3]) / ref[3]) <= 1e-2


@pytest.mark.parametrize("tau,eps", [(TAU4, 1e-6), (0.0, 1e-6), (2.5, 1e-6), (1.0, 0.0),
                                     (1.0, 0.3)])
def test_bwd_dilution_tau_eps(tau, eps):
    inp = draw_qkv(2, 2, 200, 64, "bf16", seed=1234)
    g = draw_grad(2, 2, 200, 64, seed=1234)
    got = run_bwd(inp, g, tau, 1, eps)
    ref = oracle_grads(inp, g, tau, 1, eps)
    if tau == 0.0:   # bids independent of q and k
        assert np.all(got[0] == 0.0) and np.all(got[1] == 0.0)
        check_grads(got[2:3], ref[2:3], f"tau={tau} eps={eps}")
    else:
        check_grads(got[:3], ref[:3], f"tau={tau} eps={eps}")


@pytest.mark.parametrize("mode", [0, 1], ids=["tempered", "dilution"])
def test_bwd_heavy_keys_t1024(mode):
    """The dilution_t16k recipe (5 % of key rows at 3x norm) at T=1024."""
    w = PREFILL["dilution_t16k"]
    inp = prefill_inputs(w, T=1024, H=2)
    g = draw_grad(1, 2, 1024, 64, seed=w.seed)
    got = run_bwd(inp, g, 1.0, mode, w.eps)
    ref = oracle_grads(inp, g, 1.0, mode, w.eps)
    check_grads(got[:3], ref[:3], f"heavy mode={mode}")


def test_bwd_value_totals_t16k():
    """At the full T=16384 workload: every row of A sums to one, so the dV
    rows sum to the dO rows' sum (per head, per dim) in either mode."""
    import torch

    w = PREFILL["dilution_t16k"]
    inp = prefill_inputs(w, H=4)
    g = draw_grad(1, 4, w.T, 64, seed=w.seed)
    for mode in (0, 1):
        got = run_bwd(inp, g, 1.0, mode, w.eps)
        dv_sum = got[2].astype(np.float64).sum(axis=2)
        do_sum = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64).sum(axis=2)
        err = np.max(np.abs(dv_sum - do_sum)) / np.max(np.abs(do_sum))
        print(f"t16k mode={mode} dV total rel err {err:.3e}")
        assert err <= 5e-3
        assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1]))
        torch.cuda.empty_cache()


def test_bwd_deterministic():
    inp = draw_qkv(1, 2, 300, 64, "bf16", seed=77)
    g = draw_grad(1, 2, 300, 64, seed=77)
    a = run_bwd(inp, g, 1.0, 1)
    b = run_bwd(inp, g, 1.0, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
