"""GPU parity at head dimension 128 (the focal models' heads) and with
per-(batch, head) temperature multipliers, against the fp64 oracle through
the C ABI: forward of both operators, chunked prefill, and decode."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import (DEMAND_TOTAL_REL, assert_close, assert_workload, oracle_qkv,
                      oracle_view, to_device, say)
from transformer_attention_causal_amd import binding as ab
from transformer_attention_causal_amd.workloads import (PREFILL, decode_initial_demand,
                                                        decode_queries, draw_qkv, learned_tau,
                                                        prefill_inputs)

pytestmark = pytest.mark.gpu

TAU4 = math.sqrt(0.1 * math.log(4.0) + 1.0)


def head_inputs(inp, bh_list):
    """The oracle's view of the listed flattened heads, each as a [1,1,T,d] array."""
    B, H = inp.q.shape[:2]
    out = []
    for bh in bh_list:
        b, h = divmod(bh, H)
        out.append(tuple(oracle_view(np.ascontiguousarray(x[b:b + 1, h:h + 1]), inp.dtype)
                         for x in (inp.q, inp.k, inp.v)))
    return out


def run_prefill(inp, tau, mode, eps=1e-6, tau_bh=None, want_demand=False):
    import torch

    q, k, v = (to_device(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    B, H, T, _ = q.shape
    dem = torch.zeros((B, H, T), dtype=torch.float32, device="cuda") if want_demand else None
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    tb = torch.from_numpy(tau_bh).cuda() if tau_bh is not None else None
    out = ab.prefill(q, k, v, T, tau=tau, mode=mode, eps=eps, demand_in=dem, demand_out=dem,
                     lse_out=lse, tau_bh=tb)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy(), lse.cpu().numpy(),
            dem.cpu().numpy() if dem is not None else None)


# bars on the LSE and on each key's final demand (relative to the largest)
LSE_TOL = {"bf16": 2e-3, "f32": 1e-5}
DEMAND_TOL = {"bf16": 2e-2, "f32": 1e-5}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 7, 33, 64, 129, 300, 1000])
def test_d128_ragged_lengths(T, dtype):
    inp = draw_qkv(2, 2, T, 128, dtype, seed=6000 + T, heavy_frac=0.05)
    out, lse, dem = run_prefill(inp, 1.0, ab.ATTN_DILUTION, want_demand=True)
    ref, rlse, rdem = oracle.dilution_fwd(*oracle_qkv(inp), 1.0, 1e-6)
    assert_close(out, ref, dtype, f"d128 {dtype} dilution T={T}")
    assert np.max(np.abs(lse - rlse)) <= LSE_TOL[dtype]
    assert np.max(np.abs(dem.sum(axis=-1) / T - 1.0)) <= DEMAND_TOTAL_REL
    assert np.max(np.abs(dem - rdem)) <= DEMAND_TOL[dtype] * max(1.0, float(np.max(rdem)))
    out, lse, _ = run_prefill(inp, TAU4, ab.ATTN_TEMPERED)
    ref, rlse = oracle.tempered_fwd(*oracle_qkv(inp), TAU4)
    assert_close(out, ref, dtype, f"d128 {dtype} tempered T={T}")
    assert np.max(np.abs(lse - rlse)) <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_per_head_tau(dtype, d):
    """Per-(b,h) multipliers sqrt(d)/t, t ~ U[5, 10] (learned-temperature
    range): every head matches the oracle run with its own scalar tau."""
    B, H, T = 2, 3, 300
    inp = draw_qkv(B, H, T, d, dtype, seed=6100 + d, heavy_frac=0.05)
    taus = learned_tau(B, H, d, seed=6100 + d)
    for mode in (ab.ATTN_TEMPERED, ab.ATTN_DILUTION):
        out, lse, _ = run_prefill(inp, 1.0, mode, tau_bh=taus)
        for bh, (q1, k1, v1) in enumerate(head_inputs(inp, range(B * H))):
            b, h = divmod(bh, H)
            tau = float(taus[b, h])
            if mode == ab.ATTN_TEMPERED:
                ref, rlse = oracle.tempered_fwd(q1, k1, v1, tau)
            else:
                ref, rlse, _ = oracle.dilution_fwd(q1, k1, v1, tau, 1e-6)
            assert_close(out[b:b + 1, h:h + 1], ref, dtype,
                         f"{dtype} d={d} mode={mode} head {bh} tau={tau:.3f}")
            assert np.max(np.abs(lse[b, h] - rlse[0, 0])) <= (2e-3 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_d128_chunks_and_carried_demand(dtype):
    """Chunked prefill at d = 128 with per-head multipliers: chunks over a
    NaN-tailed cache reproduce the whole prefill and its column totals."""
    import torch

    B, H, T, d, Lcap = 1, 2, 700, 128, 769
    inp = draw_qkv(B, H, T, d, dtype, seed=6200, heavy_frac=0.05)
    taus = learned_tau(B, H, d, seed=6200)
    q, k, v = (to_device(a, dtype) for a in (inp.q, inp.k, inp.v))
    kc = torch.full((B, H, Lcap, d), float("nan"), dtype=q.dtype, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    D = torch.full((B, H, Lcap), 7.0, dtype=torch.float32, device="cuda")
    D[:, :, :T] = 0.0
    tb = torch.from_numpy(taus).cuda()
    outs = []
    for a, b in zip((0, 200, 333, 640), (200, 333, 640, 700)):
        kc[:, :, a:b] = k[:, :, a:b]
        vc[:, :, a:b] = v[:, :, a:b]
        outs.append(ab.prefill(q[:, :, a:b].contiguous(), kc, vc, b, tau=1.0,
                               mode=ab.ATTN_DILUTION, eps=1e-6, demand_in=D, demand_out=D,
                               tau_bh=tb))
    torch.cuda.synchronize()
    out = torch.cat(outs, dim=2).float().cpu().numpy()
    dem = D.cpu().numpy()
    assert np.all(dem[..., T:] == 7.0)
    for bh, (q1, k1, v1) in enumerate(head_inputs(inp, range(B * H))):
        tau = float(taus[0, bh])
        ref, _, rdem = oracle.dilution_fwd(q1, k1, v1, tau, 1e-6)
        assert_close(out[:, bh:bh + 1], ref, dtype, f"d128 {dtype} chunks head {bh}")
        assert (np.max(np.abs(dem[0, bh, :T] - rdem[0, 0]))
                <= DEMAND_TOL[dtype] * max(1.0, float(rdem.max())))


def test_d128_decode_steps():
    """Four cached-decode steps at d = 128 with per-(sequence, head)
    multipliers, demand carried between steps, against the oracle."""
    import torch

    S, H, L, d = 3, 4, 5000, 128
    inp = draw_qkv(S, H, L, d, "bf16", seed=6300)
    taus = learned_tau(S, H, d, seed=6300)
    D0 = decode_initial_demand(S, H, L, seed=6300)
    qs = decode_queries(4, S, H, d, seed=6300)
    kc, vc = to_device(inp.k, "bf16"), to_device(inp.v, "bf16")
    Dd = torch.from_numpy(D0.copy()).cuda()
    tb = torch.from_numpy(taus).cuda()
    kv_len = torch.tensor([L, 4097, 1], dtype=torch.int32, device="cuda")
    Dr = D0.astype(np.float64)
    for step in range(4):
        out = ab.decode(to_device(qs[step], "bf16"), kc, vc, Dd, tau=1.0, eps=1e-6,
                        kv_len=kv_len, tau_sh=tb)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        for s in range(S):
            for h in range(H):
                Dsh = np.ascontiguousarray(Dr[s:s + 1, h:h + 1])
                ref = oracle.dilution_decode_step(
                    oracle.Bf16(np.ascontiguousarray(qs[step][s:s + 1, h:h + 1])),
                    oracle.Bf16(np.ascontiguousarray(inp.k[s:s + 1, h:h + 1])),
                    oracle.Bf16(np.ascontiguousarray(inp.v[s:s + 1, h:h + 1])), Dsh,
                    float(taus[s, h]), 1e-6, kv_len=[int(kv_len[s])])
                Dr[s, h] = Dsh[0, 0]
                assert_close(got[s:s + 1, h:h + 1], ref, "bf16", f"decode step {step} s={s} h={h}")
        Dg = Dd.cpu().numpy().astype(np.float64)
        rel = np.abs(Dg.sum(-1) / Dr.sum(-1) - 1.0)
        assert np.max(rel) <= DEMAND_TOTAL_REL, f"step {step}: demand totals {np.max(rel):.2e}"


@pytest.mark.timeout(600)
def test_focal_d128_t16k_bf16_against_fp32_kernels_all_rows():
    """The whole focal workload (H=20, T=16384, d=128, learned per-head
    multipliers), every row of every head (the oracle checks every row of
    the four sharpest heads): bf16 outputs, LSE and final column demand agree
    with the fp32 kernels' on the same values, to the absolute bf16 bars (the
    fp32 kernels are held to the oracle at 1e-5)."""
    import torch

    w = PREFILL["focal_d128_t16k"]
    inp = prefill_inputs(w)
    taus = learned_tau(w.B, w.H, w.d, seed=w.seed)
    wide = {n: (getattr(inp, n).astype(np.uint32) << 16).view(np.float32) for n in ("q", "k", "v")}
    f32 = type(inp)(**{**inp.__dict__, **wide, "dtype": "f32"})
    for mode in (ab.ATTN_DILUTION, ab.ATTN_TEMPERED):
        dil = mode == ab.ATTN_DILUTION
        out, lse, dem = run_prefill(inp, 1.0, mode, w.eps, tau_bh=taus, want_demand=dil)
        torch.cuda.empty_cache()
        ref, rlse, rdem = run_prefill(f32, 1.0, mode, w.eps, tau_bh=taus, want_demand=dil)
        torch.cuda.empty_cache()
        assert_workload(out, ref.astype(np.float64), f"focal d128 mode={mode} all rows vs fp32 kernels")
        assert np.max(np.abs(lse - rlse)) <= LSE_TOL["bf16"]
        if dil:
            tot = np.max(np.abs(dem.astype(np.float64).sum(-1) / rdem.astype(np.float64).sum(-1) - 1.0))
            say(f"focal d128 demand totals bf16 vs fp32 kernels: {tot:.3e}")
            assert tot <= DEMAND_TOTAL_REL
            assert np.max(np.abs(dem - rdem)) <= DEMAND_TOL["bf16"] * max(1.0, float(rdem.max()))


def test_d128_deterministic():
    import torch

    inp = draw_qkv(1, 4, 777, 128, "bf16", seed=6400, heavy_frac=0.05)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    for mode in (ab.ATTN_TEMPERED, ab.ATTN_DILUTION):
        a = ab.fwd(q, k, v, tau=1.0, mode=mode)
        b = ab.fwd(q, k, v, tau=1.0, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_d128_decode_split_path():
    """Caches longer than 32768 keys take the chunked decode path (scores
    through the workspace, per-chunk partials combined in order): two steps
    at d = 128 with per-(sequence, head) multipliers and mixed lengths,
    demand carried between steps."""
    import torch

    S, H, L, d = 2, 2, 40000, 128
    inp = draw_qkv(S, H, L, d, "bf16", seed=6500)
    taus = learned_tau(S, H, d, seed=6500)
    D0 = decode_initial_demand(S, H, L, seed=6500)
    qs = decode_queries(2, S, H, d, seed=6500)
    kc, vc = to_device(inp.k, "bf16"), to_device(inp.v, "bf16")
    Dd = torch.from_numpy(D0.copy()).cuda()
    tb = torch.from_numpy(taus).cuda()
    kv_len = torch.tensor([L, 32769], dtype=torch.int32, device="cuda")
    Dr = D0.astype(np.float64)
    for step in range(2):
        out = ab.decode(to_device(qs[step], "bf16"), kc, vc, Dd, tau=1.0, eps=1e-6,
                        kv_len=kv_len, tau_sh=tb)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        for s in range(S):
            for h in range(H):
                Dsh = np.ascontiguousarray(Dr[s:s + 1, h:h + 1])
                ref = oracle.dilution_decode_step(
                    oracle.Bf16(np.ascontiguousarray(qs[step][s:s + 1, h:h + 1])),
                    oracle.Bf16(np.ascontiguousarray(inp.k[s:s + 1, h:h + 1])),
                    oracle.Bf16(np.ascontiguousarray(inp.v[s:s + 1, h:h + 1])), Dsh,
                    float(taus[s, h]), 1e-6, kv_len=[int(kv_len[s])])
                Dr[s, h] = Dsh[0, 0]
                assert_close(got[s:s + 1, h:h + 1], ref, "bf16", f"split decode step {step} s={s} h={h}")
        Dg = Dd.cpu().numpy().astype(np.float64)
        rel = np.abs(Dg.sum(-1) / Dr.sum(-1) - 1.0)
        assert np.max(rel) <= DEMAND_TOTAL_REL, f"step {step}: demand totals {np.max(rel):.2e}"
        assert np.max(np.abs(Dg - Dr)) <= 1e-4 * max(1.0, float(Dr.max()))
