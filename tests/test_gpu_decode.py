"""GPU parity of the cached-decode step against the fp64 oracle, through the
C ABI.  The oracle keeps its own fp64 demand and replays the same steps from
the same fp32 initial demand."""
import numpy as np
import pytest

import oracle
from gpu_util import DEMAND_TOTAL_REL, assert_close, to_device, say
from transformer_attention_causal_amd import binding as ab
from transformer_attention_causal_amd.workloads import (decode_cache_host, decode_initial_demand,
                                                        decode_queries, draw_qkv)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("L", [1, 5, 64, 1000, 2048, 2049, 5000, 32768, 32769])
def test_decode_small_matches_oracle(L):
    import torch

    S, H, d, steps = 3, 2, 64, 4
    kc, vc = decode_cache_host(S, H, L, d, seed=5000 + L)
    D0 = decode_initial_demand(S, H, L, seed=5000 + L)
    qs = decode_queries(steps, S, H, d, seed=5000 + L)
    kc_d, vc_d = to_device(kc, "bf16"), to_device(vc, "bf16")
    D_d = torch.from_numpy(D0.copy()).cuda()
    D_ref = D0.astype(np.float64)
    for s in range(steps):
        out = ab.decode(to_device(qs[s], "bf16"), kc_d, vc_d, D_d, tau=1.0, eps=1e-6)
        ref = oracle.dilution_decode_step(oracle.Bf16(qs[s]), oracle.Bf16(kc), oracle.Bf16(vc),
                                          D_ref, 1.0, 1e-6)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().numpy(), ref, "bf16", f"decode L={L} step={s}")
        Dg = D_d.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(Dg.sum(-1) / D_ref.sum(-1) - 1.0)) <= DEMAND_TOTAL_REL
        assert np.max(np.abs(Dg - D_ref)) <= 1e-4 * max(1.0, float(D_ref.max()))


def test_decode_kv_len_and_append_matches_prefill_rows():
    """Decoding token by token with the new key appended (kv_len = i+1, its
    demand zeroed) reproduces the prefill rows of dilution attention."""
    import torch

    T, H = 70, 2
    inp = draw_qkv(1, H, T, 64, "bf16", seed=5100, heavy_frac=0.05)
    ref, _, rdem = oracle.dilution_fwd(oracle.Bf16(inp.q), oracle.Bf16(inp.k),
                                       oracle.Bf16(inp.v), 1.0, 1e-6)
    kc, vc = to_device(inp.k, "bf16"), to_device(inp.v, "bf16")
    q_all = to_device(inp.q, "bf16")
    D = torch.zeros((1, H, T), dtype=torch.float32, device="cuda")
    outs = []
    for i in range(T):
        kv_len = torch.full((1,), i + 1, dtype=torch.int32, device="cuda")
        outs.append(ab.decode(q_all[:, :, i].contiguous(), kc, vc, D, tau=1.0, eps=1e-6,
                              kv_len=kv_len).float())
    torch.cuda.synchronize()
    got = torch.stack(outs, dim=2).cpu().numpy()
    assert_close(got, ref, "bf16", "append decode vs prefill rows")
    assert np.max(np.abs(D.cpu().numpy() - rdem)) <= 1e-4 * max(1.0, float(rdem.max()))


def test_decode_deterministic_and_resumable():
    """Checkpoint/resume: running 3 steps, copying the demand, then 3 more
    equals 6 uninterrupted steps bit for bit."""
    import torch

    S, H, L = 2, 2, 3000
    kc, vc = decode_cache_host(S, H, L, 64, seed=5200)
    D0 = decode_initial_demand(S, H, L, seed=5200)
    qs = decode_queries(6, S, H, 64, seed=5200)
    kc_d, vc_d = to_device(kc, "bf16"), to_device(vc, "bf16")
    Da = torch.from_numpy(D0.copy()).cuda()
    outs_a = [ab.decode(to_device(qs[s], "bf16"), kc_d, vc_d, Da).clone() for s in range(6)]
    Db = torch.from_numpy(D0.copy()).cuda()
    outs_b = [ab.decode(to_device(qs[s], "bf16"), kc_d, vc_d, Db).clone() for s in range(3)]
    saved = Db.cpu().clone()
    Dc = saved.cuda()
    outs_b += [ab.decode(to_device(qs[s], "bf16"), kc_d, vc_d, Dc).clone() for s in range(3, 6)]
    torch.cuda.synchronize()
    assert torch.equal(Da, Dc)
    for x, y in zip(outs_a, outs_b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [64, 128])
def test_fused_and_chunked_decode_agree(d):
    """The same keys through the two decode implementations: a cache of
    exactly L = 30000 keys takes the fused path (scores in LDS), the same keys
    inside a 40000-key cache (kv_len = 30000) the chunked path (scores through
    the workspace, per-chunk partials).  Outputs and demand agree to rounding."""
    import torch

    S, H, L, Lbig = 2, 2, 30000, 40000
    inp = draw_qkv(S, H, Lbig, d, "bf16", seed=3300 + d)
    D0 = decode_initial_demand(S, H, Lbig, seed=3300 + d)
    q = to_device(decode_queries(1, S, H, d, seed=3300 + d)[0], "bf16")
    kb, vb = to_device(inp.k, "bf16"), to_device(inp.v, "bf16")
    ks, vs = kb[:, :, :L].contiguous(), vb[:, :, :L].contiguous()
    Db = torch.from_numpy(D0.copy()).cuda()
    Ds = Db[:, :, :L].contiguous()
    kv_len = torch.full((S,), L, dtype=torch.int32, device="cuda")
    o_fused = ab.decode(q, ks, vs, Ds, tau=1.0, eps=1e-6)
    o_chunk = ab.decode(q, kb, vb, Db, tau=1.0, eps=1e-6, kv_len=kv_len)
    torch.cuda.synchronize()
    a, b = o_fused.float().cpu().numpy(), o_chunk.float().cpu().numpy()
    err = float(np.max(np.abs(a - b)))
    say(f"d={d}: fused vs chunked max-abs {err:.3e}")
    assert err <= 2e-2 * max(1.0, float(np.max(np.abs(a))))
    dd = np.abs(Ds.cpu().numpy() - Db[:, :, :L].cpu().numpy())
    assert float(dd.max()) <= 1e-5 * max(1.0, float(D0.max()) + 1.0)
    assert np.array_equal(Db[:, :, L:].cpu().numpy(), D0[:, :, L:])   # past kv_len: untouched


@pytest.mark.parametrize("L", [5000, 33000])
def test_decode_per_head_tau_d64(L):
    """Per-(sequence, head) multipliers at d = 64 on both decode paths (fused
    up to 32768 keys, chunked beyond): two steps against the oracle with the
    demand carried."""
    import torch

    from transformer_attention_causal_amd.workloads import learned_tau

    S, H, d = 2, 3, 64
    inp = draw_qkv(S, H, L, d, "bf16", seed=3400 + L)
    taus = learned_tau(S, H, d, seed=3400 + L)
    D0 = decode_initial_demand(S, H, L, seed=3400 + L)
    qs = decode_queries(2, S, H, d, seed=3400 + L)
    kc, vc = to_device(inp.k, "bf16"), to_device(inp.v, "bf16")
    Dd = torch.from_numpy(D0.copy()).cuda()
    tb = torch.from_numpy(taus).cuda()
    Dr = D0.astype(np.float64)
    for step in range(2):
        got = ab.decode(to_device(qs[step], "bf16"), kc, vc, Dd, tau=1.0, eps=1e-6,
                        tau_sh=tb).float().cpu().numpy()
        for s in range(S):
            for h in range(H):
                Dsh = np.ascontiguousarray(Dr[s:s + 1, h:h + 1])
                ref = oracle.dilution_decode_step(
                    oracle.Bf16(np.ascontiguousarray(qs[step][s:s + 1, h:h + 1])),
                    oracle.Bf16(np.ascontiguousarray(inp.k[s:s + 1, h:h + 1])),
                    oracle.Bf16(np.ascontiguousarray(inp.v[s:s + 1, h:h + 1])), Dsh,
                    float(taus[s, h]), 1e-6)
                Dr[s, h] = Dsh[0, 0]
                assert_close(got[s:s + 1, h:h + 1], ref, "bf16",
                             f"L={L} step {step} s={s} h={h} tau={taus[s, h]:.3f}")
        Dg = Dd.cpu().numpy().astype(np.float64)
        assert np.max(np.abs(Dg.sum(-1) / Dr.sum(-1) - 1.0)) <= DEMAND_TOTAL_REL
        assert np.max(np.abs(Dg - Dr)) <= 1e-4 * max(1.0, float(Dr.max()))


@pytest.mark.parametrize("Lcap", [5000, 40000])
def test_decode_kv_len_out_of_range_is_clamped(Lcap):
    """kv_len values outside [1, Lcap] are clamped on the device: 0 and a
    negative length act as 1 and a length past the cache as Lcap, on the
    fused path (Lcap <= 32768) and the chunked one.  Outputs and demand equal
    those of the clamped lengths bit for bit."""
    import torch

    S, H = 3, 2
    kc, vc = decode_cache_host(S, H, Lcap, 64, seed=5300 + Lcap)
    D0 = decode_initial_demand(S, H, Lcap, seed=5300 + Lcap)
    q = to_device(decode_queries(1, S, H, 64, seed=5300 + Lcap)[0], "bf16")
    kc_d, vc_d = to_device(kc, "bf16"), to_device(vc, "bf16")
    outs, dems = [], []
    for lens in ([0, -7, Lcap + 100], [1, 1, Lcap]):
        D = torch.from_numpy(D0.copy()).cuda()
        kv_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
        outs.append(ab.decode(q, kc_d, vc_d, D, tau=1.0, eps=1e-6, kv_len=kv_len))
        dems.append(D)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(dems[0], dems[1])
    # a one-key decode attends to key 0 alone: the output is v_0
    v0 = to_device(vc[:2, :, 0], "bf16")
    assert torch.equal(outs[0][:2], v0)
