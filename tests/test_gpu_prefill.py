"""GPU parity of chunked prefill (attn_prefill) against the fp64 oracle,
through the C ABI: chunks of query rows over cached keys, dilution carrying
the committed demand from chunk to chunk in place, both operators and both
storage types.  Cache rows past the keys hold NaN and must never be read;
demand entries past the keys hold 7.0 and must never be written."""
import math

import numpy as np
import pytest

import oracle
from gpu_util import DEMAND_TOTAL_REL, assert_close, oracle_qkv, oracle_view, to_device, say
from transformer_attention_causal_amd import binding as ab
from transformer_attention_causal_amd.workloads import draw_qkv

pytestmark = pytest.mark.gpu

TAU4 = math.sqrt(0.1 * math.log(4.0) + 1.0)


def _nan_cache(B, H, Lcap, d, dtype):
    import torch

    if dtype == "bf16":
        return torch.full((B, H, Lcap, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    return torch.full((B, H, Lcap, d), float("nan"), dtype=torch.float32, device="cuda")


def run_chunks(inp, bounds, Lcap, tau, mode, eps, demand0=None):
    """Prefill rows [bounds[i], bounds[i+1]) chunk by chunk, appending each
    chunk's keys/values to the caches first.  Returns (out, lse, demand) as
    host arrays (demand: the whole [B,H,Lcap] array, or None for tempered)."""
    import torch

    q, k, v = (to_device(a, inp.dtype) for a in (inp.q, inp.k, inp.v))
    B, H, T, d = q.shape
    kc, vc = _nan_cache(B, H, Lcap, d, inp.dtype), _nan_cache(B, H, Lcap, d, inp.dtype)
    D = None
    if mode == ab.ATTN_DILUTION:
        D = torch.full((B, H, Lcap), 7.0, dtype=torch.float32, device="cuda")
        D[:, :, :T] = 0.0 if demand0 is None else torch.from_numpy(demand0).cuda()
    outs, lses = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        kc[:, :, a:b] = k[:, :, a:b]
        vc[:, :, a:b] = v[:, :, a:b]
        lse = torch.empty((B, H, b - a), dtype=torch.float32, device="cuda")
        out = ab.prefill(q[:, :, a:b].contiguous(), kc, vc, b, tau=tau, mode=mode, eps=eps,
                         demand_in=D, demand_out=D, lse_out=lse)
        outs.append(out)
        lses.append(lse)
    torch.cuda.synchronize()
    out = torch.cat(outs, dim=2).float().cpu().numpy()
    lse = torch.cat(lses, dim=2).cpu().numpy()
    return out, lse, (D.cpu().numpy() if D is not None else None)


def check_demand(dem, rdem, T, dtype, what):
    assert np.all(dem[..., T:] == 7.0), f"{what}: demand past the keys was written"
    dem = dem[..., :T]
    if dtype == "f32":
        err = float(np.max(np.abs(dem - rdem) / np.maximum(1.0, np.abs(rdem))))
        say(f"{what} demand: max rel {err:.3e}")
        assert err <= 1e-5
    else:
        tot = float(np.max(np.abs(dem.sum(axis=-1) / rdem.sum(axis=-1) - 1.0)))
        err = float(np.max(np.abs(dem - rdem)) / max(1.0, float(np.max(rdem))))
        say(f"{what} demand: totals rel {tot:.3e} per-key {err:.3e}")
        assert tot <= DEMAND_TOTAL_REL and err <= 2e-2


CHUNKS_F32 = [(0, 300), (0, 100, 300), (0, 128, 256, 300), (0, 1, 2, 150, 299, 300)]
CHUNKS_BF16 = [(0, 700), (0, 200, 333, 640, 700), (0, 384, 700), (0, 699, 700),
               (0, 31, 32, 33, 500, 700)]


@pytest.mark.parametrize("bounds", CHUNKS_F32, ids=str)
def test_fp32_chunks_equal_whole_prefill(bounds):
    inp = draw_qkv(1, 2, 300, 64, "f32", seed=5000)
    for tau, eps in ((1.3, 1e-6), (1.0, 0.0)):
        out, lse, dem = run_chunks(inp, bounds, 333, tau, ab.ATTN_DILUTION, eps)
        ref, rlse, rdem = oracle.dilution_fwd(*oracle_qkv(inp), tau, eps)
        assert_close(out, ref, "f32", f"dilution chunks {bounds} tau={tau} eps={eps}")
        assert np.max(np.abs(lse - rlse)) <= 1e-5
        check_demand(dem, rdem, 300, "f32", f"chunks {bounds}")
    out, lse, _ = run_chunks(inp, bounds, 333, TAU4, ab.ATTN_TEMPERED, 0.0)
    ref, rlse = oracle.tempered_fwd(*oracle_qkv(inp), TAU4)
    assert_close(out, ref, "f32", f"tempered chunks {bounds}")
    assert np.max(np.abs(lse - rlse)) <= 1e-5


@pytest.mark.parametrize("bounds", CHUNKS_BF16, ids=str)
def test_bf16_chunks_equal_whole_prefill(bounds):
    inp = draw_qkv(2, 2, 700, 64, "bf16", seed=5100, heavy_frac=0.05)
    out, lse, dem = run_chunks(inp, bounds, 769, 1.0, ab.ATTN_DILUTION, 1e-6)
    ref, rlse, rdem = oracle.dilution_fwd(*oracle_qkv(inp), 1.0, 1e-6)
    assert_close(out, ref, "bf16", f"dilution chunks {bounds}")
    assert np.max(np.abs(lse - rlse)) <= 2e-3
    check_demand(dem, rdem, 700, "bf16", f"chunks {bounds}")
    out, lse, _ = run_chunks(inp, bounds, 769, TAU4, ab.ATTN_TEMPERED, 0.0)
    ref, rlse = oracle.tempered_fwd(*oracle_qkv(inp), TAU4)
    assert_close(out, ref, "bf16", f"tempered chunks {bounds}")
    assert np.max(np.abs(lse - rlse)) <= 2e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Tk,Tq", [(1000, 300), (1000, 1000), (513, 1), (4096, 129)])
def test_chunk_from_carried_demand(dtype, Tk, Tq):
    """One chunk over cached keys whose demand is already non-zero (uniform on
    [0, 4) for the cached keys, zero for the chunk's own), out of place: the
    input demand is left as it was."""
    import torch

    B, H, d, Lcap = 1, 2, 64, Tk + 40
    inp = draw_qkv(B, H, Tk, d, dtype, seed=5200 + Tk + Tq, heavy_frac=0.05)
    P = Tk - Tq
    rng = np.random.Generator(np.random.PCG64(5300 + Tq))
    D0 = np.zeros((B, H, Lcap))
    D0[:, :, :P] = rng.random((B, H, P)) * 4.0
    D0 = D0.astype(np.float32)
    qc = np.ascontiguousarray(inp.q[:, :, P:])
    kc = np.zeros((B, H, Lcap, d), dtype=inp.k.dtype)
    vc = np.zeros((B, H, Lcap, d), dtype=inp.v.dtype)
    kc[:, :, :Tk] = inp.k
    vc[:, :, :Tk] = inp.v
    din = torch.from_numpy(D0).cuda()
    dout = torch.full_like(din, 7.0)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device="cuda")
    out = ab.prefill(to_device(qc, dtype), to_device(kc, dtype), to_device(vc, dtype), Tk,
                     tau=1.0, mode=ab.ATTN_DILUTION, eps=1e-6, demand_in=din, demand_out=dout,
                     lse_out=lse)
    torch.cuda.synchronize()
    Dref = D0.astype(np.float64)
    ref, rlse = oracle.prefill(oracle_view(qc, dtype), oracle_view(kc, dtype),
                               oracle_view(vc, dtype), Tk, 1.0, 1e-6, 1, Dref)
    assert_close(out.float().cpu().numpy(), ref, dtype, f"carried demand Tk={Tk} Tq={Tq}")
    assert np.max(np.abs(lse.cpu().numpy() - rlse)) <= (1e-5 if dtype == "f32" else 2e-3)
    assert np.array_equal(din.cpu().numpy(), D0)
    got = dout.cpu().numpy()
    assert np.all(got[..., Tk:] == 7.0)
    tol = 1e-5 if dtype == "f32" else 2e-2
    err = np.max(np.abs(got[..., :Tk] - Dref[..., :Tk]) / np.maximum(1.0, Dref[..., :Tk]))
    say(f"carried demand Tk={Tk} Tq={Tq}: demand max rel {err:.3e}")
    assert err <= tol
    # the chunk adds one unit of demand per row
    added = got[..., :Tk].astype(np.float64).sum(-1) - D0[..., :Tk].astype(np.float64).sum(-1)
    assert np.max(np.abs(added / Tq - 1.0)) <= 1e-4


def test_one_row_chunk_is_a_decode_step():
    """A one-row chunk whose key was just appended is one cached-decode step
    with kv_len = Tk (two different kernels), with the same demand update."""
    import torch

    S, H, d, Lcap, Tk = 2, 4, 64, 5000, 4097
    inp = draw_qkv(S, H, Lcap, d, "bf16", seed=5400)
    rng = np.random.Generator(np.random.PCG64(5401))
    D0 = (rng.random((S, H, Lcap)) * 4.0).astype(np.float32)
    D0[:, :, Tk - 1:] = 0.0
    kc, vc = to_device(inp.k, "bf16"), to_device(inp.v, "bf16")
    qrow = np.ascontiguousarray(inp.q[:, :, Tk - 1])
    q = to_device(qrow, "bf16")
    d_pre = torch.from_numpy(D0).cuda()
    d_dec = d_pre.clone()
    out_p = ab.prefill(q[:, :, None, :].contiguous(), kc, vc, Tk, tau=1.0,
                       mode=ab.ATTN_DILUTION, eps=1e-6, demand_in=d_pre, demand_out=d_pre)
    kv_len = torch.full((S,), Tk, dtype=torch.int32, device="cuda")
    out_d = ab.decode(q, kc, vc, d_dec, tau=1.0, eps=1e-6, kv_len=kv_len)
    torch.cuda.synchronize()
    Dref = D0.astype(np.float64)
    ref = oracle.dilution_decode_step(oracle.Bf16(qrow), oracle.Bf16(inp.k), oracle.Bf16(inp.v),
                                      Dref, 1.0, 1e-6, kv_len=[Tk] * S)
    assert_close(out_p[:, :, 0].float().cpu().numpy(), ref, "bf16", "one-row chunk")
    assert_close(out_d.float().cpu().numpy(), ref, "bf16", "decode step")
    a, b = d_pre.cpu().numpy(), d_dec.cpu().numpy()
    assert np.max(np.abs(a - Dref)) <= 1e-4 * max(1.0, float(Dref.max()))
    assert np.max(np.abs(a - b)) <= 1e-4 * max(1.0, float(Dref.max()))


@pytest.mark.timeout(600)
def test_long_chunk_after_long_cache():
    """A 1536-row chunk after 18464 cached keys (20000 keys in all, heavy keys),
    starting from the demand the cached rows would have committed (uniform on
    [0, 4 (T-j)/T), the decode workload's recipe); sampled rows of both heads
    against the oracle, and the added demand per head."""
    import torch

    from transformer_attention_causal_amd.workloads import decode_initial_demand

    B, H, d, Tk, Tq = 1, 2, 64, 20000, 1536
    inp = draw_qkv(B, H, Tk, d, "bf16", seed=5500, heavy_frac=0.05)
    P = Tk - Tq
    D0 = decode_initial_demand(B, H, Tk, seed=5501)
    D0[:, :, P:] = 0.0
    qc = np.ascontiguousarray(inp.q[:, :, P:])
    din = torch.from_numpy(D0).cuda()
    out = ab.prefill(to_device(qc, "bf16"), to_device(inp.k, "bf16"), to_device(inp.v, "bf16"),
                     Tk, tau=1.0, mode=ab.ATTN_DILUTION, eps=1e-6, demand_in=din,
                     demand_out=din)
    torch.cuda.synchronize()
    Dref = D0.astype(np.float64)
    ref, _ = oracle.prefill(oracle.Bf16(qc), oracle.Bf16(inp.k), oracle.Bf16(inp.v), Tk, 1.0,
                            1e-6, 1, Dref)
    assert_close(out.float().cpu().numpy(), ref, "bf16", "chunk 1536 after 18464")
    got = din.cpu().numpy().astype(np.float64)
    added = got.sum(-1) - D0.astype(np.float64).sum(-1)
    assert np.max(np.abs(added / Tq - 1.0)) <= 1e-3
    assert np.max(np.abs(got - Dref)) <= 2e-2 * max(1.0, float(Dref.max()))


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_whole_prefill_is_the_forward(dtype, d):
    """attn_prefill over a whole sequence (Tq = Tk = T, no carried demand) runs
    the forward's launches: out, lse, row sums and final column demand equal
    attn_fwd_ex's bit for bit (tempered: out and lse)."""
    import torch

    B, H, T = 2, 3, 300
    inp = draw_qkv(B, H, T, d, dtype, seed=5600 + d)
    q, k, v = (to_device(a, dtype) for a in (inp.q, inp.k, inp.v))

    def f32(*shape):
        return torch.empty(shape, dtype=torch.float32, device="cuda")

    for mode in (ab.ATTN_TEMPERED, ab.ATTN_DILUTION):
        dil = mode == ab.ATTN_DILUTION
        l1, l2 = f32(B, H, T), f32(B, H, T)
        r1, r2 = (f32(B, H, T), f32(B, H, T)) if dil else (None, None)
        d1, d2 = (f32(B, H, T), f32(B, H, T)) if dil else (None, None)
        o1 = ab.fwd(q, k, v, tau=TAU4, mode=mode, eps=1e-6, lse_out=l1, rowsum_out=r1,
                    demand_out=d1)
        o2 = ab.prefill(q, k, v, T, tau=TAU4, mode=mode, eps=1e-6, lse_out=l2, rowsum_out=r2,
                        demand_out=d2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (dtype, d, mode)
        if dil:
            assert torch.equal(r1, r2) and torch.equal(d1, d2), (dtype, d, mode)


def test_chunk_row_sums_match_whole_prefill():
    """The row sums a chunked prefill returns (rowsum_out, what the backward
    needs) agree with the whole prefill's, chunk by chunk (bf16, d = 64)."""
    import torch

    B, H, T, d = 1, 2, 700, 64
    inp = draw_qkv(B, H, T, d, "bf16", seed=5700, heavy_frac=0.05)
    q, k, v = (to_device(a, "bf16") for a in (inp.q, inp.k, inp.v))
    rs_whole = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    ab.prefill(q, k, v, T, tau=1.0, mode=ab.ATTN_DILUTION, eps=1e-6, rowsum_out=rs_whole)
    D = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    parts = []
    for a, b in zip((0, 200, 333, 640), (200, 333, 640, 700)):
        rs = torch.empty((B, H, b - a), dtype=torch.float32, device="cuda")
        ab.prefill(q[:, :, a:b].contiguous(), k, v, b, tau=1.0, mode=ab.ATTN_DILUTION, eps=1e-6,
                   demand_in=D, demand_out=D, rowsum_out=rs)
        parts.append(rs)
    torch.cuda.synchronize()
    got = torch.cat(parts, dim=2).cpu().numpy().astype(np.float64)
    ref = rs_whole.cpu().numpy().astype(np.float64)
    rel = float(np.max(np.abs(got / ref - 1.0)))
    say(f"chunk row sums vs whole: max rel {rel:.3e}")
    assert np.all(ref > 0) and rel <= 5e-3


@pytest.mark.timeout(600)
def test_bench_chunking_t16k_against_oracle():
    """The measured chunked-prefill configuration at full length: T = 16384
    (the dilution workload's recipe, heavy keys) as 8 chunks of 2048 rows over
    the cache, demand carried in place, 2 heads; every row and the final
    demand per key against the oracle's whole prefill."""
    from transformer_attention_causal_amd.workloads import PREFILL, prefill_inputs

    w = PREFILL["dilution_t16k"]
    inp = prefill_inputs(w, H=2)
    bounds = tuple(range(0, w.T + 1, 2048))
    out, lse, dem = run_chunks(inp, bounds, w.T + 64, 1.0, ab.ATTN_DILUTION, w.eps)
    ref, rlse, rdem = oracle.dilution_fwd(*oracle_qkv(inp), 1.0, w.eps)
    assert_close(out, ref, "bf16", "8 x 2048 chunks at T=16384")
    lse_err = float(np.max(np.abs(lse - rlse)))
    say(f"8 x 2048 chunks lse: max-abs {lse_err:.3e}")
    assert lse_err <= 2e-3
    check_demand(dem, rdem, w.T, "bf16", "8 x 2048 chunks")
