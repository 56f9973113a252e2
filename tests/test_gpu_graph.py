"""Graph capture: the library allocates, clears and synchronises nothing, so a
step of its launches captures into a HIP graph as it is.  Every replay is
checked against eager runs, with eager work between the replays."""
import numpy as np
import pytest

from gpu_util import to_device
from transformer_attention_causal_amd import binding as ab
from transformer_attention_causal_amd.workloads import (decode_initial_demand, decode_queries,
                                                        draw_grad, draw_qkv)

pytestmark = pytest.mark.gpu


def test_step_replays_in_a_hip_graph():
    """Dilution forward and backward, tempered forward (a small grid, so the
    key-split row stages and their combine kernels are captured too) and one
    decode step that updates the demand in place: three replays equal three
    eager steps bit for bit, outputs, gradients and demand."""
    import torch

    B, H, T, d = 1, 4, 1000, 64
    inp = draw_qkv(B, H, T, d, "bf16", seed=7000, heavy_frac=0.05)
    q, k, v = (to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    ws, _ = ab.fwd_workspace(B, H, T, ab.ATTN_DILUTION, ab.ATTN_BF16, q.device, d)
    S, Hd, L = 4, 4, 3000
    cache = draw_qkv(S, Hd, L, d, "bf16", seed=7001)
    kc, vc = to_device(cache.k, "bf16"), to_device(cache.v, "bf16")
    D0 = torch.from_numpy(decode_initial_demand(S, Hd, L, seed=7001)).cuda()
    qd = to_device(decode_queries(1, S, Hd, d, seed=7001)[0], "bf16")
    dws, _ = ab.decode_workspace(S, Hd, L, q.device, d)
    dout = to_device(draw_grad(B, H, T, d, seed=7002), "bf16")
    bws, _ = ab.bwd_workspace(B, H, T, ab.ATTN_DILUTION, ab.ATTN_BF16, q.device, d)
    f32 = dict(dtype=torch.float32, device="cuda")

    # eager reference: forward and backward once, the decode step three times
    lse, rs = torch.empty((B, H, T), **f32), torch.empty((B, H, T), **f32)
    out_d = ab.fwd(q, k, v, tau=1.0, mode=ab.ATTN_DILUTION, eps=1e-6, workspace=ws, lse_out=lse,
                   rowsum_out=rs)
    grads = ab.bwd(q, k, v, out_d, dout, lse, rs, tau=1.0, mode=ab.ATTN_DILUTION, eps=1e-6,
                   workspace=bws)
    out_t = ab.fwd(q, k, v, tau=1.1, mode=ab.ATTN_TEMPERED)
    dem = D0.clone()
    dec_ref, dem_ref = [], []
    for _ in range(3):
        dec_ref.append(ab.decode(qd, kc, vc, dem, tau=1.0, eps=1e-6, workspace=dws).clone())
        dem_ref.append(dem.clone())
    torch.cuda.synchronize()

    # the same step captured once
    g_out_d, g_out_t = torch.empty_like(q), torch.empty_like(q)
    g_lse, g_rs = torch.empty((B, H, T), **f32), torch.empty((B, H, T), **f32)
    g_grads = [torch.empty_like(q) for _ in range(3)]
    g_dec = torch.empty_like(qd)
    g_dem = D0.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ab.fwd(q, k, v, tau=1.0, mode=ab.ATTN_DILUTION, eps=1e-6, out=g_out_d, workspace=ws,
               lse_out=g_lse, rowsum_out=g_rs)
        ab.bwd(q, k, v, g_out_d, dout, g_lse, g_rs, tau=1.0, mode=ab.ATTN_DILUTION, eps=1e-6,
               dq=g_grads[0], dk=g_grads[1], dv=g_grads[2], workspace=bws)
        ab.fwd(q, k, v, tau=1.1, mode=ab.ATTN_TEMPERED, out=g_out_t)
        ab.decode(qd, kc, vc, g_dem, tau=1.0, eps=1e-6, out=g_dec, workspace=dws)
    torch.cuda.synchronize()
    # capture records without running: the demand is still the initial one
    assert torch.equal(g_dem, D0)
    for r in range(3):
        for t in [g_out_d, g_out_t] + g_grads:
            t.fill_(0.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_out_d, out_d), f"replay {r}: dilution forward"
        for name, a, b in zip(("dq", "dk", "dv"), g_grads, grads):
            assert torch.equal(a, b), f"replay {r}: {name}"
        assert torch.equal(g_out_t, out_t), f"replay {r}: tempered forward"
        assert torch.equal(g_dec, dec_ref[r]), f"replay {r}: decode output"
        assert torch.equal(g_dem, dem_ref[r]), f"replay {r}: demand"
        # eager work between replays, on the same device
        x = torch.randn(4096, device="cuda")
        assert np.isfinite(float((x * x).sum()))
