"""The library's device memory cache, on the GPU: a plan or an attend returns
to its caller while earlier GPU work is still queued (the runtime's
stream-ordered pool would have made the host wait for that work), blocks
reused across calls of other sizes and on other streams give bit-identical
outputs, and fp_workspace_trim leaves later calls working."""
import time

import numpy as np
import pytest

from synth import BY_NAME, LayerGen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_long_context_last_amd as F
    return F


def layer(cfg):
    return LayerGen(cfg).torch_layer("cuda")


def plan_of(F, cfg, q, k, **kw):
    return F.plan(q, k, block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget, **kw)


def test_calls_do_not_wait_for_queued_gpu_work(F):
    cfg = BY_NAME["llama8b_32k"].with_(N=8192)
    q, k, v = layer(cfg)
    out = torch.empty_like(q)
    # warm the cache: these calls allocate, later ones reuse
    for _ in range(2):
        P = plan_of(F, cfg, q, k)
        F.attend(P, q, k, v, out=out)
    torch.cuda.synchronize()
    ref = out.clone()
    x = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(40):
        y = x @ x                       # tens of ms or more of queued matrix work (0.23 s measured)
    e1.record()
    t0 = time.perf_counter()
    plans = []
    for _ in range(3):
        P = plan_of(F, cfg, q, k)
        F.attend(P, q, k, v, out=out)
        plans.append(P)
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    queued_ms = e0.elapsed_time(e1)
    print(f"[workspace] 3 x (plan + attend) returned after {host_ms:.1f} ms with {queued_ms:.1f} ms of GPU work "
          f"queued ahead", flush=True)
    assert queued_ms > 20.0
    assert host_ms < 0.5 * queued_ms, (host_ms, queued_ms)
    assert torch.equal(out, ref)


def test_reuse_across_sizes_and_streams_is_exact(F):
    cfgs = [BY_NAME["llama8b_32k"].with_(N=8192),
            BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=2, N=3000, block=64, min_budget=256,
                                         explicit_types=("V", "S", "QA", "N") * 2),
            BY_NAME["tiny_fp32_4k"].with_(N=1000)]
    layers = [layer(c) for c in cfgs]
    # references, each computed from an emptied cache and synchronized
    refs = []
    for c, (q, k, v) in zip(cfgs, layers):
        F.workspace_trim()
        P = plan_of(F, c, q, k, vs_granularity="token" if c.block == 64 else "block")
        o = torch.full_like(q, float("nan"))
        F.attend(P, q, k, v, out=o)
        torch.cuda.synchronize()
        refs.append((P.copy_out(), o.clone()))
        del P
    # the same calls back to back without synchronizing, alternating two
    # streams, largest first: every call reuses blocks released by others
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    order = [(rep, i) for rep in range(2) for i in range(len(cfgs))]
    bufs = [torch.full_like(layers[i][0], float("nan")) for _, i in order]
    torch.cuda.synchronize()
    outs = []
    for (rep, i), o in zip(order, bufs):
        c, (q, k, v) = cfgs[i], layers[i]
        sp, sa = (s1, s2) if (i + rep) % 2 == 0 else (s2, s1)
        with torch.cuda.stream(sp):
            P = plan_of(F, c, q, k, vs_granularity="token" if c.block == 64 else "block")
        F.attend(P, q, k, v, out=o, stream=sa)
        outs.append((i, P, o))
    torch.cuda.synchronize()
    for i, P, o in outs:
        (pat, djs, rp, ci), ro = refs[i]
        pat2, djs2, rp2, ci2 = P.copy_out()
        assert np.array_equal(pat, pat2) and np.array_equal(djs, djs2)
        assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2)
        assert torch.equal(o, ro), f"layer {i}"
    print(f"[workspace] {len(outs)} reused calls bit-identical", flush=True)


def test_trim_then_calls_still_work(F):
    cfg = BY_NAME["tiny_fp32_4k"].with_(N=2048)
    q, k, v = layer(cfg)
    P = plan_of(F, cfg, q, k)
    o1 = torch.empty_like(q)
    F.attend(P, q, k, v, out=o1)
    F.workspace_trim()             # the live plan keeps its buffers
    o2 = torch.empty_like(q)
    F.attend(P, q, k, v, out=o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    del P
    F.workspace_trim()
    P = plan_of(F, cfg, q, k)
    o3 = torch.empty_like(q)
    F.attend(P, q, k, v, out=o3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3)
