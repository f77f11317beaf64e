"""fp_prefill_attend_noalloc (the attention call that allocates nothing and
works in the library's static per-GPU workspace) against fp_prefill_attend
on the same plans: outputs bit-identical, on calls in a row whose sizes
shrink (so the second call runs over what the first left in the workspace),
for both dtypes, a token-granular plan, a packed batch of ragged sequences
and an attend on a stream other than the plan's; a plan whose workspace
exceeds the static array is refused before anything is enqueued."""
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
    q, k, v = LayerGen(cfg).torch_layer("cuda")
    return q, k, v


def both(F, P, q, k, v, stream=None):
    ref = torch.full_like(q, float("nan"))
    got = torch.full_like(q, float("nan"))
    F.attend(P, q, k, v, out=ref)
    F.attend(P, q, k, v, out=got, noalloc=True, stream=stream)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_attend_on_shrinking_calls(F):
    base = BY_NAME["llama8b_32k"]
    # 1: 32 query / 8 kv heads, 16k tokens, bf16, block 128 (V^T: 32 MiB of the 64)
    c1 = base.with_(N=16384)
    q, k, v = layer(c1)
    P = F.plan(q, k, block=c1.block, gamma=c1.gamma, tau=c1.tau, min_budget=c1.min_budget)
    ref, got = both(F, P, q, k, v)
    print(f"[noalloc] call 1: {c1.Hq}q/{c1.Hkv}kv N={c1.N} bf16 block {c1.block}", flush=True)
    assert not torch.isnan(ref).any()
    assert torch.equal(ref, got)
    del P, q, k, v, ref, got
    # 2: smaller, ragged length, block 64, token-granular columns (gathered tiles in the workspace too)
    c2 = base.with_(Hq=8, Hkv=2, N=3000, block=64, min_budget=256, explicit_types=("V", "S", "QA", "N") * 2)
    q, k, v = layer(c2)
    P = F.plan(q, k, block=c2.block, gamma=c2.gamma, tau=c2.tau, min_budget=c2.min_budget, vs_granularity="token")
    ref, got = both(F, P, q, k, v)
    print(f"[noalloc] call 2: {c2.Hq}q/{c2.Hkv}kv N={c2.N} bf16 block 64 token columns", flush=True)
    assert not torch.isnan(ref).any()
    assert torch.equal(ref, got)
    del P, q, k, v, ref, got
    # 3: smaller still, fp32, block 128
    c3 = BY_NAME["tiny_fp32_4k"].with_(N=1000)
    q, k, v = layer(c3)
    P = F.plan(q, k, block=c3.block, gamma=c3.gamma, tau=c3.tau, min_budget=c3.min_budget)
    ref, got = both(F, P, q, k, v)
    print(f"[noalloc] call 3: {c3.Hq}q/{c3.Hkv}kv N={c3.N} fp32", flush=True)
    assert torch.equal(ref, got)


def test_noalloc_packed_batch_and_other_stream(F):
    cfg = BY_NAME["llama8b_32k"].with_(Hq=4, Hkv=2, N=5000, explicit_types=("V", "S", "QA", "N"))
    q4, k4, v4 = layer(cfg)
    lens = [2100, 0, 1, 1777, 1122]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = torch.cat([q4[0, :, :L].transpose(0, 1) for L in lens if L], 0).contiguous()
    k = torch.cat([k4[0, :, :L].transpose(0, 1) for L in lens if L], 0).contiguous()
    v = torch.cat([v4[0, :, :L].transpose(0, 1) for L in lens if L], 0).contiguous()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        P = F.plan_varlen(q, k, cu, block=128, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget)
    # the allocation-free call on the current stream, the plan on stream s
    ref, got = both(F, P, q, k, v, stream=torch.cuda.current_stream())
    print(f"[noalloc] packed batch {lens}", flush=True)
    assert not torch.isnan(ref).any()
    assert torch.equal(ref, got)


def test_noalloc_refuses_oversized_workspace(F):
    # 8 kv heads x 65536 tokens x 128 x 2 bytes of V^T = 128 MiB > 64 MiB
    cfg = BY_NAME["llama8b_32k"].with_(Hq=8, Hkv=8, N=65536, explicit_types=("N",) * 8)
    q = torch.randn(1, 8, cfg.N, 128, device="cuda", dtype=torch.bfloat16)
    k = torch.randn_like(q)
    v = torch.randn_like(q)
    P = F.plan(q, k, block=128, gamma=0.95, tau=0.1, min_budget=1024)
    out = torch.zeros_like(q)
    with pytest.raises(F.FpError) as e:
        F.attend(P, q, k, v, out=out, noalloc=True)
    assert e.value.status == -3 and "workspace" in str(e.value)
    torch.cuda.synchronize()
    assert not out.any()          # nothing was enqueued
