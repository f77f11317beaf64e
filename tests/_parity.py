"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding and compare it with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np

import oracle as O

BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
FP32_MAX_ABS = 1e-4


def gpu_plan(F, q, k, cfg_like):
    return F.plan(q, k, block=cfg_like.block, gamma=cfg_like.gamma, tau=cfg_like.tau,
                  min_budget=cfg_like.min_budget)


def compare_head(P, gpu_dbg: dict, gpu_pattern, gpu_djs, gpu_lists, bh: int, hp: O.HeadPlan,
                 intermediates: bool = True):
    """Bit-exact comparison of one head's plan (and intermediates) with the oracle."""
    nb = hp.A.shape[0]
    if intermediates:
        np.testing.assert_array_equal(gpu_dbg["qbar"][bh], hp.qbar)
        # the GPU keeps `block` representative rows; with fewer tokens the
        # first ones do not exist and read 0
        R = hp.stats.M.shape[0]
        skip = gpu_dbg["rowmax"][bh].shape[0] - R
        np.testing.assert_array_equal(gpu_dbg["rowmax"][bh][skip:], hp.stats.M)
        np.testing.assert_array_equal(gpu_dbg["rowsum"][bh][skip:], hp.stats.Z)
        assert not gpu_dbg["rowmax"][bh][:skip].any() and not gpu_dbg["rowsum"][bh][:skip].any()
        np.testing.assert_array_equal(gpu_dbg["colsum"][bh], hp.stats.c)
        np.testing.assert_array_equal(gpu_dbg["diagsum"][bh], hp.stats.g)
        np.testing.assert_array_equal(gpu_dbg["atrue"][bh], hp.stats.a_true)
        np.testing.assert_array_equal(gpu_dbg["ahat"][bh], O.tri_values(hp.A))
    assert gpu_djs[bh] == hp.D, (bh, gpu_djs[bh], hp.D)
    assert int(gpu_pattern[bh]) == hp.pattern, bh
    assert len(gpu_lists[bh]) == nb
    for r in range(nb):
        if not np.array_equal(gpu_lists[bh][r], hp.lists[r]):
            raise AssertionError(f"head {bh} row {r}: gpu {gpu_lists[bh][r][:20]} "
                                 f"oracle {hp.lists[r][:20]}")


def check_attention(out_gpu: np.ndarray, ref: np.ndarray, dtype: str, where: str = ""):
    err = np.abs(out_gpu.astype(np.float64) - ref)
    if dtype == "bf16":
        assert err.max() <= BF16_MAX_ABS, f"{where} max abs {err.max():.3g}"
        assert err.mean() <= BF16_MEAN_ABS, f"{where} mean abs {err.mean():.3g}"
    else:
        assert err.max() <= FP32_MAX_ABS, f"{where} max abs {err.max():.3g}"
    return float(err.max()), float(err.mean())


def list_properties(lists, nb: int, floor_blocks: int):
    """Properties every plan has at any size: per row a strictly ascending list
    of key blocks in [0, row] with at least min(row + 1, floor) entries."""
    for r, x in enumerate(lists):
        assert len(x) >= min(r + 1, floor_blocks), (r, len(x))
        assert x.min() >= 0 and x.max() <= r
        assert np.all(np.diff(x) > 0)
