"""GPU parity on seeded random small shapes (and packed batches of them): batch, query / key-value heads
(grouped 1:1 up to 6:1, three key-value heads), head dim, block, dtype,
sequence length (ragged tails, lengths below one block), gamma, tau and
minimum budget drawn at collection from a fixed seed.  Every head is
compared with the oracle as in the ragged-layer tests: intermediates and
lists bit-exact, sparse and dense outputs within tolerance."""
import numpy as np
import pytest

from synth import BY_NAME
from tests.test_gpu_ragged import check_layer, check_packed

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TYPES = ("V", "S", "QA", "N")


def _cases(n=32, seed=2026):
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(n):
        block = int(rng.choice([64, 128]))
        dtype = "fp32" if rng.random() < 0.25 else "bf16"
        Hkv = int(rng.choice([1, 2, 3]))
        group = int(rng.choice([1, 2, 3, 4, 6]))
        Hq = Hkv * group
        B = int(rng.choice([1, 1, 2]))
        N = int(rng.choice([int(rng.integers(1, block)), int(rng.integers(block, 1700))]))
        base = BY_NAME["tiny_fp32_4k"] if dtype == "fp32" else BY_NAME["llama8b_32k"]
        cfg = base.with_(B=B, Hq=Hq, Hkv=Hkv, d=int(rng.choice([64, 128])), block=block,
                         gamma=float(rng.choice([0.8, 0.9, 0.95, 1.0, round(float(rng.uniform(0.3, 1.0)), 3)])),
                         tau=float(rng.choice([0.0, 0.1, 0.3, 0.84])),
                         min_budget=int(rng.choice([0, block, 3 * block, 1024])),
                         explicit_types=tuple(TYPES[int(x)] for x in rng.integers(0, 4, Hq)),
                         seed=int(rng.integers(1, 1 << 30)))
        out[f"shape{i}_B{B}_H{Hq}x{Hkv}_d{cfg.d}_bs{block}_{dtype}_N{N}"] = (cfg, N)
    return out


CASES = _cases()


@pytest.fixture(scope="module")
def F():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_long_context_last_amd as F
    return F


@pytest.mark.parametrize("name", list(CASES))
def test_random_shape_parity(F, name):
    cfg, N = CASES[name]
    check_layer(F, cfg, N, name)


def _packed_cases(n=12, seed=2027):
    rng = np.random.default_rng(seed)
    out = {}
    for i, (cfg, _) in enumerate(_cases(n, seed).values()):
        nseq = int(rng.integers(1, 6))
        lens = [int(rng.choice([0, int(rng.integers(1, cfg.block)), int(rng.integers(cfg.block, 1500))]))
                for _ in range(nseq)]
        if not any(lens):
            lens[0] = int(rng.integers(1, 700))
        out[f"packed{i}_H{cfg.Hq}x{cfg.Hkv}_d{cfg.d}_bs{cfg.block}_{cfg.dtype}_" + "-".join(map(str, lens))] = \
            (cfg.with_(B=1), lens)
    return out


PACKED_CASES = _packed_cases()


@pytest.mark.parametrize("name", list(PACKED_CASES))
def test_random_packed_parity(F, name):
    cfg, lens = PACKED_CASES[name]
    check_packed(F, cfg, lens, name)
