"""The oracle against hand-worked examples stored under tests/golden/ (no GPU).

Each fixture states its source (the FlexPrefill section it follows) and, per
case, how the expected value was worked out from the definition; none of
them is produced by the oracle or the GPU path.
"""
import json
import math
from pathlib import Path

import numpy as np
import pytest

import oracle as O

GOLDEN = Path(__file__).parent / "golden"


def _cases(name):
    return json.loads((GOLDEN / name).read_text())["cases"]


@pytest.mark.parametrize("case", _cases("selection_worked.json"), ids=lambda c: c["why"][:40])
def test_selection_worked_examples(case):
    sel = O.select_cumulative(np.asarray(case["values"], np.float32), case["gamma"])
    assert set(np.nonzero(sel)[0].tolist()) == set(case["selected"])


@pytest.mark.parametrize("case", _cases("vs_blocks_worked.json"), ids=lambda c: c["why"][:40])
def test_vs_block_conversion_worked_examples(case):
    N, bs = case["N"], case["bs"]
    cols = np.zeros(N, bool)
    cols[case["cols"]] = True
    offs = np.zeros(N, bool)
    offs[case["offsets"]] = True
    mask = O.vs_block_mask(cols, offs, bs)
    got = {(int(a), int(b)) for a, b in zip(*np.nonzero(mask))}
    assert got == {tuple(x) for x in case["blocks"]}


@pytest.mark.parametrize("case", _cases("jsd_worked.json"), ids=lambda c: c["why"][:40])
def test_jsd_worked_examples(case):
    jsd, D = O.jsd_canonical(np.asarray(case["P"], np.float32), np.asarray(case["Q"], np.float32))
    want = sum(c * (math.log(num) - math.log(den)) for c, num, den in case["jsd"])
    assert jsd == pytest.approx(want, rel=1e-12, abs=1e-15)
    assert D == pytest.approx(math.sqrt(want), rel=1e-12, abs=1e-15)
