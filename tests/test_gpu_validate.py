"""The opt-in offsets check (pqm_validate_offsets) on hand-made arrays with
one known defect each, on several defects at once (the smallest index wins),
on a long array (a defect past the first thread's stride), and on the
offsets the routing and padding kernels produce (valid)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import precision_quantization_moe_amd as pqm
from precision_quantization_moe_amd import workloads as wl
from gpu_util import dev, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _check(off, M, align=1):
    r = pqm.validate_offsets(dev(np.asarray(off, np.int64)), M, align)
    torch.cuda.synchronize()
    return tuple(int(v) for v in r.cpu())


@pytest.mark.parametrize("off,M,align,want", [
    ([0, 5, 5, 37, 100], 100, 1, (0, -1)),
    ([0, 5, 5, 37, 90], 100, 1, (0, -1)),                      # offsets[G] < M_total is legal
    ([3, 5, 10], 10, 1, (pqm.OFFSETS_FIRST_NOT_ZERO, 0)),
    ([0, 10, 20, 15, 30], 30, 1, (pqm.OFFSETS_DECREASING, 2)),
    ([0, 32, 64, 70, 96], 96, 32, (pqm.OFFSETS_MISALIGNED, 3)),
    ([0, 10, 200], 100, 1, (pqm.OFFSETS_PAST_END, 2)),
    ([0], 0, 1, (0, -1)),                                       # no groups
    ([7], 10, 1, (pqm.OFFSETS_FIRST_NOT_ZERO, 0)),
    ([0, 32, 40, 30, 64], 64, 32, (pqm.OFFSETS_DECREASING, 2)),  # two defects at index 2: the first check
    ([0, 31, 64, 30, 96], 96, 32, (pqm.OFFSETS_MISALIGNED, 1)),  # defects at 1 and 2: the first index
])
def test_validate_offsets_cases(off, M, align, want):
    assert _check(off, M, align) == want


def test_validate_offsets_long_array():
    G = 3000
    off = np.arange(G + 1, dtype=np.int64) * 4
    assert _check(off, 4 * G) == (0, -1)
    bad = off.copy()
    bad[2501] = bad[2500] - 1                     # decreasing at index 2500
    bad[2900] = 1                                 # and again later
    assert _check(bad, 4 * G) == (pqm.OFFSETS_DECREASING, 2500)
    assert _check(off, 4 * G - 1) == (pqm.OFFSETS_PAST_END, G)


def test_validate_offsets_of_routing_and_padding():
    T, E, k = 1000, 64, 4
    ids = torch.from_numpy(wl.zipf_routing(T, E, k)).cuda()
    off, _, _, _ = pqm.moe_route(ids, E)
    assert _check(off.cpu().numpy(), T * k) == (0, -1)
    x = torch.zeros((T * k, 64), dtype=torch.bfloat16, device="cuda")
    _, poff = pqm.moe_pad_rows(x, off)
    Mp = int(poff[-1].item())
    assert _check(poff.cpu().numpy(), Mp, 32) == (0, -1)
    assert _check(off.cpu().numpy(), T * k, 32)[0] in (0, pqm.OFFSETS_MISALIGNED)
