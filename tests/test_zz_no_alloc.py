"""The standalone row for callers that cannot allocate
(fpi8_matrix_rows_packed_noalloc), through the C ABI: its output equals
fpi8_matrix_rows_packed's, bit for bit, on calls in a row that reuse the
library's per-GPU workspace array, each later one smaller; sizes beyond its
limits are rejected."""
import numpy as np
import pytest

import workloads as W
from fixed_point_int8_amd import binding as B
from gpu_helpers import require_gpu, say

pytestmark = pytest.mark.gpu


def packed_operands(torch, rows, cols, batch, seed, adversarial=False):
    Wm, s, x = W.row_operands(rows, cols, batch, seed)
    if adversarial:
        x = W.adversarial_row_inputs(batch, cols, seed)
    dW = torch.from_numpy(np.ascontiguousarray(Wm)).cuda()
    n_p = B.fpi8_matrix_packed_size(rows, cols)
    dP = torch.empty(n_p, dtype=torch.uint8, device="cuda")
    assert B.fpi8_matrix_pack(dW, rows, cols, dP, n_p) == 0
    dS = torch.from_numpy(np.ascontiguousarray(s).view(np.int32)).cuda()
    dX = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return dP, dS, dX


def with_workspace(torch, dP, dS, dX, rows, cols, batch):
    dY = torch.zeros((batch, rows), dtype=torch.int64, device="cuda")
    n = B.fpi8_matrix_rows_workspace_size(rows, cols, batch)
    work = torch.zeros(n, dtype=torch.uint8, device="cuda")
    assert B.fpi8_matrix_rows_packed(dP, dS, rows, cols, dX, batch, dY, work, n) == 0
    torch.cuda.synchronize()
    return dY.cpu().numpy()


def without_allocation(torch, dP, dS, dX, rows, cols, batch):
    dY = torch.full((batch, rows), -1, dtype=torch.int64, device="cuda")
    assert B.fpi8_matrix_rows_packed_noalloc(dP, dS, rows, cols, dX, batch, dY) == 0
    torch.cuda.synchronize()
    return dY.cpu().numpy()


@pytest.mark.parametrize("calls", [
    # a call with digit planes over the whole array, then smaller ones
    [(4096, 16384, 128, False), (300, 1000, 5, False), (37, 64, 1, False)],
    # the persistent streaming kernel, then a call on the exact path
    [(65536, 4096, 8, False), (100, 200, 40, True)],
    # the exact path first, then a smaller call whose inputs fit three digits
    [(512, 2048, 64, True), (64, 128, 17, False)],
])
def test_noalloc_matches_workspace_call(calls):
    torch = require_gpu()
    for i, (rows, cols, batch, adv) in enumerate(calls):
        say(f"noalloc call {i}: {rows}x{cols} batch {batch}{' adversarial' if adv else ''}")
        dP, dS, dX = packed_operands(torch, rows, cols, batch, 100 + i + rows, adv)
        want = with_workspace(torch, dP, dS, dX, rows, cols, batch)
        got = without_allocation(torch, dP, dS, dX, rows, cols, batch)
        assert np.array_equal(got, want), (rows, cols, batch)


def test_noalloc_limits():
    torch = require_gpu()
    dP, dS, dX = packed_operands(torch, 16, 64, 1, 5)
    dY = torch.zeros((B.NOALLOC_MAX_BATCH + 1, 16), dtype=torch.int64, device="cuda")
    assert B.fpi8_matrix_rows_packed_noalloc(dP, dS, 16, 64, dX, B.NOALLOC_MAX_BATCH + 1, dY) == 102
    assert B.fpi8_matrix_rows_packed_noalloc(dP, dS, 16, B.NOALLOC_MAX_COLS + 1, dX, 1, dY) == 102
    assert B.fpi8_matrix_rows_packed_noalloc(0, dS, 16, 64, dX, 1, dY) == 102
