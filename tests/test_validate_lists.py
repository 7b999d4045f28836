"""The host-side list validator (block_sparse_attention_major_amd.validate)
on index lists built by the oracle: valid lists pass, and each planted
corruption (an unsorted row, a key tile out of range, a wrong row offset, a
wrong work order) is reported."""

import numpy as np
import pytest

import oracle
from block_sparse_attention_major_amd import validate


def _lists(seed=3, heads=2, nT=12, p=0.4):
    M = (np.random.default_rng(seed).random((heads, nT, nT)) < p).astype(np.uint8)
    rp, cl, od = oracle.csr(M)
    return M, rp.copy(), cl.copy(), od.copy(), nT


def test_valid_lists_pass():
    M, rp, cl, od, nT = _lists()
    rows = validate.check_row_lists(rp, cl, od, nT, int(M.sum()))
    assert sum(r.size for r in rows) == int(M.sum())
    for h in range(M.shape[0]):
        for i in range(nT):
            assert np.array_equal(rows[h * nT + i], np.nonzero(M[h, i])[0])


def test_empty_mask_passes():
    M, rp, cl, od, nT = _lists(p=0.0)
    validate.check_row_lists(rp, cl, od, nT, 0)


@pytest.mark.parametrize("corrupt", ["unsorted", "range", "offset", "order", "count"])
def test_corruptions_are_reported(corrupt):
    M, rp, cl, od, nT = _lists()
    nnz = int(M.sum())
    r = int(np.argmax(np.diff(rp)))  # a row with at least two entries
    if corrupt == "unsorted":
        cl[rp[r]], cl[rp[r] + 1] = cl[rp[r] + 1], cl[rp[r]]
    elif corrupt == "range":
        cl[rp[r]] = nT
    elif corrupt == "offset":
        rp[r + 1] -= 1
    elif corrupt == "order":
        od[[0, -1]] = od[[-1, 0]]
    else:
        nnz += 1
    with pytest.raises(ValueError):
        validate.check_row_lists(rp, cl, od, nT, nnz)
