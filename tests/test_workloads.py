"""The synthetic inputs' recipes (host only): the sparse workload's block
mask keeps a fixed share of every query tile's key blocks."""

import numpy as np

import workloads


def test_sparse_mask_keeps_a_fixed_share_of_each_query_tile():
    w = workloads.get("sparse", H=3, Nq=300, Nkv=1000, seed=11)
    m = workloads.block_mask(w)
    nkc = -(-1000 // 64)
    assert m.shape == (1, 3, 3, nkc) and m.dtype == np.uint8
    assert set(np.unique(m)) <= {0, 1}
    assert (m.sum(-1) == round(0.25 * nkc)).all()
    # tiles draw independently: not all tiles keep the same blocks
    rows = m.reshape(-1, nkc)
    assert len({r.tobytes() for r in rows}) > 1
    # seeded: the same workload gives the same mask, another seed another
    assert np.array_equal(m, workloads.block_mask(workloads.get("sparse", H=3, Nq=300, Nkv=1000, seed=11)))
    assert not np.array_equal(m, workloads.block_mask(workloads.get("sparse", H=3, Nq=300, Nkv=1000, seed=12)))


def test_sparse_workload_mask_at_full_size():
    w = workloads.get("sparse")
    m = workloads.block_mask(w)
    assert m.shape == (1, 40, 591, 1182)
    assert (m.sum(-1) == 296).all()
