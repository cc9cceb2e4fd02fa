"""CPU checks of the BigBird BlockMask builder against the seeded workload
generator ("4.3 Block-Sparse Attention"; BigBird reference [9]).  The two are
written separately; they must agree block for block for the same seed."""
import numpy as np
import pytest
import torch

import attention_attnfuse_fwd_amd as af
import workloads


@pytest.mark.parametrize("N,block,seed,kw", [
    (4096, 64, 4, {}),
    (1000, 64, 7, {}),
    (512, 32, 1, dict(n_window=2, n_global=1, n_random=5)),
    (256, 64, 3, dict(n_random=10)),
])
def test_matches_generator(N, block, seed, kw):
    bm = af.bigbird_block_mask(N, block, seed=seed, **kw)
    nb = -(-N // block)
    rp, ci = workloads.bigbird_csr(nb, nb, seed, **kw)
    assert bm.block_m == bm.block_n == block and not bm.per_head
    assert bm.row_ptr.dtype == bm.col_idx.dtype == torch.int32
    np.testing.assert_array_equal(bm.row_ptr.numpy(), rp)
    np.testing.assert_array_equal(bm.col_idx.numpy(), ci)


def test_headline_mask_shape():
    # 64 x 64 blocks of 64 rows: 505 active blocks; rows 0, 1, 2 and 63 hold 5, 6, 7, 7.
    bm = af.bigbird_block_mask(4096, 64, seed=4)
    counts = np.diff(bm.row_ptr.numpy())
    assert bm.nnz == 505
    assert list(counts[[0, 1, 2, 63]]) == [5, 6, 7, 7] and np.all(counts[3:63] == 8)


def test_degenerate_cases():
    empty = af.bigbird_block_mask(0, 64)
    assert empty.row_ptr.tolist() == [0] and empty.nnz == 0
    diag = af.bigbird_block_mask(300, 64, n_window=0, n_global=0, n_random=0)
    assert diag.row_ptr.tolist() == [0, 1, 2, 3, 4, 5] and diag.col_idx.tolist() == [0, 1, 2, 3, 4]
    full = af.bigbird_block_mask(128, 64, n_random=3)
    assert full.row_ptr.tolist() == [0, 2, 4] and full.col_idx.tolist() == [0, 1, 0, 1]
    rect = af.bigbird_block_mask(128, 64, n_window=0, n_global=0, n_random=0, N_k=640)
    assert rect.row_ptr.tolist() == [0, 1, 2] and rect.col_idx.tolist() == [0, 1]
    with pytest.raises(ValueError):
        af.bigbird_block_mask(64, 0)
    with pytest.raises(ValueError):
        af.bigbird_block_mask(64, 64, n_random=-1)
