"""The seeded input generators and block-mask patterns (CPU; no attention arithmetic)."""

import torch

from exact_tiled_attention_forward_amd.workloads import (WORKLOADS, butterfly_block_mask, local_global_block_mask,
                                                         make_inputs, workload_block_mask)


def test_inputs_are_seeded_and_rounded():
    a = make_inputs(1, 2, 33, 64, "bf16", seed_base=5)
    b = make_inputs(1, 2, 33, 64, "bf16", seed_base=5)
    assert all(torch.equal(a[x], b[x]) for x in ("q", "k", "v"))
    assert a["q"].dtype == torch.bfloat16 and a["q"].shape == (1, 2, 33, 64)


def test_butterfly_mask_pattern():
    for n, nb in ((16384, 128), (1024, 8), (1000, 8)):
        m = butterfly_block_mask(n)[0].bool()
        assert m.shape == (nb, nb)
        assert torch.equal(m, m.T) and m.diagonal().all()
        logn = nb.bit_length() - 1
        assert (m.sum(1) == 1 + logn).all()
        for i in range(nb):
            for j in range(nb):
                x = i ^ j
                assert bool(m[i, j]) == (x & (x - 1) == 0)
    assert float(butterfly_block_mask(16384).float().mean()) == 8 / 128


def test_named_masks():
    assert workload_block_mask(WORKLOADS["large_head_causal"]) is None
    assert torch.equal(workload_block_mask(WORKLOADS["block_sparse_local"]), local_global_block_mask(16384))
    assert torch.equal(workload_block_mask(WORKLOADS["block_sparse_butterfly"]), butterfly_block_mask(16384))
