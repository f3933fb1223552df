"""The full-size GPU parity tests compute the oracle's attention with every
(sequence, head) pair handed over as a sequence of its own and the pairs split
over host threads (gpu_common.oracle_attend_batch).  On the CPU: that output is
bit-identical to one plain oracle call on the original layout, for dense rows
and block-aligned words, several sequences and heads, and a ragged block."""
import numpy as np
import pytest

import varq_inputs as vi
from gpu_common import oracle_attend_batch


@pytest.mark.parametrize("pack_mode", [0, 2])
def test_threaded_pairs_equal_one_call(oracle, pack_mode):
    wl = vi.Workload("threads", 1, 3, 5, 64, 3, (1, 7, 40, 97), "bf16", rope=True, seed=31)
    Lo = oracle.layout_of(wl)
    Lo.pack_mode = pack_mode
    kc, vc = oracle.alloc_cache(Lo), oracle.alloc_cache(Lo)
    for j in range(len(wl.blocks)):
        assert oracle.quantize_block(Lo, j, vi.kv_block(wl, 0, "k", j), vi.kv_block(wl, 0, "v", j),
                                     kc, vc) == 0
        q = vi.q_block(wl, 0, j)
        one = oracle.attend(Lo, j, q, kc, vc).astype(np.float64)
        threaded = oracle_attend_batch(oracle, Lo, j, q, kc, vc)
        assert threaded.shape == one.shape
        assert np.array_equal(threaded, one), j
