"""Host logic of the whole-population parity tests: the worker-process oracle gives the same results, in row
order, as the oracle called on all rows at once (blocks of uneven size, T = 0 and T > 0)."""

import numpy as np

import workloads as W
from parity_util import CORE_KEYS, OraclePool, oracle_block


def test_pool_matches_direct_oracle():
    w = W.workload(1)
    a, b = W.make_logits_numpy(w)
    a, b = a[:50], b[:50]
    pos = W.positions(w)[:50]
    with OraclePool(workers=2, block=16) as pool:
        for T in (0.0, 1.0):
            got = pool.rows(a, b, "fp32", T, 3, pos)
            ref = oracle_block((a, b, "fp32", T, 3, pos))
            for k in CORE_KEYS:
                np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
        empty = pool.rows(a[:0], b[:0], "fp32", 1.0, 3, pos[:0])
        assert all(len(v) == 0 for v in empty.values())
