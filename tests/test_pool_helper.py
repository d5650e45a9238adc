"""The head-by-head oracle pool used by the full-size GPU parity tests gives the oracle's own
results (mask groups of block-sparse plans, GQA sums of dK / dV)."""
import numpy as np

import _pool
from _cases import sparse_spec
from oracle import attention as A
from oracle import masks as M


def _rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_pool_matches_oracle():
    T, Hq, Hkv, d = 600, 4, 2, 6  # 600 rows: two row ranges per head
    q, k, v, do = _rnd(1, T, Hq, d), _rnd(2, T, Hkv, d), _rnd(3, T, Hkv, d), _rnd(4, T, Hq, d)
    for spec in (M.MaskSpec("SLIDING_WINDOW", T, T, window=37), sparse_spec(T, 40, 4, 50, seed=3)):
        O, L = A.attn_fwd(q, k, v, spec, 0.4)
        g = A.attn_bwd(q, k, v, do, spec, 0.4)
        r = _pool.oracle_heads(q, k, v, do, spec, 0.4, range(Hq))
        assert np.max(np.abs(r["o"] - O)) < 1e-13 and np.array_equal(np.isinf(r["lse"]), np.isinf(L))
        for n in ("dq", "dk", "dv"):
            assert np.max(np.abs(r[n] - g[n])) < 1e-12, n
        keys = [0, 15, 16, 99, 599]
        dk, dv = _pool.oracle_keys(q, k, v, do, spec, 0.4, keys, 1)
        assert np.max(np.abs(dk - g["dk"][keys, 1])) < 1e-12 and np.max(np.abs(dv - g["dv"][keys, 1])) < 1e-12
