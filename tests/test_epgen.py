"""The seeded workload generator: determinism, shapes, routing structure."""

import numpy as np
import pytest

from epgen import CONFIGS, make_hidden, make_routing, spec


@pytest.mark.parametrize("name", list(CONFIGS))
def test_routing_deterministic_and_valid(name):
    s = spec(name, T=min(CONFIGS[name].T, 1024))
    a_idx, a_w = make_routing(s)
    b_idx, b_w = make_routing(s)
    assert np.array_equal(a_idx, b_idx) and np.array_equal(a_w, b_w)
    assert a_idx.dtype == np.int64 and a_w.dtype == np.float32
    assert a_idx.shape == (s.T, s.K) and a_w.shape == (s.T, s.K)
    assert a_idx.min() >= -1 and a_idx.max() < s.E
    for t in range(s.T):
        r = a_idx[t][a_idx[t] >= 0]
        assert len(np.unique(r)) == len(r)
    assert np.all(a_w[a_idx < 0] == 0)
    routed = (a_idx >= 0).any(axis=1)
    np.testing.assert_allclose(a_w[routed].sum(axis=1), 1.0, rtol=1e-6)


def test_prefix_property():
    s = spec("skewed_t16384", T=512, H=64)
    idx_full, w_full = make_routing(s)
    idx_pre, w_pre = make_routing(s.replace(T=100))
    assert np.array_equal(idx_full[:100], idx_pre)
    assert np.array_equal(w_full[:100], w_pre)
    x_full = make_hidden(s)
    assert np.array_equal(x_full[:100], make_hidden(s, rows=100))


def test_seed_changes_inputs():
    a, _ = make_routing(spec("tiny"))
    b, _ = make_routing(spec("tiny", seed=1))
    assert not np.array_equal(a, b)


def test_skewed_routing_is_skewed():
    s = spec("skewed_t16384", T=4096)
    idx, _ = make_routing(s)
    frac_unrouted = (idx < 0).mean()
    assert 0.04 < frac_unrouted < 0.06
    counts = np.bincount(idx[idx >= 0], minlength=s.E)
    # Zipf(1.2) over 256 experts: the hottest expert takes far more than 1/E
    assert counts.max() > 20 * counts.mean()
