"""Property tests of the oracle over random small shapes (CPU only):
invariants that hold for any input -- counts sum to M*k, offsets are the
exclusive prefix sum, the permutation is a stable bijection into the right
segments, routing equals a stable argsort, the weights sum to one."""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle


@st.composite
def routing_case(draw):
    E = draw(st.integers(1, 40))
    k = draw(st.integers(1, min(E, 16)))
    M = draw(st.integers(0, 120))
    S = draw(st.integers(1, 6))
    seed = draw(st.integers(0, 2**31 - 1))
    ties = draw(st.booleans())
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((M, E)).astype(np.float32)
    if ties:  # coarse values make many exact ties
        logits = np.round(logits * 2).astype(np.float32) / 2
    src = rng.integers(0, S, size=M).astype(np.int32)
    return M, E, k, S, logits, src


@settings(max_examples=60, deadline=None)
@given(routing_case())
def test_routing_and_permutation_invariants(case):
    M, E, k, S, logits, src = case
    idx, w = oracle.route(logits, k)
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, order)
    if M:
        assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= 4 * k * 2.0 ** -24)
    counts, offsets = oracle.counts_offsets(idx, E, S, src if S > 1 else None)
    s2f, f2s = oracle.permutation(idx, E, S, src if S > 1 else None)
    R = M * k
    assert counts.sum() == R and offsets[0] == 0 and offsets[-1] == R
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(s2f), np.arange(R))
    assert np.array_equal(f2s[s2f], np.arange(R))
    seg = ((src[:, None] if S > 1 else 0) * E + idx).reshape(-1) if R else np.zeros(0, np.int64)
    for g in range(S * E):
        part = s2f[offsets[g]:offsets[g + 1]]
        assert np.all(np.diff(part) > 0)
        assert np.all(seg[part] == g)
