"""Pins of the oracle's expert indexing, gather, combine and unpermute-sum.

* counts and offsets: numpy's bincount (the counting the unsloth PR #3812
  review suggests) and a cumulative sum; counts have shape [E], not [E, T]
  (the bug that review found) and sum to T*k;
* the permutation: numpy's stable argsort of the flattened expert ids (again
  the review's suggested definition), a brute-force O((Tk)^2) rank formula,
  and the invariants (both arrays are permutations, mutual inverses, expert
  ids non-decreasing along the sorted order, token order kept inside each
  expert);
* gather then combine is the identity when no experts sit between them
  (weights sum to 1), and gather then unpermute-sum is exactly k times X.
"""
import numpy as np
import pytest

from mixture_experts_expert_amd import synth


def _random_idx(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 3, 3), (64, 8, 2), (200, 16, 4), (0, 4, 2), (33, 128, 8)])
def test_counts_offsets_and_stable_argsort(oracle, T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    idx = _random_idx(rng, T, E, k) if T > 0 else np.zeros((0, k), np.int32)
    counts, offsets, s2f, f2s = oracle.permute_index(idx, E)
    flat = idx.reshape(-1)
    assert counts.shape == (E,)
    assert (counts == np.bincount(flat, minlength=E)).all()
    assert counts.sum() == T * k and offsets[-1] == T * k and offsets[0] == 0
    assert (offsets[1:] == np.cumsum(counts)).all()
    assert (s2f == np.argsort(flat, kind="stable")).all()
    assert (f2s[s2f] == np.arange(T * k)).all()


def test_permutation_brute_force_rank(oracle):
    rng = np.random.default_rng(5)
    T, E, k = 23, 6, 3
    idx = _random_idx(rng, T, E, k)
    counts, offsets, s2f, f2s = oracle.permute_index(idx, E)
    flat = idx.reshape(-1)
    for f in range(T * k):
        e = flat[f]
        pos = offsets[e] + sum(1 for g in range(f) if flat[g] == e)
        assert f2s[f] == pos and s2f[pos] == f


def test_permutation_invariants(oracle):
    rng = np.random.default_rng(6)
    T, E, k = 300, 11, 4
    idx = _random_idx(rng, T, E, k)
    counts, offsets, s2f, f2s = oracle.permute_index(idx, E)
    flat = idx.reshape(-1)
    assert sorted(s2f) == list(range(T * k)) and sorted(f2s) == list(range(T * k))
    assert (np.diff(flat[s2f]) >= 0).all()
    tok = s2f // k
    for e in range(E):
        seg = tok[offsets[e]:offsets[e + 1]]
        assert (np.diff(seg) > 0).all()  # tokens ascend inside each expert
    # The gather index is a permutation of (token, slot) pairs, not a token
    # index (the second bug the unsloth review found): s2f // k repeats each
    # token exactly k times.
    assert (np.bincount(tok, minlength=T) == k).all()


def test_out_of_range_expert_is_rejected(oracle):
    with pytest.raises(ValueError):
        oracle.permute_index(np.array([[0, 5]], np.int32), 4)


@pytest.mark.parametrize("k", [1, 2, 8])
def test_gather_then_combine_is_identity(oracle, k):
    cfg = synth.MoEConfig("t", T=40, H=96, E=16, k=k, I=8, dtype="bf16", backward=False)
    inp = synth.make_inputs(cfg, 11, router_only=True)
    x = inp.f32("x")
    _, idx, w = oracle.route(x, inp.f32("w_router"), k)
    counts, offsets, s2f, f2s = oracle.permute_index(idx, cfg.E)
    x_perm = oracle.gather(x, s2f, k)
    y = oracle.combine(x_perm, w, f2s, cfg.T, k)
    np.testing.assert_allclose(y, x, rtol=4 * k * 2.0 ** -24, atol=0)
    assert (x_perm == x[s2f // k]).all()


def test_gather_then_unpermute_sum_is_k_times_x(oracle):
    k = 8
    cfg = synth.MoEConfig("t", T=37, H=64, E=12, k=k, I=8, dtype="bf16", backward=False)
    inp = synth.make_inputs(cfg, 12, router_only=True)
    x = inp.f32("x")
    _, idx, _ = oracle.route(x, inp.f32("w_router"), k)
    _, _, s2f, f2s = oracle.permute_index(idx, cfg.E)
    dx = oracle.unpermute_sum(oracle.gather(x, s2f, k), f2s, cfg.T, k)
    assert (dx == np.float32(k) * x).all()  # j*x needs <= 12 significant bits: exact
