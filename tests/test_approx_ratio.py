"""The approximation-ratio diagnostic of the DropKV selection (CPU).

Pins: the joint objective of a single token equals that token's DropKV score
(the closed form, itself pinned to delete-and-recompute elsewhere), the empty
set costs nothing, with k = 1 and no pooling the DropKV choice is the exact
optimum, and the brute-force minimum is never above the DropKV set's cost.
The ratio distribution over seeds is printed (a diagnostic, not a target:
the pages' median 1.16 comes from trained models).
"""

import numpy as np
import pytest

import oracle
from brute_force import brute_force_joint
from oracle.joint import approx_ratio, joint_objective


def _case(seed, Hq=4, Hkv=2, d=8, n=14, w=3):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, w, d))
    k = rng.standard_normal((Hkv, n, d)) * 1.5
    v = rng.standard_normal((Hkv, n, d))
    return q, k, v, dict(n=n, window=w, Hq=Hq, Hkv=Hkv, d=d)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_single_token_joint_objective_is_the_score(seed):
    q, k, v, s = _case(seed)
    G = s["Hq"] // s["Hkv"]
    for g in range(s["Hkv"]):
        S = oracle.head_scores(q, k, v, g, G, s["n"], s["window"])["S"]
        for j in range(s["n"] - s["window"]):
            J = joint_objective(q, k, v, g, G, s["n"], s["window"], [j])
            assert abs(J - S[j]) <= 1e-12 * max(S[j], 1e-300)
        assert joint_objective(q, k, v, g, G, s["n"], s["window"], []) == 0.0


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_joint_objective_of_sets_equals_literal_deletion(seed):
    """|E| >= 2: the joint objective against removing the whole set literally
    (brute force: re-softmax over the visible keys outside E), including sets
    that hold every evictable token of a row's view but one."""
    q, k, v, s = _case(seed)
    G = s["Hq"] // s["Hkv"]
    n, w = s["n"], s["window"]
    rng = np.random.default_rng(1000 + seed)
    sets = [sorted(rng.choice(n - w, size=size, replace=False).tolist()) for size in (2, 3, 5, 8)]
    sets.append(list(range(n - w)))          # every evictable token
    sets.append(list(range(1, n - w)))       # all but the first
    sets.append([0, n - w - 1])              # both ends of the evictable range
    for g in range(s["Hkv"]):
        for E in sets:
            J = joint_objective(q, k, v, g, G, n, w, E)
            B = brute_force_joint(q, k, v, g, G, n, w, E)
            assert abs(J - B) <= 1e-12 * max(B, 1e-300), (g, E, J, B)


def test_joint_objective_is_not_additive():
    """Removing two tokens together differs from the sum of removing each:
    a check that the set objective really renormalises once over the rest."""
    q, k, v, s = _case(7)
    G = s["Hq"] // s["Hkv"]
    n, w = s["n"], s["window"]
    J12 = joint_objective(q, k, v, 0, G, n, w, [1, 2])
    J1 = joint_objective(q, k, v, 0, G, n, w, [1])
    J2 = joint_objective(q, k, v, 0, G, n, w, [2])
    assert abs(J12 - (J1 + J2)) > 1e-6 * J12
    assert abs(J12 - brute_force_joint(q, k, v, 0, G, n, w, [1, 2])) <= 1e-12 * J12


@pytest.mark.parametrize("seed", range(4))
def test_k1_unpooled_choice_is_optimal(seed):
    q, k, v, s = _case(seed)
    r = approx_ratio(q, k, v, n_evict=1, pool_kernel=1, **s)
    assert np.allclose(r["ratio"], 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("ne,pool", [(3, 3), (3, 1), (5, 1)])
def test_ratio_distribution(ne, pool):
    ratios = []
    for seed in range(12):
        q, k, v, s = _case(100 + seed)
        r = approx_ratio(q, k, v, n_evict=ne, pool_kernel=pool, **s)
        assert np.all(r["J_opt"] > 0)
        assert np.all(r["ratio"] >= 1.0 - 1e-12) and np.all(r["ratio_unpooled"] >= 1.0 - 1e-12)
        for g in range(s["Hkv"]):  # the brute-force minimiser is a valid set outside the window
            E = r["E_opt"][g]
            assert E.size == ne and np.all(np.diff(E) > 0) and E.max() < s["n"] - s["window"]
        ratios += list(r["ratio"])
    print(f"\napprox ratio, n=14 w=3 evict {ne} of 11, pool {pool}, {len(ratios)} head cases: "
          f"median {np.median(ratios):.4f}, max {np.max(ratios):.4f}")
