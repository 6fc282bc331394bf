"""Pins of the oracle's load-balance loss and statistics (no GPU).

The pages name the balancing loss and its failure mode but print no formula;
the oracle uses the Switch Transformer loss. These tests fix it by closed
forms (uniform and one-expert routing, where every statistic is known), by
finite differences of the loss (the gradient, with the counts held fixed),
by invariants of the softmax (probabilities sum to one, each token's
gradient sums to zero), and by the failure mode itself: a router whose
probabilities are perfectly even (the loss at its uniform value) while the
hard load sits on one expert."""
import numpy as np
import pytest

import oracle


def test_uniform_closed_form():
    T, E, k, alpha = 64, 8, 2, 0.01
    logits = np.full((T, E), 0.3)
    counts = np.full(E, T * k // E)
    st, g = oracle.load_balance(logits, counts, k, alpha)
    np.testing.assert_allclose(st, [alpha, 1, 1, 1, 1, 1, 0, 0], atol=1e-12)
    assert np.abs(g).max() < 1e-15


def test_one_expert_closed_form():
    T, E, k = 32, 16, 1
    counts = np.zeros(E); counts[3] = T
    logits = np.zeros((T, E)); logits[:, 3] = 60.0        # p -> one-hot on expert 3
    st, _ = oracle.load_balance(logits, counts, k, 1.0)
    assert st[0] == pytest.approx(E, rel=1e-12)           # loss at its maximum alpha*E
    assert st[2] == pytest.approx(E)                       # E sum f^2
    assert st[4] == pytest.approx(E) and st[5] == 0.0
    assert st[6] == pytest.approx(np.sqrt(E - 1))          # population CV of [N, 0, ..., 0]
    assert st[7] == E - 1


def test_gradient_finite_differences():
    rng = np.random.default_rng(3)
    T, E, k, alpha = 12, 6, 2, 0.3
    logits = rng.standard_normal((T, E))
    counts = rng.integers(0, 9, E)
    counts[0] += T * k - counts.sum() if counts.sum() < T * k else 0
    _, g = oracle.load_balance(logits, counts, k, alpha)
    h = 1e-6
    for t, e in [(0, 0), (3, 2), (7, 5), (11, 1)]:
        lp = logits.copy(); lp[t, e] += h
        lm = logits.copy(); lm[t, e] -= h
        fd = (oracle.load_balance(lp, counts, k, alpha)[0][0] -
              oracle.load_balance(lm, counts, k, alpha)[0][0]) / (2 * h)
        assert g[t, e] == pytest.approx(fd, rel=1e-6, abs=1e-10)


def test_invariants():
    rng = np.random.default_rng(4)
    T, E, k = 50, 10, 3
    logits = rng.standard_normal((T, E)) * 2
    counts = rng.multinomial(T * k, np.ones(E) / E)
    st, g = oracle.load_balance(logits, counts, k, 1.0)
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-15)
    # with even counts the loss no longer depends on the router: f = 1/E gives E sum P/E = 1
    st_even, g_even = oracle.load_balance(logits, np.full(E, T * k / E), k, 1.0)
    assert st_even[1] == pytest.approx(1.0, rel=1e-12)
    assert np.abs(g_even).max() < 1e-15
    assert 1.0 <= st[2] <= E and st[5] <= 1.0 <= st[4]


def test_gerrymandering_is_visible():
    """Even router probabilities with all rows on one expert: the balance
    term the loss measures reads 1 (perfectly balanced), the hard-load
    statistics read the worst case -- the divergence the monitor exists for."""
    T, E, k = 40, 8, 1
    logits = np.zeros((T, E))
    counts = np.zeros(E); counts[0] = T
    st, _ = oracle.load_balance(logits, counts, k, 1.0)
    assert st[1] == pytest.approx(1.0)
    assert st[2] == pytest.approx(E) and st[4] == pytest.approx(E) and st[7] == E - 1


def test_zero_tokens():
    st, g = oracle.load_balance(np.zeros((0, 4)), np.zeros(4), 2, 1.0)
    assert np.all(st == 0) and g.shape == (0, 4)


# ---------------------------------------------------------------------------
# planted mistakes in a private copy of the function must fail the pins above


LB_MUTATIONS = {
    "balance_without_E": ("balance = E * np.dot(f, P)", "balance = np.dot(f, P)"),
    "fraction_without_k": ("f = counts / (T * k)", "f = counts / T"),
    "gradient_sign": ("(f[None, :] - (p @ f)[:, None])", "((p @ f)[:, None] - f[None, :])"),
    "probability_of_first_token": ("P = p.mean(axis=0)", "P = p[0]"),
    "sample_std": ("counts.std() / mean", "counts.std(ddof=1) / mean"),
    "gradient_without_alpha": ("grad = (alpha * E / T)", "grad = (E / T)"),
}


def _mutated(name):
    import inspect
    import textwrap
    old, new = LB_MUTATIONS[name]
    src = textwrap.dedent(inspect.getsource(oracle.load_balance))
    assert src.count(old) == 1, name
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    return ns["load_balance"]


def _pins_hold(lb) -> bool:
    saved = oracle.load_balance
    oracle.load_balance = lb
    try:
        for pin in (test_uniform_closed_form, test_one_expert_closed_form,
                    test_gradient_finite_differences, test_invariants,
                    test_gerrymandering_is_visible, test_zero_tokens):
            pin()
        return True
    except AssertionError:
        return False
    finally:
        oracle.load_balance = saved


def test_unmutated_load_balance_passes():
    assert _pins_hold(oracle.load_balance)


@pytest.mark.parametrize("name", sorted(LB_MUTATIONS))
def test_load_balance_mutation_is_caught(name):
    assert not _pins_hold(_mutated(name)), f"planted mistake '{name}' went unnoticed"
