"""The CPU oracle against its pins (hand fixtures, invariants, closed forms,
brute force).  CPU only."""
import numpy as np
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def test_mask_golden(o):
    pins.pin_mask_golden(o)


def test_mask_all(o):
    pins.all_mask_pins(o)


def test_rope(o):
    pins.all_rope_pins(o)


def test_attention_bruteforce(o):
    for seed, P in ((11, 32), (12, 0), (13, 7), (15, 1)):
        pins.pin_attn_bruteforce(o, pins.tiny_attn_inputs(seed, B=8, P=P), 1e4)
    # long positions, large theta, head_dim 64 as in the fp32 workload
    pins.pin_attn_bruteforce(o, pins.tiny_attn_inputs(16, B=4, P=40, Hq=4, Hkv=4, d=64), 1e6)


def test_attention_identity_order_bruteforce(o):
    inp = pins.tiny_attn_inputs(17, B=8, P=16)
    inp["tau"] = np.arange(1, 9, dtype=np.int32)
    pins.pin_attn_bruteforce(o, inp, 1e4)


def test_attention_special_cases(o):
    pins.pin_attn_single_key(o)
    pins.pin_attn_two_keys_scale(o)
    pins.pin_attn_gqa_mapping(o)
    pins.pin_attn_constant_values(o)
    pins.pin_attn_copy_alignment(o)
    for s in (21, 22, 23):
        pins.pin_attn_equivariance(o, s)


def test_attention_tau_sort_reduces_to_identity(o):
    """Sorting slots by tau turns any order into the identity order."""
    inp = pins.tiny_attn_inputs(24, B=7, P=4, Hq=2, Hkv=1, d=8)
    B = 7
    sigma = np.argsort(inp["tau"])
    rows = np.concatenate([sigma, B + sigma])
    out = o.attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                      inp["tau"], 0.0)
    out2 = o.attention(inp["q"][rows], inp["k_new"][rows], inp["v_new"][rows], inp["k_cache"],
                       inp["v_cache"], np.arange(1, B + 1, dtype=np.int32), 0.0)
    assert np.abs(out2 - out[rows]).max() < 1e-13


def test_accept(o):
    pins.all_accept_pins(o, exact=False)


def test_accept_exact_distribution(o):
    pins.pin_accept_exact_distribution(o, V=4, seed=31, N=4000)
    pins.pin_accept_exact_distribution(o, V=5, seed=36, N=2000)


def test_accept_monte_carlo(o):
    """1e6 trials on V = 8: the token emitted at the first step follows
    p_theta (the accept + resample rule preserves the target distribution),
    the acceptance rate is 1 - D_TV, and conditioned on step 1 accepted the
    token emitted for step 2 follows that slot's p_theta."""
    from scipy.stats import chisquare
    r = np.random.default_rng(77)
    V, B, n = 8, 2, 1_000_000
    lt = (r.standard_normal((B, V)) * 1.3).astype(np.float32)
    pd = r.dirichlet(np.ones(V), B)
    pd = (pd / pd.sum(axis=1, keepdims=True)).astype(np.float32)
    pt = np.stack([o.softmax(lt[k])[0] for k in range(B)])
    tau = np.array([[2, 1]] * n, np.int32)   # step 1 -> slot 1, step 2 -> slot 0
    cdfs = np.cumsum(pd.astype(np.float64), axis=1)
    toks = np.stack([np.minimum(np.searchsorted(cdfs[k], r.random(n) * cdfs[k, -1], side="right"), V - 1)
                     for k in range(B)], axis=1).astype(np.int32)
    u = r.random((n, B + 1)).astype(np.float32)
    L, ot, al, rs = o.accept(np.broadcast_to(lt, (n, B, V)), np.broadcast_to(pd, (n, B, V)),
                             toks, tau, u, B)
    first = ot[:, 1]
    cnt = np.bincount(first, minlength=V)
    assert chisquare(cnt, pt[1] * n).pvalue > 1e-4
    tv = 0.5 * np.abs(pt[1] - pd[1]).sum()
    acc = (L >= 1).mean()
    assert abs(acc - (1 - tv)) < 5 * np.sqrt(0.25 / n)
    sel = L >= 1
    cnt2 = np.bincount(ot[sel, 0], minlength=V)
    assert chisquare(cnt2, pt[0] * sel.sum()).pvalue > 1e-4


def test_coupled_greedy(o):
    pins.pin_coupled_greedy(o)


def test_coupled_gumbel_max_law(o):
    pins.pin_coupled_gumbel_max_law(o)


def test_coupled_coupling_bounds(o):
    pins.pin_coupled_coupling_bounds(o)


def test_coupled_accept_closed_form(o):
    pins.pin_coupled_accept_closed_form(o)


def test_coupled_preserves_target_law(o):
    pins.pin_coupled_preserves_target_law(o)


def test_route_closed_forms(o):
    pins.pin_route_closed_forms(o)


def test_route_margin_counts(o):
    pins.pin_route_margin_counts(o)


def test_route_entropy_library(o):
    pins.pin_route_entropy_library(o)


def test_route_expected_prefix(o):
    pins.pin_route_expected_prefix(o)


def test_copies_single_textbook(o):
    pins.pin_copies_single_textbook(o)


def test_copies_decompose(o):
    pins.pin_copies_decompose(o)


def test_gather_roundtrip(o):
    pins.pin_gather_roundtrip(o)


def test_paged_attention_lengths(o):
    pins.pin_paged_attention_lengths(o)


def test_commit_golden(o):
    pins.pin_commit_golden(o)


def test_commit_invariants(o):
    pins.pin_commit_invariants(o)


def test_append_roundtrip(o):
    pins.pin_append_roundtrip(o)


def test_append_rotation(o):
    pins.pin_append_rotation(o)


def test_tree_golden(o):
    pins.pin_tree_golden(o)


def test_tree_chain_is_coupled(o):
    pins.pin_tree_chain_is_coupled(o)


def test_tree_bruteforce(o):
    pins.pin_tree_bruteforce(o)


def test_tree_rejects_bad_parent(o):
    pins.pin_tree_rejects_bad_parent(o)


def test_states_golden(o):
    pins.pin_states_golden(o)


def test_confidence_closed_forms(o):
    pins.pin_confidence_closed_forms(o)


def test_transition_rule(o):
    pins.pin_transition_rule(o)


def test_state_walk_bruteforce(o):
    pins.pin_state_walk_bruteforce(o)


def test_states_one_commit_is_tree_verify(o):
    pins.pin_states_one_commit_is_tree_verify(o)


def test_states_reject_bad_parent(o):
    pins.pin_states_reject_bad_parent(o)
