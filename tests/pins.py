"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each pin takes an ``oracle.Oracle`` handle and raises AssertionError when the
oracle disagrees with an independent fact: a hand-worked fixture under
``tests/golden/``, an invariant that follows from the pages' definitions, a
closed form, a special case that reduces to a textbook computation, or brute
force on a tiny input.  None of them retypes the oracle's own formula.  The
same pins run against deliberately broken copies of the oracle
(``test_oracle_mutants.py``) to show that each plausible mistake is caught.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- fixtures
def load_mask_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(t) for t in line.split()])
    B, P = rows[0]
    tau = np.array(rows[1], np.int32)
    M = np.array(rows[2:], np.uint8)
    return B, P, tau, M


def load_accept_golden():
    with open(os.path.join(GOLDEN, "accept_tiny.json")) as f:
        return json.load(f)["cases"]


def rng(seed):
    return np.random.default_rng(seed)


def random_tau(B, seed):
    return (rng(seed).permutation(B) + 1).astype(np.int32)


# --------------------------------------------------------------------- mask
def pin_mask_golden(o):
    for name in ("mask_B3_tau213_P2.txt", "mver_B4.txt"):
        B, P, tau, M = load_mask_golden(name)
        got = o.mask(tau, P)
        assert got.shape == M.shape, name
        assert np.array_equal(got, M), f"{name}: oracle mask differs from the hand-worked fixture"


def pin_mask_invariants(o, tau, P):
    """Every response row sees the whole prompt, exactly one of D_k / D~_k for
    each slot k, hence exactly P + B keys (follows from the four cases being
    complementary per slot)."""
    B = len(tau)
    M = o.mask(tau, P).astype(np.int64)
    assert M.shape == (2 * B, P + 2 * B)
    assert (M[:, :P] == 1).all(), "prompt must be visible to every response row"
    pair = M[:, P:P + B] + M[:, P + B:]
    assert (pair == 1).all(), "exactly one of D_k, D~_k must be visible per row and slot"
    assert (M.sum(axis=1) == P + B).all()


def pin_mask_extremes(o, tau, P):
    """The mask slot decoded first (tau = 1) has no earlier data: it sees no
    D and every D~.  The data row decoded last (tau = B) sees all of D and no
    D~.  Each D~ row never sees its own data slot (no leak of the token it
    predicts) and each D row sees its own token."""
    B = len(tau)
    M = o.mask(tau, P)
    k1 = int(np.where(tau == 1)[0][0])
    kB = int(np.where(tau == B)[0][0])
    assert (M[B + k1, P:P + B] == 0).all() and (M[B + k1, P + B:] == 1).all()
    assert (M[kB, P:P + B] == 1).all() and (M[kB, P + B:] == 0).all()
    for k in range(B):
        assert M[B + k, P + k] == 0, "a mask slot must not see its own data token"
        assert M[k, P + k] == 1, "a data slot sees its own token"
        assert M[B + k, P + B + k] == 1, "a mask slot sees itself"


def pin_mask_identity(o, B, P):
    """tau = identity gives the block-triangular 2L verification view."""
    tau = np.arange(1, B + 1, dtype=np.int32)
    M = o.mask(tau, P)
    one = np.ones((B, B), np.uint8)
    ref = np.block([[np.tril(one), np.triu(one, 1)], [np.tril(one, -1), np.triu(one)]])
    assert np.array_equal(M[:, P:], ref)
    assert (M[:, :P] == 1).all()


def slot_perm_index(sigma, P):
    """Column/row index map for a slot permutation: new slot k holds old slot
    sigma[k] (prompt positions fixed)."""
    B = len(sigma)
    rows = np.concatenate([sigma, B + sigma])
    cols = np.concatenate([np.arange(P), P + sigma, P + B + sigma])
    return rows, cols


def pin_mask_equivariance(o, tau, sigma, P):
    """Relabelling slots permutes rows and columns of the mask: the mask
    depends on kinds and step labels only, not on slot indices."""
    tau2 = tau[sigma]
    M = o.mask(tau, P)
    M2 = o.mask(tau2, P)
    rows, cols = slot_perm_index(sigma, P)
    assert np.array_equal(M2, M[np.ix_(rows, cols)])


def pin_mask_rejects_bad_tau(o):
    import oracle as om
    for bad in ([1, 1, 2], [0, 1, 2], [1, 2, 4]):
        try:
            o.mask(np.array(bad, np.int32), 3)
        except om.OracleError:
            continue
        raise AssertionError(f"tau {bad} accepted")


def all_mask_pins(o):
    pin_mask_golden(o)
    for B in (1, 2, 3):
        for perm in itertools.permutations(range(1, B + 1)):
            tau = np.array(perm, np.int32)
            for P in (0, 3):
                pin_mask_invariants(o, tau, P)
                pin_mask_extremes(o, tau, P)
    for s in range(20):
        B = (8, 16, 64)[s % 3]
        tau = random_tau(B, 100 + s)
        pin_mask_invariants(o, tau, 5)
        pin_mask_extremes(o, tau, 5)
        pin_mask_equivariance(o, tau, rng(200 + s).permutation(B), 5)
        pin_mask_equivariance(o, tau, np.argsort(tau), 0)
    for B in (1, 4, 8, 32):
        pin_mask_identity(o, B, 7)
    pin_mask_rejects_bad_tau(o)


# --------------------------------------------------------------------- RoPE
def pin_rope_zero_position(o):
    x = rng(1).standard_normal((3, 2, 16))
    y = o.rope(x, np.zeros(3), 1e4)
    assert np.array_equal(x, y)


def pin_rope_2d(o):
    """d = 2: the only pair turns by exactly pos radians (theta^0 = 1), the
    textbook plane rotation."""
    x = rng(2).standard_normal((5, 2))
    pos = np.array([0.0, 1.0, 2.5, -3.0, 100.0])
    y = o.rope(x, pos, 1e4)
    c, s = np.cos(pos), np.sin(pos)
    ref = np.stack([x[:, 0] * c - x[:, 1] * s, x[:, 0] * s + x[:, 1] * c], axis=1)
    assert np.allclose(y, ref, rtol=0, atol=1e-12)


def pin_rope_pairs_and_frequencies(o, d=16, theta=1e4):
    """Unit vector e_i (i < d/2) at position p stays in the plane (i, i+d/2)
    and turns by p * theta^(-2i/d) counter-clockwise."""
    half = d // 2
    for i in range(half):
        e = np.zeros((1, d))
        e[0, i] = 1.0
        p = 0.7
        y = o.rope(e, np.array([p]), theta)[0]
        others = np.delete(y, [i, i + half])
        assert np.abs(others).max() < 1e-15, "rotate-half pairs (i, i + d/2)"
        ang = np.arctan2(y[i + half], y[i])
        assert abs(ang - p * theta ** (-2.0 * i / d)) < 1e-12


def pin_rope_norm_and_relative(o, d=64, theta=1e4):
    """Rotation preserves norms, and <R_m q, R_n k> = <R_{m-n} q, k>."""
    r = rng(3)
    q = r.standard_normal((1, d))
    k = r.standard_normal((1, d))
    for m, n in ((5, 2), (100, 37), (2080, 3), (16400, 16400)):
        qm = o.rope(q, np.array([float(m)]), theta)
        kn = o.rope(k, np.array([float(n)]), theta)
        qd = o.rope(q, np.array([float(m - n)]), theta)
        assert abs(np.linalg.norm(qm) - np.linalg.norm(q)) < 1e-12
        assert abs(np.dot(qm[0], kn[0]) - np.dot(qd[0], k[0])) < 1e-9


def all_rope_pins(o):
    pin_rope_zero_position(o)
    pin_rope_2d(o)
    pin_rope_pairs_and_frequencies(o)
    pin_rope_pairs_and_frequencies(o, d=128, theta=1e6)
    pin_rope_norm_and_relative(o)


# ---------------------------------------------------------------- attention
def tiny_attn_inputs(seed, B=8, P=32, Hq=4, Hkv=2, d=16):
    r = rng(seed)
    R = 2 * B
    return dict(
        q=r.standard_normal((R, Hq, d)).astype(np.float32),
        k_new=r.standard_normal((R, Hkv, d)).astype(np.float32),
        v_new=r.standard_normal((R, Hkv, d)).astype(np.float32),
        k_cache=r.standard_normal((Hkv, P, d)).astype(np.float32),
        v_cache=r.standard_normal((Hkv, P, d)).astype(np.float32),
        tau=random_tau(B, seed + 1),
    )


def textbook_attention(q, K, V, scale):
    """Ordinary unmasked softmax attention of one query over rows of K, V."""
    s = scale * (K @ q)
    w = np.exp(s - s.max())
    return (w / w.sum()) @ V


def pin_attn_bruteforce(o, inp, theta):
    """One-layer invariant: each response row equals plain unmasked attention
    over its explicitly rebuilt context.  D~_i: prompt, data tokens D_k with
    tau(k) < tau(i), mask tokens D~_k for the other slots.  D_i: prompt, D_k
    with tau(k) <= tau(i), D~_k otherwise.  Every token is rotated at its true
    position (prompt already rotated; slot k at P + k)."""
    q, kn, vn, kc, vc, tau = (inp[k] for k in ("q", "k_new", "v_new", "k_cache", "v_cache", "tau"))
    R, Hq, d = q.shape
    B = R // 2
    Hkv, P = kc.shape[0], kc.shape[1]
    g = Hq // Hkv
    got = o.attention(q, kn, vn, kc, vc, tau, theta)
    slot_pos = P + np.arange(B, dtype=np.float64)
    kD = o.rope(kn[:B].astype(np.float64), slot_pos, theta) if theta > 0 else kn[:B].astype(np.float64)
    kM = o.rope(kn[B:].astype(np.float64), slot_pos, theta) if theta > 0 else kn[B:].astype(np.float64)
    qD = o.rope(q[:B].astype(np.float64), slot_pos, theta) if theta > 0 else q[:B].astype(np.float64)
    qM = o.rope(q[B:].astype(np.float64), slot_pos, theta) if theta > 0 else q[B:].astype(np.float64)
    vD, vM = vn[:B].astype(np.float64), vn[B:].astype(np.float64)
    worst = 0.0
    for i in range(B):
        for is_mask in (False, True):
            use_data = (tau < tau[i]) if is_mask else (tau <= tau[i])
            for h in range(Hq):
                kv = h // g
                Kctx = np.concatenate([kc[kv].astype(np.float64),
                                       np.where(use_data[:, None], kD[:, kv], kM[:, kv])])
                Vctx = np.concatenate([vc[kv].astype(np.float64),
                                       np.where(use_data[:, None], vD[:, kv], vM[:, kv])])
                qi = (qM if is_mask else qD)[i, h]
                ref = textbook_attention(qi, Kctx, Vctx, 1.0 / np.sqrt(d))
                row = (B + i) if is_mask else i
                worst = max(worst, np.abs(got[row, h] - ref).max())
    assert worst < 1e-12, f"brute-force context mismatch {worst}"


def pin_attn_single_key(o):
    """P = 0, B = 1: D_1 sees only itself and D~_1 only itself, so each
    output is that token's value vector exactly."""
    inp = tiny_attn_inputs(5, B=1, P=0, Hq=2, Hkv=1, d=8)
    out = o.attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                      inp["tau"], 1e4)
    for h in range(2):
        assert np.abs(out[0, h] - inp["v_new"][0, 0]).max() < 1e-14
        assert np.abs(out[1, h] - inp["v_new"][1, 0]).max() < 1e-14


def pin_attn_two_keys_scale(o):
    """P = 1, B = 1, no rotation: D_1 sees the prompt key and itself, so the
    output is a logistic mix with weight sigmoid((s0 - s1)/sqrt(d))."""
    d = 8
    inp = tiny_attn_inputs(6, B=1, P=1, Hq=1, Hkv=1, d=d)
    out = o.attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                      inp["tau"], 0.0)
    q = inp["q"][0, 0].astype(np.float64)
    s0 = q @ inp["k_cache"][0, 0] / np.sqrt(d)
    s1 = q @ inp["k_new"][0, 0] / np.sqrt(d)
    w0 = 1.0 / (1.0 + np.exp(s1 - s0))
    ref = w0 * inp["v_cache"][0, 0] + (1 - w0) * inp["v_new"][0, 0]
    assert np.abs(out[0, 0] - ref).max() < 1e-13
    out2 = o.attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                       inp["tau"], 0.0, scale=1.0 / np.sqrt(d))
    assert np.abs(out2 - out).max() == 0.0


def pin_attn_gqa_mapping(o):
    """Query heads 2k and 2k+1 read kv-head k when Hq = 4, Hkv = 2: zero
    values on kv-head 1 zero exactly heads 2 and 3."""
    inp = tiny_attn_inputs(7, B=4, P=6, Hq=4, Hkv=2, d=8)
    inp["v_new"][:, 1] = 0
    inp["v_cache"][1] = 0
    out = o.attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                      inp["tau"], 1e4)
    assert (out[:, 2:] == 0).all()
    assert (np.abs(out[:, :2]).max(axis=2) > 0).all()


def pin_attn_constant_values(o):
    """Softmax weights sum to one: constant value rows give that constant."""
    inp = tiny_attn_inputs(8, B=5, P=9, Hq=2, Hkv=1, d=8)
    inp["v_new"][:] = 0.75
    inp["v_cache"][:] = 0.75
    out = o.attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                      inp["tau"], 1e4)
    assert np.abs(out - 0.75).max() < 1e-14


def pin_attn_equivariance(o, seed):
    """Relabelling slots (rows and keys of D and D~ together, tau' = tau o
    sigma) permutes the outputs in the same way (pre-rotated inputs)."""
    inp = tiny_attn_inputs(seed, B=6, P=5, Hq=2, Hkv=1, d=8)
    B = 6
    sigma = rng(seed + 9).permutation(B)
    out = o.attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                      inp["tau"], 0.0)
    rows = np.concatenate([sigma, B + sigma])
    out2 = o.attention(inp["q"][rows], inp["k_new"][rows], inp["v_new"][rows], inp["k_cache"],
                       inp["v_cache"], inp["tau"][sigma], 0.0)
    assert np.abs(out2 - out[rows]).max() < 1e-13


def pin_attn_copy_alignment(o):
    """Identical raw query rows for D_k and D~_k are rotated at the same
    position: with every key made visible-equivalent (identical D and D~
    keys/values), D_k and D~_k see the same multiset of tokens and give the
    same output."""
    inp = tiny_attn_inputs(9, B=4, P=3, Hq=1, Hkv=1, d=8)
    B = 4
    inp["q"][B:] = inp["q"][:B]
    inp["k_new"][B:] = inp["k_new"][:B]
    inp["v_new"][B:] = inp["v_new"][:B]
    out = o.attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"],
                      inp["tau"], 1e4)
    assert np.abs(out[:B] - out[B:]).max() < 1e-13


def all_attention_pins(o):
    for seed, P in ((11, 32), (12, 0), (13, 7)):
        inp = tiny_attn_inputs(seed, B=8, P=P)
        pin_attn_bruteforce(o, inp, 1e4)
    pin_attn_bruteforce(o, tiny_attn_inputs(14, B=3, P=5, Hq=2, Hkv=2, d=8), 0.0)
    pin_attn_single_key(o)
    pin_attn_two_keys_scale(o)
    pin_attn_gqa_mapping(o)
    pin_attn_constant_values(o)
    pin_attn_equivariance(o, 21)
    pin_attn_copy_alignment(o)


# ------------------------------------------------------------------- accept
def pin_accept_golden(o):
    for c in load_accept_golden():
        tp = np.array(c["target_probs"], np.float64)
        logits = np.log(tp).astype(np.float32)[None]
        probs = np.array(c["draft_probs"], np.float32)[None]
        L, ot, al, _ = o.accept(logits, probs, np.array([c["draft_tokens"]], np.int32),
                                np.array([c["tau"]], np.int32),
                                np.array([c["uniforms"]], np.float32), c["gamma"])
        assert int(L[0]) == c["accept_len"], c["note"]
        assert ot[0].tolist() == c["out_tokens"], c["note"]
        assert np.allclose(al[0], c["alpha"], rtol=1e-6, atol=0), c["note"]


def pin_softmax(o):
    """V = 2 gives the logistic function; shifting logits changes nothing;
    probabilities sum to one."""
    p, m, s = o.softmax(np.array([1.5, -0.5], np.float32))
    assert abs(p[0] - 1.0 / (1.0 + np.exp(-2.0))) < 1e-15
    # logits on a 2^-10 grid so that adding 64 is exact in float32
    l = (np.round(rng(4).standard_normal(1000) * 3 * 1024) / 1024).astype(np.float32)
    p1, _, _ = o.softmax(l)
    p2, _, _ = o.softmax(l + np.float32(64.0))
    assert abs(p1.sum() - 1) < 1e-13 and np.abs(p1 - p2).max() < 1e-12


def _one_slot(o, lt, pd, x, u0, u1, temperature=1.0):
    L, ot, al, _ = o.accept(lt[None, None], pd[None, None], np.array([[x]], np.int32),
                            np.array([[1]], np.int32), np.array([[u0, u1]], np.float32), 1, temperature)
    return int(L[0]), int(ot[0, 0]), float(al[0, 0])


def pin_accept_tv_identity(o, V=6, seed=30):
    """E_{x ~ p_phi}[alpha(x)] = sum_v min(p_theta, p_phi) = 1 - D_TV
    (the acceptance rate of rejection sampling equals one minus the total
    variation distance)."""
    r = rng(seed)
    lt = (r.standard_normal(V) * 1.5).astype(np.float32)
    pt, _, _ = o.softmax(lt)
    pd = r.dirichlet(np.ones(V)).astype(np.float32)
    acc = sum(float(pd[x]) * _one_slot(o, lt, pd, x, 0.0, 0.5)[2] for x in range(V))
    tv = 0.5 * np.abs(pt - pd.astype(np.float64)).sum()
    ref = np.minimum(pt, pd.astype(np.float64)).sum()
    assert abs(acc - ref) < 1e-12
    assert abs(ref - (1 - tv)) < 1e-6  # p_phi sums to one only up to float32


def pin_accept_exact_distribution(o, V=4, seed=31, N=4000):
    """Exact law of the emitted token at a slot, by enumeration: draft token
    x with probability p_phi(x); accept with probability alpha(x) (measure of
    u < alpha); otherwise the resample, whose law is the measure of the
    resample uniform mapping to each token (a fine midpoint grid).  The
    result must be the target distribution p_theta."""
    r = rng(seed)
    lt = (r.standard_normal(V) * 1.2).astype(np.float32)
    pt, _, _ = o.softmax(lt)
    pd = r.dirichlet(np.ones(V)).astype(np.float64)
    pd /= pd.sum()
    pd32 = pd.astype(np.float32)
    law = np.zeros(V)
    grid = (np.arange(N) + 0.5) / N
    for x in range(V):
        a = _one_slot(o, lt, pd32, x, 0.0, 0.5)[2]
        law[x] += float(pd32[x]) * a
        counts = np.zeros(V)
        for u1 in grid:
            L, t, _ = _one_slot(o, lt, pd32, x, 0.999999, float(u1))
            if L == 0:
                counts[t] += 1
        if counts.sum():
            law += float(pd32[x]) * (1 - a) * counts / N
    assert np.abs(law - pt).max() < 2.0 / N + 1e-6, (law, pt)


def pin_accept_special_cases(o):
    r = rng(32)
    V = 50
    lt = r.standard_normal(V).astype(np.float32)
    pt, _, _ = o.softmax(lt)
    pd = pt.astype(np.float32)
    # p_theta == p_phi: every step accepted (alpha = 1 up to float32 rounding)
    B = 5
    lts = np.stack([lt] * B)[None]
    pds = np.stack([pd] * B)[None]
    tau = random_tau(B, 33)[None]
    toks = r.integers(0, V, (1, B)).astype(np.int32)
    u = np.full((1, B + 1), 0.99, np.float32)
    L, ot, al, rs = o.accept(lts, pds, toks, tau, u, B)
    assert L[0] == B and (ot == toks).all() and rs[0] == -1
    assert np.abs(al - 1).max() < 1e-6
    # p_theta(x) = 0: rejected even with u = 0
    lt0 = lt.copy()
    lt0[7] = np.float32(-3e38)
    Lx, tx, ax = _one_slot(o, lt0, pd, 7, 0.0, 0.5)
    assert Lx == 0 and ax == 0.0 and tx != 7
    # p_phi >= p_theta everywhere: the residual is empty and the target is used
    pd_big = (pt * 1.25).astype(np.float32)
    tok, cdf, Z, used = o.residual(lt, pd_big, 0.5)
    assert used and abs(Z - 1) < 1e-12 and cdf[tok] > 0.5 and (tok == 0 or cdf[tok - 1] <= 0.5)


def pin_residual_boundaries(o):
    """The inverse CDF at the ends of the uniform's range, on a row whose
    residual (p_theta - p_phi)^+ is positive at tokens 1 and 4 only: u = 0
    takes the first token with mass; a u just below 1 crosses at token 4,
    the last one with mass; at u = 1 (one past the documented range) no
    running sum exceeds u * Z and the rule falls back to the last token
    with positive mass -- still 4, not the later zero-mass tokens 5..7.
    With p_phi >= p_theta everywhere the target itself is sampled, and the
    fallback then skips tokens whose target mass is 0 (-inf logits)."""
    lt = np.log(np.arange(1, 9, dtype=np.float64)).astype(np.float32)
    pt, _, _ = o.softmax(lt)
    pd = np.where(np.isin(np.arange(8), [1, 4]), 0.5 * pt, 1.5 * pt).astype(np.float32)
    for u, want in ((0.0, 1), (float(np.float32(1.0 - 2 ** -24)), 4), (1.0, 4)):
        tok, cdf, Z, used = o.residual(lt, pd, u)
        assert not used and tok == want, (u, tok, want)
        assert Z > 0 and cdf[-1] == cdf[4] == Z and cdf[0] == 0.0
    lt2 = lt.copy()
    lt2[6:] = -np.inf
    pt2, _, _ = o.softmax(lt2)
    tok, cdf, Z, used = o.residual(lt2, (1.5 * pt2).astype(np.float32), 1.0)
    assert used and tok == 5 and abs(Z - 1.0) < 1e-12, (tok, Z)


def pin_accept_assembly(o, seed=34):
    """Output layout: tokens of steps 1..L are the draft tokens, the slot of
    step L+1 holds the resample, slots of later steps and of steps > gamma
    hold -1; alpha is reported for every step in draft order."""
    r = rng(seed)
    n, B, V = 200, 6, 16
    lt = (r.standard_normal((n, B, V)) * 1.5).astype(np.float32)
    pd = r.dirichlet(np.ones(V), (n, B)).astype(np.float32)
    toks = r.integers(0, V, (n, B)).astype(np.int32)
    tau = np.stack([random_tau(B, 1000 + i) for i in range(n)])
    u = r.random((n, B + 1)).astype(np.float32)
    for gamma in (B, 3):
        uu = u[:, :gamma + 1].copy()
        L, ot, al, rs = o.accept(lt, pd, toks, tau, uu, gamma)
        for b in range(n):
            l = int(L[b])
            assert 0 <= l <= gamma
            steps = tau[b]
            # leading accepts: every step r <= L has u < alpha, step L+1 fails
            assert all(uu[b, s] < al[b, s] for s in range(l))
            if l < gamma:
                assert not (uu[b, l] < al[b, l])
            for k in range(B):
                if steps[k] <= l:
                    assert ot[b, k] == toks[b, k]
                elif steps[k] == l + 1 and l < gamma:
                    assert rs[b] == k and 0 <= ot[b, k] < V
                else:
                    assert ot[b, k] == -1
            # alpha in draft order: step s verifies the slot with tau = s
            for s in range(gamma):
                k = int(np.where(steps == s + 1)[0][0])
                x = toks[b, k]
                pt, _, _ = o.softmax(lt[b, k])
                assert abs(al[b, s] - min(1.0, pt[x] / float(pd[b, k, x]))) < 1e-12


def pin_accept_energy(o, seed=35):
    """S2D2's residual-energy form: alpha = min(1, exp(-E)), with
    E = -log q + log p (q the verifier's, p the draft's probability)."""
    r = rng(seed)
    V = 12
    for _ in range(10):
        lt = (r.standard_normal(V) * 2).astype(np.float32)
        pd = r.dirichlet(np.ones(V)).astype(np.float32)
        x = int(r.integers(V))
        pt, _, _ = o.softmax(lt)
        a = _one_slot(o, lt, pd, x, 0.0, 0.5)[2]
        E = -np.log(pt[x]) + np.log(float(pd[x]))
        assert abs(a - min(1.0, np.exp(-E))) < 1e-12


def pin_accept_tempered(o, V=4, seed=37, N=1000):
    """Sampling at temperature T: draft token x ~ p_phi, acceptance with
    alpha and the resample emit tokens distributed as the tempered target
    softmax(l / T) -- scipy's softmax of the float64 quotient (the float32
    rounding of l * (1/T) moves the law by ~1e-7) -- and the acceptance rate
    is sum_v min(softmax(l / T), p_phi).  At T = 0.5 and T = 2, where
    untempered logits, or logits multiplied by T, give other laws."""
    from scipy.special import softmax
    r = rng(seed)
    lt = (r.standard_normal(V) * 1.2).astype(np.float32)
    pd = r.dirichlet(np.ones(V))
    pd32 = (pd / pd.sum()).astype(np.float32)
    grid = (np.arange(N) + 0.5) / N
    for T in (0.5, 2.0):
        pt = softmax(lt.astype(np.float64) / T)
        law, rate = np.zeros(V), 0.0
        for x in range(V):
            a = _one_slot(o, lt, pd32, x, 0.0, 0.5, T)[2]
            rate += float(pd32[x]) * a
            law[x] += float(pd32[x]) * a
            counts = np.zeros(V)
            for u1 in grid:
                L, t, _ = _one_slot(o, lt, pd32, x, 0.999999, float(u1), T)
                if L == 0:
                    counts[t] += 1
            if counts.sum():
                law += float(pd32[x]) * (1 - a) * counts / N
        assert np.abs(law - pt).max() < 2.0 / N + 1e-6, (T, law, pt)
        assert abs(rate - np.minimum(pt, pd32.astype(np.float64)).sum()) < 1e-6, (T, rate)


def all_accept_pins(o, exact=True):
    pin_accept_golden(o)
    pin_softmax(o)
    pin_accept_tv_identity(o)
    pin_accept_special_cases(o)
    pin_residual_boundaries(o)
    pin_accept_assembly(o)
    pin_accept_energy(o)
    pin_accept_tempered(o)
    if exact:
        pin_accept_exact_distribution(o, N=1000)


# ----------------------------------------------- shared-noise verification
def gumbel(r, shape):
    """Standard Gumbel noise, -log(-log U), U uniform on (0, 1)."""
    u = r.random(shape)
    u = np.where(u <= 0.0, np.finfo(np.float64).tiny, u)
    return (-np.log(-np.log(u))).astype(np.float32)


def pin_coupled_greedy(o):
    """T = 0 is the greedy transition: the choice is the first maximal logit
    (numpy's argmax returns the first occurrence), ties included."""
    r = rng(40)
    for V in (1, 7, 1000):
        for _ in range(5):
            l = r.standard_normal(V).astype(np.float32)
            assert o.coupled_choice(l, None, 0.0) == int(np.argmax(l))
    l = np.array([0.5, 2.0, -1.0, 2.0, 2.0], np.float32)
    assert o.coupled_choice(l, None, 0.0) == 1


def pin_coupled_gumbel_max_law(o, N=30000):
    """Gumbel-max: argmax_v (l_v / T + G_v) with iid standard Gumbel G is a
    sample of softmax(l / T).  Two temperatures, so that T and 1/T, the sign
    of the noise and argmax vs argmin are all distinguished."""
    r = rng(41)
    l = np.array([0.3, -1.2, 1.1, 0.0, 0.6], np.float32)
    for T in (0.5, 2.0):
        counts = np.zeros(l.shape[0])
        for g in gumbel(r, (N, l.shape[0])):
            counts[o.coupled_choice(l, g, T)] += 1
        z = l.astype(np.float64) / np.float64(np.float32(T))
        p = np.exp(z - z.max())
        p /= p.sum()
        sd = np.sqrt(p * (1 - p) / N)
        assert (np.abs(counts / N - p) < 4.5 * sd + 1e-12).all(), (T, counts / N, p)


def pin_coupled_coupling_bounds(o, N=30000):
    """Shared noise couples two Gumbel-max samples: with delta = D_TV(p, q),
    P[choice under p == choice under q] is at least (1 - delta)/(1 + delta)
    (the bound the SPOT page quotes) and at most 1 - delta (no coupling does
    better)."""
    r = rng(42)
    V = 8
    for scale in (0.3, 1.0):
        lp = r.standard_normal(V).astype(np.float32)
        lq = (lp + scale * r.standard_normal(V)).astype(np.float32)
        p, _, _ = o.softmax(lp)
        q, _, _ = o.softmax(lq)
        delta = 0.5 * np.abs(p - q).sum()
        agree = 0
        for g in gumbel(r, (N, V)):
            agree += o.coupled_choice(lp, g, 1.0) == o.coupled_choice(lq, g, 1.0)
        rate = agree / N
        sd = np.sqrt(0.25 / N)
        assert rate >= (1 - delta) / (1 + delta) - 4.5 * sd, (rate, delta)
        assert rate <= 1 - delta + 4.5 * sd, (rate, delta)


def pin_coupled_accept_closed_form(o):
    """Draft tokens built to match the target's choice for exactly k leading
    steps (draft order given by tau): L = k, the draft tokens are kept for
    steps 1..k, the target's own choice is committed at step k+1, later steps
    and steps past gamma stay -1; matching every step accepts all gamma with
    no extra token."""
    r = rng(43)
    B, V = 6, 40
    for T in (0.0, 0.7):
        for gamma in (B, 4):
            for k in range(gamma + 1):
                logits = (r.standard_normal((1, B, V)) * 2).astype(np.float32)
                noise = gumbel(r, (1, B, V))
                tau = random_tau(B, 500 + 7 * k + gamma)[None]
                choice = np.array([o.coupled_choice(logits[0, j], noise[0, j], T) for j in range(B)])
                toks = choice.copy()
                step_slot = {int(tau[0, j]): j for j in range(B)}
                if k < gamma:
                    j = step_slot[k + 1]
                    toks[j] = (choice[j] + 1) % V   # the first mismatch
                for s in range(k + 2, B + 1):      # later steps: anything
                    toks[step_slot[s]] = int(r.integers(V))
                L, ot, tt = o.accept_coupled(logits, noise, toks[None].astype(np.int32), tau, gamma, T)
                assert int(L[0]) == k, (T, gamma, k, int(L[0]))
                for j in range(B):
                    t = int(tau[0, j])
                    assert tt[0, j] == (choice[j] if t <= gamma else -1)
                    if t <= k:
                        assert ot[0, j] == toks[j]
                    elif t == k + 1 and k < gamma:
                        assert ot[0, j] == choice[j] and ot[0, j] != toks[j]
                    else:
                        assert ot[0, j] == -1


def pin_coupled_preserves_target_law(o, N=20000):
    """The committed token at a verified slot follows the target's sampling
    law softmax(l / T) whatever the draft proposes (the step either accepts a
    draft equal to the target's choice or commits that choice): here the
    draft is a shared-noise sample of a different distribution."""
    r = rng(44)
    V, T = 6, 1.5
    lt = np.array([0.2, 1.4, -0.7, 0.9, 0.0, -1.5], np.float32)
    ld = np.array([1.6, -0.3, 0.4, -1.0, 0.8, 0.1], np.float32)
    noise = gumbel(r, (N, 1, V))
    inv_t = np.float32(1.0) / np.float32(T)
    draft = np.argmax(ld[None, None, :] * inv_t + noise, axis=2).astype(np.int32)
    L, ot, tt = o.accept_coupled(np.broadcast_to(lt, (N, 1, V)), noise, draft,
                                 np.ones((N, 1), np.int32), 1, T)
    counts = np.bincount(ot[:, 0], minlength=V)
    z = lt.astype(np.float64) / np.float64(np.float32(T))
    p = np.exp(z - z.max())
    p /= p.sum()
    sd = np.sqrt(p * (1 - p) / N)
    assert (np.abs(counts / N - p) < 4.5 * sd).all(), (counts / N, p)
    assert 0 < L.mean() < 1  # both outcomes occur


def all_coupled_pins(o):
    pin_coupled_greedy(o)
    pin_coupled_gumbel_max_law(o)
    pin_coupled_coupling_bounds(o)
    pin_coupled_accept_closed_form(o)
    pin_coupled_preserves_target_law(o)


# ---------------------------------------------- multi-copy verification
def tiny_copy_inputs(seed, L=6, C=3, P=10, Hq=4, Hkv=2, d=16):
    r = rng(seed)
    R = C * L
    return dict(
        q=r.standard_normal((R, Hq, d)).astype(np.float32),
        k_new=r.standard_normal((R, Hkv, d)).astype(np.float32),
        v_new=r.standard_normal((R, Hkv, d)).astype(np.float32),
        k_cache=r.standard_normal((Hkv, P, d)).astype(np.float32),
        v_cache=r.standard_normal((Hkv, P, d)).astype(np.float32),
    )


def pin_copies_single_textbook(o, theta=1e4):
    """One copy is a plain block: each row is ordinary unmasked attention over
    [prompt ; the block], the block rotated at positions P + i."""
    inp = tiny_copy_inputs(70, C=1)
    L, Hq, d = inp["q"].shape
    Hkv, P = inp["k_cache"].shape[0], inp["k_cache"].shape[1]
    out = o.attention_copies(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], 1, theta)
    pos = P + np.arange(L, dtype=np.float64)
    qr = o.rope(inp["q"], pos, theta)
    kr = o.rope(inp["k_new"], pos, theta)
    g = Hq // Hkv
    for i in range(L):
        for h in range(Hq):
            kv = h // g
            K = np.concatenate([inp["k_cache"][kv].astype(np.float64), kr[:, kv]])
            V = np.concatenate([inp["v_cache"][kv].astype(np.float64), inp["v_new"][:, kv].astype(np.float64)])
            ref = textbook_attention(qr[i, h], K, V, 1 / np.sqrt(d))
            assert np.abs(out[i, h] - ref).max() < 1e-12


def pin_copies_decompose(o, theta=1e4):
    """Each copy's rows equal a one-copy run on that copy's rows alone; a
    change to one copy leaves every other copy bit-identical; permuting the
    copies permutes the output."""
    L, C = 5, 4
    inp = tiny_copy_inputs(71, L=L, C=C, P=7)
    args = (inp["k_cache"], inp["v_cache"])
    out = o.attention_copies(inp["q"], inp["k_new"], inp["v_new"], *args, C, theta)
    for c in range(C):
        sl = slice(c * L, (c + 1) * L)
        one = o.attention_copies(inp["q"][sl], inp["k_new"][sl], inp["v_new"][sl], *args, 1, theta)
        assert np.array_equal(out[sl], one), c
    k2, v2 = inp["k_new"].copy(), inp["v_new"].copy()
    k2[L:2 * L] += 1.0
    v2[L:2 * L] -= 2.0
    out2 = o.attention_copies(inp["q"], k2, v2, *args, C, theta)
    for c in range(C):
        sl = slice(c * L, (c + 1) * L)
        if c == 1:
            assert np.abs(out2[sl] - out[sl]).max() > 1e-3
        else:
            assert np.array_equal(out2[sl], out[sl]), c
    perm = np.array([2, 0, 3, 1])
    rows = np.concatenate([np.arange(c * L, (c + 1) * L) for c in perm])
    out3 = o.attention_copies(inp["q"][rows], inp["k_new"][rows], inp["v_new"][rows], *args, C, theta)
    assert np.array_equal(out3, out[rows])


def all_copies_pins(o):
    pin_copies_single_textbook(o)
    pin_copies_decompose(o)


# ------------------------------------------------ verify-routing estimator
def pin_route_closed_forms(o):
    """Uniform rows have normalised entropy 1, so alpha = exp(-beta) and K is
    the geometric sum; one-hot rows have margin 1 and entropy 0, so K = gamma
    for both estimators; a two-point row has entropy -q ln q - (1-q) ln(1-q)."""
    B, V, gamma = 5, 16, 5
    tau = random_tau(B, 60)[None]
    for beta in (0.3, 1.7):
        kh, ah = o.route(np.full((1, B, V), 1.0 / V, np.float32), tau, gamma, "entropy", beta)
        a = np.exp(-beta)
        assert np.abs(ah - a).max() < 1e-12
        assert abs(kh[0] - a * (1 - a ** gamma) / (1 - a)) < 1e-12
    onehot = np.zeros((1, B, V), np.float32)
    onehot[0, np.arange(B), (np.arange(B) * 3) % V] = 1.0
    for est, prm in (("margin", 0.9), ("entropy", 5.0)):
        kh, ah = o.route(onehot, tau, gamma, est, prm)
        assert kh[0] == gamma and (ah == 1).all()
    q = np.float32(0.3)
    two = np.zeros((1, 1, V), np.float32)
    two[0, 0, 3], two[0, 0, 9] = q, np.float32(1) - q
    qd = float(q)
    h = -(qd * np.log(qd) + (1 - qd) * np.log(1 - qd)) / np.log(V)
    kh, ah = o.route(two, np.ones((1, 1), np.int32), 1, "entropy", 2.0)
    assert abs(ah[0, 0] - np.exp(-2.0 * h)) < 1e-9


def pin_route_margin_counts(o, seed=61):
    """Margin estimator: alpha is 1 while the draft margin p_(1) - p_(2)
    reaches the threshold, so K counts the leading steps in draft order that
    do; rows are built with known margins and shuffled positions."""
    r = rng(seed)
    n, B, V, thr = 40, 7, 12, 0.25
    probs = np.zeros((n, B, V), np.float32)
    margins = r.choice([0.1, 0.2, 0.3, 0.6], size=(n, B))
    for b in range(n):
        for k in range(B):
            top, rest = 0.5 + margins[b, k] / 2, 0.5 - margins[b, k] / 2
            row = np.zeros(V)
            idx = r.permutation(V)
            row[idx[0]] = top
            row[idx[1]] = rest * 0.99
            row[idx[2]] = rest * 0.01
            probs[b, k] = row
    tau = np.stack([random_tau(B, 700 + b) for b in range(n)])
    for gamma in (B, 4):
        kh, ah = o.route(probs, tau, gamma, "margin", thr)
        for b in range(n):
            m = [float(probs[b, int(np.where(tau[b] == s)[0][0])].max()) -
                 float(np.sort(probs[b, int(np.where(tau[b] == s)[0][0])])[-2]) for s in range(1, gamma + 1)]
            lead = next((i for i, x in enumerate(m) if not x >= thr), gamma)
            assert kh[b] == lead, (b, kh[b], lead, m)


def pin_route_entropy_library(o, seed=62):
    """The entropy estimator against scipy's entropy terms -x ln x (entr,
    which also maps 0 to 0) of the same rows, without renormalising."""
    from scipy.special import entr
    r = rng(seed)
    n, B, V, beta = 6, 4, 300, 0.8
    probs = r.dirichlet(np.full(V, 0.3), (n, B)).astype(np.float32)
    probs[0, 0, :10] = 0.0  # zero entries contribute nothing
    tau = np.stack([random_tau(B, 800 + b) for b in range(n)])
    kh, ah = o.route(probs, tau, B, "entropy", beta)
    for b in range(n):
        for s in range(B):
            k = int(np.where(tau[b] == s + 1)[0][0])
            ref = np.exp(-beta * entr(probs[b, k].astype(np.float64)).sum() / np.log(V))
            assert abs(ah[b, s] - ref) < 1e-12, (b, s, ah[b, s], ref)


def pin_route_expected_prefix(o, seed=63):
    """K is the expected accepted prefix length when step r is accepted
    independently with probability alpha_r: enumerate all 2^gamma outcomes."""
    r = rng(seed)
    B, V, gamma = 4, 20, 4
    probs = r.dirichlet(np.full(V, 0.5), (1, B)).astype(np.float32)
    tau = random_tau(B, 900)[None]
    kh, ah = o.route(probs, tau, gamma, "entropy", 1.3)
    a = ah[0]
    e = 0.0
    for bits in itertools.product((0, 1), repeat=gamma):
        pr = np.prod([a[i] if bits[i] else 1 - a[i] for i in range(gamma)])
        L = next((i for i, x in enumerate(bits) if not x), gamma)
        e += pr * L
    assert abs(kh[0] - e) < 1e-12, (kh[0], e)


def all_route_pins(o):
    pin_route_closed_forms(o)
    pin_route_margin_counts(o)
    pin_route_entropy_library(o)
    pin_route_expected_prefix(o)


def all_pins(o):
    all_mask_pins(o)
    all_rope_pins(o)
    all_attention_pins(o)
    all_accept_pins(o)
    all_coupled_pins(o)
    all_route_pins(o)
    all_copies_pins(o)
    all_cache_pins(o)
    all_tree_pins(o)
    all_states_pins(o)


# ---------------------------------------------------------------- paged cache, commit, append
def _paged_from_contiguous(cache, page_size, n_pages, perm):
    """Page a contiguous [Hkv][P][d] cache by reshaping it into page blocks:
    block k (rows k*ps .. k*ps+ps-1) goes to page perm[k]; other pages hold NaN."""
    Hkv, P, d = cache.shape
    npg = -(-P // page_size)
    padded = np.full((Hkv, npg * page_size, d), np.nan, np.float32)
    padded[:, :P] = cache
    blocks = padded.reshape(Hkv, npg, page_size, d).transpose(1, 0, 2, 3)
    pages = np.full((n_pages, Hkv, page_size, d), np.nan, np.float32)
    pages[perm[:npg]] = blocks
    return pages


def pin_gather_roundtrip(o):
    """Gathering a cache paged by a reshape into page blocks gives it back."""
    r = np.random.default_rng(110)
    for P, ps in ((13, 4), (16, 4), (1, 8), (0, 4), (9, 1)):
        cache = r.standard_normal((3, P, 5)).astype(np.float32)
        n_pages = -(-P // ps) + 3
        perm = r.permutation(n_pages).astype(np.int32)
        pages = _paged_from_contiguous(cache, ps, n_pages, perm)
        g = o.gather_prefix(pages, perm, P, ps)
        assert np.array_equal(g, cache), (P, ps)


def pin_paged_attention_lengths(o, theta=1e4):
    """Per-sequence prompt lengths over a paged cache: each sequence equals the
    one-sequence attention over its own P_b prompt rows; rows past P_b (NaN in
    the pages) are never read."""
    r = np.random.default_rng(111)
    B, Hq, Hkv, d, ps = 3, 4, 2, 8, 4
    lens = np.array([10, 0, 7], np.int32)
    Pmax = 12
    n_pages = 3 * (Pmax // ps) + 1
    perm = r.permutation(n_pages).astype(np.int32)
    table = perm[:3 * (Pmax // ps)].reshape(3, Pmax // ps)
    kc = r.standard_normal((3, Hkv, Pmax, d)).astype(np.float32)
    vc = r.standard_normal((3, Hkv, Pmax, d)).astype(np.float32)
    kp = np.full((n_pages, Hkv, ps, d), np.nan, np.float32)
    vp = np.full((n_pages, Hkv, ps, d), np.nan, np.float32)
    for b in range(3):
        for k in range(-(-int(lens[b]) // ps)):
            rows = slice(k * ps, min((k + 1) * ps, int(lens[b])))
            n = rows.stop - rows.start
            kp[table[b, k], :, :n] = kc[b][:, rows]
            vp[table[b, k], :, :n] = vc[b][:, rows]
    q = r.standard_normal((3, 2 * B, Hq, d)).astype(np.float32)
    kn = r.standard_normal((3, 2 * B, Hkv, d)).astype(np.float32)
    vn = r.standard_normal((3, 2 * B, Hkv, d)).astype(np.float32)
    tau = np.stack([r.permutation(B) + 1 for _ in range(3)]).astype(np.int32)
    out = o.attention_paged(q, kn, vn, kp, vp, table, lens, tau, ps, theta)
    assert np.isfinite(out).all()
    for b in range(3):
        P = int(lens[b])
        ref = o.attention(q[b], kn[b], vn[b], kc[b][:, :P], vc[b][:, :P], tau[b], theta)
        assert np.array_equal(out[b], ref), b


def pin_commit_golden(o):
    g = json.load(open(os.path.join(GOLDEN, "commit_tiny.json")))
    bt, rem, state, napp = o.commit(np.array(g["out_tokens"], np.int32), np.array(g["block_before"], np.int32),
                                    g["gamma"])
    assert bt.tolist() == g["block_after"]
    assert rem.tolist() == g["remaining"]
    assert state.tolist() == g["state"]
    assert napp.tolist() == g["n_append"]


def pin_commit_invariants(o):
    """Committed slots take the committed token, other slots keep theirs; R is
    the number of masked slots left; the state is decided by R against gamma at
    every boundary (R = 0, gamma - 1, gamma)."""
    r = np.random.default_rng(112)
    B, gamma, n = 8, 4, 400
    before = np.where(r.random((n, B)) < 0.5, r.integers(0, 50, (n, B)), -1).astype(np.int32)
    out = np.where(r.random((n, B)) < 0.3, r.integers(0, 50, (n, B)), -1).astype(np.int32)
    bt, rem, state, napp = o.commit(out, before, gamma)
    for b in range(n):
        for k in range(B):
            assert bt[b, k] == (out[b, k] if out[b, k] >= 0 else before[b, k])
        R = int((bt[b] == -1).sum())
        assert rem[b] == R
        assert state[b] == {True: 2, False: 1 if R < gamma else 0}[R == 0]
        assert napp[b] == (B if R == 0 else 0)
    seen = {int(x) for x in rem}
    assert {0, gamma - 1, gamma} <= seen, seen


def pin_append_roundtrip(o):
    """Appending n rows at P_b and gathering P_b + n rows gives the old prompt
    followed by the rows (theta = 0: stored as given); nothing else changes;
    an append that would pass the capacity changes nothing; one that fits
    exactly is made."""
    r = np.random.default_rng(113)
    Hkv, d, ps, mp, n_pages, S = 2, 4, 4, 4, 16, 6
    table = r.permutation(n_pages)[:3 * mp].reshape(3, mp).astype(np.int32)
    kp = r.standard_normal((n_pages, Hkv, ps, d)).astype(np.float32)
    vp = r.standard_normal((n_pages, Hkv, ps, d)).astype(np.float32)
    lens = np.array([5, 10, 16], np.int32)       # capacity 16: the third is full
    nap = np.array([6, 6, 1], np.int32)          # 10 + 6 = 16 fits exactly; 16 + 1 does not
    kr = r.standard_normal((3, S, Hkv, d)).astype(np.float32)
    vr = r.standard_normal((3, S, Hkv, d)).astype(np.float32)
    kp2, vp2, lens2, st = o.kv_append(kr, vr, nap, kp, vp, table, lens, ps, 0.0, round_bf16=False)
    assert st.tolist() == [0, 0, 1]
    assert lens2.tolist() == [11, 16, 16]
    changed = 0
    for b in range(3):
        P, P2 = int(lens[b]), int(lens2[b])
        for pages, pages2, rows in ((kp, kp2, kr), (vp, vp2, vr)):
            g0 = o.gather_prefix(pages, table[b], P, ps)
            g1 = o.gather_prefix(pages2, table[b], P2, ps)
            assert np.array_equal(g1[:, :P], g0)
            assert np.array_equal(g1[:, P:P2], rows[b][:P2 - P].transpose(1, 0, 2))
        changed += (P2 - P) * Hkv * d
    assert int((kp2 != kp).sum()) == changed and int((vp2 != vp).sum()) == changed


def pin_append_rotation(o):
    """With theta > 0 an appended key is rotated at its position P_b + i: the
    unit vector on dims (i, i + d/2) becomes (cos, sin) of P_b + i times the
    pair's frequency theta^(-2i/d); stored rounded to bfloat16 (contiguous
    cache, row stride 12)."""
    theta, d, S = 100.0, 4, 3
    lens = np.array([0, 7], np.int32)
    for i in range(d // 2):
        kr = np.zeros((2, S, 1, d), np.float32)
        kr[:, :, 0, i] = 1.0
        vr = np.zeros_like(kr)
        kc = np.zeros((2, 1, 12, d), np.float32)
        kc2, _, lens2, st = o.kv_append(kr, vr, np.array([3, 3], np.int32), kc, kc.copy(), None, lens, 12, theta)
        assert st.tolist() == [0, 0] and lens2.tolist() == [3, 10]
        w = theta ** (-2.0 * i / d)
        for b in range(2):
            for j in range(3):
                p = lens[b] + j
                got = kc2[b, 0, p]
                want = np.zeros(d)
                want[i], want[i + d // 2] = np.cos(p * w), np.sin(p * w)
                ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
                assert (np.abs(got - want) <= ulp + 1e-30).all(), (i, b, j, got, want)


def all_cache_pins(o):
    pin_gather_roundtrip(o)
    pin_paged_attention_lengths(o)
    pin_commit_golden(o)
    pin_commit_invariants(o)
    pin_append_roundtrip(o)
    pin_append_rotation(o)


# ---------------------------------------------------------------- draft-tree verification
def pin_tree_golden(o):
    g = json.load(open(os.path.join(GOLDEN, "tree_tiny.json")))
    pl, path, cp, ct, tt = o.tree_verify(np.array([g["logits"]], np.float32), None, np.array([g["parent"]]),
                                         np.array([g["node_pos"]]), np.array([g["node_tok"]]),
                                         np.array([g["target_pos"]]), g["temperature"])
    assert int(pl[0]) == g["path_len"] and path[0].tolist() == g["path"]
    assert int(cp[0]) == g["commit_pos"] and int(ct[0]) == g["commit_tok"]
    assert tt[0].tolist() == g["target_tok"]


def _chain_from_coupled(lt, gum, tok, tau, gamma):
    """A draft chain of gamma commits in draft order as a tree: node r (1..gamma)
    commits slot o_r; node r's target row is slot o_{r+1}'s."""
    n, B, V = lt.shape
    N = gamma + 1
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (n, 1))
    node_pos, node_tok = np.full((n, N), -1, np.int32), np.full((n, N), -1, np.int32)
    tpos = np.zeros((n, N), np.int32)
    L_rows = np.zeros((n, N, V), np.float32)
    G_rows = np.zeros((n, N, V), np.float32)
    for b in range(n):
        o = np.argsort(tau[b])                 # o[r - 1] = slot with tau = r
        for r in range(1, N):
            node_pos[b, r], node_tok[b, r] = o[r - 1], tok[b, o[r - 1]]
        for r in range(N):
            s = o[min(r, gamma - 1)] if r < gamma else o[gamma - 1]
            tpos[b, r] = s
            L_rows[b, r], G_rows[b, r] = lt[b, s], gum[b, s]
    return L_rows, G_rows, parent, node_pos, node_tok, tpos


def pin_tree_chain_is_coupled(o):
    """A chain of draft commits in draft order is verified exactly as the
    shared-noise verification of the same steps: the same number of accepted
    edges, and the same committed target token after a rejection."""
    r = np.random.default_rng(120)
    n, B, V, gamma = 40, 6, 7, 5
    for T in (1.0, 0.0):
        lt = r.normal(0, 1, (n, B, V)).astype(np.float32)
        gum = (-np.log(-np.log(r.random((n, B, V))))).astype(np.float32)
        tau = np.stack([r.permutation(B) + 1 for _ in range(n)]).astype(np.int32)
        choice = np.stack([[o.coupled_choice(lt[b, k], gum[b, k], T) for k in range(B)] for b in range(n)])
        tok = np.where(r.random((n, B)) < 0.7, choice, (choice + 1) % V).astype(np.int32)
        L_c, ot_c, _ = o.accept_coupled(lt, gum if T > 0 else None, tok, tau, gamma, T)
        rows = _chain_from_coupled(lt, gum, tok, tau, gamma)
        pl, path, cp, ct, tt = o.tree_verify(rows[0], rows[1] if T > 0 else None, *rows[2:], T)
        assert np.array_equal(pl, L_c), (pl, L_c)
        for b in range(n):
            if L_c[b] < gamma:
                o_next = int(np.argsort(tau[b])[L_c[b]])
                assert ct[b] == ot_c[b, o_next] and cp[b] == o_next
            assert path[b, :pl[b] + 1].tolist() == list(range(pl[b] + 1))


def pin_tree_bruteforce(o):
    """Random trees (siblings commit distinct (position, token) pairs): the
    walk visits exactly the nodes whose every edge from the root equals the
    target's own commit at the edge's parent, in depth order, and commits the
    target's own at the deepest of them."""
    r = np.random.default_rng(121)
    for trial in range(300):
        N, V, P = int(r.integers(1, 10)), int(r.integers(2, 4)), 3
        parent = [-1] + [int(r.integers(0, n)) for n in range(1, N)]
        used = {}
        pos, tok = [-1] * N, [-1] * N
        for n in range(1, N):
            while True:
                pv = (int(r.integers(0, P)), int(r.integers(0, V)))
                if pv not in used.setdefault(parent[n], set()):
                    used[parent[n]].add(pv)
                    break
            pos[n], tok[n] = pv
        tpos = [int(r.integers(0, P)) for _ in range(N)]
        T = float(r.choice([0.0, 0.7]))
        lt = r.normal(0, 1, (1, N, V)).astype(np.float32)
        gum = (-np.log(-np.log(r.random((1, N, V))))).astype(np.float32)
        pl, path, cp, ct, tt = o.tree_verify(lt, gum, np.array([parent]), np.array([pos]), np.array([tok]),
                                             np.array([tpos]), T)
        own = [o.coupled_choice(lt[0, n], gum[0, n], T) for n in range(N)]
        ok = [False] * N
        ok[0] = True
        for n in range(1, N):                  # parents come first
            p = parent[n]
            ok[n] = ok[p] and pos[n] == tpos[p] and tok[n] == own[p]
        chain = [n for n in range(N) if ok[n]]
        assert path[0, :pl[0] + 1].tolist() == chain, (trial, chain, path[0])
        last = chain[-1]
        assert cp[0] == tpos[last] and ct[0] == own[last] and tt[0].tolist() == own


def pin_tree_rejects_bad_parent(o):
    bad = np.array([[-1, 0, 3, 1]], np.int32)   # node 2's parent comes after it
    z = np.zeros((1, 4), np.int32)
    try:
        o.tree_verify(np.zeros((1, 4, 3), np.float32), None, bad, z, z, z, 0.0)
    except oracle_error():
        return
    raise AssertionError("a parent after its child was accepted")


def oracle_error():
    import oracle
    return oracle.OracleError


def all_tree_pins(o):
    pin_tree_golden(o)
    pin_tree_chain_is_coupled(o)
    pin_tree_bruteforce(o)
    pin_tree_rejects_bad_parent(o)


# ---------------------------------------------------------------- trees of block states
def _frac(x):
    if isinstance(x, str):
        a, b = x.split("/")
        return int(a) / int(b)
    return float(x)


def pin_states_golden(o):
    """The hand-worked fixture: confidences, per-node commits, walk and next
    state at T = 0 (one-commit and threshold decoders) and at T = 1, and the
    strict threshold comparison."""
    g = json.load(open(os.path.join(GOLDEN, "tree_states_tiny.json")))
    w = np.array(g["weights"], np.float64)
    lt = np.log(w).astype(np.float32)[None]
    noise = np.array(g["noise"], np.float32)[None]
    parent, state = np.array([g["parent"]], np.int32), np.array([g["state"]], np.int32)
    conf_ref = np.array([[_frac(x) for x in row] for row in g["conf"]])
    for c in g["cases"]:
        pl, path, ns, commit, conf = o.tree_states(lt, noise, parent, state, c["temperature"], c["threshold"])
        assert int(pl[0]) == c["path_len"] and path[0].tolist() == c["path"], (c, pl, path)
        assert ns[0].tolist() == c["next_state"], (c, ns)
        assert commit[0].tolist() == c["commit"], (c, commit)
        assert np.allclose(conf[0], conf_ref, rtol=1e-6, atol=0), (conf[0], conf_ref)
    s = g["strict"]
    for c in s["cases"]:
        commit, conf, n = o.transition(np.array(s["logits"], np.float32), None, np.array(s["state"]), 0.0,
                                       c["threshold"])
        assert commit.tolist() == c["commit"], (c, commit, conf)
        assert n == sum(t >= 0 for t in c["commit"])


def pin_confidence_closed_forms(o):
    """max_v softmax(l)_v: 1/V for a constant row; 1 when one entry is finite
    and the rest -inf; unchanged by a constant shift of the row (also a large
    one); equal to the largest probability of a softmax summed exactly."""
    import math
    r = np.random.default_rng(130)
    for V in (1, 2, 7, 1000):
        assert abs(o.confidence(np.full(V, 3.25, np.float32)) - 1.0 / V) <= 1e-15
        row = np.full(V, -np.inf, np.float32)
        row[V // 2] = 0.5
        assert o.confidence(row) == 1.0
    for _ in range(30):
        V = int(r.integers(2, 300))
        l = (r.standard_normal(V) * r.choice([0.5, 3.0, 20.0])).astype(np.float32)
        e = [math.exp(float(x) - float(l.max())) for x in l]
        ref = max(e) / math.fsum(e)
        c = o.confidence(l)
        assert abs(c - ref) <= 1e-13 * ref, (c, ref)
        for shift in (1000.0, -1000.0, 37.0):   # exact in float32 for these rows
            ls = (l.astype(np.float64) + shift).astype(np.float32)
            if np.array_equal(ls.astype(np.float64) - shift, l.astype(np.float64)):
                assert abs(o.confidence(ls) - c) <= 1e-12 * c


def _check_transition_rule(commit, conf, state, lt, gum, T, threshold, o):
    L = state.shape[0]
    masked = [s for s in range(L) if state[s] < 0]
    assert all(commit[s] == -1 and conf[s] == -1.0 for s in range(L) if state[s] >= 0)
    if not masked:
        assert (commit == -1).all()
        return
    above = [s for s in masked if conf[s] > np.float64(np.float32(threshold))]
    if above:
        chosen = above
    else:
        top = max(conf[s] for s in masked)
        chosen = [min(s for s in masked if conf[s] == top)]
    assert sorted(s for s in range(L) if commit[s] >= 0) == chosen, (chosen, commit, conf)
    for s in chosen:
        assert commit[s] == o.coupled_choice(lt[s], gum[s] if T > 0 else None, T)


def pin_transition_rule(o):
    """Random states (several identical rows to make exact ties): decided
    slots are never committed; the committed set is every masked slot above
    the threshold, or else the first masked slot of highest confidence, each
    with the target's own (coupled) token; a threshold of 1 or more commits
    exactly one slot, a negative one every masked slot; the confidences
    agree with an exactly summed softmax."""
    import math
    r = np.random.default_rng(131)
    for trial in range(400):
        L, V = int(r.integers(1, 7)), int(r.integers(1, 6))
        lt = (r.standard_normal((L, V)) * r.choice([0.3, 2.0, 6.0])).astype(np.float32)
        for s in range(1, L):
            if r.random() < 0.3:
                lt[s] = lt[int(r.integers(0, s))]
        gum = (-np.log(-np.log(r.random((L, V))))).astype(np.float32)
        state = np.where(r.random(L) < 0.4, r.integers(0, V, L), -1).astype(np.int32)
        T = float(r.choice([0.0, 1.0, 0.6]))
        threshold = float(r.choice([1.0, 1.5, 0.5, 0.3, 0.9, -0.1]))
        commit, conf, n = o.transition(lt, gum, state, T, threshold)
        _check_transition_rule(commit, conf, state, lt, gum, T, threshold, o)
        masked = int((state < 0).sum())
        assert n == int((commit >= 0).sum())
        if threshold >= 1.0:
            assert n == min(1, masked)
        if threshold < 0:
            assert n == masked
        for s in range(L):
            if state[s] < 0:
                e = [math.exp(float(x) - float(lt[s].max())) for x in lt[s]]
                assert abs(conf[s] - max(e) / math.fsum(e)) <= 1e-13


def pin_state_walk_bruteforce(o):
    """Random trees and commits: the walk visits exactly the nodes whose every
    edge from the root equals its parent with the parent's commit applied,
    never leaving a node without masked slots -- the smallest index where
    siblings are equal -- and applies the last node's commit."""
    r = np.random.default_rng(132)
    for trial in range(400):
        N, L, V = int(r.integers(1, 9)), int(r.integers(1, 5)), int(r.integers(1, 4))
        st = [np.where(r.random(L) < 0.3, r.integers(0, V, L), -1).astype(np.int32)]
        par, commits = [-1], []
        for n in range(N):
            y = st[n]
            masked = np.flatnonzero(y < 0)
            c = np.full(L, -1, np.int32)
            if len(masked):                    # any nonempty set of masked slots
                k = int(r.integers(1, len(masked) + 1))
                c[r.choice(masked, k, replace=False)] = r.integers(0, V, k)
            commits.append(c)
            if n + 1 < N:                      # the next node: a child of an earlier one
                p = int(r.integers(0, n + 1))
                yp = st[p]
                if r.random() < 0.6:           # its parent plus the parent's commit
                    z = np.where(commits[p] >= 0, commits[p], yp)
                else:                          # a random commit, or none at all
                    z = yp.copy()
                    mp = np.flatnonzero(yp < 0)
                    if len(mp) and r.random() < 0.9:
                        z[r.choice(mp)] = int(r.integers(0, V))
                st.append(z.astype(np.int32))
                par.append(p)
        S, C = np.stack(st), np.stack(commits)
        pl, path, ns = o.state_walk(np.array([par], np.int32), S[None], C[None])
        ok = [True] + [False] * (N - 1)
        for n in range(1, N):
            p = par[n]
            applied = np.where(C[p] >= 0, C[p], S[p])
            ok[n] = ok[p] and bool((S[p] < 0).any()) and np.array_equal(S[n], applied)
        walk, cur = [0], 0
        while True:
            kids = [n for n in range(1, N) if par[n] == cur and ok[n]]
            if not kids:
                break
            cur = kids[0]
            walk.append(cur)
        assert path[0, :pl[0] + 1].tolist() == walk and (path[0, pl[0] + 1:] == -1).all(), (trial, walk, path)
        assert ns[0].tolist() == np.where(C[cur] >= 0, C[cur], S[cur]).tolist()


def pin_states_one_commit_is_tree_verify(o):
    """With the one-commit decoder every edge is one (position, token) commit:
    trees of states verify exactly as the (separately pinned) draft-tree
    verification given each node's commit position and its row there."""
    r = np.random.default_rng(133)
    compared = 0
    for trial in range(150):
        N, L, V = int(r.integers(2, 9)), int(r.integers(2, 6)), int(r.integers(2, 5))
        T = float(r.choice([0.0, 0.8]))
        lt = (r.standard_normal((N, L, V)) * 2).astype(np.float32)
        gum = (-np.log(-np.log(r.random((L, V))))).astype(np.float32)
        root = np.where(r.random(L) < 0.3, r.integers(0, V, L), -1).astype(np.int32)
        root[int(r.integers(0, L))] = -1
        states, parent, commits = [root], [-1], []
        for n in range(N):
            commits.append(o.transition(lt[n], gum, states[n], T, 1.0)[0])
            if n + 1 == N:
                break
            open_nodes = [p for p in range(n + 1) if (states[p] < 0).sum() >= 2]
            if not open_nodes:                 # every child must keep a masked slot
                break
            p = int(r.choice(open_nodes))
            y = states[p]
            if r.random() < 0.6:
                z = np.where(commits[p] >= 0, commits[p], y)
            else:
                z = y.copy()
                z[r.choice(np.flatnonzero(y < 0))] = int(r.integers(0, V))
            parent.append(p)
            states.append(z.astype(np.int32))
        N = len(states)
        S = np.stack(states)
        pl, path, ns, commit, conf = o.tree_states(lt[None, :N], gum[None], np.array([parent]), S[None], T, 1.0)
        node_pos, node_tok = np.full(N, -1, np.int32), np.full(N, -1, np.int32)
        for n in range(1, N):
            d = np.flatnonzero(S[n] != S[parent[n]])
            node_pos[n], node_tok[n] = d[0], S[n, d[0]]
        tpos = np.array([int(np.flatnonzero(commit[0, n] >= 0)[0]) for n in range(N)], np.int32)
        rows = np.stack([lt[n, tpos[n]] for n in range(N)])[None]
        grow = np.stack([gum[tpos[n]] for n in range(N)])[None]
        pl2, path2, cp2, ct2, tt2 = o.tree_verify(rows, grow if T > 0 else None, np.array([parent]),
                                                  node_pos[None], node_tok[None], tpos[None], T)
        assert pl[0] == pl2[0] and np.array_equal(path, path2), (trial, path, path2)
        assert ns[0, cp2[0]] == ct2[0] and commit[0, path[0, pl[0]], cp2[0]] == ct2[0]
        assert (commit[0] >= 0).sum(axis=1).tolist() == [1] * N
        compared += 1
    assert compared == 150


def pin_states_reject_bad_parent(o):
    try:
        o.tree_states(np.zeros((1, 3, 2, 2), np.float32), None, np.array([[-1, 2, 0]]),
                      np.full((1, 3, 2), -1), 0.0)
    except oracle_error():
        return
    raise AssertionError("a parent after its child was accepted")


def all_states_pins(o):
    pin_states_golden(o)
    pin_confidence_closed_forms(o)
    pin_transition_rule(o)
    pin_state_walk_bruteforce(o)
    pin_states_one_commit_is_tree_verify(o)
    pin_states_reject_bad_parent(o)
