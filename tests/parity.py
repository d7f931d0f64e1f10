"""Comparison rules between the HIP path and the CPU oracle.

Tolerances of the verification step's parity bar:
  attention, float32 inputs: max |gpu - oracle| <= 1e-5
  attention, bf16 inputs:    max |gpu - oracle| <= 2e-2 and
                             ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2
  accepted prefix lengths and resampled tokens: identical, except where the
  decision is a tie: |u - alpha| < 1e-6 for an acceptance test, or u * Z
  within 1e-6 * Z of a running-sum boundary for the resample; ties are
  counted and returned.
  trees of block states: every masked slot's confidence within 1e-5
  relative of the oracle's float64 value (the GPU sums float32 exponentials
  into a float64 normaliser: a few 1e-6 relative at most); committed tokens
  identical; each node's commit set identical unless a decision is within
  that band (a confidence within 1e-5 of the threshold, or the two highest
  within 1e-5 of each other when none exceeds it): such a node is a counted
  tie, its GPU commit set must satisfy the rule within the band, and the
  walk is then checked against the oracle's walk over the GPU's commits.
"""
from __future__ import annotations

import numpy as np

TIE = 1e-6

# running totals over the session (reported at the end of the test run)
TOTALS = {"sequences": 0, "ties": 0, "tree_sequences": 0, "tree_ties": 0}
CONF_TIE = 1e-5


def attn_errors(gpu: np.ndarray, ref: np.ndarray):
    d = gpu.astype(np.float64) - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def check_attn(gpu, ref, dtype: str, what=""):
    mx, rel = attn_errors(gpu, ref)
    if dtype == "f32":
        assert mx <= 1e-5, f"{what}: max abs {mx:.3e} > 1e-5"
    else:
        assert mx <= 2e-2, f"{what}: max abs {mx:.3e} > 2e-2"
        assert rel <= 1e-2, f"{what}: relative RMS {rel:.3e} > 1e-2"
    return mx, rel


def check_accept(o, inp, gamma, L_g, tok_g, alpha_g, seqs=None, temperature=1.0):
    """Compare GPU acceptance outputs with the oracle on sequences `seqs`
    (indices into the batch), at `temperature`.  Returns the number of
    counted ties."""
    n = inp["tau"].shape[0]
    seqs = range(n) if seqs is None else seqs
    seqs = list(seqs)
    lt = inp["target_logits"][seqs]
    pd = inp["draft_probs"][seqs]
    toks = inp["draft_tokens"][seqs]
    tau = inp["tau"][seqs]
    u = inp["uniforms"][seqs]
    L_o, tok_o, al_o, rs_o = o.accept(lt, pd, toks, tau, u, gamma, temperature)
    if temperature != 1.0:   # the tempered rows the oracle's resample used
        lt = lt * (np.float32(1.0) / np.float32(temperature))
    ties = 0
    for i, b in enumerate(seqs):
        # alpha of every step: float32 output of a float64 value
        assert np.abs(alpha_g[b] - al_o[i]).max() <= 2e-6 + 1e-6 * 0, (b, alpha_g[b], al_o[i])
        lg, lo = int(L_g[b]), int(L_o[i])
        if lg != lo:
            r = min(lg, lo)
            assert abs(float(u[i, r]) - al_o[i, r]) < TIE, f"seq {b}: accept_len {lg} vs oracle {lo}"
            ties += 1
            continue
        if not np.array_equal(tok_g[b], tok_o[i]):
            diff = np.nonzero(tok_g[b] != tok_o[i])[0]
            slot = int(rs_o[i])
            assert diff.tolist() == [slot], f"seq {b}: tokens differ at {diff.tolist()} (resample slot {slot})"
            v = int(tok_g[b, slot])
            _, cdf, Z, _ = o.residual(lt[i, slot], pd[i, slot], float(u[i, gamma]))
            thr = float(u[i, gamma]) * Z
            lo_b = cdf[v - 1] if v > 0 else 0.0
            assert lo_b - TIE * Z <= thr <= cdf[v] + TIE * Z, f"seq {b}: resampled {v} is not a tie"
            ties += 1
    TOTALS["sequences"] += len(seqs)
    TOTALS["ties"] += ties
    return ties


def _valid_commit_set(taken, conf, masked, threshold):
    """The GPU's commit set of one node obeys the threshold rule within the
    confidence band (conf: the oracle's float64 values)."""
    thr = float(np.float32(threshold))
    near = {s for s in masked if abs(conf[s] - thr) <= CONF_TIE * max(conf[s], abs(thr))}
    above = {s for s in masked if conf[s] > thr and s not in near}
    t = set(taken)
    if not masked:
        return not t
    if t and above <= t <= above | near:         # the threshold branch
        return True
    if not above and len(t) == 1:                 # the fallback: (one of) the highest
        top = max(conf[s] for s in masked)
        return conf[taken[0]] >= top * (1 - CONF_TIE)
    return False


def check_states(o, inp, T, threshold, pl_g, path_g, ns_g, commit_g, conf_g, seqs=None, count=True):
    """Compare the GPU's verification of trees of block states with the
    oracle on sequences `seqs`.  Returns the number of counted ties."""
    n = inp["st_parent"].shape[0]
    seqs = list(range(n) if seqs is None else seqs)
    lt, par, st = inp["st_logits"][seqs], inp["st_parent"][seqs], inp["st_state"][seqs]
    gum = inp["st_gumbel"][seqs] if T > 0 else None
    pl_o, path_o, ns_o, commit_o, conf_o = o.tree_states(lt, gum, par, st, T, threshold)
    ties = 0
    for i, b in enumerate(seqs):
        N, L = st[i].shape
        tied = False
        for k in range(N):
            masked = [s for s in range(L) if st[i, k, s] < 0]
            dec = [s for s in range(L) if st[i, k, s] >= 0]
            assert (conf_g[b, k, dec] == -1).all() and (commit_g[b, k, dec] == -1).all(), (b, k)
            if masked:
                err = np.abs(conf_g[b, k, masked].astype(np.float64) - conf_o[i, k, masked])
                assert (err <= CONF_TIE * conf_o[i, k, masked] + 1e-30).all(), \
                    (b, k, conf_g[b, k, masked], conf_o[i, k, masked])
            both = (commit_g[b, k] >= 0) & (commit_o[i, k] >= 0)
            assert np.array_equal(commit_g[b, k, both], commit_o[i, k, both]), (b, k, "committed tokens differ")
            if not np.array_equal(commit_g[b, k] >= 0, commit_o[i, k] >= 0):
                taken = [s for s in range(L) if commit_g[b, k, s] >= 0]
                assert _valid_commit_set(taken, conf_o[i, k], masked, threshold), \
                    (b, k, taken, np.flatnonzero(commit_o[i, k] >= 0), conf_o[i, k])
                for s in taken:   # tokens of slots only the GPU committed: the oracle's choice there
                    row = lt[i, k, s]
                    assert commit_g[b, k, s] == o.coupled_choice(row, gum[i, s] if T > 0 else None, T)
                tied = True
        if tied:
            ties += 1
            pl_w, path_w, ns_w = o.state_walk(par[i:i + 1], st[i:i + 1], commit_g[b:b + 1])
            ref = (pl_w[0], path_w[0], ns_w[0])
        else:
            ref = (pl_o[i], path_o[i], ns_o[i])
        assert int(pl_g[b]) == int(ref[0]) and np.array_equal(path_g[b], ref[1]), (b, pl_g[b], path_g[b], ref)
        assert np.array_equal(ns_g[b], ref[2]), (b, ns_g[b], ref[2])
    if count:
        TOTALS["tree_sequences"] += len(seqs)
        TOTALS["tree_ties"] += ties
    return ties
