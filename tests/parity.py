"""Comparison rules between the HIP path and the CPU oracle.

Tolerances of the verification step's parity bar:
  attention, float32 inputs: max |gpu - oracle| <= 1e-5
  attention, bf16 inputs:    max |gpu - oracle| <= 2e-2 and
                             ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2
  accepted prefix lengths and resampled tokens: identical, except where the
  decision is a tie: |u - alpha| < 1e-6 for an acceptance test, or u * Z
  within 1e-6 * Z of a running-sum boundary for the resample; ties are
  counted and returned.
"""
from __future__ import annotations

import numpy as np

TIE = 1e-6

# running totals over the session (reported at the end of the test run)
TOTALS = {"sequences": 0, "ties": 0}


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
