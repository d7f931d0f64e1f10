"""The comparison rules of parity.py on the CPU: the oracle's own outputs
pass with no counted tie, and plausible GPU mistakes fail."""
import numpy as np
import pytest

import oracle
import parity
from diffusion_speculative_verification_amd import synth


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


@pytest.mark.parametrize("T,thr", [(0.0, 1.0), (1.0, 0.9)])
def test_states_rules(o, T, thr):
    case = synth.Case("rules", 4, 0, 8, 8, 4, 4, 64, 300, "f32", 1e6, "perturb", 3.0, 1.0, 0, seed=150,
                      n_copies=6, temperature=T, threshold=thr)
    inp = synth.make_inputs(case, parts=("states",))
    pl, path, ns, commit, conf = o.tree_states(inp["st_logits"], inp["st_gumbel"], inp["st_parent"],
                                               inp["st_state"], T, thr)
    good = (pl, path, ns, commit, conf.astype(np.float32))
    assert parity.check_states(o, inp, T, thr, *good, count=False) == 0

    def fails(**change):
        bad = dict(zip(("pl", "path", "ns", "commit", "conf"), [x.copy() for x in good]))
        for k, f in change.items():
            f(bad[k])
        with pytest.raises(AssertionError):
            parity.check_states(o, inp, T, thr, *bad.values(), count=False)

    b, k = 1, 0
    s = int(np.flatnonzero(commit[b, k] >= 0)[0])
    fails(commit=lambda c: c.__setitem__((b, k, s), c[b, k, s] + 1))           # another token
    fails(conf=lambda c: c.__setitem__((b, k, s), c[b, k, s] * (1 + 1e-3)))     # confidence off
    fails(pl=lambda x: x.__setitem__(b, x[b] + 1))                              # walk length
    fails(ns=lambda x: x.__setitem__((b, 0), x[b, 0] + 1))                      # next state
    other = [t for t in np.flatnonzero(inp["st_state"][b, k] < 0) if commit[b, k, t] < 0]
    if other:                                                                    # a far lower slot taken
        def swap(c):
            c[b, k, other[0]] = 0
        fails(commit=swap)
