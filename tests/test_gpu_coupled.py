"""Shared-noise (Gumbel-coupled) and greedy verification: the HIP path vs the
CPU oracle, through the C-ABI, on the same seeded inputs.

The target's choice at a slot is an argmax, decided on both sides in the same
float32 arithmetic (one fused multiply-add per entry with the float32
reciprocal of T, ties to the smallest index), so accept_len, out_tokens and
the per-slot target choices must be identical."""
import numpy as np
import pytest

import oracle
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

EDGE = synth.Case("coupled-edge", 6, 0, 8, 8, 4, 4, 64, 1000, "bf16", 1e6, "perturb", 3.0, 1.0, 0, seed=60)


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(case, inp, T):
    from diffusion_speculative_verification_amd.device import StepBuffers
    buf = StepBuffers(case, inp, parts=("coupled",))
    buf.accept_coupled(temperature=T)
    torch.cuda.synchronize()
    return (buf.cpl_accept_len.cpu().numpy(), buf.cpl_out_tokens.cpu().numpy(),
            buf.cpl_target_tokens.cpu().numpy())


def check(o, case, inp, T, seqs=None):
    print(f"[case] {case.name} T={T} batch={case.batch} B={case.block} gamma={case.gamma} V={case.vocab}",
          flush=True)
    _cuda()
    L, ot, tt = run(case, inp, T)
    idx = list(range(case.batch)) if seqs is None else list(seqs)
    Lo, oto, tto = o.accept_coupled(inp["target_logits"][idx], inp["gumbel"][idx] if T > 0 else None,
                                    inp["coupled_tokens"][idx], inp["tau"][idx], case.gamma, T)
    assert np.array_equal(tt[idx], tto), "target choices differ"
    assert np.array_equal(L[idx], Lo), (L[idx], Lo)
    assert np.array_equal(ot[idx], oto), "out_tokens differ"
    print(f"[result] {case.name} T={T}: mean accept_len {L[idx].mean():.2f} of {case.gamma}", flush=True)
    return L, ot, tt


@pytest.mark.parametrize("T", [1.0, 0.0, 0.6, 2.0])
def test_coupled_small(o, T):
    case = EDGE.with_(temperature=T)
    check(o, case, synth.make_inputs(case, parts=("coupled",)), T)


@pytest.mark.parametrize("name", ["small", "headline"])
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_coupled_workloads(o, name, T):
    """Full size, in the launch configuration the benchmark times; every
    sequence compared (the oracle's argmax is one pass over each row)."""
    case = synth.config_by_name(name).with_(temperature=T)
    check(o, case, synth.make_inputs(case, parts=("coupled",)), T)


@pytest.mark.parametrize("kw", [
    dict(vocab=1001),                      # scalar loads
    dict(vocab=1),                         # one token: the choice is 0
    dict(vocab=6151),                      # several vocab splits, ragged
    dict(gamma=5),                         # slots tau > gamma stay -1
    dict(batch=1, block=1, gamma=1),       # B = 1
    dict(vocab=100000, batch=2),           # vocab splits of uneven size
])
def test_coupled_edges(o, kw):
    for T in (1.0, 0.0):
        case = EDGE.with_(temperature=T, **kw)
        check(o, case, synth.make_inputs(case, parts=("coupled",)), T)


def test_coupled_ties(o):
    """Equal scores go to the smallest index on both sides: repeated maxima
    for the greedy choice, and equal logit + noise for the coupled one."""
    _cuda()
    case = EDGE.with_(vocab=4096)
    inp = synth.make_inputs(case, parts=("coupled",))
    r = np.random.default_rng(61)
    lt = np.round(inp["target_logits"] * 2) / 2  # few distinct values: many ties
    inp["target_logits"] = lt.astype(np.float32)
    check(o, case.with_(temperature=0.0), inp, 0.0)
    inp["gumbel"] = np.zeros_like(inp["gumbel"])    # T = 1 with zero noise: ties of the logits
    inp["gumbel"][:, :, r.integers(0, 4096, 50)] = np.float32(0.5)
    check(o, case.with_(temperature=1.0), inp, 1.0)


def test_coupled_all_accepted_and_all_rejected(o):
    _cuda()
    case = EDGE.with_(vocab=5000)
    inp = synth.make_inputs(case, parts=("coupled",))
    for T in (1.0, 0.0):
        _, _, tto = o.accept_coupled(inp["target_logits"], inp["gumbel"] if T > 0 else None,
                                     inp["coupled_tokens"], inp["tau"], case.gamma, T)
        inp["coupled_tokens"] = tto.astype(np.int32)          # drafts equal the target's choices
        L, _, _ = check(o, case, inp, T)
        assert (L == case.gamma).all()
        inp["coupled_tokens"] = ((tto + 1) % case.vocab).astype(np.int32)  # every draft differs
        L, ot, tt = check(o, case, inp, T)
        assert (L == 0).all()
        first = inp["tau"] == 1
        assert np.array_equal(ot[first], tt[first])           # the target's own choice is committed
