"""S2D2's verify-routing estimator: the HIP path vs the CPU oracle, through
the C-ABI, on the same seeded draft distributions.

The margin estimator's alpha is a decision (a float64 difference of two
float32 entries against the threshold, exact on both sides), so K must be
identical; the entropy estimator's K is compared within 1e-5 relative (the
kernel takes log2 in hardware float32 and sums in float64)."""
import numpy as np
import pytest

import oracle
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

EDGE = synth.Case("route-edge", 5, 0, 8, 8, 4, 4, 64, 1000, "bf16", 1e6, "perturb", 3.0, 1.0, 0, seed=70)


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check(o, case, inp, estimator, param):
    print(f"[case] {case.name} {estimator}={param} batch={case.batch} B={case.block} gamma={case.gamma} "
          f"V={case.vocab}", flush=True)
    _cuda()
    from diffusion_speculative_verification_amd.device import StepBuffers
    buf = StepBuffers(case, inp, parts=("route",))
    buf.route(estimator, param)
    torch.cuda.synchronize()
    kh, ah = buf.khat.cpu().numpy(), buf.alpha_hat.cpu().numpy()
    kho, aho = o.route(inp["draft_probs"], inp["tau"], case.gamma, estimator, param)
    if estimator == "margin":
        assert np.array_equal(ah, aho.astype(np.float32))
        assert np.array_equal(kh, kho.astype(np.float32))
    else:
        assert np.abs(ah - aho).max() <= 1e-5 * np.abs(aho).max() + 1e-7, np.abs(ah - aho).max()
        assert (np.abs(kh - kho) <= 1e-5 * np.abs(kho) + 1e-6).all(), (kh, kho)
    print(f"[result] {case.name} {estimator}: mean K {kh.mean():.3f} of {case.gamma}", flush=True)
    return kh


@pytest.mark.parametrize("estimator,param", [("margin", 0.02), ("margin", 0.2), ("entropy", 1.0),
                                             ("entropy", 4.0)])
def test_route_small(o, estimator, param):
    check(o, EDGE, synth.make_inputs(EDGE, parts=("accept",)), estimator, param)


@pytest.mark.parametrize("name", ["small", "headline"])
def test_route_workloads(o, name):
    """Full size, every sequence (the oracle is one pass per draft row)."""
    case = synth.config_by_name(name)
    inp = synth.make_inputs(case, parts=("accept",))
    check(o, case, inp, "entropy", 2.0)
    check(o, case, inp, "margin", 1e-3)


@pytest.mark.parametrize("kw", [dict(vocab=1001), dict(vocab=1), dict(vocab=6151), dict(gamma=3),
                                dict(batch=1, block=1, gamma=1), dict(vocab=100000, batch=2)])
def test_route_edges(o, kw):
    case = EDGE.with_(**kw)
    inp = synth.make_inputs(case, parts=("accept",))
    check(o, case, inp, "entropy", 1.5)
    check(o, case, inp, "margin", 0.05)


def test_route_special_rows(o):
    """Uniform rows (normalised entropy 1), one-hot rows (margin 1, entropy
    0), rows with exact zeros and ties at the top (margin 0)."""
    _cuda()
    case = EDGE.with_(vocab=4096)
    inp = synth.make_inputs(case, parts=("accept",))
    p = inp["draft_probs"]
    p[0] = np.float32(1.0 / 4096)
    p[1] = 0.0
    p[1, :, 17] = 1.0
    p[2, :, :100] = 0.0
    p[3, :, 5] = p[3, :, 6] = p[3].max(axis=1)
    for est, prm in (("entropy", 1.0), ("margin", 1e-6), ("margin", 0.0)):
        check(o, case, inp, est, prm)
