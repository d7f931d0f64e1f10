"""Rejection-sampling verification at temperature T: the HIP path
(spec_verify_accept_temperature) against the CPU oracle through the C-ABI on
the same seeded inputs.  Acceptance lengths and tokens bit-exact outside the
counted ties, alpha within 2e-6; T = 1 reproduces spec_verify_accept
exactly."""
import numpy as np
import pytest

import oracle
import parity
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def run(case, inp, T):
    print(f"[case] tempered accept {case.name} batch={case.batch} B={case.block} gamma={case.gamma} "
          f"V={case.vocab} T={T}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    buf = StepBuffers(case, inp, parts=("accept",))
    buf.accept(temperature=T)
    torch.cuda.synchronize()
    return (buf.accept_len.cpu().numpy(), buf.out_tokens.cpu().numpy(), buf.alpha.cpu().numpy())


@pytest.mark.parametrize("T", [0.5, 0.8, 2.0])
def test_small_workload(o, T):
    case = synth.config_by_name("small")
    inp = synth.make_inputs(case, parts=("accept",))
    L, tok, al = run(case, inp, T)
    ties = parity.check_accept(o, inp, case.gamma, L, tok, al, temperature=T)
    print(f"[result] ties {ties}, mean accept_len {L.mean():.2f}", flush=True)


@pytest.mark.parametrize("kw,T", [
    (dict(vocab=1001, batch=5), 1.5),             # scalar loads, ragged last chunk
    (dict(vocab=100000, batch=3, block=8, gamma=5), 0.6),
    (dict(vocab=4096, batch=4, block=64, gamma=64), 0.9),
])
def test_shapes(o, kw, T):
    case = synth.config_by_name("small").with_(**kw)
    inp = synth.make_inputs(case, parts=("accept",))
    L, tok, al = run(case, inp, T)
    parity.check_accept(o, inp, case.gamma, L, tok, al, temperature=T)


def test_headline_sampled(o):
    """The headline shape (batch 32, B = gamma = 32, vocab 151936) at T = 0.7,
    checked on sampled sequences."""
    case = synth.config_by_name("headline")
    inp = synth.make_inputs(case, parts=("accept",))
    L, tok, al = run(case, inp, 0.7)
    parity.check_accept(o, inp, case.gamma, L, tok, al, seqs=[0, 9, 17, 31], temperature=0.7)


def test_unit_temperature_is_the_plain_call():
    case = synth.config_by_name("small")
    inp = synth.make_inputs(case, parts=("accept",))
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    buf = StepBuffers(case, inp, parts=("accept",))
    buf.accept()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (buf.accept_len, buf.out_tokens, buf.alpha)]
    buf.accept(temperature=1.0)
    torch.cuda.synchronize()
    for t, r in zip((buf.accept_len, buf.out_tokens, buf.alpha), ref):
        assert torch.equal(t, r)
