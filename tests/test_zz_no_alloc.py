"""spec_verify_accept_noalloc (static device scratch, no workspace argument)
against spec_verify_accept (caller's workspace), through the C-ABI: two
calls in a row, the second with a smaller input, each compared with the
workspace call on the same inputs (the same kernels: identical outputs)."""
import numpy as np
import pytest

from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run_both(case, inp):
    from diffusion_speculative_verification_amd import binding as sv
    from diffusion_speculative_verification_amd.device import StepBuffers
    buf = StepBuffers(case, inp, parts=("accept",))
    buf.accept()
    c = case
    L = torch.full((c.batch,), -5, dtype=torch.int32, device="cuda")
    tok = torch.full((c.batch, c.block), -5, dtype=torch.int32, device="cuda")
    al = torch.full((c.batch, c.gamma), -5.0, dtype=torch.float32, device="cuda")
    assert buf.acc_ws_bytes <= sv.SCRATCH_BYTES
    sv.spec_verify_accept_noalloc(buf.target_logits, buf.draft_probs, buf.draft_tokens, buf.tau, buf.uniforms,
                                  c.batch, c.block, c.gamma, c.vocab, L, tok, al)
    torch.cuda.synchronize()
    return (buf.accept_len.cpu().numpy(), buf.out_tokens.cpu().numpy(), buf.alpha.cpu().numpy(),
            L.cpu().numpy(), tok.cpu().numpy(), al.cpu().numpy())


def test_noalloc_matches_workspace_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # the headline workload, then a smaller one (fewer sequences, slots and
    # vocabulary, a vocabulary that takes the scalar-load path): the second
    # call finds the first call's contents in the scratch buffer
    big = synth.config_by_name("headline")
    small = synth.Case("noalloc-small", 5, 64, 12, 8, 8, 2, 128, 30001, "bf16", 1e6, "perturb", 3.0, 1.0, 0,
                       seed=71).with_(gamma=9)
    for case in (big, small):
        print(f"[case] noalloc {case.name} batch={case.batch} block={case.block} gamma={case.gamma} "
              f"vocab={case.vocab}", flush=True)
        inp = synth.make_inputs(case, parts=("accept",))
        L_w, tok_w, al_w, L_n, tok_n, al_n = _run_both(case, inp)
        assert np.array_equal(L_w, L_n), (L_w, L_n)
        assert np.array_equal(tok_w, tok_n)
        assert np.array_equal(al_w, al_n)
        assert (L_n < case.gamma).any() and (L_n >= 0).all()
        print(f"[result] noalloc {case.name}: identical (mean accept_len {L_n.mean():.2f})", flush=True)


def test_noalloc_rejects_sizes_beyond_scratch():
    """A shape whose scratch exceeds the static buffer is refused before any
    launch, and leaves the outputs untouched."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd import binding as sv
    batch, block, gamma, vocab = 1 << 12, 64, 64, 1 << 14   # 2^18 slots: ~8 MiB of partials
    assert sv.spec_verify_accept_workspace_size(batch, block, gamma, vocab) > sv.SCRATCH_BYTES
    dummy = torch.zeros(64, dtype=torch.int32, device="cuda")
    L = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    with pytest.raises(sv.SpecVerifyError) as e:
        # pointers are never dereferenced: the size check comes first
        sv.spec_verify_accept_noalloc(dummy, dummy, dummy, dummy, dummy, batch, block, gamma, vocab, L, dummy, None)
    assert e.value.status == sv.SV_E_SCRATCH
    torch.cuda.synchronize()
    assert (L.cpu().numpy() == 7).all()
