"""The library's calls under HIP graph capture: they allocate nothing, set no
memory with memset and never synchronise, so a step captured once replays
correctly.  Each replay is checked against the eager result, with eager work
(the outputs overwritten) and a synchronisation between replays."""
import numpy as np
import pytest

from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _graph_check(buf, step, outputs, restore=None, replays=4):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm up on a side stream, as capture requires
        if restore:
            restore()
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    if restore:
        restore()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    g = torch.cuda.CUDAGraph()
    if restore:
        restore()
    with torch.cuda.graph(g):
        step()
    for k in range(replays):
        for t in outputs:        # eager work between replays: clobber the outputs
            t.fill_(-7 if t.dtype in (torch.int32, torch.int64) else 3.0)
        if restore:
            restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs, ref):
            assert torch.equal(t, r), f"replay {k} differs"
    print(f"[result] {replays} replays equal the eager step", flush=True)


def test_graph_headline_step():
    print("[case] graph: small workload, attention + accept", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = synth.config_by_name("small")
    buf = StepBuffers(case, synth.make_inputs(case))
    _graph_check(buf, lambda: (buf.attn(), buf.accept()), [buf.out, buf.accept_len, buf.out_tokens, buf.alpha])


def test_graph_coupled_and_route():
    print("[case] graph: shared-noise verification + routing estimate", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = synth.config_by_name("small")
    inp = synth.make_inputs(case, parts=("attn", "accept", "coupled"))
    buf = StepBuffers(case, inp, parts=("attn", "accept", "coupled", "route"))
    _graph_check(buf, lambda: (buf.route("entropy", 1.0), buf.accept_coupled(temperature=1.0)),
                 [buf.khat, buf.alpha_hat, buf.cpl_accept_len, buf.cpl_out_tokens, buf.cpl_target_tokens])


def test_graph_paged_commit_append():
    print("[case] graph: paged attention, accept, commit, append", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = synth.config_by_name("small").with_(page_size=64, ragged=True)
    inp = synth.make_inputs(case, parts=("attn", "accept", "paged"))
    buf = StepBuffers(case, inp, parts=("attn", "accept", "paged"))
    k0, v0 = buf.k_pages.clone(), buf.v_pages.clone()

    def restore():
        buf.prefix_lens.copy_(buf.prefix_lens0)
        buf.block_tokens.copy_(buf.block_tokens0)
        buf.k_pages.copy_(k0)
        buf.v_pages.copy_(v0)

    def step():
        buf.attn_paged()
        buf.accept()
        buf.commit(buf.out_tokens)
        buf.kv_append(buf.k_new, buf.v_new, 2 * case.block)

    _graph_check(buf, step, [buf.out_paged, buf.accept_len, buf.out_tokens, buf.block_tokens, buf.prefix_lens,
                             buf.remaining, buf.state, buf.n_append], restore=restore)


def test_graph_copies_and_tree():
    print("[case] graph: multi-copy attention + draft-tree verification", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = synth.config_by_name("small").with_(n_copies=9, gamma=8, temperature=1.0)
    inp = synth.make_inputs(case, parts=("copies", "tree"))
    buf = StepBuffers(case, inp, parts=("copies", "tree"))
    _graph_check(buf, lambda: (buf.attn_copies(), buf.tree(temperature=1.0)),
                 [buf.out_c, buf.path_len, buf.path, buf.commit_pos, buf.commit_tok, buf.tree_target_tok])


def test_graph_tree_states():
    print("[case] graph: multi-copy attention + verification of a tree of block states", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    for T, thr in ((1.0, 1.0), (0.0, 0.9)):
        case = synth.config_by_name("small").with_(n_copies=5, gamma=4, temperature=T, threshold=thr, vocab=20000)
        inp = synth.make_inputs(case, parts=("copies", "states"))
        buf = StepBuffers(case, inp, parts=("copies", "states"))
        _graph_check(buf, lambda: (buf.attn_copies(), buf.tree_states()),
                     [buf.out_c, buf.st_path_len, buf.st_path, buf.st_next, buf.st_commit, buf.st_conf])


def test_graph_paged_step_with_restore():
    """The benchmark's paged step as one graph: the commit and append, then
    the two device copies that restore the prompt lengths and the block."""
    print("[case] graph: paged step with the restoring copies inside the graph", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = synth.config_by_name("small").with_(page_size=64, ragged=True)
    inp = synth.make_inputs(case, parts=("attn", "accept", "paged"))
    buf = StepBuffers(case, inp, parts=("attn", "accept", "paged"))

    def step():
        buf.attn_paged()
        buf.accept()
        buf.commit(buf.out_tokens)
        buf.kv_append(buf.k_new, buf.v_new, 2 * case.block)
        buf.prefix_lens.copy_(buf.prefix_lens0)
        buf.block_tokens.copy_(buf.block_tokens0)

    def restore():   # the clobbered state back before each replay; the graph's own copies restore it after
        buf.prefix_lens.copy_(buf.prefix_lens0)
        buf.block_tokens.copy_(buf.block_tokens0)

    # after a replay the block and the prompt lengths must hold the restored
    # values (the in-graph copies ran after the commit and the append)
    _graph_check(buf, step, [buf.out_paged, buf.accept_len, buf.out_tokens, buf.block_tokens, buf.prefix_lens,
                             buf.remaining, buf.state, buf.n_append], restore=restore)
