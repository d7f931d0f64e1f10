"""Draft-tree verification ("SPOT"): the HIP path vs the CPU oracle through
the C-ABI on the same seeded trees.  The target's own token at each node is
an argmax decided in the same float32 arithmetic on both sides, so the walk,
the committed token and every node's target token must be identical."""
import numpy as np
import pytest

import oracle
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE = synth.Case("tree", 6, 0, 32, 32, 4, 4, 64, 1000, "bf16", 1e6, "perturb", 3.0, 1.0, 0, seed=130,
                  n_copies=9)


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def run(o, case, inp, T, check_seqs=None):
    print(f"[case] tree batch={case.batch} nodes={case.n_copies} V={case.vocab} T={T}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    buf = StepBuffers(case, inp, parts=("tree",))
    buf.tree(temperature=T)
    torch.cuda.synchronize()
    idx = list(range(case.batch)) if check_seqs is None else list(check_seqs)
    pl, path, cp, ct, tt = o.tree_verify(inp["tree_logits"][idx], inp["tree_gumbel"][idx] if T > 0 else None,
                                         inp["parent"][idx], inp["node_pos"][idx], inp["node_tok"][idx],
                                         inp["target_pos"][idx], T)
    assert np.array_equal(buf.tree_target_tok.cpu().numpy()[idx], tt), "target tokens differ"
    assert np.array_equal(buf.path_len.cpu().numpy()[idx], pl)
    assert np.array_equal(buf.path.cpu().numpy()[idx], path)
    assert np.array_equal(buf.commit_pos.cpu().numpy()[idx], cp)
    assert np.array_equal(buf.commit_tok.cpu().numpy()[idx], ct)
    print(f"[result] accepted edges {pl.tolist()[:12]}", flush=True)
    return pl


@pytest.mark.parametrize("T", [1.0, 0.0, 0.5])
@pytest.mark.parametrize("kw", [
    dict(),                                   # 9 nodes (root + 8 draft states)
    dict(n_copies=1),                         # the root alone: nothing to walk
    dict(n_copies=64, block=64, batch=3),     # 64 nodes: one wave's worth
    dict(vocab=1001),                         # scalar loads
    dict(vocab=100000, batch=2, n_copies=21), # several vocab splits, D = 20
])
def test_tree(o, kw, T):
    case = BASE.with_(temperature=T, **kw)
    run(o, case, synth.make_inputs(case, parts=("tree",)), T)


def test_tree_headline_shape(o):
    """Batch 32, vocab 151936, the root and 8 draft states, as the benchmark's
    tree step runs it; every sequence checked."""
    case = synth.config_by_name("headline").with_(n_copies=9, temperature=1.0)
    run(o, case, synth.make_inputs(case, parts=("tree",)), 1.0)


def test_tree_chain_matches_coupled(o):
    """A chain in draft order verified as a tree gives the shared-noise
    verification's accepted length on the GPU."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = synth.Case("chain", 8, 0, 16, 12, 4, 4, 64, 3000, "bf16", 1e6, "perturb", 3.0, 1.0, 0, seed=131,
                      temperature=1.0)
    inp = synth.make_inputs(case, parts=("coupled",))
    buf = StepBuffers(case, inp, parts=("coupled",))
    buf.accept_coupled(temperature=1.0)
    import pins
    rows = pins._chain_from_coupled(inp["target_logits"], inp["gumbel"], inp["coupled_tokens"], inp["tau"], case.gamma)
    tcase = case.with_(n_copies=case.gamma + 1)
    tinp = {"tau": inp["tau"], "tree_logits": rows[0], "tree_gumbel": rows[1], "parent": rows[2],
            "node_pos": rows[3], "node_tok": rows[4], "target_pos": rows[5]}
    tb = StepBuffers(tcase, tinp, parts=("tree",))
    tb.tree(temperature=1.0)
    torch.cuda.synchronize()
    assert np.array_equal(tb.path_len.cpu().numpy(), buf.cpl_accept_len.cpu().numpy())


def test_tree_malformed_parents_end():
    """Parents that point forward or form a cycle give some path but the
    call ends (a walk has at most n_nodes - 1 edges) and reads nothing
    outside its buffers."""
    print("[case] tree malformed parents", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = BASE.with_(batch=2, n_copies=6, temperature=0.0)
    inp = synth.make_inputs(case, parts=("tree",))
    inp["parent"][:] = np.array([[3, 0, 1, 2, 3, 4], [5, 2, 1, 0, 0, 1]], np.int32)
    # make every edge match the target so the walk runs as long as it can
    buf = StepBuffers(case, inp, parts=("tree",))
    buf.tree(temperature=0.0)
    torch.cuda.synchronize()
    tt = buf.tree_target_tok.cpu().numpy()
    inp["node_pos"][:] = inp["target_pos"][np.arange(2)[:, None], np.clip(inp["parent"], 0, 5)]
    inp["node_tok"][:] = tt[np.arange(2)[:, None], np.clip(inp["parent"], 0, 5)]
    buf = StepBuffers(case, inp, parts=("tree",))
    buf.tree(temperature=0.0)
    torch.cuda.synchronize()
    pl = buf.path_len.cpu().numpy()
    assert ((pl >= 0) & (pl <= case.n_copies - 1)).all(), pl
