"""Trees of block states ("SPOT", the target's own transition computed from
every copy's logits): the HIP path vs the CPU oracle through the C-ABI on
the same seeded trees.  Confidences within the band of parity.py, committed
tokens identical (an argmax taken in the same float32 arithmetic on both
sides), commit sets and walks identical outside counted ties."""
import numpy as np
import pytest

import oracle
import parity
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE = synth.Case("states", 6, 0, 32, 32, 4, 4, 64, 20000, "bf16", 1e6, "perturb", 3.0, 1.0, 0, seed=140,
                  n_copies=9)


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def run(o, case, inp, T, thr, check_seqs=None, gpu_inp=None):
    print(f"[case] states batch={case.batch} nodes={case.n_copies} block={case.block} V={case.vocab} T={T} "
          f"threshold={thr}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    buf = StepBuffers(case, gpu_inp if gpu_inp is not None else inp, parts=("states",))
    buf.tree_states(temperature=T, threshold=thr)
    torch.cuda.synchronize()
    g = [t.cpu().numpy() for t in (buf.st_path_len, buf.st_path, buf.st_next, buf.st_commit, buf.st_conf)]
    ties = parity.check_states(o, inp, T, thr, *g, seqs=check_seqs)
    print(f"[result] accepted edges {g[0].tolist()[:16]}, commits per node {float((g[3] >= 0).sum(2).mean()):.2f}, "
          f"ties {ties}", flush=True)
    return g


@pytest.mark.parametrize("T,thr", [(0.0, 1.0), (1.0, 1.0), (0.5, 1.0), (0.0, 0.9), (1.0, 0.9)])
@pytest.mark.parametrize("kw", [
    dict(),                                      # root + 8 draft states, 16-byte loads
    dict(n_copies=1),                            # the root alone
    dict(n_copies=64, block=64, batch=2),        # 64 nodes of 64 slots
    dict(vocab=1001),                            # scalar loads
    dict(vocab=1),                               # one token
    dict(block=5, n_copies=4, vocab=4099),       # ragged block, scalar loads, several splits
    dict(logit_model="iid"),                     # no planted peaks: close confidences
    dict(vocab=151936, batch=2, n_copies=21),    # D = 20
], ids=lambda kw: "-".join(f"{k}={v}" for k, v in kw.items()) or "base")
def test_states(o, kw, T, thr):
    case = BASE.with_(temperature=T, threshold=thr, **kw)
    run(o, case, synth.make_inputs(case, parts=("states",)), T, thr)


@pytest.mark.parametrize("T,thr", [(0.0, 1.0), (1.0, 1.0), (0.0, 0.9)])
def test_states_headline_shape(o, T, thr):
    """Batch 32, block 32, vocab 151936, the root and 8 draft states, as the
    benchmark's tree step runs it; every sequence checked."""
    case = synth.config_by_name("headline").with_(n_copies=9, temperature=T, threshold=thr)
    run(o, case, synth.make_inputs(case, parts=("states",)), T, thr)


def test_states_every_slot_committed(o):
    """A negative threshold commits every masked slot at every node; a
    root without masked slots ends the walk at once."""
    case = BASE.with_(threshold=-0.5)
    inp = synth.make_inputs(case, parts=("states",))
    g = run(o, case, inp, 0.0, -0.5)
    assert ((g[3] >= 0) == (inp["st_state"] < 0)).all()
    inp["st_state"][:, 0] = np.abs(inp["st_state"][:, 0])   # every root slot decided
    g = run(o, case, inp, 0.0, 1.0)
    assert (g[0] == 0).all() and np.array_equal(g[2], inp["st_state"][:, 0])


def test_states_masked_logits(o):
    """-inf logits have probability 0: a leading run of them on some rows,
    every 7th entry on others, and a row that is -inf everywhere
    (confidence 0, token 0 when committed)."""
    case = BASE.with_(vocab=20000, batch=4)
    inp = synth.make_inputs(case, parts=("states",))
    lt = inp["st_logits"]
    lt[:, :, ::2, :5000] = -np.inf
    lt[:, :, 1::2, ::7] = -np.inf
    lt[:, :, 3, :] = -np.inf
    for T in (0.0, 1.0):
        for thr in (1.0, 0.9):
            run(o, case, inp, T, thr)


def test_states_bad_parent_never_entered(o):
    """A node whose parent is not an earlier node is never entered (the call
    still ends): the same walk as a tree where that node cannot match."""
    case = BASE.with_(batch=4)
    inp = synth.make_inputs(case, parts=("states",))
    k = 3
    gpu_inp = dict(inp)
    gpu_inp["st_parent"] = inp["st_parent"].copy()
    gpu_inp["st_parent"][:, k] = k                  # its own index: not before it
    inp = dict(inp)
    inp["st_state"] = inp["st_state"].copy()
    inp["st_state"][:, k] = np.abs(inp["st_state"][:, k]) + 7   # decided everywhere, equal to no child of 0
    gpu_inp["st_state"] = inp["st_state"]
    inp["st_parent"] = inp["st_parent"].copy()
    inp["st_parent"][:, k] = 0
    g = run(o, case, inp, 0.0, 1.0, gpu_inp=gpu_inp)
    assert not (g[1] == k).any()


def test_states_repeat_bit_identical(o):
    """Two runs give identical bytes (no reduction races)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = BASE.with_(temperature=1.0, vocab=151936, batch=4)
    buf = StepBuffers(case, synth.make_inputs(case, parts=("states",)), parts=("states",))
    outs = []
    for _ in range(2):
        buf.tree_states()
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().copy() for t in (buf.st_path_len, buf.st_path, buf.st_next, buf.st_commit,
                                                       buf.st_conf)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_states_irregular_trees(o):
    """Trees the synthetic drafter never builds: a chain of 16 single commits
    from a fully masked root, each node its parent with the target's own
    commit applied, ending in a finished block; a child of that finished
    node identical to it (the walk stops at a finished block); a child equal
    to its parent (no commit: never an edge); and a sibling equal to a chain
    node but with a larger index (the smaller index is taken).  At threshold
    1 the walk must run the whole chain; at 0.5 it is checked against the
    oracle only."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    case = BASE.with_(batch=4, n_copies=20, block=16, vocab=3000, temperature=0.0)
    inp = synth.make_inputs(case, parts=("states",))
    st, par, lt = inp["st_state"], inp["st_parent"], inp["st_logits"]
    r = np.random.default_rng(77)

    def fresh_rows(b, n):   # N(0, 3) rows at the masked slots, NaN at the decided ones
        lt[b, n] = (r.standard_normal((case.block, case.vocab)) * np.sqrt(3.0)).astype(np.float32)
        lt[b, n][st[b, n] >= 0] = np.nan

    for b in range(case.batch):
        st[b, 0] = -1
        fresh_rows(b, 0)
        for n in range(1, 17):   # the chain 0 -> 1 -> ... -> 16
            par[b, n] = n - 1
            commit, _, _ = o.transition(lt[b, n - 1], None, st[b, n - 1], 0.0, 1.0)
            st[b, n] = np.where(commit >= 0, commit, st[b, n - 1])
            fresh_rows(b, n)
        assert (st[b, 16] >= 0).all()           # 16 commits fill the block
        par[b, 17], st[b, 17] = 16, st[b, 16]   # a finished node's identical child
        par[b, 18], st[b, 18] = 3, st[b, 3]     # a child equal to its parent
        par[b, 19], st[b, 19] = 15, st[b, 16]   # equal to node 16, a larger index
        for n in (17, 18, 19):
            fresh_rows(b, n)
    for thr in (1.0, 0.5):
        g = run(o, case, inp, 0.0, thr)
        if thr == 1.0:
            assert (g[0] == 16).all() and (g[1][:, :17] == np.arange(17)).all() and (g[1][:, 17:] == -1).all()
            assert np.array_equal(g[2], st[:, 16])
