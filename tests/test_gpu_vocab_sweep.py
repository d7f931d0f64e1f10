"""A seeded sweep of random shapes through the calls that stream a
vocabulary -- rejection sampling (at T = 1 and at another temperature),
shared-noise or greedy verification, the routing estimate (both estimators),
draft-tree verification and the verification of a tree of block states (the
target's own transition at one-commit and dynamic thresholds) -- against the
CPU oracle through the C-ABI:
batch, block, gamma, node counts and vocabulary sizes (multiples of 4 and
not, one vocabulary split and several) drawn within the documented limits.
Integer results must be identical (ties of the rejection sampler counted),
alpha within 2e-6, the entropy estimate within 1e-5."""
import numpy as np
import pytest

import oracle
import parity
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

VOCABS = [1, 3, 4, 17, 1000, 4097, 16384, 50001, 100000, 151936, 262144]


def _shapes(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        block = int(r.choice([1, 2, 5, 16, 33, 64]))
        vocab = VOCABS[i % len(VOCABS)]                   # every vocabulary size meets a random shape
        batch = int(r.integers(1, 6))
        while batch > 1 and batch * block * vocab > 12_000_000:  # keeps the oracle to seconds
            batch -= 1
        if batch * block * vocab > 12_000_000:
            block = max(1, 12_000_000 // vocab)
        # a draft tree of at most `block` nodes: every path has a free position
        # left for each later node
        out.append(dict(batch=batch, block=block, gamma=int(r.integers(1, block + 1)), vocab=vocab,
                        T=float(r.choice([0.5, 1.7, 0.0])), nodes=min(block, int(r.integers(1, 65))),
                        seed=500 + i))
    return out


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


# the largest vocabulary the calls accept (2^21: 1024 published half-chunk
# sums in the resample), and one below it on the scalar-load path
MAX_VOCAB = [dict(batch=2, block=3, gamma=3, vocab=1 << 21, T=0.8, nodes=3, seed=590),
             dict(batch=1, block=4, gamma=2, vocab=(1 << 21) - 1, T=0.0, nodes=4, seed=591)]


@pytest.mark.parametrize("sh", _shapes(22, 11) + MAX_VOCAB,
                         ids=lambda sh: f"b{sh['batch']}-B{sh['block']}-g{sh['gamma']}-V{sh['vocab']}-T{sh['T']}")
def test_vocab_sweep(o, sh):
    print(f"[case] {sh}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    T = sh["T"]
    case = synth.Case("vsweep", sh["batch"], 0, sh["block"], sh["gamma"], 4, 4, 64, sh["vocab"], "bf16", 1e6,
                      "perturb", 3.0, 1.0, 0, seed=sh["seed"], temperature=T, n_copies=sh["nodes"])
    inp = synth.make_inputs(case, parts=("accept", "coupled", "tree"))
    buf = StepBuffers(case, inp, parts=("accept", "coupled", "route", "tree"))
    idx = list(range(case.batch))

    # rejection sampling at T = 1, then at the case's temperature (T = 0 has no
    # rejection-sampling form: 1.3 stands in)
    Ta = T if T > 0 else 1.3
    for temp in (None, Ta):
        buf.accept(temperature=temp)
        torch.cuda.synchronize()
        parity.check_accept(o, inp, case.gamma, buf.accept_len.cpu().numpy(), buf.out_tokens.cpu().numpy(),
                            buf.alpha.cpu().numpy(), temperature=1.0 if temp is None else temp)

    # shared-noise (T > 0) or greedy (T = 0) verification
    buf.accept_coupled(temperature=T)
    torch.cuda.synchronize()
    Lo, oto, tto = o.accept_coupled(inp["target_logits"], inp["gumbel"] if T > 0 else None, inp["coupled_tokens"],
                                    inp["tau"], case.gamma, T)
    assert np.array_equal(buf.cpl_target_tokens.cpu().numpy(), tto), "target choices differ"
    assert np.array_equal(buf.cpl_accept_len.cpu().numpy(), Lo)
    assert np.array_equal(buf.cpl_out_tokens.cpu().numpy(), oto)

    # routing estimate, both estimators
    for est, param in (("margin", 0.05), ("entropy", 2.0)):
        buf.route(est, param)
        torch.cuda.synchronize()
        kh, ah = buf.khat.cpu().numpy(), buf.alpha_hat.cpu().numpy()
        kho, aho = o.route(inp["draft_probs"], inp["tau"], case.gamma, est, param)
        if est == "margin":
            assert np.array_equal(ah, aho.astype(np.float32)) and np.array_equal(kh, kho.astype(np.float32))
        else:
            assert np.abs(ah - aho).max() <= 1e-5 * np.abs(aho).max() + 1e-7
            assert (np.abs(kh - kho) <= 1e-5 * np.abs(kho) + 1e-6).all()

    # draft-tree verification over the case's nodes
    buf.tree(temperature=T)
    torch.cuda.synchronize()
    pl, path, cp, ct, tt = o.tree_verify(inp["tree_logits"], inp["tree_gumbel"] if T > 0 else None, inp["parent"],
                                         inp["node_pos"], inp["node_tok"], inp["target_pos"], T)
    assert np.array_equal(buf.tree_target_tok.cpu().numpy(), tt)
    assert np.array_equal(buf.path_len.cpu().numpy(), pl) and np.array_equal(buf.path.cpu().numpy(), path)
    assert np.array_equal(buf.commit_pos.cpu().numpy(), cp) and np.array_equal(buf.commit_tok.cpu().numpy(), ct)
    # a tree of block states: every masked slot of every copy streams the
    # vocabulary (node count capped to keep the logits within 160 MB)
    ns = max(1, min(sh["nodes"], 40_000_000 // (case.batch * case.block * case.vocab)))
    thr = float(np.random.default_rng(sh["seed"]).choice([1.0, 0.9, 0.5]))
    scase = case.with_(n_copies=ns, threshold=thr)
    sinp = synth.make_inputs(scase, parts=("states",))
    sbuf = StepBuffers(scase, sinp, parts=("states",))
    sbuf.tree_states(temperature=T, threshold=thr)
    torch.cuda.synchronize()
    g = [t.cpu().numpy() for t in (sbuf.st_path_len, sbuf.st_path, sbuf.st_next, sbuf.st_commit, sbuf.st_conf)]
    st_ties = parity.check_states(o, sinp, T, thr, *g)
    print(f"[result] ok: accept_len {buf.accept_len.cpu().numpy().tolist()[:6]}, "
          f"tree edges {pl.tolist()[:6]}, state-tree edges {g[0].tolist()[:6]} ({ns} nodes, threshold {thr}, "
          f"ties {st_ties})", flush=True)
