"""Attention on random shapes (fixed seed): the paired layout with random step
labels (some sequences in identity order), block sizes 1 to 64, prompt
lengths that are and are not multiples of the 64-key tile, several GQA shapes
and head sizes; and the multi-copy layout with random copy counts.  Every
sequence is compared with the oracle to the bf16 tolerance.  The cases put
the first response key anywhere inside a tile, so the masked tile's 64-key
visibility window starts at every offset class, and they reach the largest
block (two 64-bit visibility words) and the 1024-row copy limit."""
import numpy as np
import pytest

import oracle
import parity
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GQA = [(4, 1), (8, 2), (32, 8), (16, 16), (64, 8)]


def _cases(n=45, seed=123):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 65))
        P = int(rng.choice([0, int(rng.integers(1, 200)), int(rng.integers(200, 1500))]))
        hq, hkv = GQA[int(rng.integers(0, len(GQA)))]
        d = int(rng.choice([64, 128]))
        batch = int(rng.integers(1, 4))
        if i % 3 == 2:
            C = int(rng.integers(1, max(2, min(32, 1024 // B)) + 1))
            out.append(synth.Case(f"random{i}", batch, P, B, B, hq, hkv, d, 64, "bf16", 1e6, "iid", 2.0, 2.0, 0,
                                  seed=9000 + i, n_copies=C))
        else:
            out.append(synth.Case(f"random{i}", batch, P, B, B, hq, hkv, d, 64, "bf16", 1e6, "iid", 2.0, 2.0,
                                  int(rng.choice([0, 1, 2])), seed=9000 + i, n_copies=0))
    # the two extremes of the window's word arithmetic: B = 64 and B = 1, the
    # response keys starting at the last key of a tile
    out.append(synth.Case("random-B64", 2, 63, 64, 64, 8, 2, 128, 64, "bf16", 1e6, "iid", 2.0, 2.0, 2, seed=9101,
                          n_copies=0))
    out.append(synth.Case("random-B1", 3, 127, 1, 1, 8, 2, 64, 64, "bf16", 1e6, "iid", 2.0, 2.0, 0, seed=9102,
                          n_copies=0))
    return out


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c.name)
def test_random_shape(o, case):
    copies = case.n_copies > 0
    print(f"[case] {case.name} {'copies C=' + str(case.n_copies) if copies else 'paired'} B={case.block} "
          f"P={case.prefix_len} heads={case.n_qh}/{case.n_kvh} d={case.head_dim} batch={case.batch}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    inp = synth.make_inputs(case, parts=("copies",) if copies else ("attn",))
    buf = StepBuffers(case, inp, parts=("copies",) if copies else ("attn",))
    if copies:
        buf.attn_copies()
    else:
        buf.attn()
    torch.cuda.synchronize()
    out = (buf.out_c if copies else buf.out).float().cpu().numpy()
    for b in range(case.batch):
        if copies:
            ref = o.attention_copies(inp["q_c"][b], inp["k_new_c"][b], inp["v_new_c"][b], inp["k_cache"][b],
                                     inp["v_cache"][b], case.n_copies, case.theta)
        else:
            ref = o.attention(inp["q"][b], inp["k_new"][b], inp["v_new"][b], inp["k_cache"][b], inp["v_cache"][b],
                              inp["tau"][b], case.theta)
        parity.check_attn(out[b], ref, "bf16", f"{case.name} seq {b}")
