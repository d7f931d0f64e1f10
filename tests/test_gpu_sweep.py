"""A seeded sweep of shapes through the attention entry points (paired,
multi-copy, paged with ragged lengths) against the CPU oracle: block sizes,
prompt lengths, GQA group sizes, head dims, copy counts and page sizes drawn
within the documented limits, each compared element by element within the
bf16 tolerance."""
import numpy as np
import pytest

import oracle
import parity
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _shapes(n, seed):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(r.choice([1, 3, 8, 16, 24, 32, 48, 64]))
        g = int(r.choice([1, 2, 4, 8]))
        n_kvh = int(r.choice([1, 2]))
        d = int(r.choice([64, 128]))
        P = [0, 1, 63, 64, 65, 200, 777, 2100][(i * 3) % 8]   # every prompt length meets every layout
        C = int(r.integers(1, max(2, min(12, 1024 // B)) + 1))
        ps = int(r.choice([64, 128, 256]))
        layout = ["paired", "copies", "paged", "paged_copies"][i % 4]
        out.append(dict(B=B, g=g, n_kvh=n_kvh, d=d, P=P, C=C, ps=ps, layout=layout,
                        batch=int(r.integers(1, 4)), theta=float(r.choice([1e4, 1e6, 0.0])), seed=300 + i))
    return out


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


@pytest.mark.parametrize("sh", _shapes(24, 7), ids=lambda sh: f"{sh['layout']}-B{sh['B']}-P{sh['P']}-g{sh['g']}-d{sh['d']}")
def test_sweep(o, sh):
    print(f"[case] {sh}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    case = synth.Case("sweep", sh["batch"], sh["P"], sh["B"], sh["B"], sh["g"] * sh["n_kvh"], sh["n_kvh"], sh["d"],
                      64, "bf16", 1e6 if sh["theta"] == 0.0 else sh["theta"], "perturb", 3.0, 1.0, 0,
                      seed=sh["seed"], n_copies=sh["C"], page_size=sh["ps"], ragged=True)
    copies = sh["layout"] in ("copies", "paged_copies")
    paged = sh["layout"].startswith("paged")
    parts = (("copies",) if copies else ("attn",)) + (("paged",) if paged else ())
    inp = synth.make_inputs(case, parts=parts)
    buf = StepBuffers(case, inp, parts=parts)
    theta = sh["theta"]
    if paged:
        buf.attn_paged(n_copies=sh["C"] if copies else 0, rope_theta=theta)
        got = buf.out_paged
    elif copies:
        buf.attn_copies(rope_theta=theta)
        got = buf.out_c
    else:
        buf.attn(rope_theta=theta)
        got = buf.out
    torch.cuda.synchronize()
    got = got.float().cpu().numpy()
    q, kn, vn = (inp["q_c"], inp["k_new_c"], inp["v_new_c"]) if copies else (inp["q"], inp["k_new"], inp["v_new"])
    for b in range(case.batch):
        if paged:
            ref = o.attention_paged(q[b:b + 1], kn[b:b + 1], vn[b:b + 1], inp["k_pages"], inp["v_pages"],
                                    inp["block_table"][b:b + 1], inp["prefix_lens"][b:b + 1], inp["tau"][b:b + 1],
                                    case.page_size, theta, sh["C"] if copies else 0)[0]
        elif copies:
            ref = o.attention_copies(q[b], kn[b], vn[b], inp["k_cache"][b], inp["v_cache"][b], sh["C"], theta)
        else:
            ref = o.attention(q[b], kn[b], vn[b], inp["k_cache"][b], inp["v_cache"][b], inp["tau"][b], theta)
        parity.check_attn(got[b], ref, "bf16", f"sweep {sh} seq {b}")
    print(f"[result] ok", flush=True)
