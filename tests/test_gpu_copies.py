"""Multi-copy verification attention (the root and the draft states of the
block as copies, each bidirectional over its own block, the prompt shared):
the HIP path vs the CPU oracle, through the C-ABI, on the same seeded inputs.
Tolerances as for the paired-layout attention (bf16 inputs)."""
import numpy as np
import pytest

import oracle
import parity
from diffusion_speculative_verification_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BASE = synth.Case("copies", 2, 300, 16, 16, 8, 2, 128, 1000, "bf16", 1e6, "perturb", 3.0, 1.0, 0, seed=80,
                  n_copies=5)


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


def check(o, case, rope_theta=None, check_seqs=None):
    print(f"[case] {case.name} batch={case.batch} P={case.prefix_len} L={case.block} copies={case.n_copies} "
          f"heads={case.n_qh}/{case.n_kvh} d={case.head_dim}", flush=True)
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from diffusion_speculative_verification_amd.device import StepBuffers
    inp = synth.make_inputs(case, parts=("copies",))
    buf = StepBuffers(case, inp, parts=("copies",))
    buf.attn_copies(rope_theta=rope_theta)
    torch.cuda.synchronize()
    out = buf.out_c.float().cpu().numpy()
    th = case.theta if rope_theta is None else rope_theta
    worst = (0.0, 0.0)
    for i in (range(case.batch) if check_seqs is None else check_seqs):
        ref = o.attention_copies(inp["q_c"][i], inp["k_new_c"][i], inp["v_new_c"][i], inp["k_cache"][i],
                                 inp["v_cache"][i], case.n_copies, th)
        mx, rel = parity.check_attn(out[i], ref, case.dtype, f"{case.name} seq {i}")
        worst = (max(worst[0], mx), max(worst[1], rel))
    print(f"[result] {case.name}: max {worst[0]:.3e} relrms {worst[1]:.3e}", flush=True)


@pytest.mark.parametrize("kw", [
    dict(),                                    # 5 copies of 16: 80 response rows
    dict(n_copies=1),                          # the root alone: a plain block
    dict(block=32, n_copies=9, prefix_len=2048, n_qh=32, n_kvh=8, batch=2),   # SPOT budget D = 8 at the headline shape
    dict(block=32, n_copies=21, prefix_len=512),   # D = 20: 672 response rows
    dict(block=8, n_copies=4, prefix_len=0),   # no prompt
    dict(block=32, n_copies=32, prefix_len=100, n_qh=4, n_kvh=4),  # 1024 response rows (the limit)
    dict(head_dim=64, prefix_len=77),          # head_dim 64, ragged tail
    dict(batch=1, prefix_len=9000, n_qh=8, n_kvh=1, n_copies=3),   # prefix splits + combine
    dict(batch=2, block=64, n_copies=16, prefix_len=1000, n_qh=64, n_kvh=8),   # B = 64, 1024 rows, g = 8
    dict(block=24, n_copies=7, prefix_len=130),   # copies not aligned to 32-row waves or 64-key tiles
])
def test_copies(o, kw):
    check(o, BASE.with_(**kw))


def test_copies_pre_rotated(o):
    check(o, BASE.with_(prefix_len=40), rope_theta=0.0)


def test_copies_headline_d20_sampled(o):
    """The headline shape with the root and 20 draft states (672 response
    rows per sequence), batch 32; sampled sequences checked."""
    case = synth.config_by_name("headline").with_(n_copies=21)
    check(o, case, check_seqs=[5, 30])


def test_copies_headline_budget_sampled(o):
    """The headline shape with the root and 8 draft states, batch 32, in the
    launch configuration a benchmark would time; sampled sequences checked."""
    case = synth.config_by_name("headline").with_(n_copies=9)
    check(o, case, check_seqs=[0, 13, 31])
