"""The benchmark's algorithmic figures (CPU only): the bytes and FLOPs that the
roofline fractions divide by, recomputed here per unit of work from the
shapes alone, and the command-line refusals that end the run before any GPU
work."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from diffusion_speculative_verification_amd import synth  # noqa: E402


def test_headline_attention_figures():
    c = synth.config_by_name("headline")
    # one (sequence, kv head): its prompt K and V, the 2B response K and V
    # rows, and the g * 2B query and output rows, bf16
    g = c.n_qh // c.n_kvh
    per_unit = 2 * (2 * c.prefix_len * c.head_dim + 2 * (2 * c.block) * c.head_dim
                    + 2 * g * (2 * c.block) * c.head_dim)
    assert per_unit == 1_212_416
    assert bench.attn_bytes(c) == per_unit * c.batch * c.n_kvh == 310_378_496
    # every response row of every query head meets P + B keys, QK^T and PV
    flops = c.batch * c.n_qh * (2 * c.block) * (c.prefix_len + c.block) * c.head_dim * 2 * 2
    assert bench.attn_flops(c) == flops
    assert abs(flops / 1e9 - 69.79) < 0.01


def test_headline_accept_figures():
    c = synth.config_by_name("headline")
    logits = 4 * c.batch * c.gamma * c.vocab
    assert logits == 622_329_856
    # every sequence rejecting: two float32 rows more per sequence
    full = bench.accept_bytes(c, c.batch)
    assert full - bench.accept_bytes(c, 0) == c.batch * 2 * 4 * c.vocab
    assert abs(full / 1e6 - 661.25) < 0.01
    # the roofline of the whole step at 8 TB/s
    step_us = (bench.attn_bytes(c) + full) / (bench.HBM_PEAK_GBS * 1e9) * 1e6
    assert abs(step_us - 121.45) < 0.05


def test_copies_and_coupled_figures():
    c = synth.config_by_name("headline").with_(n_copies=9, gamma=8)
    R = 9 * c.block
    # the multi-copy layout: C * B response rows instead of 2B
    assert bench.attn_bytes(c, copies=9) - bench.attn_bytes(c) == 2 * c.batch * (R - 2 * c.block) * (
        c.n_qh + c.n_kvh) * c.head_dim * 2
    assert bench.attn_flops(c, copies=9) == 4.0 * R * c.n_qh * c.head_dim * c.batch * (c.prefix_len + c.block)
    h = synth.config_by_name("headline")
    rows = 4.0 * h.batch * h.gamma * h.vocab
    assert bench.coupled_bytes(h, greedy=True) - rows == bench.coupled_bytes(h, greedy=False) - 2 * rows


def test_states_bytes_count_masked_rows():
    c = synth.config_by_name("headline").with_(n_copies=3, block=4, batch=2, vocab=10)
    state = np.array([[[-1, -1, 5, 6], [-1, 7, 5, 6], [3, 7, 5, 6]],
                      [[-1, -1, -1, -1], [2, -1, -1, -1], [2, 3, -1, -1]]])
    masked_rows = 2 + 1 + 0 + 4 + 3 + 2          # logits rows of masked slots
    noise_rows = 2 + 4                           # slots masked in at least one copy
    small = c.batch * (c.n_copies * (c.block + 2) * 4 + c.block * 4 + 4)
    assert bench.states_bytes(c, state, greedy=True) == 4 * 10 * masked_rows + small
    assert bench.states_bytes(c, state, greedy=False) == 4 * 10 * (masked_rows + noise_rows) + small


@pytest.mark.parametrize("argv,needle", [
    (["--gpus", "2"], "one GPU only"),
    (["--gpus", "8"], "one GPU only"),
])
def test_refusals_before_gpu_work(argv, needle):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert needle in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_attention_agreement():
    """The CPU leg's attention comparison: zero against the oracle's own rows,
    and the planted error's size when one element is moved."""
    import oracle
    c = synth.config_by_name("tiny")
    inp = synth.make_inputs(c, parts=("attn", "accept"))
    o = oracle.Oracle()
    ref = np.stack([o.attention(inp["q"][b], inp["k_new"][b], inp["v_new"][b], inp["k_cache"][b],
                                inp["v_cache"][b], inp["tau"][b], c.theta) for b in range(c.batch)])
    same = bench.cpu_baseline(c, inp, gpu_attn=ref.copy())
    assert same["attn_agreement"] == {"sequences": c.batch, "max_abs_err": 0.0, "rel_rms_err": 0.0}
    moved = ref.copy()
    moved[c.batch - 1, 3, 1, 2] += 0.25
    got = bench.cpu_baseline(c, inp, gpu_attn=moved)["attn_agreement"]
    assert abs(got["max_abs_err"] - 0.25) < 1e-12
    assert abs(got["rel_rms_err"] - 0.25 / np.linalg.norm(ref)) < 1e-12
    assert bench.cpu_baseline(c, inp)["attn_agreement"] is None
