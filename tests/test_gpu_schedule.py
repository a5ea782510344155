"""GPU tests of the per-layer schedule (skiparse_attn_schedule through the C ABI).

Bars: every layer of a schedule equals a separate skiparse_attn call bit for bit (the same
kernel on the same inputs); one layer per mode is also checked against the fp64 oracle at
the attention bars of test_gpu_parity.py; a HIP-graph capture of the schedule replays
bit-exactly, three times, with eager work on the outputs between the replays.
"""

import numpy as np
import pytest
import torch

import oracle
import skiparse_sparse_attention_amd as sk
from skiparse_sparse_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

GRID = (4, 8, 16)        # N = 512: k up to 8 divides N and N / k^2 in both modes
HEADS, D = 2, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    sk.lib()
    yield


def _layers(n_layers, k_max, seed):
    w = wl.Workload("sched", 1, *GRID, HEADS, D, 1, oracle.SINGLE, "bf16")
    sched = sk.u_schedule(n_layers, k_max)
    layers = []
    for i, (k, mode) in enumerate(sched):
        q, kk, v = (x.cuda() for x in wl.make_inputs(w, seed=seed + i, device="cpu"))
        layers.append((q, kk, v, torch.empty_like(q), k, mode))
    return layers


def test_schedule_equals_separate_calls_and_the_oracle():
    layers = _layers(6, 8, seed=10)
    print("schedule", [(k, m) for *_, k, m in layers], flush=True)
    sk.attn_schedule(layers, GRID)
    torch.cuda.synchronize()
    checked = set()
    for q, kk, v, out, k, mode in layers:
        ref = sk.attn(q, kk, v, GRID, k, mode)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (k, mode)
        if mode not in checked and k > 1:
            checked.add(mode)
            want = oracle.skiparse_attention(*(x.float().cpu().numpy() for x in (q, kk, v)), *GRID, k, mode)
            err = np.abs(out.float().cpu().numpy() - want)
            print(f"layer k={k} mode={mode}: max {err.max():.3e} mean {err.mean():.3e}", flush=True)
            assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_schedule_graph_replays_bit_exactly():
    layers = _layers(8, 8, seed=30)
    sk.attn_schedule(layers, GRID)
    torch.cuda.synchronize()
    eager = [layer[3].clone() for layer in layers]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on the capture stream
        sk.attn_schedule(layers, GRID)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sk.attn_schedule(layers, GRID)
    torch.cuda.synchronize()
    for rep in range(3):
        for layer in layers:
            layer[3].fill_(float(rep + 1))      # eager work on the outputs between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for layer, ref in zip(layers, eager):
            assert torch.equal(layer[3], ref), rep


def test_rotated_schedule_equals_the_schedule():
    """Every layer run as the RoPE pass into shared scratch and the attention on rotated
    operands: the outputs equal skiparse_attn_schedule's bit for bit."""
    layers = _layers(6, 8, seed=50)
    print("rotated schedule", [(k, m) for *_, k, m in layers], flush=True)
    sk.attn_schedule(layers, GRID)
    torch.cuda.synchronize()
    ref = [layer[3].clone() for layer in layers]
    for layer in layers:
        layer[3].zero_()
    sk.attn_schedule_rotated(layers, GRID)
    torch.cuda.synchronize()
    for (q, kk, v, out, k, mode), r in zip(layers, ref):
        assert torch.equal(out, r), (k, mode)


def test_rotated_schedule_graph_replays_bit_exactly():
    layers = _layers(8, 8, seed=70)
    scratch = (torch.empty_like(layers[0][0]), torch.empty_like(layers[0][0]))
    sk.attn_schedule_rotated(layers, GRID, scratch=scratch)
    torch.cuda.synchronize()
    eager = [layer[3].clone() for layer in layers]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sk.attn_schedule_rotated(layers, GRID, scratch=scratch)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sk.attn_schedule_rotated(layers, GRID, scratch=scratch)
    torch.cuda.synchronize()
    for rep in range(3):
        for layer in layers:
            layer[3].fill_(float(rep + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for layer, r in zip(layers, eager):
            assert torch.equal(layer[3], r), rep
