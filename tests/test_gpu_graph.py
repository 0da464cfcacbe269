"""The F/S stack captured into a HIP graph (through torch's graph capture on
the current stream) and replayed: every replay, with eager work and
synchronisations between replays, reproduces the eager result exactly.

The library's calls only enqueue kernels (no allocation, no synchronisation,
no memset nodes), so a caller can capture a whole stack once per shape and
replay it each step.
"""

import numpy as np
import pytest

from synth import random_batch
from tests.gpu_helpers import device_batch, device_layer, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_token_fp8_amd as m
    return m, torch


@pytest.mark.parametrize("lengths,new,pattern", [
    ([3000, 9000, 20000, 1500, 700], 1, "FSFS"),             # decode batch, long rows
    ([2500, 1200], [200, 1], "FSSF"),                         # prefill chunk plus one decode
])
def test_stack_graph_replays_match_eager(env, lengths, new, pattern):
    m, torch = env
    wl = random_batch(6001 + len(lengths), lengths, new, k=256, num_layers=len(pattern),
                      pattern=pattern)
    say("graph stack", lengths, new, pattern)
    full = m.idx_layer_schedule(True, pattern, 1, 2, len(pattern))
    batch = device_batch(m, wl)
    devs = [device_layer(m, torch, wl, l) for l in range(len(pattern))]
    layers = [(d["k_new"], d["cache"], d["q8"], d["w"]) for d in devs]
    slots = devs[0]["slots_new"]
    topk = torch.full((wl.num_tokens, wl.k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(m.idx_score_topk_workspace_size(batch, wl.k), dtype=torch.uint8, device="cuda")

    def run():
        m.idx_indexcache_stack(layers, full, True, slots, batch, wl.k, topk, workspace=ws)

    run()
    torch.cuda.synchronize()
    eager = topk.cpu().numpy().copy()
    assert (eager[:, 0] >= 0).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()

    other = torch.empty((wl.num_tokens, wl.max_seq_len), dtype=torch.float32, device="cuda")
    for rep in range(4):
        topk.fill_(-5)
        m.idx_logits(devs[1]["q8"], devs[1]["w"], devs[1]["cache"], batch, logits=other)   # eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = topk.cpu().numpy()
        assert np.array_equal(got, eager), f"replay {rep}"
        say(f"  replay {rep} ok")
