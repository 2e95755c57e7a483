"""Concurrent use of the library: two host threads, each with its own stream,
buffers and workspace, call the forward at the same time.  The library keeps
no per-call state, so each thread's outputs must equal, bit for bit, what the
same calls give one after the other (every sum has a fixed order)."""
import threading

import pytest
import torch

from block_causal_linear_phi_amd import sva
from gpu_helpers import DEV, rand

pytestmark = pytest.mark.gpu


def test_two_threads_two_streams_match_sequential():
    print("concurrency: two threads", flush=True)
    grid, F, split = (6, 9, 13), 3, (16, 24, 24)
    N = grid[0] * grid[1] * grid[2]
    jobs = []
    for j in range(2):
        q = rand((2, 4, N, 64), 70 + 3 * j, "bf16")[1]
        k = rand((2, 4, N, 64), 71 + 3 * j, "bf16")[1]
        v = rand((2, 4, N, 64), 72 + 3 * j, "bf16")[1]
        jobs.append((q, k, v))
    ref = [sva.sva_lin_attn_fwd(q, k, v, grid, F, rope=True, split=split) for q, k, v in jobs]
    torch.cuda.synchronize()

    outs = [[None] * 20 for _ in jobs]
    errors = []

    def worker(j):
        try:
            q, k, v = jobs[j]
            stream = torch.cuda.Stream(device=DEV)  # default priority
            desc = sva.make_desc(2, 4, 64, grid, F, rope=True, split=split)
            ws = torch.zeros(sva.sva_lin_attn_fwd_workspace(desc), dtype=torch.uint8, device=DEV)
            with torch.cuda.stream(stream):
                for i in range(20):
                    outs[j][i] = sva.sva_lin_attn_fwd(q, k, v, grid, F, rope=True, split=split, ws=ws,
                                                      stream=stream)
            stream.synchronize()
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    for j in range(2):
        for i in range(20):
            assert torch.equal(outs[j][i], ref[j]), (j, i)
