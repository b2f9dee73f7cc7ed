"""The two microbenchmark exports that give the achievable peaks bench.py
reads the rooflines against: each reads what it claims to read and runs the
instructions it claims to run."""
import numpy as np
import pytest

from gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu


def test_stream_read_reads_every_word_once():
    import torch
    from resident_expert_routing_amd import binding as B
    rng = np.random.default_rng(4)
    n = 65537 * 16   # ragged: not a multiple of the four-loads-per-thread round
    host = rng.integers(0, 256, size=n, dtype=np.uint8)
    grid = 8
    src = to_dev(host)
    sink = torch.empty(grid * 256, dtype=torch.int32, device=src.device)
    say(f"stream_read over {n} bytes, {grid} workgroups")
    B.check(B.moe_test_stream_read(src, n, sink, grid), "moe_test_stream_read")
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert got == want


@pytest.mark.parametrize("fmt", [0, 1])
def test_mfma_loop_accumulates(fmt):
    import torch
    from resident_expert_routing_amd import binding as B
    grid = 2
    dev = torch.device("cuda", 0)
    s1 = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    s2 = torch.empty_like(s1)
    say(f"mfma_loop with 1 and 2 rounds, B format {fmt}")
    B.check(B.moe_test_mfma_loop(1, s1, grid, act_format=fmt), "moe_test_mfma_loop")
    B.check(B.moe_test_mfma_loop(2, s2, grid, act_format=fmt), "moe_test_mfma_loop")
    torch.cuda.synchronize()
    a, b = s1.cpu().numpy(), s2.cpu().numpy()
    assert np.isfinite(a).all() and np.abs(a).sum() > 0
    # every accumulator chain adds the same product twice: exactly doubled
    assert np.array_equal(b, 2 * a)
