"""The page-locked copies behind arena_load_slot (runtime.PinnedCopies): one
copy per host array, least recently used first out past the byte budget, and
an entry still read by an enqueued copy stays until that copy has completed."""
import numpy as np
import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def test_pinned_copies_budget_and_reuse():
    import torch
    from resident_expert_routing_amd import runtime as R
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mib = 1 << 20
    pins = R.PinnedCopies(budget=3 * mib)
    arrs = [np.full(mib, i + 1, dtype=np.uint8) for i in range(5)]
    first = pins.get(arrs[0])
    assert pins.get(arrs[0]).data_ptr() == first.data_ptr()     # one copy per array
    for a in arrs[1:]:
        pins.get(a)
    assert pins.bytes == 3 * mib and len(pins.entries) == 3
    assert [e[0] is a for e, a in zip(pins.entries.values(), arrs[2:])] == [True] * 3
    # a copy that reads an entry: the entry's bytes arrive whole, and once the
    # copy has completed the entry can go
    side = torch.cuda.Stream()
    dst = torch.empty(mib, dtype=torch.uint8, device="cuda")
    src = pins.get(arrs[2])
    with torch.cuda.stream(side):
        dst.copy_(src, non_blocking=True)
    pins.used_on(arrs[2], side)
    side.synchronize()
    assert (dst.cpu().numpy() == 3).all()
    for a in (arrs[0], arrs[1], arrs[3]):   # three newer uses: arrs[2] is now the oldest
        pins.get(a)
    assert pins.bytes == 3 * mib and id(arrs[2]) not in pins.entries
    say("  page-locked copies: budget kept, completed copies' entries dropped")
