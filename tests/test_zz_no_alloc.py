"""lrm_select_static, the selection for callers that cannot allocate: through
the C ABI, its outputs must equal lrm_select's (given a workspace) bit for bit
(integer outputs), on consecutive calls that reuse the library's scratch
array, the second smaller than the first; sizes beyond the array are refused
before any launch."""

import numpy as np
import pytest
import torch

from pruned_expert_backward_lrm_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from pruned_expert_backward_lrm_amd import lrm
    return lrm


def _case(L, T, E, k, zipf, seed, quota_fn):
    r = synth.make_routing(T, E, k, zipf, "noalloc", seed)
    pairs = L.Pairs.from_routing(r, DEV)
    g = torch.Generator(device="cpu").manual_seed(seed)
    # scores with exact ties (few distinct values) so the tie-break is exercised
    score = torch.randint(0, 50, (max(r.N, 1),), generator=g).float().to(DEV) * 0.25
    return r, pairs, score, quota_fn(r.counts).astype(np.int32)


def _both(L, r, pairs, score, quota, flags=0):
    i32 = dict(dtype=torch.int32, device=DEV)
    outs = []
    for static in (False, True):
        pos = torch.full((max(r.N, 1),), -7, **i32)
        offsets = torch.full((r.E + 1,), -7, **i32)
        kept = torch.full((max(r.N, 1),), -7, **i32)
        if static:
            L.lrm_select_static(pairs, score, quota, pos, offsets, kept, flags=flags)
        else:
            L.lrm_select(pairs, score, quota, pos, offsets, kept, flags=flags)
        torch.cuda.synchronize()
        M = int(offsets[-1].item())
        outs.append((pos[:r.N].cpu(), offsets.cpu(), kept[:M].cpu()))
    return outs


def test_static_select_equals_workspace_select_twice(L):
    # first a Qwen3-sized call, then a smaller one in the same scratch
    big = _case(L, 4096, 128, 8, 1.1, 1, lambda c: (3 * np.minimum(c, 320)) // 5)
    small = _case(L, 700, 12, 2, 1.3, 2, lambda c: c // 2 + (c % 3 == 0))
    for r, pairs, score, q in (big, small):
        (p0, o0, k0), (p1, o1, k1) = _both(L, r, pairs, score, q)
        assert torch.equal(p0, p1) and torch.equal(o0, o1) and torch.equal(k0, k1)
        assert int(o1[-1]) == int(np.minimum(q, r.counts).sum())


def test_static_select_copied_and_device_quotas(L):
    # more than 512 experts: the host quotas go through a stream copy into
    # the scratch; device quotas are read where they are; keep-all
    r, pairs, score, q = _case(L, 3000, 600, 2, 1.1, 3, lambda c: (c + 1) // 2)
    for quota, flags in ((q, 0), (torch.as_tensor(q, device=DEV), L.LRM_QUOTA_ON_DEVICE),
                         (None, L.LRM_KEEP_ALL)):
        (p0, o0, k0), (p1, o1, k1) = _both(L, r, pairs, score, quota, flags)
        assert torch.equal(p0, p1) and torch.equal(o0, o1) and torch.equal(k0, k1)


def test_static_select_refuses_sizes_beyond_its_scratch(L):
    # 8M pairs need 64 MiB of candidate lists and keys: refused on the host,
    # before any launch (the arrays are real, of the stated size)
    N, E, T = 8 << 20, 16, 1 << 20
    i32 = dict(dtype=torch.int32, device=DEV)
    token = torch.arange(N, **i32) // 8
    expert = torch.arange(N, **i32) % E
    pairs = L.Pairs(token, expert, torch.ones(N, device=DEV), T, E)
    score = torch.ones(N, device=DEV)
    pos, kept = torch.empty(N, **i32), torch.empty(N, **i32)
    offsets = torch.empty(E + 1, **i32)
    with pytest.raises(L.LrmError) as ei:
        L.lrm_select_static(pairs, score, np.full(E, 4, np.int32), pos, offsets, kept)
    assert ei.value.status == 7, str(ei.value)  # LRM_ERR_WORKSPACE
