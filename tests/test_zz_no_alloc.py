"""The PFT build that allocates nothing (xmoe_build_pft_noalloc, on the
library's static scratch) against xmoe_build_pft with a caller workspace,
through the C ABI: bitwise the same six fields on two calls in a row, the
second with a smaller input, so the scratch holds the first call's counts when
the second starts.  Also its size limit, checked on the host."""
import ctypes

import pytest
import torch

import workloads
from _helpers import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def xm():
    need_gpu()
    import padding_free_expert_amd as m
    assert m.xmoe_query_device(0)
    return m


def _both(xm, T, E, k, skew, seed):
    print(f"\n[noalloc] T={T} E={E} k={k} skew={skew} seed={seed}", flush=True)
    ids, w = workloads.random_topk(T, E, k, seed=seed, skew=skew)
    ids, w = ids.cuda(), w.cuda()
    a = xm.PFT(T, E, k)
    ws = torch.empty(max(xm.xmoe_build_pft_workspace_size(T, E, k), 16), dtype=torch.uint8, device="cuda")
    xm.xmoe_build_pft(ids, w, E, a, ws)
    b = xm.PFT(T, E, k)
    for t in b.fields().values():
        t.fill_(-7)   # every field must be written
    c = b.c()
    st = xm._lib_pft_na(ids.data_ptr(), w.data_ptr(), T, E, k, ctypes.byref(c),
                        torch.cuda.current_stream().cuda_stream)
    assert st == 0, xm._lib_last_error()
    torch.cuda.synchronize()
    for key, t in a.fields().items():
        u = b.fields()[key]
        if key == "combine_weights":
            assert torch.equal(t.view(torch.int32), u.view(torch.int32)), key
        else:
            assert torch.equal(t, u), key


@pytest.mark.parametrize("first,second", [((32768, 160, 8, 0.0, 1), (4096, 64, 6, 0.0, 2)),
                                          ((16384, 128, 8, 3.0, 3), (257, 128, 8, 3.0, 4)),
                                          ((130816, 1024, 8, 1.0, 5), (1, 8, 2, 0.0, 6))])
def test_noalloc_matches_workspace_call_twice(xm, first, second):
    _both(xm, *first)
    _both(xm, *second)


def test_noalloc_rejects_sizes_beyond_the_scratch(xm):
    mx = xm.xmoe_build_pft_noalloc_max_bytes()
    assert mx == 4 << 20
    T, E, k = 1 << 20, 1024, 2      # 4096 blocks x 1024 experts x 2 words: 32 MiB
    assert xm.xmoe_build_pft_workspace_size(T, E, k) > mx
    ids = torch.zeros((1, k), dtype=torch.int32, device="cuda")   # never read: rejected first
    pft = xm.PFT(1, E, k)
    c = pft.c()
    st = xm._lib_pft_na(ids.data_ptr(), ids.data_ptr(), T, E, k, ctypes.byref(c), None)
    assert st == 2 and b"scratch" in xm._lib_last_error()
