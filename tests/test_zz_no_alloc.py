"""The allocation-free E2-TTT chunk scan (e2ttt_chunk_scan_noalloc, for
callers that cannot allocate device memory) against e2ttt_chunk_scan on the
same inputs: two calls in a row, the second on a smaller problem (the fixed
work buffer then still holds the first call's contents), and a problem
beyond the buffer's limit rejected before any device work."""
import pytest
import torch

import synth
from tests.util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("first,second", [((16, 32768, 128, 2048), (4, 5000, 64, 640)),
                                          ((8, 6000, 128, 1024), (3, 700, 128, 256))])
def test_noalloc_matches_allocating_scan_on_consecutive_calls(first, second):
    import test_long_context_amd as tla
    for (H, T, D, C) in (first, second):
        say(f"no-alloc e2 case: H={H} T={T} D={D} C={C}")
        x = synth.gen_e2(H, T, D, seed=7, device="cuda")
        Wa, Ma = x["W"].clone(), x["M"].clone()
        Wb, Mb = x["W"].clone(), x["M"].clone()
        tla.e2ttt_chunk_scan(x["k"], x["v"], x["eta"], x["beta"], x["gamma"], Wa, Ma, C)
        tla.e2ttt_chunk_scan_noalloc(x["k"], x["v"], x["eta"], x["beta"], x["gamma"], Wb, Mb, C)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(Wb).all()) and bool(torch.isfinite(Mb).all())
        # same kernels, same order of every sum: identical bits
        assert torch.equal(Wa, Wb) and torch.equal(Ma, Mb)


def test_noalloc_rejects_problems_beyond_its_buffer():
    """A problem whose per-token coefficients alone exceed the buffer is
    refused on the host (the small tensors passed are never touched)."""
    import test_long_context_amd as tla
    limit = tla.e2ttt_chunk_scan_noalloc_max_bytes()
    H, D, C = 64, 128, 2048
    T = limit // (8 * H) + C
    kv = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    f = torch.zeros(16, dtype=torch.float32, device="cuda")
    st = tla.lib().e2ttt_chunk_scan_noalloc(kv.data_ptr(), kv.data_ptr(), f.data_ptr(), f.data_ptr(),
                                            f.data_ptr(), f.data_ptr(), f.data_ptr(), H, T, D, C,
                                            tla._stream())
    assert st == -2   # TTT_ERR_UNSUPPORTED
