"""greedy_argmax_noalloc (partials in the library's fixed device array)
against greedy_argmax (partials in a buffer the library allocates), through
the C ABI, on two calls in a row, the second with a smaller input."""

import numpy as np
import pytest
import torch

from autoregressive_transformer_decode_amd import binding as B
from autoregressive_transformer_decode_amd import device as dv

pytestmark = pytest.mark.gpu


def _case(Bn, V, seed):
    g = torch.Generator().manual_seed(seed)
    z = torch.randn(Bn, V, generator=g) * 3.0
    z[0, 17] = z[0, V - 3] = z[0].max() + 1.0          # a tie: the lower index wins
    z[-1, :] = 0.5                                      # a flat row
    seen = torch.zeros(Bn, dv.seen_words(V), dtype=torch.int32)
    idx = torch.randint(0, V, (Bn, 40), generator=g)
    for b in range(Bn):
        for t in idx[b].tolist():
            seen[b, t // 32] |= (1 << (t % 32)) if t % 32 < 31 else -(1 << 31)
    return z.cuda(), seen.cuda()


def _run(fn, z, seen0, penalty):
    Bn, V = z.shape
    seen = seen0.clone()
    tok = torch.full((Bn,), -1, dtype=torch.int32, device="cuda")
    margin = torch.zeros(Bn, device="cuda")
    fn(z.data_ptr(), Bn, V, seen.data_ptr(), penalty, tok.data_ptr(), margin.data_ptr(),
       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), margin.cpu().numpy(), seen.cpu().numpy()


def test_noalloc_argmax_equals_allocating_one():
    for Bn, V, seed in ((5, 151936, 1), (2, 20000, 2)):   # the second call is smaller
        z, seen0 = _case(Bn, V, seed)
        got = _run(B.greedy_argmax_noalloc, z, seen0, 1.05)
        ref = _run(B.greedy_argmax, z, seen0, 1.05)
        for a, r in zip(got, ref):
            assert np.array_equal(a, r), (Bn, V)
    with pytest.raises(B.AtdError) as ei:      # beyond the fixed array: refused
        big = torch.zeros(600, 151936, device="cuda")
        B.greedy_argmax_noalloc(big.data_ptr(), 600, 151936, None, 1.0,
                                torch.zeros(600, dtype=torch.int32, device="cuda").data_ptr(),
                                None, torch.cuda.current_stream().cuda_stream)
    assert ei.value.code == B.ATD_ERR_CAPACITY
