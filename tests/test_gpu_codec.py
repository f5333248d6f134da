"""Codec decoder convolutions on the GPU against the oracle (float64
definitions): the dilated causal convolution and the transposed convolution
by phases, on ragged shapes and on the stages of a 4-stage decoder
(strides 8, 5, 4, 3; channels 1024 -> 64).  float32 data and accumulation:
normwise max relative error <= 1e-5."""

import numpy as np
import pytest
import torch

from autoregressive_transformer_decode_amd import device as dv
from autoregressive_transformer_decode_amd import inputs
from oracle import codec as oc
from tests._models import normwise_rel

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _log(msg):
    print(msg, flush=True)


def _rand(seed, tid, shape, scale):
    return inputs.normal(seed, 7, tid, shape, scale=scale).astype(np.float32)


CONV_CASES = [   # cin, cout, T, K, dilation
    (1, 1, 20, 5, 1),
    (33, 70, 130, 7, 3),      # ragged against the 64 x 64 tiles and 16-wide chunks
    (64, 64, 1000, 7, 9),
    (256, 256, 600, 7, 1),
    (128, 128, 257, 1, 1),
    (7, 1, 300, 7, 1),        # output convolution to one channel
    (512, 512, 2400, 7, 3),   # a first-stage residual convolution at full length
]


@pytest.mark.parametrize("case", range(len(CONV_CASES)))
def test_conv1d_causal(case):
    cin, cout, T, K, d = CONV_CASES[case]
    _log(f"conv1d_causal cin {cin} cout {cout} T {T} K {K} dilation {d}")
    x = _rand(1, case, (cin, T), 1.0)
    w = _rand(2, case, (cout, cin, K), 1.0 / np.sqrt(cin * K))
    b = _rand(3, case, (cout,), 0.1)
    y = dv.conv1d_causal(torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(),
                         torch.from_numpy(b).cuda(), d)
    torch.cuda.synchronize()
    ref = oc.conv1d_causal(x, w, b, d)
    e = normwise_rel(y.cpu().numpy(), ref)
    _log(f"  normwise {e:.2e}")
    assert e <= TOL


TRANS_CASES = [   # cin, cout, T, stride
    (3, 5, 7, 3),
    (70, 33, 65, 4),
    (1024, 512, 300, 8),      # the four stages of the decoder at full length
    (512, 256, 2400, 5),
    (256, 128, 12000, 4),
    (128, 64, 48000, 3),
]


@pytest.mark.parametrize("case", range(len(TRANS_CASES)))
def test_transconv1d(case):
    cin, cout, T, s = TRANS_CASES[case]
    _log(f"transconv1d cin {cin} cout {cout} T {T} stride {s}")
    x = _rand(4, case, (cin, T), 1.0)
    w = _rand(5, case, (cin, cout, 2 * s), 1.0 / np.sqrt(2 * cin))
    b = _rand(6, case, (cout,), 0.1)
    packed = dv.transconv1d_pack(torch.from_numpy(w).cuda(), s)
    y = dv.transconv1d(torch.from_numpy(x).cuda(), packed, torch.from_numpy(b).cuda(), s)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    if cin * cout * T <= 2 ** 27:
        ref = oc.transconv1d(x, w, b, s)
        e = normwise_rel(got, ref)
    else:   # sampled output frames, from the definition restricted to their sources
        rng = np.random.default_rng(case)
        ts = np.concatenate([[0, 1, T - 1], rng.integers(0, T, 40)])
        e = 0.0
        for t in ts:
            lo = max(t - 1, 0)
            part = oc.transconv1d(x[:, lo:t + 1], w, b, s)
            seg = part[:, (t - lo) * s:(t - lo + 1) * s]
            e = max(e, normwise_rel(got[:, t * s:(t + 1) * s], seg))
    _log(f"  normwise {e:.2e}")
    assert e <= TOL
