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
    (8, 8, 1, 7, 1),          # one frame: only the last tap sees data
    (16, 8, 20, 7, 9),        # taps reaching before frame 0 for every t (shifts up to 54)
    (1024, 1024, 300, 7, 1),  # the input convolution (the smallest grid)
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
    (9, 4, 1, 2),             # one input frame: only the first tap of each phase
    (5, 3, 11, 1),            # stride 1 (kernel 2)
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


def test_conv1d_accumulate_and_stack():
    """accumulate adds the result to y (a residual connection); a reduced
    copy of the decoder stack (16 input frames, narrower channels) run layer by layer equals the
    oracle's."""
    x = _rand(7, 0, (48, 100), 1.0)
    w = _rand(8, 0, (40, 48, 3), 0.1)
    y0 = _rand(9, 0, (40, 100), 1.0)
    y = torch.from_numpy(y0.copy()).cuda()
    dv.conv1d_causal(torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda(), None, 2, y=y,
                     accumulate=True)
    torch.cuda.synchronize()
    assert normwise_rel(y.cpu().numpy(), y0 + oc.conv1d_causal(x, w, None, 2)) <= TOL
    import dataclasses
    c = dataclasses.replace(inputs.CODEC, frames=16, channels=(128, 96, 64, 48, 32))
    layers = inputs.codec_layers(c)
    ws = inputs.make_codec_weights(c, seed=1)
    h = inputs.codec_input(c, seed=1).astype(np.float32)
    hd = torch.from_numpy(h).cuda()
    h = h.astype(np.float64)
    for i, (L, (w, b)) in enumerate(zip(layers, ws)):
        wd, bd = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
        if L[0] == "trans":
            hd = dv.transconv1d(hd, dv.transconv1d_pack(wd, L[3]), bd, L[3])
            h = oc.transconv1d(h, w, b, L[3])
        elif L[6]:   # 1-tap convolution of the unit's dilated output, added back
            dv.conv1d_causal(ud, wd, bd, 1, y=hd, accumulate=True)
            h = h + oc.conv1d_causal(u, w, b, 1)
        elif i + 1 < len(layers) and layers[i + 1][0] == "conv" and layers[i + 1][6]:
            ud = dv.conv1d_causal(hd, wd, bd, L[4])
            u = oc.conv1d_causal(h, w, b, L[4])
        else:
            hd = dv.conv1d_causal(hd, wd, bd, L[4])
            h = oc.conv1d_causal(h, w, b, L[4])
    torch.cuda.synchronize()
    e = normwise_rel(hd.cpu().numpy(), h)
    _log(f"reduced decoder stack: output {tuple(hd.shape)}, normwise {e:.2e}")
    assert hd.shape == (1, 16 * 480) and e <= 1e-4
