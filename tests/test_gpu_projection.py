"""Input projection on the GPU against the oracle: a stack whose input rows
are wider than its hidden size (the Code Predictor of the 1.7B Talker takes
its inputs in the Talker's width), alone and in the 1.7B frame loop."""

import dataclasses

import numpy as np
import pytest
import torch

from autoregressive_transformer_decode_amd import device as dv
from autoregressive_transformer_decode_amd import inputs
from oracle import decoder as od
from tests._models import oracle_from_weights
from tests.gpu_util import GAIN_SD, MARGIN, lm_parity, small_shape

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_projected_stack(kind):
    """Prefill rows and token embeddings 384 wide into a 256-wide stack
    (bias on the projection), 20 teacher-forced steps with growth."""
    args = (("pb", 2, 256, 8, 2, 64, 512, 700, "bf16", True, False) if kind == "bf16"
            else ("pf", 2, 128, 4, 2, 64, 384, 500, "f32", True, True))
    shape = dataclasses.replace(small_shape(*args), input_dim=384)
    mw = inputs.make_weights(shape, seed=13, gain_sd=GAIN_SD)
    X0 = inputs.normal(13, 2, 4, (7, 384), scale=1.0)
    chk, _, _ = lm_parity(mw, X0, 20, 16)
    _log(f"projected {kind}: {chk.n} checks, worst {chk.worst:.2e}, tokens {chk.tokens_checked}")
    assert chk.tokens_checked >= 10


def test_talker17_frames():
    """The 1.7B Talker with its projected Code Predictor: graph-replayed
    frames equal eager C-ABI calls bit for bit and the oracle's free-running
    loop code for code while they agree; a difference is allowed only at a
    close call (top-2 margin <= 1e-2), where the comparison ends."""
    wl = inputs.WORKLOADS["talker1.7b-frames"]
    n_frames = 5
    tmw = inputs.make_weights(wl.model, seed=0, gain_sd=GAIN_SD)
    cmw = inputs.make_weights(wl.cp, seed=0, tables=tmw.tables, gain_sd=GAIN_SD)
    X0 = inputs.prefill_embeddings(wl, seed=0)
    text = inputs.text_embeddings(wl, seed=0)
    ot = oracle_from_weights(tmw, np.float32)
    oc = oracle_from_weights(cmw, np.float32)
    frames, _ = od.run_talker(ot, oc, X0, text, n_frames, wl.s_init, rho=wl.penalty,
                              cp_capacity=inputs.CP_CAPACITY)
    tdm = dv.DeviceModel(tmw)
    cdm = dv.DeviceModel(cmw, tables=tdm.tables)
    tdec = dv.Decoder(tdm, max_slots=1, max_rows=wl.prefill, max_ctx=wl.s_init)
    cdec = dv.Decoder(cdm, max_slots=1, max_rows=2, max_ctx=inputs.CP_CAPACITY)
    tdec.grow(0, wl.s_init)
    cdec.grow(0, inputs.CP_CAPACITY)
    h, Vt, Vc, hin = wl.model.hidden, wl.model.vocab, wl.cp.vocab, wl.cp.in_width
    assert hin == h
    text_d = torch.from_numpy(text).cuda()
    X0_d = torch.from_numpy(X0).cuda()

    def start():
        y = torch.empty(h, device="cuda")
        zt = torch.empty(Vt, device="cuda")
        codes = torch.zeros(16, dtype=torch.int32, device="cuda")
        seen = torch.zeros(dv.seen_words(Vt), dtype=torch.int32, device="cuda")
        tdec.prefill(X0_d, y_out=y, logits_out=zt)
        dv.greedy_argmax(zt, seen, wl.penalty, codes[0:1])
        return y, zt, codes, seen

    y, zt, codes, seen = start()
    out = torch.full((n_frames, 16), -1, dtype=torch.int32, device="cuda")
    dv.talker_frames(tdec, cdec, n_frames, codes, y, text_d, seen, wl.penalty, codes_out=out)
    torch.cuda.synchronize()
    native = out.cpu().numpy()

    y, zt, codes, seen = start()
    cp_x = torch.empty(2, hin, device="cuda")
    zc = torch.empty(Vc, device="cuda")
    eager = []
    for f in range(n_frames):
        if f > 0:
            tdec.step(codes.view(1, 16), list(range(16)), extra=text_d[f:f + 1], y_out=y.view(1, h),
                      logits_out=zt.view(1, Vt))
            dv.greedy_argmax(zt, seen, wl.penalty, codes[0:1])
        cp_x[0].copy_(y)
        cdec.embed(codes[0:1].view(1, 1), [0], cp_x[1:2])
        cdec.prefill(cp_x, head=0, logits_out=zc)
        dv.greedy_argmax(zc, None, 1.0, codes[1:2])
        for j in range(1, 15):
            cdec.step(codes[j:j + 1].view(1, 1), [j], head=j, logits_out=zc.view(1, Vc))
            dv.greedy_argmax(zc, None, 1.0, codes[j + 1:j + 2])
        eager.append(codes.cpu().numpy().copy())
    torch.cuda.synchronize()
    assert (np.stack(eager) == native).all()

    seq = []
    for f in range(n_frames):
        fr = frames[f]
        seq.append((int(native[f, 0]), fr["c0"], fr["margin"]))
        seq += [(int(native[f, j + 1]), fr["codes"][j], fr["cp"][j][2]) for j in range(15)]
    checked, close = 0, 0
    for i, (g, o, m) in enumerate(seq):
        if g != o:
            assert m <= MARGIN, f"code {i}: device {g} != oracle {o} (margin {m:.3g})"
            break
        checked += 1
        close += m <= MARGIN
    _log(f"1.7B frames: native == eager over {n_frames} frames; {checked} codes equal to the "
         f"oracle ({close} of them close calls) before the first difference")
    assert checked >= 16
    tdec.close()
    cdec.close()
