"""Generation controls on the GPU against the oracle: suppressed tokens,
eos blocked before min_new_tokens, the stop at eos (later choices eos, seen
set untouched, eos_step recorded), in greedy_argmax / sample_topk rows and in
the graph-replayed generate and frame loops."""

import numpy as np
import pytest
import torch

from autoregressive_transformer_decode_amd import device as dv
from autoregressive_transformer_decode_amd import inputs
from oracle import decoder as od
from tests._models import oracle_from_weights
from tests.gpu_util import GAIN_SD, MARGIN, small_shape
from tests.test_gpu_sampling import EPS, _seen_mask, _seen_words

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("V", [3072, 151936])
@pytest.mark.parametrize("sampled", [False, True])
def test_controls_rows(V, sampled):
    """Six rows: eos made the largest logit of rows 0, 1 and 4 (blocked in the
    first call, whose index is below min_new_tokens; chosen in the second),
    row 2 already stopped, suppressed tokens everywhere (the largest logit of
    row 3 among them)."""
    Bn, eos, min_new, rho = 6, 17, 2, 1.05
    z = inputs.normal(21, 9, V, (Bn, V), scale=2.0).astype(np.float32)
    rng = np.random.default_rng([21, V])
    sup = rng.random((Bn, V)) < 0.05
    sup[:, eos] = False
    for b in (0, 1, 4):
        z[b, eos] = z[b].max() + 1.0
    sup[3, int(np.argmax(z[3]))] = True
    seen = rng.random((Bn, V)) < 0.02
    sup_d = torch.from_numpy(_seen_words(sup)).cuda()
    seen_d = torch.from_numpy(_seen_words(seen)).cuda()
    zd = torch.from_numpy(z).cuda()
    eos_step = torch.tensor([-1, -1, 3, -1, -1, -1], dtype=torch.int32, device="cuda")
    ctls = [od.Controls(suppress=sup[b], eos=eos, min_new=min_new) for b in range(Bn)]
    ctls[2].eos_step = 3
    seen_o = seen.copy()
    u = inputs.uniforms(21, V, (2, Bn))
    tok = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    for call, first in enumerate((0, 2)):
        c = dv.Controls(sup_d, eos, min_new, first, eos_step)
        if sampled:
            dv.sample_topk(zd, seen_d, rho, dv.Sampling(50, 0.9, 1.0, torch.from_numpy(u[call]).cuda()),
                           tok, controls=c)
        else:
            dv.greedy_argmax(zd, seen_d, rho, tok, controls=c)
        torch.cuda.synchronize()
        got = tok.cpu().numpy()
        for b in range(Bn):
            ctls[b].count = first
            samp = (50, 0.9, 1.0, u[call][b:b + 1]) if sampled else None
            if sampled and ctls[b].eos_step < 0:
                d = od.sample_topk(ctls[b].mask(z[b]), seen_o[b].copy(), rho, 50, 0.9, 1.0,
                                   float(u[call][b]))
                if d.gap <= EPS:
                    _log(f"row {b}: draw within {EPS} of a boundary, taken from the device")
                    ctls[b].count += 1
                    if got[b] == eos:
                        ctls[b].eos_step = first
                    seen_o[b][got[b]] = True
                    continue
            t, _ = od.choose_controlled(z[b], seen_o[b], rho, ctls[b], samp, 0)
            assert int(got[b]) == t, (call, b, int(got[b]), t)
        assert np.array_equal(_seen_mask(seen_d.cpu().numpy(), V), seen_o), call
        assert eos_step.cpu().tolist() == [c.eos_step for c in ctls], (call, eos_step.cpu().tolist())
    _log(f"rows V={V} sampled={sampled}: eos_step {eos_step.cpu().tolist()}")
    assert eos_step.cpu().tolist() == [2, 2, 3, -1, 2, -1] or sampled


def test_generate_controls():
    """decoder_generate with controls over two calls (first_index continues):
    graph = eager choices bit for bit, and equal to the oracle's controlled
    run up to its first close decision; the stop makes the rest eos."""
    shape = small_shape("gen", 2, 256, 8, 2, 128, 512, 700, "bf16", True, False)
    mw = inputs.make_weights(shape, seed=7, gain_sd=GAIN_SD)
    X0 = inputs.normal(7, 2, 1, (9, 256), scale=1.0)
    om = oracle_from_weights(mw)
    n = 40
    free, _ = od.run_lm(om, X0, n, 128, rho=1.3)
    sup = np.zeros(shape.vocab, bool)
    sup[free[2][2]] = True
    probe, _ = od.run_lm(om, X0, n, 128, rho=1.3, controls=od.Controls(suppress=sup))
    min_new = 8
    for j in range(12, n):          # an eos the controlled run reaches
        eos = probe[j][2]
        ctl = od.Controls(suppress=sup, eos=eos, min_new=min_new)
        ref, _ = od.run_lm(om, X0, n, 128, rho=1.3, controls=ctl)
        if ctl.eos_step >= min_new:
            break
    _log(f"oracle: eos {eos}, eos_step {ctl.eos_step}")
    assert ctl.eos_step >= min_new

    dm = dv.DeviceModel(mw)
    sup_d = torch.from_numpy(_seen_words(sup[None])[0]).cuda()
    res = []
    for mode in ("eager", "graph"):
        dec = dv.Decoder(dm, max_slots=1, max_rows=9, max_ctx=128)
        dec.grow(0, 128)
        z = torch.empty(1, shape.vocab, device="cuda")
        dec.prefill(torch.from_numpy(X0).cuda(), logits_out=z[0])
        seen = torch.zeros(dv.seen_words(shape.vocab), dtype=torch.int32, device="cuda")
        es = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        dv.greedy_argmax(z[0], seen, 1.3, tok, controls=dv.Controls(sup_d, eos, min_new, 0, es))
        toks = [int(tok.item())]
        if mode == "eager":
            for k in range(n):
                dec.step(tok.view(1, 1), [0], logits_out=z)
                dv.greedy_argmax(z[0], seen, 1.3, tok,
                                 controls=dv.Controls(sup_d, eos, min_new, 1 + k, es))
                toks.append(int(tok.item()))
        else:
            out = torch.zeros(n, dtype=torch.int32, device="cuda")
            dec.generate(25, tok, seen=seen, penalty=1.3, tokens_out=out[:25], logits_out=z[0],
                         controls=dv.Controls(sup_d, eos, min_new, 1, es))
            dec.generate(15, tok, seen=seen, penalty=1.3, tokens_out=out[25:], logits_out=z[0],
                         controls=dv.Controls(sup_d, eos, min_new, 26, es))
            torch.cuda.synchronize()
            toks += out.cpu().tolist()
        torch.cuda.synchronize()
        res.append((toks, int(es.item()), z[0].cpu().numpy().copy(), seen.cpu().numpy().copy()))
        dec.close()
    assert res[0][0] == res[1][0] and res[0][1] == res[1][1]
    assert np.array_equal(res[0][2], res[1][2]) and np.array_equal(res[0][3], res[1][3])
    toks, es = res[1][0], res[1][1]
    checked = 0
    for k in range(n + 1):
        if toks[k] != ref[k][2]:
            assert ref[k][3] <= MARGIN, (k, toks[k], ref[k][2])
            break
        checked += 1
    else:
        assert es == ctl.eos_step
    if es >= 0:
        assert all(t == eos for t in toks[es:])
    assert sup.nonzero()[0][0] not in toks
    _log(f"generate with controls: eos_step {es}; {checked} tokens equal to the oracle")
    assert checked >= 10


def test_talker_frames_controls():
    """The 0.6B frame loop with an eos on the main code: frames equal the
    oracle's controlled loop up to its first close decision; after the stop
    c0 stays eos."""
    wl = inputs.WORKLOADS["talker0.6b"]
    n_frames = 8
    tmw = inputs.make_weights(wl.model, seed=0, gain_sd=GAIN_SD)
    cmw = inputs.make_weights(wl.cp, seed=0, tables=tmw.tables, gain_sd=GAIN_SD)
    X0 = inputs.prefill_embeddings(wl, seed=0)
    text = inputs.text_embeddings(wl, seed=0)
    ot = oracle_from_weights(tmw, np.float32)
    oc = oracle_from_weights(cmw, np.float32)
    free, _ = od.run_talker(ot, oc, X0, text, n_frames, wl.s_init, rho=wl.penalty,
                            cp_capacity=inputs.CP_CAPACITY)
    eos, min_new = free[5]["c0"], 3
    ctl = od.Controls(eos=eos, min_new=min_new)
    frames, _ = od.run_talker(ot, oc, X0, text, n_frames, wl.s_init, rho=wl.penalty,
                              cp_capacity=inputs.CP_CAPACITY, tk_controls=ctl)
    _log(f"oracle frames: eos {eos}, eos_step {ctl.eos_step}")

    tdm = dv.DeviceModel(tmw)
    cdm = dv.DeviceModel(cmw, tables=tdm.tables)
    tdec = dv.Decoder(tdm, max_slots=1, max_rows=wl.prefill, max_ctx=wl.s_init)
    cdec = dv.Decoder(cdm, max_slots=1, max_rows=2, max_ctx=inputs.CP_CAPACITY)
    tdec.grow(0, wl.s_init)
    cdec.grow(0, inputs.CP_CAPACITY)
    h, Vt = wl.model.hidden, wl.model.vocab
    y = torch.empty(h, device="cuda")
    zt = torch.empty(Vt, device="cuda")
    codes = torch.zeros(16, dtype=torch.int32, device="cuda")
    seen = torch.zeros(dv.seen_words(Vt), dtype=torch.int32, device="cuda")
    es = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    tdec.prefill(torch.from_numpy(X0).cuda(), y_out=y, logits_out=zt)
    c = dv.Controls(None, eos, min_new, 0, es)
    dv.greedy_argmax(zt, seen, wl.penalty, codes[0:1], controls=c)
    out = torch.full((n_frames, 16), -1, dtype=torch.int32, device="cuda")
    dv.talker_frames(tdec, cdec, n_frames, codes, y, torch.from_numpy(text).cuda(), seen,
                     wl.penalty, codes_out=out, tk_controls=c)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    esv = int(es.item())
    checked = 0
    for f in range(n_frames):
        fr = frames[f]
        if got[f, 0] != fr["c0"]:
            assert fr["margin"] <= MARGIN, (f, int(got[f, 0]), fr["c0"])
            break
        checked += 1
        if ctl.eos_step >= 0 and f >= ctl.eos_step:
            continue   # the codes of frames after the stop are not compared
        if any(int(got[f, j + 1]) != fr["codes"][j] for j in range(15)):
            break
    if esv >= 0:
        assert (got[esv:, 0] == eos).all()
    _log(f"frames with controls: eos_step {esv} (oracle {ctl.eos_step}); {checked} frames' c0 equal")
    assert checked >= 4
    tdec.close()
    cdec.close()
