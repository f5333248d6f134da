"""Interleaved mRoPE on the GPU (decoder_prefill_mrope, decoder_step_mrope)
against the oracle: rows whose rotary (t, h, w) positions differ from their
cache positions -- a block of image-like rows on a 6 x 8 grid inside text --
on the MFMA (bf16) and matrix-vector (float32) paths, single-stream and
batched; with t = h = w = the cache position the result equals the plain
entry points' bit for bit."""

import dataclasses

import numpy as np
import pytest
import torch

from autoregressive_transformer_decode_amd import device as dv
from autoregressive_transformer_decode_amd import inputs
from oracle import decoder as od
from tests._models import oracle_from_weights
from tests.gpu_util import GAIN_SD, MARGIN, StepCheck, small_shape

pytestmark = pytest.mark.gpu

SECTIONS = (24, 20, 20)


def _log(msg):
    print(msg, flush=True)


def _shape(kind):
    args = (("mb", 2, 256, 4, 2, 128, 512, 700, "bf16", True, False) if kind == "bf16"
            else ("mf", 2, 256, 4, 2, 128, 384, 500, "f32", True, True))
    return dataclasses.replace(small_shape(*args), mrope_sections=SECTIONS)


def grid_positions(n_text0, rows, cols, n_text1):
    """Text rows at t = h = w = index, then a rows x cols block sharing
    t = start with h = start + r, w = start + c, then text again from
    start + max(rows, cols)."""
    pos = [(i, i, i) for i in range(n_text0)]
    s = n_text0
    pos += [(s, s + r, s + c) for r in range(rows) for c in range(cols)]
    nxt = s + max(rows, cols)
    pos += [(nxt + i,) * 3 for i in range(n_text1)]
    return np.array(pos, np.int32), nxt + n_text1


@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_mrope_prefill_and_steps(kind):
    """70-row prefill (10 text rows, a 6 x 8 block, 12 text rows; MFMA chunks
    of 64 + 6 for bf16), then 8 teacher-forced steps at the following text
    positions, against the oracle."""
    shape = _shape(kind)
    mw = inputs.make_weights(shape, seed=31, gain_sd=GAIN_SD)
    X0 = inputs.normal(31, 2, 5, (70, shape.hidden), scale=1.0)
    rp, nxt = grid_positions(10, 6, 8, 12)
    assert rp.shape == (70, 3)
    om = oracle_from_weights(mw, np.float64)
    dm = dv.DeviceModel(mw)
    dec = dv.Decoder(dm, max_slots=1, max_rows=70, max_ctx=128)
    dec.grow(0, 128)
    cache = od.Cache(om, 128)
    y_ref, z_ref = od.prefill(om, cache, X0, 0, rope_pos=rp)
    y = torch.empty(1, shape.hidden, device="cuda")
    z = torch.empty(1, shape.vocab, device="cuda")
    dec.prefill(torch.from_numpy(X0.astype(np.float32)).cuda(), y_out=y[0], logits_out=z[0],
                rope_pos=torch.from_numpy(rp).cuda())
    chk = StepCheck()
    tok = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    for k in range(9):
        if k > 0:
            t = int(np.argmax(z_ref))
            p3 = (nxt + k - 1,) * 3
            y_ref, z_ref = od.step(om, cache, om.tables[0][t], 0, rope_pos=p3)
            tok.fill_(t)
            dec.step(tok, [0], y_out=y, logits_out=z,
                     rope_pos=torch.tensor([p3], dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        chk.add(y[0].cpu().numpy(), z[0].cpu().numpy(), y_ref, z_ref, f"{kind} step {k}")
        zs = np.sort(z_ref)
        if zs[-1] - zs[-2] > MARGIN:
            assert int(torch.argmax(z[0]).item()) == int(np.argmax(z_ref))
            chk.tokens_checked += 1
    assert dec.position(0)[0] == 78 and cache.pos == 78
    dec.close()
    _log(f"mrope {kind}: {chk.n} checks, worst {chk.worst:.2e}, tokens {chk.tokens_checked}")
    assert chk.tokens_checked >= 5


@pytest.mark.parametrize("kind,B", [("bf16", 3), ("bf16", 5), ("f32", 3)])
def test_mrope_batched_step(kind, B):
    """B streams with different histories step together, each row with its
    own distinct (t, h, w): bf16 at B = 3 on the vector path (two launches of
    two rows and one), at B = 5 on the matrix-core path; f32 on the vector
    path."""
    shape = _shape(kind)
    mw = inputs.make_weights(shape, seed=32, gain_sd=GAIN_SD)
    om = oracle_from_weights(mw, np.float64)
    dm = dv.DeviceModel(mw)
    dec = dv.Decoder(dm, max_slots=B, max_rows=16, max_ctx=64)
    lens = (5, 9, 16, 3, 12)[:B]
    step_pos = np.array([[7, 3, 9], [12, 12, 5], [2, 30, 31], [4, 8, 1], [20, 2, 33]],
                        np.int32)[:B]
    z_refs, toks = [], []
    for b, T in enumerate(lens):
        dec.grow(b, 64)
        X = inputs.normal(32, 2, 10 + b, (T, shape.hidden), scale=1.0)
        rp = np.stack([np.arange(T), np.arange(T)[::-1], np.full(T, b)], 1).astype(np.int32)
        cache = od.Cache(om, 64)
        od.prefill(om, cache, X, 0, rope_pos=rp)
        dec.prefill(torch.from_numpy(X.astype(np.float32)).cuda(), slot=b,
                    rope_pos=torch.from_numpy(rp).cuda())
        t = 17 * b + 3
        toks.append(t)
        z_refs.append(od.step(om, cache, om.tables[0][t], 0, rope_pos=step_pos[b]))
    z = torch.empty(B, shape.vocab, device="cuda")
    y = torch.empty(B, shape.hidden, device="cuda")
    tok = torch.tensor(toks, dtype=torch.int32, device="cuda").view(B, 1)
    dec.step(tok, [0], slot0=0, nrows=B, y_out=y, logits_out=z,
             rope_pos=torch.from_numpy(step_pos).cuda())
    torch.cuda.synchronize()
    chk = StepCheck()
    for b in range(B):
        chk.add(y[b].cpu().numpy(), z[b].cpu().numpy(), z_refs[b][0], z_refs[b][1],
                f"{kind} row {b}")
        assert dec.position(b)[0] == lens[b] + 1
    dec.close()
    _log(f"mrope batched {kind} B={B}: worst {chk.worst:.2e}")


def test_mrope_equal_positions_bitwise():
    """t = h = w = the cache position: the *_mrope entry points give the plain
    ones' logits bit for bit (prefill of 70 rows, steps of one and of three
    streams); a rotary position beyond max_ctx reads as max_ctx - 1."""
    shape = _shape("bf16")
    mw = inputs.make_weights(shape, seed=33, gain_sd=GAIN_SD)
    dm = dv.DeviceModel(mw)
    X0 = torch.from_numpy(inputs.normal(33, 2, 6, (70, shape.hidden), scale=1.0)).cuda()
    rp = torch.arange(70, dtype=torch.int32, device="cuda").view(70, 1).repeat(1, 3).contiguous()
    outs = []
    for use in (False, True):
        dec = dv.Decoder(dm, max_slots=3, max_rows=70, max_ctx=128)
        zs = []
        for b in range(3):
            dec.grow(b, 128)
            z = torch.empty(shape.vocab, device="cuda")
            dec.prefill(X0[:70 - 5 * b], slot=b, logits_out=z,
                        rope_pos=rp[:70 - 5 * b] if use else None)
            zs.append(z)
        tok = torch.tensor([[5], [6], [7]], dtype=torch.int32, device="cuda")
        z1 = torch.empty(1, shape.vocab, device="cuda")
        dec.step(tok[:1], [0], slot0=0, nrows=1, logits_out=z1,
                 rope_pos=torch.tensor([[70] * 3], dtype=torch.int32, device="cuda") if use else None)
        z3 = torch.empty(3, shape.vocab, device="cuda")
        p3 = torch.tensor([[71] * 3, [65] * 3, [60] * 3], dtype=torch.int32, device="cuda")
        dec.step(tok, [0], slot0=0, nrows=3, logits_out=z3, rope_pos=p3 if use else None)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in zs + [z1, z3]])
        dec.close()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    # clamping: rotary t beyond max_ctx = 128 reads as 127
    zc = []
    for t in (127, 5000):
        dec = dv.Decoder(dm, max_slots=1, max_rows=4, max_ctx=128)
        dec.grow(0, 128)
        z = torch.empty(shape.vocab, device="cuda")
        dec.prefill(X0[:4], logits_out=z,
                    rope_pos=torch.tensor([[t, 1, 2]] * 4, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        zc.append(z.cpu().numpy())
        dec.close()
    assert np.array_equal(zc[0], zc[1])
