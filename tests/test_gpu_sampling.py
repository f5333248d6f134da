"""On-device sampled token choice against the oracle's draw with the same
uniforms: sample_topk alone, and the sampled forms of decoder_generate and
talker_generate_frames.

Given equal logits the top-k set and its order are exact (bit for bit); the
running weights are float32 sums on the device and float64 in the oracle, so
a token is compared wherever u sits more than EPS from a boundary of the
oracle's cumulative distribution (and, with top_p < 1, the cut more than EPS
from top_p).  Elsewhere the token must still lie in the oracle's kept set.
Through the decoders the logits themselves differ within the 2e-3 bar: there
every decision must match the oracle's, except that a decision a change of
1e-2 (in probability, or in logit at the top-k cut) could flip may differ,
and the comparison ends at such a difference (both continuations are
valid)."""

import numpy as np
import pytest
import torch

from autoregressive_transformer_decode_amd import device as dv
from autoregressive_transformer_decode_amd import inputs
from oracle import decoder as od
from tests._models import oracle_from_weights
from tests.gpu_util import GAIN_SD, MARGIN, small_shape

pytestmark = pytest.mark.gpu

EPS = 1e-5


def _log(msg):
    print(msg, flush=True)


def _follow(seq):
    """seq: (device token, oracle token, oracle robustness) in decision
    order.  Counts the equal decisions up to the first difference, which
    must be at a close decision."""
    n = 0
    for i, (g, o, r) in enumerate(seq):
        if g != o:
            assert r <= MARGIN, f"decision {i}: device {g} != oracle {o} (robustness {r:.3g})"
            break
        n += 1
    return n


def _seen_words(mask):
    """[B, V] bool -> [B, ceil(V/32)] int32 bit words (bit t%32 of word t/32)."""
    B, V = mask.shape
    W = dv.seen_words(V)
    padded = np.zeros((B, W * 32), bool)
    padded[:, :V] = mask
    bits = padded.reshape(B, W, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)
    return bits.sum(axis=2).astype(np.uint32).view(np.int32)


def _seen_mask(words, V):
    w = words.view(np.uint32).astype(np.uint64)
    bits = (w[..., None] >> np.arange(32, dtype=np.uint64)) & 1
    return bits.reshape(words.shape[0], -1)[:, :V].astype(bool)


# B, V, top_k, temperature, top_p, penalty, equal-value logits
CASES = [
    (8, 3072, 50, 0.9, 1.0, 1.05, False),      # Talker defaults
    (8, 2048, 50, 0.9, 1.0, 1.0, False),       # Code Predictor defaults
    (5, 1000, 1, 0.9, 1.0, 1.05, False),       # greedy limit
    (4, 1000, 256, 1.7, 1.0, 1.05, False),     # largest k
    (4, 257, 256, 0.5, 0.8, 1.3, False),       # k near V, top-p
    (6, 3072, 50, 0.9, 1.0, 1.05, True),       # many equal logits at the cut
    (3, 8193, 50, 0.9, 0.9, 1.05, False),      # two chunks, one logit in the second
    (2, 151936, 256, 0.9, 1.0, 1.05, False),   # ASR vocabulary: 19 chunks of 8192
    (2, 151936, 50, 0.7, 0.95, 1.05, True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_sample_topk_rows(case):
    Bn, V, k, t, tp, rho, ties = CASES[case]
    _log(f"sample_topk case {case}: B={Bn} V={V} k={k} T={t} top_p={tp} rho={rho} ties={ties}")
    z = inputs.normal(3, 9, 100 + case, (Bn, V), scale=3.0)
    if ties:
        z = np.round(z * 2.0) / 2.0
    z = z.astype(np.float32)
    rng = np.random.default_rng([3, case])
    mask = rng.random((Bn, V)) < 0.1
    u = inputs.uniforms(3, case, Bn)
    seen_d = torch.from_numpy(_seen_words(mask)).cuda()
    tok_d = torch.full((Bn,), -1, dtype=torch.int32, device="cuda")
    sp = dv.Sampling(k, t, tp, torch.from_numpy(u).cuda())
    dv.sample_topk(torch.from_numpy(z).cuda(), seen_d if rho != 1.0 else None, rho, sp, tok_d)
    torch.cuda.synchronize()
    got = tok_d.cpu().numpy()
    seen_after = _seen_mask(seen_d.cpu().numpy(), V)
    compared = 0
    for b in range(Bn):
        s = mask[b].copy() if rho != 1.0 else None
        d = od.sample_topk(z[b], s, rho, k, t, tp, float(u[b]))
        kept, _, _, _ = od.sampling_distribution(z[b], mask[b] if rho != 1.0 else None, rho, k, t, tp)
        assert int(got[b]) in set(int(x) for x in kept), (b, int(got[b]))
        if d.gap > EPS and d.cut_gap > EPS:
            assert int(got[b]) == d.tok, (b, int(got[b]), d.tok, d.gap)
            compared += 1
        if rho != 1.0:
            exp = mask[b].copy()
            exp[int(got[b])] = True
            assert np.array_equal(seen_after[b], exp), b
    _log(f"  {compared}/{Bn} rows compared")
    assert compared >= Bn - 1


@pytest.mark.parametrize("V,k,t,tp", [(3072, 256, 0.9, 1.0), (3072, 50, 0.9, 0.7),
                                      (151936, 50, 0.9, 1.0)])
def test_sample_topk_uniform_grid(V, k, t, tp):
    """One row of logits drawn with a grid of uniforms (row i: u = (i+0.5)/n):
    every grid point away from a boundary gives the oracle's token, so the
    whole kept set and its order are checked."""
    n = 1024 if V <= 8192 else 64
    _log(f"uniform grid: V={V} k={k} T={t} top_p={tp} n={n}")
    row = inputs.normal(4, 9, V + k, (V,), scale=2.0).astype(np.float32)
    u = ((np.arange(n) + 0.5) / n).astype(np.float32)
    zd = torch.from_numpy(row).cuda().expand(n, V).contiguous()
    tok_d = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    dv.sample_topk(zd, None, 1.0, dv.Sampling(k, t, tp, torch.from_numpy(u).cuda()), tok_d)
    torch.cuda.synchronize()
    got = tok_d.cpu().numpy()
    kept = set(int(x) for x in od.sampling_distribution(row, None, 1.0, k, t, tp)[0])
    compared, hit = 0, set()
    for i in range(n):
        d = od.sample_topk(row, None, 1.0, k, t, tp, float(u[i]))
        if d.gap > EPS and d.cut_gap > EPS:
            assert int(got[i]) == d.tok, (i, int(got[i]), d.tok)
            compared += 1
        assert int(got[i]) in kept, (i, int(got[i]))
        hit.add(int(got[i]))
    _log(f"  {compared}/{n} compared, {len(hit)} distinct tokens of {len(kept)} kept")
    # the last candidates carry tiny probabilities, so their boundaries sit
    # closer than EPS near u = 1; every other grid point is compared
    assert compared >= 0.97 * n


def test_generate_sampled():
    """decoder_generate with sampling: the graph-replayed steps equal eager
    decoder_step + sample_topk with the same uniforms, bit for bit (two
    sampling settings in a row, so the graph key must hold the settings), and
    follow the oracle's sampled run up to its first close decision."""
    shape = small_shape("gen", 2, 256, 8, 2, 128, 512, 700, "bf16", True, False)
    mw = inputs.make_weights(shape, seed=7, gain_sd=GAIN_SD)
    X0 = inputs.normal(7, 2, 1, (9, 256), scale=1.0)
    n1, n2 = 25, 15
    u = inputs.uniforms(7, 0, n1 + n2 + 1)
    ud = torch.from_numpy(u).cuda()
    cfg1 = (50, 0.9, 1.0)
    cfg2 = (20, 1.3, 0.9)
    dm = dv.DeviceModel(mw)
    res = []
    for mode in ("eager", "graph"):
        dec = dv.Decoder(dm, max_slots=1, max_rows=9, max_ctx=128)
        dec.grow(0, 128)
        z = torch.empty(1, shape.vocab, device="cuda")
        dec.prefill(torch.from_numpy(X0).cuda(), logits_out=z[0])
        seen = torch.zeros(dv.seen_words(shape.vocab), dtype=torch.int32, device="cuda")
        tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        dv.sample_topk(z[0], seen, 1.3, dv.Sampling(*cfg1, ud[0:1]), tok)
        first = int(tok.item())
        if mode == "eager":
            toks = []
            for i in range(n1 + n2):
                cfg = cfg1 if i < n1 else cfg2
                dec.step(tok.view(1, 1), [0], logits_out=z)
                dv.sample_topk(z[0], seen, 1.3, dv.Sampling(*cfg, ud[1 + i:2 + i]), tok)
                toks.append(int(tok.item()))
        else:
            out = torch.zeros(n1 + n2, dtype=torch.int32, device="cuda")
            dec.generate(n1, tok, seen=seen, penalty=1.3, tokens_out=out[:n1], logits_out=z[0],
                         sampling=dv.Sampling(*cfg1, ud[1:1 + n1]))
            dec.generate(n2, tok, seen=seen, penalty=1.3, tokens_out=out[n1:], logits_out=z[0],
                         sampling=dv.Sampling(*cfg2, ud[1 + n1:]))
            torch.cuda.synchronize()
            toks = out.cpu().tolist()
        torch.cuda.synchronize()
        assert dec.position(0)[0] == 9 + n1 + n2
        res.append(([first] + toks, z[0].cpu().numpy().copy(), seen.cpu().numpy().copy()))
        dec.close()
    assert res[0][0] == res[1][0]
    assert np.array_equal(res[0][1], res[1][1])
    assert np.array_equal(res[0][2], res[1][2])

    # the oracle's sampled run (settings 1 throughout; compared over the
    # first n1 + 1 choices, which used settings 1 on the device too)
    om = oracle_from_weights(mw)
    ref, _ = od.run_lm(om, X0, n1, 128, rho=1.3, sampling=cfg1 + (u,))
    checked = _follow([(res[1][0][k], ref[k][2], ref[k][3]) for k in range(n1 + 1)])
    _log(f"sampled generate: graph == eager over {n1 + n2} steps; {checked} tokens equal to "
         f"the oracle before its first close decision")
    assert checked >= 8


def test_talker06_sampled_frames():
    """The 0.6B frame loop with the log's default sampling (top-k 50, top-p
    1, temperature 0.9, penalty 1.05 on the main code; the same settings
    for the Code Predictor): graph-replayed frames equal eager C-ABI calls
    with the same uniforms bit for bit, a replay reproduces them, other
    uniforms change them, and the codes follow the oracle's sampled loop up
    to its first close decision."""
    wl = inputs.WORKLOADS["talker0.6b"]
    n_frames = 6
    tmw = inputs.make_weights(wl.model, seed=0, gain_sd=GAIN_SD)
    cmw = inputs.make_weights(wl.cp, seed=0, tables=tmw.tables, gain_sd=GAIN_SD)
    X0 = inputs.prefill_embeddings(wl, seed=0)
    text = inputs.text_embeddings(wl, seed=0)
    ut = inputs.uniforms(0, 1, n_frames)
    uc = inputs.uniforms(0, 2, (n_frames, 15))
    cfg = (50, 0.9, 1.0)

    tdm = dv.DeviceModel(tmw)
    cdm = dv.DeviceModel(cmw, tables=tdm.tables)
    tdec = dv.Decoder(tdm, max_slots=1, max_rows=wl.prefill, max_ctx=wl.s_init)
    cdec = dv.Decoder(cdm, max_slots=1, max_rows=2, max_ctx=inputs.CP_CAPACITY)
    tdec.grow(0, wl.s_init)
    cdec.grow(0, inputs.CP_CAPACITY)
    h, Vt, Vc = wl.model.hidden, wl.model.vocab, wl.cp.vocab
    text_d = torch.from_numpy(text).cuda()
    X0_d = torch.from_numpy(X0).cuda()
    ut_d = torch.from_numpy(ut).cuda()
    uc_d = torch.from_numpy(uc).cuda()

    def start(ut_dev):
        y = torch.empty(h, device="cuda")
        zt = torch.empty(Vt, device="cuda")
        codes = torch.zeros(16, dtype=torch.int32, device="cuda")
        seen = torch.zeros(dv.seen_words(Vt), dtype=torch.int32, device="cuda")
        tdec.prefill(X0_d, y_out=y, logits_out=zt)
        dv.sample_topk(zt, seen, wl.penalty, dv.Sampling(*cfg, ut_dev[0:1]), codes[0:1])
        return y, zt, codes, seen

    def native(ut_dev, uc_dev):
        y, zt, codes, seen = start(ut_dev)
        out = torch.full((n_frames, 16), -1, dtype=torch.int32, device="cuda")
        dv.talker_frames(tdec, cdec, n_frames, codes, y, text_d, seen, wl.penalty, codes_out=out,
                         tk_sampling=dv.Sampling(*cfg, ut_dev),
                         cp_sampling=dv.Sampling(*cfg, uc_dev))
        torch.cuda.synchronize()
        return out.cpu().numpy(), y.cpu().numpy()

    got, y_n = native(ut_d, uc_d)
    again, _ = native(ut_d, uc_d)
    assert (again == got).all()
    other, _ = native(torch.from_numpy(inputs.uniforms(0, 3, n_frames)).cuda(),
                      torch.from_numpy(inputs.uniforms(0, 4, (n_frames, 15))).cuda())
    assert not (other == got).all()

    # eager calls with the same uniforms
    y, zt, codes, seen = start(ut_d)
    cp_x = torch.empty(2, h, device="cuda")
    zc = torch.empty(Vc, device="cuda")
    eager = []
    for f in range(n_frames):
        if f > 0:
            tdec.step(codes.view(1, 16), list(range(16)), extra=text_d[f:f + 1], y_out=y.view(1, h),
                      logits_out=zt.view(1, Vt))
            dv.sample_topk(zt, seen, wl.penalty, dv.Sampling(*cfg, ut_d[f:f + 1]), codes[0:1])
        cp_x[0].copy_(y)
        cdec.embed(codes[0:1].view(1, 1), [0], cp_x[1:2])
        cdec.prefill(cp_x, head=0, logits_out=zc)
        dv.sample_topk(zc, None, 1.0, dv.Sampling(*cfg, uc_d[f, 0:1]), codes[1:2])
        for j in range(1, 15):
            cdec.step(codes[j:j + 1].view(1, 1), [j], head=j, logits_out=zc.view(1, Vc))
            dv.sample_topk(zc, None, 1.0, dv.Sampling(*cfg, uc_d[f, j:j + 1]), codes[j + 1:j + 2])
        eager.append(codes.cpu().numpy().copy())
    torch.cuda.synchronize()
    assert (np.stack(eager) == got).all()
    assert np.array_equal(y.cpu().numpy(), y_n)

    ot = oracle_from_weights(tmw, np.float32)
    oc = oracle_from_weights(cmw, np.float32)
    frames, _ = od.run_talker(ot, oc, X0, text, n_frames, wl.s_init, rho=wl.penalty,
                              cp_capacity=inputs.CP_CAPACITY, tk_sampling=cfg + (ut,),
                              cp_sampling=cfg + (uc,))
    seq = []
    for f in range(n_frames):
        fr = frames[f]
        seq.append((int(got[f, 0]), fr["c0"], fr["margin"]))
        seq += [(int(got[f, j + 1]), fr["codes"][j], fr["cp"][j][2]) for j in range(15)]
    checked = _follow(seq)
    _log(f"sampled frames: {n_frames} frames equal to eager calls; {checked} codes equal to the "
         f"oracle before its first close decision")
    assert checked >= 16
    tdec.close()
    cdec.close()
