"""Matrix-core (MFMA) path against the CPU oracle: prefill blocks and batched
steps of 5 or more rows run as 64-row GEMM chunks (bf16 hi/lo activations,
float32 accumulation).  Same bar as the vector path: normwise max relative
error <= 2e-3 on y and logits, tokens equal where the oracle's top-2 margin
exceeds 1e-2."""

import numpy as np
import pytest
import torch

from autoregressive_transformer_decode_amd import device as dv
from autoregressive_transformer_decode_amd import inputs
from oracle import decoder as od
from tests._models import normwise_rel, oracle_from_weights
from tests.gpu_util import GAIN_SD, MARGIN, TOL, lm_parity, small_shape

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


# h, Hq*D and F multiples of 32 (MFMA-eligible); N ragged against the
# 64-row workgroup tile (o and down 288, vocab 1000) and K ragged against the
# 64-wide pipeline stage (h = 288 and F = 672 end in a half stage)
MFMA_SHAPE = ("mfma", 2, 288, 8, 2, 128, 672, 1000, "bf16", True, True)


@pytest.mark.parametrize("T", [5, 64, 66, 133, 514, 600])
def test_prefill_chunks(T):
    """Prefill of T rows: one chunk of ragged 64-row tiles (5, 64, 66, 133), a
    full 512-row chunk then a 2-row tail on the vector path (514) or a second
    MFMA chunk (600); then teacher-forced steps read the KV rows every chunk
    appended."""
    shape = small_shape(*MFMA_SHAPE)
    mw = inputs.make_weights(shape, seed=7, gain_sd=GAIN_SD)
    X0 = inputs.normal(7, 2, 11, (T, shape.hidden), scale=1.0)
    chk, ref, _ = lm_parity(mw, X0, 6, 256 if T < 256 else 1024)
    _log(f"prefill T={T}: {chk.n} checks, worst {chk.worst:.2e}, tokens {chk.tokens_checked}")


PREFILL_ATTN = [
    # name, L, h, Hq, Hkv, D, F, V, dtype, qk_norm, bias, kv dtype, T
    ("r1_d64_kvf32", 2, 256, 4, 4, 64, 512, 600, "bf16", False, True, "f32", 97),
    ("r2_d64_kvbf16", 2, 256, 4, 2, 64, 512, 600, "bf16", True, False, "bf16", 130),
    ("r2_d128_kvf32", 2, 256, 4, 2, 128, 512, 600, "bf16", True, False, "f32", 300),
    ("r4_d64_kvf32", 2, 256, 8, 2, 64, 512, 600, "bf16", True, True, "f32", 45),
    ("r8_d128_kvf32", 2, 256, 8, 1, 128, 512, 600, "bf16", True, True, "f32", 70),
    ("r8_d128_kvbf16", 2, 256, 8, 1, 128, 512, 600, "bf16", False, False, "bf16", 17),
]


@pytest.mark.parametrize("case", PREFILL_ATTN, ids=[c[0] for c in PREFILL_ATTN])
def test_prefill_attention_group_sizes(case):
    """Prefill chunks' causal attention (16 query rows x a KV head's query
    heads per workgroup, key tiles split over waves and merged) for every
    GQA group size, both head dims and both cache dtypes, T ragged against
    the 16-row and 64-key tiles; later layers and the teacher-forced steps
    read every prefill row's keys."""
    name, L, h, hq, hkv, D, F, V, dt, qk, bias, kvdt, T = case
    shape = small_shape(name, L, h, hq, hkv, D, F, V, dt, qk, bias, kv_dtype=kvdt)
    mw = inputs.make_weights(shape, seed=17, gain_sd=GAIN_SD)
    X0 = inputs.normal(17, 2, 13, (T, h), scale=1.0)
    chk, ref, _ = lm_parity(mw, X0, 4, 512)
    _log(f"prefill attention {name} T={T}: {chk.n} checks, worst {chk.worst:.2e}")


TILE_GEMM = [
    # name, L, h, Hq, Hkv, D, F, V, dtype, qk_norm, bias, T
    # 450 rows (4 row tiles of 128, the last one ragged): QKV, O, gate/up and
    # down take the 128 x 128 tiles; N = 1248 ragged against them; QKV and
    # down end in a short split; 20 / 10-stage splits take the stage loop,
    # O's 8-stage splits the unrolled ring
    ("tiles_ragged", 2, 1248, 16, 8, 128, 2496, 3001, "bf16", True, True, 450),
    # 200 rows: gate/up on the 128 x 128 tiles in 5 splits of 4 unrolled
    # stages, the last split holding one real stage (three zeroed)
    ("tiles_short_split", 2, 544, 8, 2, 128, 1792, 1000, "bf16", True, False, 200),
    # 520 rows: a 512-row chunk whose reductions take 4 columns per thread
    # (the residual's last wave on a partial 256-column block of h = 1248),
    # then an 8-row chunk on one column per thread
    ("tiles_vec4_reduce", 2, 1248, 16, 8, 128, 2496, 3001, "bf16", True, True, 520),
]


@pytest.mark.parametrize("case", TILE_GEMM, ids=[c[0] for c in TILE_GEMM])
def test_prefill_tile_gemm(case):
    """Prefill chunks whose GEMMs give every compute unit a 128 x 128-tile
    workgroup run on those tiles (the host's split rule decides per GEMM);
    shapes chosen so the tiles meet ragged N, rows past the call, short
    final splits and both the unrolled and the looped stage walk."""
    name, L, h, hq, hkv, D, F, V, dt, qk, bias, T = case
    shape = small_shape(name, L, h, hq, hkv, D, F, V, dt, qk, bias)
    mw = inputs.make_weights(shape, seed=19, gain_sd=GAIN_SD)
    X0 = inputs.normal(19, 2, 17, (T, h), scale=1.0)
    chk, ref, _ = lm_parity(mw, X0, 3, 512 if T + 3 < 512 else 1024)
    _log(f"tile GEMM {name} T={T}: {chk.n} checks, worst {chk.worst:.2e}")


@pytest.mark.parametrize("T", [200, 700])
def test_prefill_every_row_keys(T):
    """Every prefill row, not only the last: the last layer's K and V rows at
    all T positions (each one depends on the earlier layers' attention
    output of its own row, so on the causal attention over the rows before
    it) match the oracle's cache, row by row, to the bar; T = 700 spans a
    512-row chunk and a second one that reads its keys."""
    shape = small_shape("rows", 3, 256, 8, 2, 128, 512, 600, "bf16", True, False, kv_dtype="f32")
    mw = inputs.make_weights(shape, seed=29, gain_sd=GAIN_SD)
    X0 = inputs.normal(29, 2, 23, (T, shape.hidden), scale=1.0)
    om = oracle_from_weights(mw)
    cache = od.Cache(om, 1024)
    od.prefill(om, cache, X0, 0)
    dm = dv.DeviceModel(mw)
    dec = dv.Decoder(dm, max_slots=1, max_rows=T, max_ctx=1024)
    dec.grow(0, 1024)
    y = torch.empty(shape.hidden, device="cuda")
    z = torch.empty(shape.vocab, device="cuda")
    dec.prefill(torch.from_numpy(np.asarray(X0, np.float32)).cuda(), y_out=y, logits_out=z)
    torch.cuda.synchronize()
    ks, vs = dec.kv[0]
    last = shape.n_layers - 1
    Kg = ks[last].float().cpu().numpy()[:, :T]
    Vg = vs[last].float().cpu().numpy()[:, :T]
    dec.close()
    worst = 0.0
    for t in range(T):
        e = max(normwise_rel(Kg[:, t], cache.K[last][:, t]),
                normwise_rel(Vg[:, t], cache.V[last][:, t]))
        worst = max(worst, e)
        assert e <= TOL, f"row {t}: normwise error {e:.3e} > {TOL}"
    _log(f"prefill T={T}: every row's last-layer K/V, worst {worst:.2e}")


def test_prefill_mfma_equals_vector_path():
    """The same prefill through both paths agrees to the tolerance (and
    both agree with the oracle)."""
    shape = small_shape(*MFMA_SHAPE)
    mw = inputs.make_weights(shape, seed=8, gain_sd=GAIN_SD)
    X0 = torch.from_numpy(inputs.normal(8, 2, 12, (100, shape.hidden), scale=1.0)).cuda()
    dm = dv.DeviceModel(mw)
    out = []
    for mfma in (True, False):
        dec = dv.Decoder(dm, max_slots=1, max_rows=100, max_ctx=128, mfma=mfma)
        dec.grow(0, 128)
        y = torch.empty(shape.hidden, device="cuda")
        z = torch.empty(shape.vocab, device="cuda")
        dec.prefill(X0, y_out=y, logits_out=z)
        torch.cuda.synchronize()
        out.append((y.cpu().numpy(), z.cpu().numpy()))
        dec.close()
    e = max(normwise_rel(out[0][0], out[1][0]), normwise_rel(out[0][1], out[1][1]))
    _log(f"mfma vs vector prefill: {e:.2e}")
    assert e <= TOL


def test_batched_steps_across_chunks():
    """B = 69 streams (a 64-row chunk plus a 5-row chunk), each at its own
    position; every stream equals its own oracle run for several steps."""
    shape = small_shape(*MFMA_SHAPE)
    mw = inputs.make_weights(shape, seed=9, gain_sd=GAIN_SD)
    om = oracle_from_weights(mw)
    dm = dv.DeviceModel(mw)
    Bn, steps = 69, 3
    lens = [1 + (7 * b) % 40 for b in range(Bn)]
    dec = dv.Decoder(dm, max_slots=Bn, max_rows=Bn, max_ctx=64)
    caches, toks = [], []
    for b in range(Bn):
        dec.grow(b, 64)
        X = inputs.normal(9, 2, 200 + b, (lens[b], shape.hidden), scale=1.0)
        c = od.Cache(om, 64)
        _, z = od.prefill(om, c, X, 0)
        caches.append(c)
        toks.append(int(np.argmax(z)))
        dec.prefill(torch.from_numpy(X).cuda(), slot=b)
    y = torch.empty(Bn, shape.hidden, device="cuda")
    z = torch.empty(Bn, shape.vocab, device="cuda")
    worst = 0.0
    for k in range(steps):
        tok = torch.tensor(toks, dtype=torch.int32, device="cuda").view(Bn, 1)
        dec.step(tok, [0], slot0=0, nrows=Bn, y_out=y, logits_out=z)
        torch.cuda.synchronize()
        yg, zg = y.cpu().numpy(), z.cpu().numpy()
        for b in range(Bn):
            yr, zr = od.step(om, caches[b], od.embed(om, [toks[b]], [0]), 0)
            e = max(normwise_rel(yg[b], yr), normwise_rel(zg[b], zr))
            worst = max(worst, e)
            assert e <= TOL, (k, b, e)
            toks[b] = int(np.argmax(zr))
    for b in range(Bn):
        assert dec.position(b)[0] == lens[b] + steps
    dec.close()
    _log(f"batched 69 streams: worst {worst:.2e}")


def test_batched64_full_size_sampled_streams():
    """The batched workload at its full size: the 1.7B shape, 64 streams with
    seeded KV lengths in [256, 4096], bf16 weights and KV, one step per
    stream per iteration.  Eight streams are checked against the oracle over
    two iterations (the first from given inputs, the second from tokens): the
    first and last rows of each 32-row half of the 64-row tile (0, 31, 32, 63),
    the shortest and the longest context, and two in between."""
    wl = inputs.WORKLOADS["batched64"]
    s = wl.model
    lens = inputs.batched_lengths(wl, seed=0)
    X1 = inputs.batched_first_inputs(wl, seed=0)
    mw = inputs.make_weights(s, seed=0, gain_sd=GAIN_SD)
    dm = dv.DeviceModel(mw)
    Bn = wl.batch
    dec = dv.Decoder(dm, max_slots=Bn, max_rows=Bn, max_ctx=wl.s_max)
    caps = [int(l) + 8 for l in lens]
    for b in range(Bn):
        dec.grow(b, caps[b])
    sample = sorted({0, 31, 32, 63, int(np.argmin(lens)), int(np.argmax(lens)), 17, 45})
    om = oracle_from_weights(mw, np.float32)
    caches = {b: od.Cache(om, caps[b]) for b in sample}
    dv.fill_batched_caches(dec, lens, seed=0)
    for l in range(s.n_layers):
        pool = inputs.batched_kv_pool(s, l, seed=0)
        for b in sample:
            k, v = inputs.batched_kv(s, b, int(lens[b]), l, pool=pool)
            caches[b].K[l][:, :lens[b]] = inputs.bf16_bits_to_f32(k)
            caches[b].V[l][:, :lens[b]] = inputs.bf16_bits_to_f32(v)
    for b in sample:
        caches[b].pos = int(lens[b])
    torch.cuda.synchronize()
    _log(f"batched64: caches filled, sample streams {sample} lengths {[int(lens[b]) for b in sample]}")

    y = torch.empty(Bn, s.hidden, device="cuda")
    z = torch.empty(Bn, s.vocab, device="cuda")
    tok = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    margin = torch.zeros(Bn, device="cuda")
    dec.step(None, [], nrows=Bn, extra=torch.from_numpy(X1).cuda(), y_out=y, logits_out=z)
    dv.greedy_argmax(z, None, 1.0, tok, margin)
    torch.cuda.synchronize()
    worst, feed = 0.0, {}
    for b in sample:
        yr, zr = od.step(om, caches[b], X1[b].astype(np.float32), 0)
        e = max(normwise_rel(y[b].cpu().numpy(), yr), normwise_rel(z[b].cpu().numpy(), zr))
        worst = max(worst, e)
        assert e <= TOL, (0, b, e)
        top = np.sort(zr)[-2:]
        if top[1] - top[0] > MARGIN:
            assert int(tok[b].item()) == int(np.argmax(zr)), b
        feed[b] = int(np.argmax(zr))
    for b, t in feed.items():      # teacher-force the oracle's tokens
        tok[b] = t
    dec.step(tok.view(Bn, 1), [0], nrows=Bn, y_out=y, logits_out=z)
    torch.cuda.synchronize()
    for b in sample:
        yr, zr = od.step(om, caches[b], od.embed(om, [feed[b]], [0]), 0)
        e = max(normwise_rel(y[b].cpu().numpy(), yr), normwise_rel(z[b].cpu().numpy(), zr))
        worst = max(worst, e)
        assert e <= TOL, (1, b, e)
    for b in range(Bn):
        assert dec.position(b)[0] == int(lens[b]) + 2
    dec.close()
    _log(f"batched64 full size: worst {worst:.2e}")
