"""Pins of the CPU oracle: checks against closed forms, invariants, library
routines and brute force, each raising AssertionError on failure.

They are functions (not tests) so that tests/test_oracle_pins.py can run each
one on the real oracle and, with a planted mistake, show that it fails."""

from __future__ import annotations

import dataclasses
import math
import os

import numpy as np

from autoregressive_transformer_decode_amd import inputs
from oracle import brute
from oracle import decoder as od
from oracle import quant as oq
from oracle import codec as oc
from tests._models import tiny_model

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, tol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)
    assert err <= tol, f"normwise error {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- RMSNorm

def check_rms_closed_form():
    """[3, 4] has mean square 12.5; unit gains give [3, 4] / sqrt(12.5 + eps)."""
    x = np.array([3.0, 4.0])
    got = od.rms_norm(x, np.ones(2), 1e-6)
    exp = np.array([3.0, 4.0]) / math.sqrt(12.5 + 1e-6)
    _close(got, exp, 1e-15)
    # gains multiply the normalised value (x_hat * g)
    got2 = od.rms_norm(x, np.array([2.0, 0.5]), 1e-6)
    _close(got2, exp * np.array([2.0, 0.5]), 1e-15)


def check_rms_invariant():
    """With g = 1 the output's root-mean-square is 1/sqrt(1 + eps/mean(x^2))."""
    rng = np.random.default_rng(3)
    for scale in (1e-3, 1.0, 50.0):
        x = rng.standard_normal(64) * scale
        eps = 1e-6
        y = od.rms_norm(x, np.ones(64), eps)
        ms = np.mean(x * x)
        assert abs(math.sqrt(np.mean(y * y)) - 1 / math.sqrt(1 + eps / ms)) < 1e-12


# ---------------------------------------------------------------- bf16

def check_bf16_vs_torch():
    """Round-to-nearest-even to bf16 agrees with torch's float32 -> bfloat16."""
    import torch
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 3,
        np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, 2**-130,
                  65504.0, 1.00390625, 1.01171875], np.float32)])
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = od.bf16_round(x)
    assert np.array_equal(got, t), "oracle bf16 rounding differs from torch"
    got_b = np.array([brute._bf16(float(v)) for v in x], np.float32)
    normal = np.abs(x) >= 2**-126
    assert np.array_equal(got_b[normal], t[normal]), "brute bf16 differs from torch"


# ---------------------------------------------------------------- RoPE

def check_rope_hand_values():
    """D = 4, theta = 100, position 1: channel pairs (0,2) and (1,3) turn by
    1 rad and 0.1 rad (omega_i = theta^(-2i/D)), counter-clockwise."""
    cos, sin = od.rope_cos_sin(1, 4, 100.0)
    e0 = od.rope(np.array([1.0, 0, 0, 0]), cos, sin)
    e1 = od.rope(np.array([0, 1.0, 0, 0]), cos, sin)
    e2 = od.rope(np.array([0, 0, 1.0, 0]), cos, sin)
    _close(e0, [math.cos(1), 0, math.sin(1), 0], 1e-7)
    _close(e1, [0, math.cos(0.1), 0, math.sin(0.1)], 1e-7)
    _close(e2, [-math.sin(1), 0, math.cos(1), 0], 1e-7)


def check_rope_complex_form():
    """Rotate-half RoPE equals multiplying z = a + ib (a = v[:D/2], b =
    v[D/2:]) by exp(i*phi); position 0 is the identity; norms of every pair
    are preserved."""
    rng = np.random.default_rng(7)
    D = 16
    v = rng.standard_normal(D)
    for p in (0, 1, 5, 1000):
        cos, sin = od.rope_cos_sin(p, D, 1.0e6)
        got = od.rope(v, cos, sin)
        phi = p * 1.0e6 ** (-2.0 * np.arange(D // 2) / D)
        z = (v[:D // 2] + 1j * v[D // 2:]) * np.exp(1j * phi)
        _close(got, np.concatenate([z.real, z.imag]), 1e-6)
        pairs = got[:D // 2] ** 2 + got[D // 2:] ** 2
        _close(pairs, v[:D // 2] ** 2 + v[D // 2:] ** 2, 1e-6)
        if p == 0:
            assert np.array_equal(got, v)


def check_rope_relative():
    """RoPE_m(q) . RoPE_n(k) depends only on m - n."""
    rng = np.random.default_rng(8)
    D = 32
    q, k = rng.standard_normal(D), rng.standard_normal(D)

    def dot(m, n):
        cm, sm = od.rope_cos_sin(m, D, 1.0e4)
        cn, sn = od.rope_cos_sin(n, D, 1.0e4)
        return od.rope(q, cm, sm) @ od.rope(k, cn, sn)

    for m, n, s in ((3, 1, 10), (7, 7, 100), (2, 9, 33)):
        assert abs(dot(m, n) - dot(m + s, n + s)) < 1e-5


def check_mrope_degenerates():
    """Interleaved mRoPE with equal t/h/w positions is plain RoPE (ncnn port,
    Talker section: for TTS the three positions agree and the interleave
    reduces to ordinary RoPE), bit for bit, for [24, 20, 20] at D = 128."""
    D = 128
    for p in (0, 1, 37, 4095):
        c, s = od.mrope_cos_sin((p, p, p), D, 1.0e6, (24, 20, 20))
        c0, s0 = od.rope_cos_sin(p, D, 1.0e6)
        assert np.array_equal(c, c0) and np.array_equal(s, s0)


def check_mrope_sections():
    """The frequency map of [24, 20, 20] at D = 128 is the one the ncnn port
    derives per channel: base = c mod (D/2), modality base mod 3 when
    base < 60, else 0 (t); it gives 24 / 20 / 20 frequencies to t / h / w."""
    D = 128
    m = od.mrope_modality(D // 2, (24, 20, 20))
    for c in range(D):
        base = c % (D // 2)
        assert m[base] == (base % 3 if base < 60 else 0)
    assert [int(np.sum(m == k)) for k in range(3)] == [24, 20, 20]


def check_mrope_single_component():
    """Positions (0, p, 0): the channel pairs of the h frequencies turn by
    p omega_i, the rest are left as they are (a turn by angle 0); likewise
    for w, and for t with (p, 0, 0)."""
    D = 128
    rng = np.random.default_rng(10)
    v = rng.standard_normal(D)
    half = D // 2
    i = np.arange(half)
    for comp in range(3):
        p = 29
        pos3 = [0, 0, 0]
        pos3[comp] = p
        got = od.rope(v, *od.mrope_cos_sin(pos3, D, 1.0e6, (24, 20, 20)))
        if comp == 0:
            moving = (i % 3 == 0) | (i >= 60)
        else:
            moving = (i % 3 == comp) & (i < 60)
        turned = od.rope(v, *od.rope_cos_sin(p, D, 1.0e6))
        keep = np.concatenate([~moving, ~moving])
        assert np.array_equal(got[keep], v[keep])
        _close(got[~keep], turned[~keep], 1e-15)


def check_mrope_relative():
    """q turned at (t1, h1, w1) against k at (t2, h2, w2): the dot product
    depends only on the three differences (up to the float32 rounding of
    cos and sin); a change of one difference alone changes it."""
    D = 64
    rng = np.random.default_rng(11)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    sec = (12, 10, 10)

    def dot(a, b):
        return (od.rope(q, *od.mrope_cos_sin(a, D, 1.0e4, sec)) @
                od.rope(k, *od.mrope_cos_sin(b, D, 1.0e4, sec)))

    a, b = (9, 3, 5), (4, 1, 7)
    base = dot(a, b)
    for sh in ((10, 0, 0), (0, 6, 0), (0, 0, 13), (2, 40, 7)):
        a2 = tuple(x + y for x, y in zip(a, sh))
        b2 = tuple(x + y for x, y in zip(b, sh))
        assert abs(dot(a2, b2) - base) < 1e-5      # cos / sin are float32
    for comp in range(3):
        a3 = list(a)
        a3[comp] += 3
        assert abs(dot(tuple(a3), b) - base) > 1e-3


def check_mrope_model_brute():
    """A stack with interleaved sections (4, 2, 2) at D = 16 and distinct
    t/h/w positions: the cached prefill and the following steps equal the
    brute-force recompute, which turns every frequency by its own position
    in scalar loops; the cache rows still go to positions 0, 1, 2, ..."""
    m = dataclasses.replace(tiny_model(L=2, h=16, hq=2, hkv=1, D=16, F=16, V=24, qk_norm=True,
                                       bias=True, seed=24, scale=0.5),
                            mrope_sections=(4, 2, 2))
    rng = np.random.default_rng(25)
    rows = [rng.standard_normal(16) for _ in range(7)]
    # vision-like rows share t and walk a 2 x 2 grid; text rows continue at t = h = w
    rpos = np.array([[0, 0, 0], [1, 1, 1], [2, 2, 2], [2, 2, 3], [2, 3, 2], [2, 3, 3],
                     [4, 4, 4]])
    cache = od.Cache(m, 8)
    y, z = od.prefill(m, cache, np.stack(rows[:4]), 0, rope_pos=rpos[:4])
    yb, zb = brute.last_outputs(m, rows[:4], rope_pos=rpos[:4])
    _close(y, yb, 1e-9)
    _close(z, zb, 1e-9)
    for t in range(4, 7):
        y, z = od.step(m, cache, rows[t], 0, rope_pos=rpos[t])
        yb, zb = brute.last_outputs(m, rows[:t + 1], rope_pos=rpos[:t + 1])
        _close(y, yb, 1e-9)
        _close(z, zb, 1e-9)
    assert cache.pos == 7
    # rotary positions that differ from the row index change the outcome
    _, z_plain = od.prefill(m, od.Cache(m, 8), np.stack(rows), 0)
    assert np.max(np.abs(z_plain - z)) > 1e-6


# ---------------------------------------------------------------- attention

def check_attention_closed_form():
    """q = 1 (D = 4), keys [1,1,1,1] and 0: scores 4/sqrt(4) = 2 and 0, so the
    weights are e^2/(e^2+1) and 1/(e^2+1) on values e0 and e1."""
    q = np.ones(4)
    K = np.array([[1.0, 1, 1, 1], [0, 0, 0, 0], [9, 9, 9, 9]])
    V = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0], [5, 5, 5, 5]])
    o = od.attention(q, K, V, 2)      # the third row is beyond the valid length
    a0 = math.e ** 2 / (math.e ** 2 + 1)
    _close(o, [a0, 1 - a0, 0, 0], 1e-14)


def check_attention_invariants():
    """One cached row returns its V; q = 0 gives the mean of V; the weights
    equal scipy's softmax of the scaled scores and sum to 1."""
    from scipy.special import softmax
    rng = np.random.default_rng(11)
    D, n = 8, 13
    K, V = rng.standard_normal((n + 3, D)), rng.standard_normal((n + 3, D))
    q = rng.standard_normal(D)
    _close(od.attention(q, K, V, 1), V[0], 1e-14)
    _close(od.attention(np.zeros(D), K, V, n), V[:n].mean(0), 1e-13)
    eye = np.eye(n + 3, n + 3)
    w = od.attention(q, K, eye, n)
    ref = softmax(K[:n] @ q / math.sqrt(D))
    _close(w[:n], ref, 1e-13)
    assert abs(w.sum() - 1.0) < 1e-13


def check_gqa_equals_mha():
    """GQA over Hkv heads equals MHA over K, V repeated r times per head
    (numpy repeat = repeat_interleave: query head h reads KV head h // r)."""
    rng = np.random.default_rng(12)
    hq, hkv, S, D, n = 8, 2, 10, 4, 7
    q = rng.standard_normal((hq, D))
    K, V = rng.standard_normal((hkv, S, D)), rng.standard_normal((hkv, S, D))
    r = hq // hkv
    mha = od.gqa_attention(q, np.repeat(K, r, axis=0), np.repeat(V, r, axis=0), n)
    _close(od.gqa_attention(q, K, V, n), mha, 1e-14)


# ---------------------------------------------------------------- MLP

def check_mlp_closed_form():
    """Gate W_g = 2I, up W_u = I, down W_d = I, unit gains: the residual adds
    silu(2w) * w with w = RMSNorm(x); silu(z) = z * expit(z)."""
    from scipy.special import expit
    m = tiny_model(L=1, h=4, hq=2, hkv=1, D=2, F=4, bias=False, gains_random=False)
    L = m.layers[0]
    L["w_gate"], L["w_up"], L["w_down"] = 2 * np.eye(4), np.eye(4), np.eye(4)
    x = np.array([0.5, -1.0, 2.0, 0.25])
    w = x / math.sqrt(np.mean(x * x) + 1e-6)
    exp = x + (2 * w) * expit(2 * w) * w
    _close(od._mlp(m, L, x), exp, 1e-14)


def check_projection_orientation():
    """Weights are [out, in]: a permutation matrix permutes the input."""
    m = tiny_model(L=1, h=4, hq=2, hkv=1, D=2, F=4, bias=False, qk_norm=False,
                   gains_random=False)
    L = m.layers[0]
    P = np.eye(4)[[2, 0, 3, 1]]
    L["wq"] = P
    u = np.array([1.0, 2.0, 3.0, 4.0])
    q, _, _ = od._qkv(m, L, u)
    _close(q.reshape(-1), [3.0, 1.0, 4.0, 2.0], 0)


# ---------------------------------------------------------------- cache / stack

def _brute_model(kv_bf16, qk_norm=True, bias=True, hq=4, hkv=2):
    return tiny_model(L=2, h=12, hq=hq, hkv=hkv, D=4, F=16, V=24, qk_norm=qk_norm,
                      bias=bias, kv_bf16=kv_bf16, seed=21, scale=0.5)


def check_cached_equals_recompute(kv_bf16=False, qk_norm=True, bias=True, hq=4, hkv=2):
    """Cached decode (prefill 3 rows, then steps with bucket growth from
    capacity 4) equals a from-scratch recompute of the whole sequence at every
    step (float64 brute force, no cache)."""
    m = _brute_model(kv_bf16, qk_norm, bias, hq, hkv)
    rng = np.random.default_rng(22)
    rows = [rng.standard_normal(12) for _ in range(9)]
    cache = od.Cache(m, 4)
    y, z = od.prefill(m, cache, np.stack(rows[:3]), 0)
    yb, zb = brute.last_outputs(m, rows[:3])
    _close(y, yb, 1e-9)
    _close(z, zb, 1e-9)
    for t in range(3, 9):
        cap = od.bucket_for(cache.pos, cache.capacity)
        if cap != cache.capacity:
            cache.grow(cap)
        y, z = od.step(m, cache, rows[t], 0)
        yb, zb = brute.last_outputs(m, rows[:t + 1])
        _close(y, yb, 1e-9)
        _close(z, zb, 1e-9)
    assert cache.pos == 9 and cache.capacity == 16


def check_input_projection():
    """A stack with an input projection (inputs 10 wide, hidden 12): cached
    decode equals the brute-force recompute, which applies the projection to
    every row by scalar loops; with the projection the identity and no bias
    the stack equals the same stack without one."""
    m = _brute_model(False)
    rng = np.random.default_rng(23)
    W = rng.standard_normal((12, 10)) * 0.4
    bvec = rng.standard_normal(12) * 0.1
    mp = dataclasses.replace(m, in_proj=W, in_proj_bias=bvec,
                             tables=[rng.standard_normal((24, 10))])
    assert mp.input_dim == 10
    rows = [rng.standard_normal(10) for _ in range(6)]
    cache = od.Cache(mp, 8)
    y, z = od.prefill(mp, cache, np.stack(rows[:2]), 0)
    yb, zb = brute.last_outputs(mp, rows[:2])
    _close(z, zb, 1e-9)
    for t in range(2, 6):
        y, z = od.step(mp, cache, rows[t], 0)
        yb, zb = brute.last_outputs(mp, rows[:t + 1])
        _close(y, yb, 1e-9)
        _close(z, zb, 1e-9)
    x = od.embed(mp, [3], [0], rows[0])
    _close(x, mp.tables[0][3] + rows[0], 1e-15)
    mi = dataclasses.replace(m, in_proj=np.eye(12), in_proj_bias=None)
    r12 = [rng.standard_normal(12) for _ in range(3)]
    _close(od.prefill(mi, od.Cache(mi, 4), np.stack(r12), 0)[1],
           od.prefill(m, od.Cache(m, 4), np.stack(r12), 0)[1], 1e-12)


def check_prefill_equals_steps():
    """The block (matrix) prefill equals feeding its rows one at a time."""
    m = tiny_model(kv_bf16=True, seed=31)
    rng = np.random.default_rng(32)
    X = rng.standard_normal((6, 16))
    c1, c2 = od.Cache(m, 8), od.Cache(m, 8)
    y1, z1 = od.prefill(m, c1, X, 0)
    for t in range(6):
        y2, z2 = od.step(m, c2, X[t], 0)
    _close(y1, y2, 1e-12)
    _close(z1, z2, 1e-12)
    for l in range(m.n_layers):
        _close(c1.K[l][:, :6], c2.K[l][:, :6], 1e-12)


def check_bucket_copy_invariance():
    """Growing the cache 4 -> 8 -> 16 leaves every output bit-identical to a
    run that starts at capacity 16."""
    m = tiny_model(kv_bf16=True, seed=41)
    rng = np.random.default_rng(42)
    X = rng.standard_normal((12, 16))
    a, b = od.Cache(m, 4), od.Cache(m, 16)
    od.prefill(m, a, X[:2], 0)
    od.prefill(m, b, X[:2], 0)
    for t in range(2, 12):
        cap = od.bucket_for(a.pos, a.capacity)
        if cap != a.capacity:
            a.grow(cap)
        ya, za = od.step(m, a, X[t], 0)
        yb, zb = od.step(m, b, X[t], 0)
        assert np.array_equal(ya, yb) and np.array_equal(za, zb)
    assert a.capacity == 16


def check_code_predictor_recompute():
    """A Code Predictor pass with its per-frame cache (2-row prefill, then a
    step per group, head j for group j) equals recomputing every prefix from
    scratch (the ncnn port recomputes the Code Predictor each frame)."""
    m = tiny_model(L=2, h=12, hq=4, hkv=2, D=4, F=16, V=10, n_heads=4,
                   tables=(12, 10, 10, 10), bias=False, seed=51, scale=0.5)
    rng = np.random.default_rng(52)
    y_talker = rng.standard_normal(12)
    codes, trace = od.code_predictor_frame(m, y_talker, c0=5, cp_capacity=8)
    rows = [y_talker, m.tables[0][5]]
    for j in range(4):
        yb, zb = brute.last_outputs(m, rows, head=j)
        _close(trace[j][0], yb, 1e-9)
        _close(trace[j][1], zb, 1e-9)
        assert codes[j] == int(np.argmax(zb))
        if j + 1 < 4:
            rows.append(m.tables[j + 1][codes[j]])


def check_frame_input():
    """Talker frame input = E_tk[c0] + sum_j E_cp[j][c_j] + text: with
    one-hot tables the sum lands on known coordinates."""
    m = tiny_model(L=1, h=20, tables=(4, 3, 3), seed=61)
    m.tables = [np.eye(4, 20), np.eye(3, 20, k=4), np.eye(3, 20, k=7)]
    text = np.zeros(20)
    text[19] = 0.5
    x = od.embed(m, [2, 1, 0], [0, 1, 2], text)
    exp = np.zeros(20)
    exp[[2, 5, 7]] = 1.0
    exp[19] = 0.5
    _close(x, exp, 0)


# ---------------------------------------------------------------- loops

def _greedy_f32(z, seen, rho):
    """Penalised greedy choice written as a scalar float32 loop (independent of
    penalized_argmax): a seen token's logit is divided by rho when positive and
    multiplied by it otherwise; the lowest index of the maximum wins.  Returns
    (token, margin to the runner-up)."""
    r = np.float32(rho)
    vals = []
    for i, v in enumerate(np.asarray(z, np.float64)):
        v = np.float32(v)
        if seen is not None and i in seen:
            v = np.float32(v / r) if v > 0 else np.float32(v * r)
        vals.append(v)
    tok = 0
    for i in range(1, len(vals)):
        if vals[i] > vals[tok]:
            tok = i
    second = max(v for i, v in enumerate(vals) if i != tok)
    return tok, float(vals[tok] - second)


def check_run_lm_brute():
    """The plain LM loop against a from-scratch recompute (RKNN page:
    stepwise decode equals full recompute; Audio8-ASR report: growth when the
    write position reaches the bucket).  The prefill's last row gives token 1,
    step k feeds the embedding of token k (the previous choice), and every
    step's (y, z) equals the float64 brute force over all rows fed so far.
    The bucket starts at 4 and doubles right before a row lands on the
    capacity: 4 -> 8 before writing row 4, 8 -> 16 before row 8."""
    m = _brute_model(False)
    rng = np.random.default_rng(24)
    X0 = rng.standard_normal((3, 12))
    caps = []
    out, cache = od.run_lm(m, X0, 7, 4,
                           on_step=lambda k, c: caps.append((k, c.pos, c.capacity)))
    assert len(out) == 8, len(out)
    rows = list(X0)
    for k in range(8):
        yb, zb = brute.last_outputs(m, rows)
        _close(out[k][0], yb, 1e-9)
        _close(out[k][1], zb, 1e-9)
        tok, margin = _greedy_f32(zb, None, 1.0)
        assert margin > 1e-4, "fixture has a near tie"
        assert out[k][2] == tok, (k, out[k][2], tok)
        rows.append(m.tables[0][tok])
    assert caps == [(0, 3, 4), (1, 4, 4), (2, 5, 8), (3, 6, 8), (4, 7, 8), (5, 8, 8),
                    (6, 9, 16), (7, 10, 16)], caps


def check_run_lm_asr_stress_golden():
    """The Audio8-ASR report's 256->512 migration stress run through run_lm: an
    85-row prefill and 180 decoder steps give 181 tokens (the prefill's
    included); the bucket starts at 128 and migrates twice, to 256 in the step
    that writes row 128 (step 44) and to 512 in the step that writes row 256
    (step 172), ending at 512."""
    rows = {r[0]: r[1:] for r in read_golden("asr_bucket_runs.txt")}
    pre, toks, final, migr = (int(v) for v in rows["stress"])
    m = tiny_model(L=1, h=8, hq=2, hkv=1, D=4, F=8, V=16, tables=(16,), bias=True,
                   qk_norm=False, seed=71)
    X0 = np.random.default_rng(72).standard_normal((pre, 8))
    caps = []
    out, cache = od.run_lm(m, X0, toks - 1, 128,
                           on_step=lambda k, c: caps.append(c.capacity))
    assert len(out) == toks, len(out)
    moves = [k for k in range(1, len(caps)) if caps[k] != caps[k - 1]]
    assert (cache.capacity, len(moves)) == (final, migr), (cache.capacity, moves)
    assert moves == [128 - pre + 1, 256 - pre + 1], moves
    assert cache.pos == pre + toks - 1


def _talker_pair(seed):
    """A 1-layer Talker (6 main codes, 16 code tables) and a 1-layer Code
    Predictor (15 heads of 5 codes) sharing the code tables, as the 0.6B
    Talker and its Code Predictor do."""
    tk = tiny_model(L=1, h=16, hq=2, hkv=1, D=4, F=8, V=6, n_heads=1,
                    tables=(6,) + (5,) * 15, bias=False, seed=seed, scale=0.6)
    cp = tiny_model(L=1, h=16, hq=2, hkv=1, D=4, F=8, V=5, n_heads=15,
                    tables=(6,) + (5,) * 14, bias=False, seed=seed + 1, scale=0.6)
    cp.tables = tk.tables[:15]
    return tk, cp


def check_run_talker_brute(rho=4.0):
    """The two-level frame loop against a from-scratch recompute ("Qwen3-TTS
    ncnn port", Talker section).  The Talker's prefill gives frame 0's main
    code c0 (penalty over an empty seen set).  Frame f: the Code Predictor
    recomputes from rows [y_f, E_tk[c0_f]]; head j's greedy code is c_{j+1}
    and its table-j embedding is the next row.  The next Talker row is the sum
    of the frame's 16 code embeddings (table g holds group g) plus text row
    f + 1, and the next c0 is the penalised greedy choice over the c0 codes
    chosen so far.  rho = 4 makes the seen set decide choices: the same run
    with rho = 1 picks different main codes."""
    tk, cp = _talker_pair(81)
    rng = np.random.default_rng(82)
    X0 = rng.standard_normal((3, 16))
    n_frames = 4
    text = rng.standard_normal((n_frames, 16))
    frames, _ = od.run_talker(tk, cp, X0, text, n_frames, 8, rho=rho, cp_capacity=16)
    assert len(frames) == n_frames
    rows = list(X0)
    seen = set()
    y, z = brute.last_outputs(tk, rows)
    c0, margin = _greedy_f32(z, seen, rho)
    assert margin > 1e-4, "fixture has a near tie"
    main = []
    for f in range(n_frames):
        _close(frames[f]["y"], y, 1e-9)
        _close(frames[f]["z"], z, 1e-9)
        assert frames[f]["c0"] == c0, (f, frames[f]["c0"], c0)
        seen.add(c0)
        main.append(c0)
        cp_rows = [np.asarray(y), tk.tables[0][c0]]
        codes = []
        for j in range(15):
            yy, zz = brute.last_outputs(cp, cp_rows, head=j)
            _close(frames[f]["cp"][j][1], zz, 1e-9)
            c, mg = _greedy_f32(zz, None, 1.0)
            assert mg > 1e-4, "fixture has a near tie"
            codes.append(c)
            if j < 14:
                cp_rows.append(cp.tables[j + 1][c])
        assert frames[f]["codes"] == codes, (f, frames[f]["codes"], codes)
        if f + 1 == n_frames:
            break
        x = tk.tables[0][c0] + sum(tk.tables[g][codes[g - 1]] for g in range(1, 16)) + text[f + 1]
        rows.append(x)
        y, z = brute.last_outputs(tk, rows)
        c0, margin = _greedy_f32(z, seen, rho)
        assert margin > 1e-4, "fixture has a near tie"
    if rho != 1.0:
        plain, _ = od.run_talker(tk, cp, X0, text, n_frames, 8, rho=1.0, cp_capacity=16)
        assert [fr["c0"] for fr in plain] != main, "the penalty decides no choice here"


# ---------------------------------------------------------------- penalty / argmax

def check_penalty_and_argmax():
    z = np.array([2.0, -1.0, 2.05, 0.5], np.float32)
    # rho = 1: plain argmax, margin to the runner-up
    t, mg = od.penalized_argmax(z, None, 1.0)
    assert t == 2 and abs(mg - 0.05) < 1e-6
    # positive logit divided: 2.05 / 1.05 = 1.952 < 2.0
    seen = np.array([False, False, True, False])
    t, mg = od.penalized_argmax(z, seen, 1.05)
    assert t == 0 and abs(mg - (2.0 - np.float32(2.05) / np.float32(1.05))) < 1e-6
    assert seen[0] and seen[2]
    # negative logit multiplied: -1.0 * 1.05 = -1.05 < -1.02
    z2 = np.array([-1.0, -1.02], np.float32)
    t, _ = od.penalized_argmax(z2, np.array([True, False]), 1.05)
    assert t == 1
    # ties: lowest index, margin 0
    t, mg = od.penalized_argmax(np.array([1.0, 3.0, 3.0], np.float32), None, 1.0)
    assert t == 1 and mg == 0.0


# ---------------------------------------------------------------- sampling

# logits log(1), log(2), log(3), log(4): at temperature 1 the softmax is
# 0.1, 0.2, 0.3, 0.4
_LOG4 = np.log(np.array([1.0, 2.0, 3.0, 4.0])).astype(np.float32)


def _draw(z, k, t, top_p, u, seen=None, rho=1.0):
    return od.sample_topk(z, seen, rho, k, t, top_p, u).tok


def check_sampling_inverse_cdf():
    """Temperature 1, k = 4: the tokens in descending order of logit carry
    0.4, 0.3, 0.2, 0.1; the draw takes the first whose cumulative
    probability exceeds u (boundaries 0.4, 0.7, 0.9)."""
    toks, p, _, _ = od.sampling_distribution(_LOG4, None, 1.0, 4, 1.0)
    assert list(toks) == [3, 2, 1, 0]
    _close(p, [0.4, 0.3, 0.2, 0.1], 1e-6)
    for u, exp in [(0.0, 3), (0.35, 3), (0.45, 2), (0.75, 1), (0.95, 0), (0.99999, 0)]:
        assert _draw(_LOG4, 4, 1.0, 1.0, u) == exp, u


def check_sampling_temperature():
    """The temperature divides the logits: at 0.5 the weights are the squares
    1, 4, 9, 16 (/30), at 2 the square roots."""
    _, p, _, _ = od.sampling_distribution(_LOG4, None, 1.0, 4, 0.5)
    _close(p, np.array([16.0, 9.0, 4.0, 1.0]) / 30.0, 1e-6)
    r = np.sqrt(np.array([4.0, 3.0, 2.0, 1.0]))
    _, p2, _, _ = od.sampling_distribution(_LOG4, None, 1.0, 4, 2.0)
    _close(p2, r / r.sum(), 1e-6)
    # u = 0.35 lies below the first boundary at 0.5 (16/30 = 0.533) and 1.0
    # (0.4), above it at 2.0 (0.325)
    assert _draw(_LOG4, 4, 0.5, 1.0, 0.35) == 3
    assert _draw(_LOG4, 4, 1.0, 1.0, 0.35) == 3
    assert _draw(_LOG4, 4, 2.0, 1.0, 0.35) == 2
    assert _draw(_LOG4, 4, 0.5, 1.0, 0.9) == 1


def check_sampling_topk():
    """Top-k keeps the k largest and renormalises: k = 2 gives 4/7, 3/7;
    k = 3 gives 4/9, 3/9, 2/9."""
    toks, p, _, _ = od.sampling_distribution(_LOG4, None, 1.0, 2, 1.0)
    assert list(toks) == [3, 2]
    _close(p, [4 / 7, 3 / 7], 1e-6)
    toks, p, _, _ = od.sampling_distribution(_LOG4, None, 1.0, 3, 1.0)
    assert list(toks) == [3, 2, 1]
    _close(p, [4 / 9, 3 / 9, 2 / 9], 1e-6)
    assert _draw(_LOG4, 2, 1.0, 1.0, 0.5) == 3      # 0.5 < 4/7
    assert _draw(_LOG4, 2, 1.0, 1.0, 0.6) == 2
    assert _draw(_LOG4, 2, 1.0, 1.0, 0.99) == 2     # never a token outside the set


def check_sampling_top_p():
    """Top-p keeps the shortest descending prefix whose probability reaches
    top_p, over the top-k set."""
    cases = [(4, 0.6, [3, 2]), (4, 0.35, [3]), (4, 0.75, [3, 2, 1]), (4, 1.0, [3, 2, 1, 0]),
             (3, 0.8, [3, 2, 1]), (3, 0.7, [3, 2])]   # k = 3: cumulative 4/9, 7/9, 1
    for k, tp, exp in cases:
        toks, p, _, _ = od.sampling_distribution(_LOG4, None, 1.0, k, 1.0, tp)
        assert list(toks) == exp, (k, tp, list(toks))
        _close(p, np.array([4.0, 3.0, 2.0, 1.0])[:len(exp)] / (10 - sum(range(1, 5 - len(exp)))), 1e-6)
    assert _draw(_LOG4, 4, 1.0, 0.35, 0.99) == 3


def check_sampling_ties_and_penalty():
    """Equal logits: the set takes the lowest indices and shares the mass
    equally.  The penalty acts before the set is taken."""
    z = np.zeros(10, np.float32)
    toks, p, _, _ = od.sampling_distribution(z, None, 1.0, 3, 0.9)
    assert list(toks) == [0, 1, 2]
    _close(p, [1 / 3] * 3, 1e-12)
    assert _draw(z, 3, 0.9, 1.0, 0.5) == 1
    z2 = np.array([1.0, 2.0, 2.0, 2.0, 0.0], np.float32)
    toks, _, _, _ = od.sampling_distribution(z2, None, 1.0, 2, 1.0)
    assert list(toks) == [1, 2]
    z3 = np.array([3.0, 2.9, 1.0], np.float32)
    seen = np.array([True, False, False])
    assert _draw(z3, 1, 1.0, 1.0, 0.3, seen.copy(), 1.2) == 1    # 3.0 / 1.2 = 2.5 < 2.9
    toks, _, _, _ = od.sampling_distribution(z3, seen, 1.2, 2, 1.0)
    assert list(toks) == [1, 0]
    s2 = seen.copy()
    od.sample_topk(z3, s2, 1.2, 1, 1.0, 1.0, 0.3)
    assert s2[1] and s2[0] and not s2[2]


def check_sampling_greedy_limit():
    """k = 1 is the penalized argmax for every u (ties included)."""
    z = inputs.normal(5, 9, 1, (300,), scale=1.0)
    z[17] = z[200] = z.max() + 1.0          # the penalty breaks this tie
    seen = np.zeros(300, bool)
    seen[[3, 17, 50]] = True
    z2 = z.copy()
    z2[260] = z2[250] = z.max() + 2.0       # an exact tie: the lower index
    for zz, exp in ((z, 200), (z2, 250)):
        for u in (0.0, 0.3, 0.999):
            t = od.sample_topk(zz, seen.copy(), 1.05, 1, 0.9, 1.0, u).tok
            g, _ = od.penalized_argmax(zz, seen.copy(), 1.05)
            assert t == g == exp, (t, g, exp)


def _brute_distribution(z, seen, rho, k, t, top_p):
    """Scalar float64 definition: penalise, sort (value desc, index asc), keep
    k, exp(z / t) normalised, shortest prefix reaching top_p."""
    zp = []
    for i, v in enumerate(z.tolist()):
        if seen is not None and seen[i]:
            v = v / rho if v > 0 else v * rho
        zp.append(v)
    order = sorted(range(len(zp)), key=lambda i: (-zp[i], i))[:k]
    w = [math.exp(zp[i] / t) for i in order]
    tot = sum(w)
    keep, acc = [], 0.0
    for i, wi in zip(order, w):
        keep.append((i, wi))
        acc += wi / tot
        if acc >= top_p:
            break
    s = sum(wi for _, wi in keep)
    return {i: wi / s for i, wi in keep}


def check_sampling_frequencies():
    """Brute force: over a uniform grid of u the draw hits each token with
    its probability (within one grid step) and never a token outside the
    kept set."""
    z = inputs.normal(6, 9, 2, (60,), scale=1.5)
    seen = np.zeros(60, bool)
    seen[::7] = True
    n = 4000
    for k, t, tp in [(10, 0.7, 1.0), (25, 1.3, 0.8), (60, 0.9, 1.0)]:
        exp = _brute_distribution(z, seen, 1.05, k, t, tp)
        hits = {}
        for i in range(n):
            tok = _draw(z, k, t, tp, (i + 0.5) / n, seen.copy(), 1.05)
            hits[tok] = hits.get(tok, 0) + 1
        assert set(hits) <= set(exp), (k, set(hits) - set(exp))
        for tok, p in exp.items():
            assert abs(hits.get(tok, 0) / n - p) <= 1.0 / n + 1e-6, (k, tok, hits.get(tok, 0) / n, p)


# ---------------------------------------------------------------- generation controls

def check_controls():
    """A suppressed token is never chosen, even as the largest logit; eos is
    masked until min_new choices were made; choosing eos stops the sequence:
    later choices are eos and leave the seen set alone; without controls the
    choice is the plain one."""
    z = np.array([0.1, 3.0, 2.0, 2.5, -1.0], np.float32)
    sup = np.array([False, True, False, False, False])
    ctl = od.Controls(suppress=sup, eos=3, min_new=2)
    seen = np.zeros(5, bool)
    t0, _ = od.choose_controlled(z, seen, 1.0, ctl)      # 1 suppressed, eos masked -> 2
    t1, _ = od.choose_controlled(z, seen, 1.0, ctl)      # still below min_new -> 2
    t2, _ = od.choose_controlled(z, seen, 1.0, ctl)      # eos allowed: 2.5 > 2.0 -> 3, stop
    assert (t0, t1, t2) == (2, 2, 3) and ctl.eos_step == 2
    seen_before = seen.copy()
    t3, _ = od.choose_controlled(np.array([9, 0, 0, 0, 0], np.float32), seen, 1.0, ctl)
    assert t3 == 3 and np.array_equal(seen, seen_before) and ctl.count == 4
    # the penalty still acts on the unmasked logits: 2.5 / 1.5 < 2.0 once 3 is seen
    ctl2 = od.Controls(eos=-1)
    seen2 = np.array([False, False, False, True, False])
    t, _ = od.choose_controlled(np.array([0, 1.0, 2.0, 2.5, 0], np.float32), seen2, 1.5, ctl2)
    assert t == 2
    # sampled: the suppressed token has no mass
    zs = np.log(np.array([1, 2, 3, 4], np.float32))
    ctl3 = od.Controls(suppress=np.array([False, False, False, True]))
    hits = {od.choose_controlled(zs, None, 1.0, od.Controls(suppress=ctl3.suppress),
                                 (4, 1.0, 1.0, np.array([u])))[0]
            for u in np.linspace(0.01, 0.99, 40)}
    assert hits == {0, 1, 2}
    # no controls: the plain choice
    g, _ = od.penalized_argmax(z, None, 1.0)
    t, _ = od.choose_controlled(z, None, 1.0, od.Controls())
    assert t == g == 1


# ---------------------------------------------------------------- codec convolutions

def check_conv_causal():
    """Single channel, dilation 1: numpy's full convolution with the reversed
    kernel, cut to T; an impulse at frame t0 comes out as the taps at
    t0 + (K-1-j) d; a 1-tap convolution is the channel matrix product."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((1, 20))
    w = rng.standard_normal((1, 1, 5))
    y = oc.conv1d_causal(x, w, None, 1)
    _close(y[0], np.convolve(x[0], w[0, 0, ::-1])[:20], 1e-13)
    xi = np.zeros((3, 30))
    xi[1, 4] = 1.0
    wi = rng.standard_normal((2, 3, 4))
    bi = np.array([0.5, -0.25])
    yi = oc.conv1d_causal(xi, wi, bi, 3)
    exp = np.zeros((2, 30)) + bi[:, None]
    for j in range(4):
        exp[:, 4 + (3 - j) * 3] += wi[:, 1, j]
    _close(yi, exp, 1e-15)
    x2 = rng.standard_normal((6, 9))
    w2 = rng.standard_normal((4, 6, 1))
    _close(oc.conv1d_causal(x2, w2, None, 7), w2[:, :, 0] @ x2, 1e-13)


def check_transconv_phases():
    """The qwen3-tts-hip log's phase form, out[t s + p] = in[t] W[p] +
    in[t-1] W[p+s] + bias (in[-1] = 0), equals the transposed convolution's
    scatter definition; one frame in gives the kernel laid out once."""
    rng = np.random.default_rng(32)
    for s_, cin, cout, T in [(3, 4, 5, 7), (8, 2, 3, 4), (1, 3, 2, 5)]:
        x = rng.standard_normal((cin, T))
        w = rng.standard_normal((cin, cout, 2 * s_))
        b = rng.standard_normal(cout)
        y = oc.transconv1d(x, w, b, s_)
        assert y.shape == (cout, T * s_)
        ph = np.zeros((cout, T * s_))
        for t in range(T):
            for p in range(s_):
                v = b + w[:, :, p].T @ x[:, t]
                if t > 0:
                    v = v + w[:, :, p + s_].T @ x[:, t - 1]
                ph[:, t * s_ + p] = v
        _close(y, ph, 1e-13)
    x1 = np.zeros((2, 3))
    x1[0, 0] = 1.0
    w1 = rng.standard_normal((2, 2, 8))
    y1 = oc.transconv1d(x1, w1, None, 4)
    _close(y1[:, :8], w1[0], 1e-15)
    assert not y1[:, 8:].any()


# ---------------------------------------------------------------- block quantization

def check_quant_closed_form():
    """d = 2^-7 makes every value exact: amax 127 d gives codes 127; 2.5 d
    rounds away from zero to 3 (and -2.5 d to -3); a zero block has scale 0
    and codes 0; the 4-bit form packs weight 2i low and 2i+1 high."""
    d = 2.0 ** -7
    w = np.zeros((2, 32), np.float32)
    w[0, 0] = 127 * d
    w[0, 1] = 2.5 * d
    w[0, 2] = -2.5 * d
    w[0, 3] = -1.49 * d
    codes, scales = oq.quantize(w, oq.Q8)
    assert list(codes[0, :4]) == [127, 3, -3, -1]
    assert scales[0, 0] == np.float16(d).view(np.uint16) and scales[1, 0] == 0
    assert not codes[1].any()
    # a scale that fp16 cannot hold: 0.1 / 127 is stored rounded, and the
    # block's largest weight reads back as that rounded scale times 127
    w2 = np.zeros((1, 32), np.float32)
    w2[0, 5] = 0.1
    c2, s2 = oq.quantize(w2, oq.Q8)
    d16 = float(np.float16(np.float32(0.1) / np.float32(127)))
    assert c2[0, 5] == 127 and d16 != float(np.float32(0.1) / np.float32(127))
    assert oq.dequantize(c2, s2, oq.Q8, 32)[0, 5] == d16 * 127
    # 4-bit: amax 7 d -> d; 2.5 d -> 3 -> nibble 11; -2.5 d -> -3 -> nibble 5
    w4 = np.zeros((1, 32), np.float32)
    w4[0, 0], w4[0, 1], w4[0, 2], w4[0, 3] = 7 * d, 2.5 * d, -2.5 * d, -7 * d
    c4, s4 = oq.quantize(w4, oq.Q4)
    assert c4.shape == (1, 16)
    assert c4[0, 0] == (15 | (11 << 4)) and c4[0, 1] == (5 | (1 << 4)), (c4[0, 0], c4[0, 1])
    assert (c4[0, 2:] == (8 | (8 << 4))).all()
    assert s4[0, 0] == np.float16(d).view(np.uint16)
    _close(oq.dequantize(c4, s4, oq.Q4, 32)[0, :4], [7 * d, 3 * d, -3 * d, -7 * d], 0)


def check_quant_error_bound():
    """Every read-back weight lies within half a step of the input, plus the
    fp16 rounding of the scale over the largest code; the largest |w| of a
    block reads back as +-QMAX steps; read-back is idempotent."""
    w = inputs.normal(8, 9, 3, (16, 256), scale=0.02)
    w[3, :32] *= 1e-3           # a block with a small (fp16-subnormal-free) scale
    for fmt in (oq.Q8, oq.Q4):
        codes, scales = oq.quantize(w, fmt)
        back = oq.dequantize(codes, scales, fmt, 256)
        d = np.repeat(oq.block_scales(w, fmt).astype(np.float64), 32, axis=1)
        d16 = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
        bound = d / 2 * (1 + 1e-6) + np.abs(d16 - d) * oq.QMAX[fmt]
        assert (np.abs(back - w) <= bound + 1e-12).all(), fmt
        q = oq.codes_of(codes, fmt, 256).reshape(16, 8, 32)
        assert (np.abs(q).max(axis=2) == oq.QMAX[fmt]).all(), fmt
        c2, s2 = oq.quantize(back.astype(np.float32), fmt)
        assert np.array_equal(oq.dequantize(c2, s2, fmt, 256), back), fmt


def check_quant_bytes_golden():
    """Byte accounting of the formats against the RKNN page's table: the
    0.6B Talker matmuls in the 4-bit form (18 bytes per 32, Q4_K's rate) with
    the head at Q8_0 move 251.0 MB per token.  This count gives 251.07: the
    page's figure is taken to within 0.1 MB (its Q8_0 row, 471.3, matches
    this count to the printed digit)."""
    from autoregressive_transformer_decode_amd import inputs as inp
    g = {k: float(v) for k, v in read_golden("talker_q8_bytes.txt")}
    s = inp.TALKER06
    assert oq.bytes_per_weight(oq.Q8) == g["q8_0_bytes_per_block"] / g["q8_0_weights_per_block"]
    assert oq.bytes_per_weight(oq.Q4) == g["q4_k_bytes_per_superblock"] / g["q4_k_weights_per_superblock"]
    head = s.vocab * s.hidden
    body = s.weight_elems(with_head=True) - head
    mb = (body * oq.bytes_per_weight(oq.Q4) + head * oq.bytes_per_weight(oq.Q8)) / 1e6
    assert abs(mb - g["q4_k_mb_per_token"]) <= 0.1, mb


# ---------------------------------------------------------------- golden

def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def check_bucket_schedule_golden():
    """Growing before a write at position == capacity (start 128, doubling)
    reproduces the buckets and migration counts of the Audio8-ASR runs.  A
    run of N tokens (first token and EOS included) is a prefill and N - 1
    decode steps; step k writes KV position prefill + k - 1."""
    for label, pre, toks, final, migr in read_golden("asr_bucket_runs.txt"):
        pre, toks, final, migr = int(pre), int(toks), int(final), int(migr)
        cap, moves = od.bucket_for(pre - 1, 128), 0
        assert cap == 128
        for k in range(1, toks):
            p = pre + k - 1
            new = od.bucket_for(p, cap)
            if new != cap:
                moves += 1
                cap = new
        assert (cap, moves) == (final, migr), (label, cap, moves)


def check_talker_bytes_golden():
    """The 0.6B Talker shape (28 layers x 7 matmuls + a 3072-row head, h 1024,
    q 2048, kv 1024, FFN 3072) at Q8_0 moves 471.3 MB per token."""
    from autoregressive_transformer_decode_amd import inputs
    g = {k: float(v) for k, v in read_golden("talker_q8_bytes.txt")}
    s = inputs.TALKER06
    assert s.n_layers * 7 == g["matmuls"]
    n = s.weight_elems(with_head=True)
    mb = n * g["q8_0_bytes_per_block"] / g["q8_0_weights_per_block"] / 1e6
    assert round(mb, 1) == g["mb_per_token"], mb
