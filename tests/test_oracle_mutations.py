"""Planted mistakes in the oracle (CPU only): each plausible slip -- a dropped
term, a wrong sign or index, a transposed operand -- must make at least one
pin fail.  The mistakes are planted by monkeypatching oracle.decoder."""

import numpy as np
import pytest

from oracle import decoder as od
from oracle import quant as oq
from oracle import codec as oc
from tests import pins
from tests.test_oracle_pins import PINS

_orig = {k: getattr(od, k) for k in dir(od) if not k.startswith("__")}
_orig_q = {k: getattr(oq, k) for k in dir(oq) if not k.startswith("__")}
_orig_c = {k: getattr(oc, k) for k in dir(oc) if not k.startswith("__")}


def _all_pins():
    yield from PINS
    yield lambda: pins.check_cached_equals_recompute(False, True, True, 4, 2)
    yield lambda: pins.check_cached_equals_recompute(True, False, True, 4, 4)


def _rms_one_plus(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * (1 + g)


def _rms_no_eps(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) * g


def _rope_adjacent(v, cos, sin):
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = b * cos + a * sin
    return out


def _rope_sign(v, cos, sin):
    h = v.shape[-1] // 2
    a, b = v[..., :h], v[..., h:]
    return np.concatenate([a * cos + b * sin, b * cos - a * sin], axis=-1)


def _freq_wrong(pos, D, theta):
    i = np.arange(D // 2, dtype=np.float64)
    phi = pos * theta ** (-i / D)
    return np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)


def _attn_scale_d(q, K, V, n):
    s = K[:n] @ q / q.shape[-1]
    e = np.exp(s - s.max())
    return (e / e.sum()) @ V[:n]


def _attn_short(q, K, V, n):
    return _orig["attention"](q, K, V, max(n - 1, 1))


def _gqa_modulo(q, K, V, n):
    hkv = K.shape[0]
    return np.stack([od.attention(q[h], K[h % hkv], V[h % hkv], n)
                     for h in range(q.shape[0])])


def _mlp_swapped(model, L, x):
    w = od.rms_norm(x, L["mlp_norm"], model.rms_eps)
    a = (w @ L["w_gate"].T) * od.silu(w @ L["w_up"].T)
    return x + a @ L["w_down"].T


def _qkv_transposed(model, L, u):
    L2 = dict(L)
    for k in ("wq", "wk", "wv"):
        W = L[k]
        L2[k] = W.T.reshape(W.shape) if W.shape[0] != W.shape[1] else W.T
    return _orig["_qkv"](model, L2, u)


def _penalty_mul_pos(z, seen, rho):
    z = np.array(z, np.float32, copy=True)
    if seen is None or rho == 1.0:
        return z
    idx = np.nonzero(seen)[0]
    z[idx] = z[idx] * np.float32(rho)
    return z


def _argmax_last(z, seen, rho):
    zp = od.penalized_logits(z, seen, rho)
    tok = int(len(zp) - 1 - np.argmax(zp[::-1]))
    rest = np.delete(zp, tok)
    if seen is not None:
        seen[tok] = True
    return tok, float(zp[tok] - rest.max())


def _bf16_trunc(a):
    f = np.asarray(a, np.float32)
    u = f.view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.asarray(a).dtype)


def _embed_no_extra(model, toks, table_ids, extra=None):
    return _orig["embed"](model, toks, table_ids, None)


class _ShortGrowCache(od.Cache):
    def grow(self, capacity):
        keep = self.pos
        self.pos = max(keep - 1, 0)
        super().grow(capacity)
        self.pos = keep


def _prefill_no_mask(model, cache, X, head=0):
    real = np.tril
    np.tril = lambda m: np.ones_like(m)
    try:
        return _orig["prefill"](model, cache, X, head)
    finally:
        np.tril = real


def _cp_head0(cp, y_talker, c0, cp_capacity=16, forced=None):
    real_step = od.step
    try:
        od.step = lambda m, c, x, head=0: real_step(m, c, x, 0)
        return _orig["code_predictor_frame"](cp, y_talker, c0, cp_capacity, forced)
    finally:
        od.step = real_step


def _dist_ascending(z, seen, rho, k, t, top_p=1.0):
    toks, p, cum, zp = _orig["sampling_distribution"](z, seen, rho, k, t, top_p)
    return toks[::-1], p[::-1], cum, zp


def _dist_temp_multiplies(z, seen, rho, k, t, top_p=1.0):
    return _orig["sampling_distribution"](z, seen, rho, k, 1.0 / t, top_p)


def _dist_top_p_ignored(z, seen, rho, k, t, top_p=1.0):
    return _orig["sampling_distribution"](z, seen, rho, k, t, 1.0)


def _dist_not_renormalised(z, seen, rho, k, t, top_p=1.0):
    toks, p, cum, zp = _orig["sampling_distribution"](z, seen, rho, k, t, top_p)
    v = zp.astype(np.float64)
    w = np.exp((v - v.max()) / t)
    return toks, w[toks] / w.sum(), cum, zp


def _dist_penalty_after_set(z, seen, rho, k, t, top_p=1.0):
    cand = od.topk_candidates(np.asarray(z, np.float32), k)
    zp = od.penalized_logits(z, seen, rho)
    order = cand[np.lexsort((cand, -zp[cand].astype(np.float64)))]
    v = zp[order].astype(np.float64)
    w = np.exp((v - v[0]) / t)
    return order, w / w.sum(), np.cumsum(w) / w.sum(), zp


def _topk_high_index_ties(zp, k):
    order = np.lexsort((-np.arange(zp.size), -zp.astype(np.float64)))
    return order[:k]


def _topk_one_more(zp, k):
    return _orig["topk_candidates"](zp, k + 1)


def _quant_half_even(w, fmt):
    real = oq._round_half_away
    oq._round_half_away = np.round
    try:
        return _orig_q["quantize"](w, fmt)
    finally:
        oq._round_half_away = real


def _quant_scale_128(w, fmt):
    real = dict(oq.QMAX)
    oq.QMAX[fmt] = real[fmt] + 1
    try:
        c, s = _orig_q["quantize"](w, fmt)
    finally:
        oq.QMAX.update(real)
    return np.clip(c, -real[fmt], real[fmt]) if fmt == oq.Q8 else c, s


def _dequant_scale_misread(codes, scales, fmt, k):
    d = scales.view(np.float16).astype(np.float64)
    return oq.codes_of(codes, fmt, k) * np.repeat(d, 32, axis=1) * (1 + 2.0 ** -12)


def _quant_nibbles_swapped(w, fmt):
    c, s = _orig_q["quantize"](w, fmt)
    if fmt == oq.Q4:
        c = ((c >> 4) | (c << 4)).astype(np.uint8)
    return c, s


def _conv_taps_forward(x, w, b, dilation=1):
    return _orig_c["conv1d_causal"](x, w[:, :, ::-1], b, dilation)


def _transconv_keep_last(x, w, b, stride):
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    cin, T = x.shape
    full = np.zeros((w.shape[1], (T - 1) * stride + w.shape[2]))
    for t in range(T):
        full[:, t * stride:t * stride + w.shape[2]] += np.einsum("ick,i->ck", w, x[:, t])
    y = full[:, full.shape[1] - T * stride:]
    return y + (np.asarray(b)[:, None] if b is not None else 0)


MUTATIONS_C = {
    "conv_taps_reversed": ("conv1d_causal", _conv_taps_forward),
    "transconv_keeps_last_window": ("transconv1d", _transconv_keep_last),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS_C))
def test_planted_codec_mistake_is_caught(name, monkeypatch):
    attr, repl = MUTATIONS_C[name]
    monkeypatch.setattr(oc, attr, repl)
    caught = []
    for pin in _all_pins():
        try:
            pin()
        except Exception as e:  # noqa: BLE001 -- an error also flags the slip
            caught.append(type(e).__name__)
            break
    assert caught, f"no pin catches the planted mistake {name}"


MUTATIONS_Q = {
    "quant_rounds_half_even": ("quantize", _quant_half_even),
    "quant_scale_amax_over_qmax_plus_1": ("quantize", _quant_scale_128),
    "dequant_scale_misread": ("dequantize", _dequant_scale_misread),
    "quant_nibbles_swapped": ("quantize", _quant_nibbles_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS_Q))
def test_planted_quant_mistake_is_caught(name, monkeypatch):
    attr, repl = MUTATIONS_Q[name]
    monkeypatch.setattr(oq, attr, repl)
    caught = []
    for pin in _all_pins():
        try:
            pin()
        except Exception as e:  # noqa: BLE001 -- an error also flags the slip
            caught.append(type(e).__name__)
            break
    assert caught, f"no pin catches the planted mistake {name}"


class _CtlEosAtMin(od.Controls):
    def mask(self, z):
        z = np.array(z, dtype=np.float32, copy=True)
        if self.suppress is not None:
            z[np.asarray(self.suppress, bool)] = -np.inf
        if self.eos >= 0 and self.count < self.min_new - 1:
            z[self.eos] = -np.inf
        return z


def _choose_no_stop(z, seen, rho, ctl, sampling=None, i=0):
    tok, r = od.choose(ctl.mask(z), seen, rho, sampling, i)
    if ctl.eos >= 0 and tok == ctl.eos and ctl.eos_step < 0:
        ctl.eos_step = ctl.count
    ctl.count += 1
    return tok, r


def _project_no_bias(model, x):
    x = np.asarray(x, model.dtype)
    return x if model.in_proj is None else x @ model.in_proj.T


def _mrope_hw_swapped(half, sections):
    m = _orig["mrope_modality"](half, sections)
    return np.where(m == 1, 2, np.where(m == 2, 1, m))


def _mrope_no_cutoff(half, sections):
    return np.arange(half) % 3 if sections is not None else np.zeros(half, np.int64)


def _mrope_t_only(pos3, head_dim, theta, sections):
    return od.rope_cos_sin(pos3[0], head_dim, theta)


def _step_cache_position(model, cache, x, head=0, rope_pos=None):
    return _orig["step"](model, cache, x, head)


def _prefill_row_index(model, cache, X, head=0, rope_pos=None):
    return _orig["prefill"](model, cache, X, head)


def _run_lm_slip(slip):
    """run_lm with one slip: 'feed_prev' feeds token k-1 to step k, 'grow_early'
    grows one row before the write position reaches the capacity, 'short'
    runs one step fewer."""
    def run(model, X0, n_steps, s_init, forced=None, head=0, rho=1.0, on_step=None,
            sampling=None, controls=None):
        cache = od.Cache(model, s_init)
        y, z = od.prefill(model, cache, X0, head)
        tok, margin = od.penalized_argmax(z, None, 1.0)
        out = [(y, z, tok, margin)]
        if on_step:
            on_step(0, cache)
        last = n_steps if slip != "short" else n_steps - 1
        for k in range(1, last + 1):
            fed = out[-1][2] if slip != "feed_prev" or len(out) < 2 else out[-2][2]
            pos = cache.pos + (1 if slip == "grow_early" else 0)
            cap = od.bucket_for(pos, cache.capacity)
            if cap != cache.capacity:
                cache.grow(cap)
            y, z = od.step(model, cache, od.embed(model, [fed], [0]), head)
            tok, margin = od.penalized_argmax(z, None, 1.0)
            out.append((y, z, tok, margin))
            if on_step:
                on_step(k, cache)
        return out, cache
    return run


def _run_talker_slip(slip):
    """run_talker (greedy, no forcing) with one slip: 'text_f' adds text row f
    instead of f + 1, 'seen_early' marks the unpenalised best token seen before
    the penalised choice, 'no_c0' leaves c0's embedding out of the next input,
    'cp_penalty' applies the penalty to the Code Predictor's codes too."""
    def run(talker, cp, X0, text, n_frames, s_init, rho=1.05, cp_capacity=16, forced=None,
            tk_sampling=None, cp_sampling=None, tk_controls=None):
        cache = od.Cache(talker, s_init)
        seen = np.zeros(talker.heads[0].shape[0], bool)

        def pick(z):
            if slip == "seen_early":
                seen[int(np.argmax(z))] = True
            return od.penalized_argmax(z, seen, rho)

        y, z = od.prefill(talker, cache, X0, 0)
        c0, m0 = pick(z)
        frames = []
        for f in range(n_frames):
            cc = od.Cache(cp, cp_capacity)
            cseen = np.zeros(cp.heads[0].shape[0], bool)
            yy, zz = od.prefill(cp, cc, np.stack([y, cp.tables[0][c0]]), 0)
            choice = (lambda v: od.penalized_argmax(v, cseen, rho)) if slip == "cp_penalty" \
                else (lambda v: od.penalized_argmax(v, None, 1.0))
            c, m = choice(zz)
            codes, trace = [c], [(yy, zz, m)]
            for j in range(1, len(cp.heads)):
                yy, zz = od.step(cp, cc, od.embed(cp, [codes[-1]], [j]), j)
                c, m = choice(zz)
                codes.append(c)
                trace.append((yy, zz, m))
            frames.append(dict(y=y, z=z, c0=c0, margin=m0, codes=codes, cp=trace))
            if f == n_frames - 1:
                break
            used = [c0] + codes
            ids = list(range(16))
            if slip == "no_c0":
                used, ids = used[1:], ids[1:]
            x = od.embed(talker, used, ids, text[f] if slip == "text_f" else text[f + 1])
            y, z = od.step(talker, cache, x, 0)
            c0, m0 = pick(z)
        return frames, cache
    return run


MUTATIONS = {
    "mrope_h_w_swapped": ("mrope_modality", _mrope_hw_swapped),
    "mrope_interleave_to_the_end": ("mrope_modality", _mrope_no_cutoff),
    "mrope_t_position_only": ("mrope_cos_sin", _mrope_t_only),
    "step_rotates_at_cache_position": ("step", _step_cache_position),
    "prefill_rotates_at_row_index": ("prefill", _prefill_row_index),
    "controls_eos_one_early": ("Controls", _CtlEosAtMin),
    "input_projection_drops_bias": ("project_input", _project_no_bias),
    "controls_no_stop": ("choose_controlled", _choose_no_stop),
    "sample_walks_ascending": ("sampling_distribution", _dist_ascending),
    "sample_temperature_multiplies": ("sampling_distribution", _dist_temp_multiplies),
    "sample_top_p_ignored": ("sampling_distribution", _dist_top_p_ignored),
    "sample_not_renormalised": ("sampling_distribution", _dist_not_renormalised),
    "sample_penalty_after_set": ("sampling_distribution", _dist_penalty_after_set),
    "topk_ties_high_index": ("topk_candidates", _topk_high_index_ties),
    "topk_one_more": ("topk_candidates", _topk_one_more),
    "rms_gain_one_plus_g": ("rms_norm", _rms_one_plus),
    "rms_no_eps": ("rms_norm", _rms_no_eps),
    "rope_adjacent_pairs": ("rope", _rope_adjacent),
    "rope_sign": ("rope", _rope_sign),
    "rope_frequency": ("rope_cos_sin", _freq_wrong),
    "attention_scale_1_over_D": ("attention", _attn_scale_d),
    "attention_one_row_short": ("attention", _attn_short),
    "gqa_modulo_mapping": ("gqa_attention", _gqa_modulo),
    "swiglu_gate_up_swapped": ("_mlp", _mlp_swapped),
    "qkv_transposed": ("_qkv", _qkv_transposed),
    "penalty_multiplies_positive": ("penalized_logits", _penalty_mul_pos),
    "argmax_last_tie": ("penalized_argmax", _argmax_last),
    "bf16_truncates": ("bf16_round", _bf16_trunc),
    "embed_drops_extra": ("embed", _embed_no_extra),
    "grow_copies_short": ("Cache", _ShortGrowCache),
    "prefill_no_causal_mask": ("prefill", _prefill_no_mask),
    "code_predictor_one_head": ("code_predictor_frame", _cp_head0),
    "lm_feeds_previous_token": ("run_lm", _run_lm_slip("feed_prev")),
    "lm_grows_one_row_early": ("run_lm", _run_lm_slip("grow_early")),
    "lm_one_step_short": ("run_lm", _run_lm_slip("short")),
    "talker_text_row_f": ("run_talker", _run_talker_slip("text_f")),
    "talker_seen_before_choice": ("run_talker", _run_talker_slip("seen_early")),
    "talker_input_drops_c0": ("run_talker", _run_talker_slip("no_c0")),
    "talker_penalty_on_code_predictor": ("run_talker", _run_talker_slip("cp_penalty")),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, repl = MUTATIONS[name]
    monkeypatch.setattr(od, attr, repl)
    caught = []
    for pin in _all_pins():
        try:
            pin()
        except Exception as e:  # noqa: BLE001 -- an error also flags the slip
            caught.append(type(e).__name__)
            break
    assert caught, f"no pin catches the planted mistake {name}"
