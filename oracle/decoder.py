"""Plain CPU definition of the decode step (numpy; float64 unless asked).

Sources, by page title and section:

* "Qwen3-TTS ncnn port" (ncnn discussion 6799), section "Talker: non-standard
  structure and two-level generation": 28-layer Qwen3-style Talker, QK RMSNorm
  over head_dim after the q/k projections, 8 KV heads broadcast to 16 query
  heads, interleaved mRoPE ([24, 20, 20] sections over the frequencies; it
  reduces to plain RoPE for TTS, where the t/h/w positions agree), and the
  two-level frame loop (one Talker token, then 15 Code Predictor codes; the
  sum of the 16 code embeddings plus the text embedding is the next Talker
  input), repetition penalty 1.05 on the main token.
* "Audio8-ASR dynamic KV-cache bucket" (RK3576 acceptance report), section
  "dynamic window mechanism": Qwen2 decoder, no sliding window, external
  [heads, Smax, head_dim] cache, growth by copying the valid region into a
  larger buffer and continuing at the same token and RoPE position.
* "qwen3-tts-hip OPTIMIZATION_LOG", entries on the DecodeStepStack profile
  (input norm, QKV, q/k layout + cache, attention, output projection +
  residual, post norm, gate/up, SwiGLU, down + residual) and on the
  configurable repetition penalty.

Readings where the pages are silent (each listed in the design notes):
RMSNorm eps 1e-6 and gain form x_hat*g; rotate-half RoPE pairing c with
c + D/2, angles in float64 rounded to fp32; attention scale 1/sqrt(D), causal,
no window; query head h reads KV head h // (Hq/Hkv); the KV cache stores bf16
(round to nearest even) for bf16 models; argmax ties go to the lowest index;
the penalty divides positive logits and multiplies the others.  Sampling
(the log's GenerateOptions defaults and device-sampler entries): the top-k set
is unique under (value descending, index ascending); the temperature divides
the logits inside the softmax; top-p keeps the shortest descending prefix
whose probability reaches top_p; the draw inverts the cumulative distribution
over the candidates in descending order with a uniform that the caller passes
in.  Controls: suppressed tokens (and eos before min_new_tokens) are masked to
-inf before the penalty; choosing eos stops the sequence, every later choice
being eos.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, NamedTuple, Optional, Sequence, Tuple

import numpy as np


# --------------------------------------------------------------------------
# model container (plain arrays; built by the caller)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Model:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    rope_theta: float
    rms_eps: float
    qk_norm: bool
    kv_bf16: bool                     # cache rows rounded to bf16 when stored
    layers: List[dict]                # per layer: see LAYER_KEYS
    final_norm: np.ndarray
    heads: List[np.ndarray]           # [V, h]
    tables: List[np.ndarray]          # [V_g, h_in]
    dtype: type = np.float64
    in_proj: Optional[np.ndarray] = None       # [h, h_in] input projection, or None
    in_proj_bias: Optional[np.ndarray] = None  # [h] or None
    mrope_sections: Optional[Tuple[int, int, int]] = None  # (s_t, s_h, s_w), or plain RoPE

    @property
    def input_dim(self) -> int:
        """Width of the input rows (tables, extra, prefill rows)."""
        return self.hidden if self.in_proj is None else self.in_proj.shape[1]


LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "q_norm",
              "k_norm", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def make_model(hp: dict, layers: Sequence[dict], final_norm, heads, tables,
               dtype=np.float64, in_proj=None, in_proj_bias=None) -> Model:
    """Copy the given arrays into the compute dtype (None stays None)."""
    def cv(a):
        return None if a is None else np.asarray(a, dtype=dtype)
    return Model(layers=[{k: cv(L.get(k)) for k in LAYER_KEYS} for L in layers],
                 final_norm=cv(final_norm), heads=[cv(h) for h in heads],
                 tables=[cv(t) for t in tables], dtype=dtype, in_proj=cv(in_proj),
                 in_proj_bias=cv(in_proj_bias), **hp)


# --------------------------------------------------------------------------
# elementary operations
# --------------------------------------------------------------------------

def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), returned in a's dtype.

    The value goes through float32 first (numpy rounds to nearest even), then
    the low 16 bits of the float32 pattern are rounded away."""
    f = np.asarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.asarray(a).dtype)


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.

    Used as the input norm, the post-attention norm, the final norm and, per
    head over head_dim, as the QK norm (ncnn port, Talker section)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_cos_sin(pos: int, head_dim: int, theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """Angles of rotary position pos: omega_i = theta^(-2i/D), phi = pos*omega_i,
    i < D/2, evaluated in float64; cos and sin are then rounded to float32."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    omega = theta ** (-2.0 * i / head_dim)
    phi = float(pos) * omega
    return np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)


def mrope_modality(half: int, sections: Optional[Tuple[int, int, int]]) -> np.ndarray:
    """Which position (0 = t, 1 = h, 2 = w) drives each rotary frequency
    i < D/2 under interleaved sections (s_t, s_h, s_w).  The ncnn port's
    Talker section gives the map for [24, 20, 20] at D = 128: frequency i
    takes i mod 3 while i < 60 and t from there on.  For other sections the
    reading is the same interleave: i takes h when i mod 3 = 1 and i < 3 s_h,
    w when i mod 3 = 2 and i < 3 s_w, and t otherwise (so s_t + s_h + s_w =
    D/2 with 3 max(s_h, s_w) <= D/2).  None: every frequency takes t."""
    m = np.zeros(half, np.int64)
    if sections is None:
        return m
    s_t, s_h, s_w = sections
    if s_t + s_h + s_w != half or 3 * max(s_h, s_w) > half or min(sections) < 0:
        raise ValueError(f"mRoPE sections {sections} do not fit D/2 = {half}")
    i = np.arange(half)
    m[(i % 3 == 1) & (i < 3 * s_h)] = 1
    m[(i % 3 == 2) & (i < 3 * s_w)] = 2
    return m


def mrope_cos_sin(pos3: Sequence[int], head_dim: int, theta: float,
                  sections: Optional[Tuple[int, int, int]]) -> Tuple[np.ndarray, np.ndarray]:
    """Angles of a row with rotary positions (t, h, w): frequency i turns by
    pos3[modality(i)] * omega_i, evaluated and rounded as in rope_cos_sin.
    With t = h = w this is rope_cos_sin(t) (the ncnn port's observation that
    the interleave reduces to plain RoPE for TTS)."""
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    omega = theta ** (-2.0 * i / head_dim)
    p = np.asarray(pos3, np.float64)[mrope_modality(half, sections)]
    phi = p * omega
    return np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)


def rope(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on the last axis: channel i pairs with i + D/2 and
    the pair (a, b) becomes (a cos - b sin, b cos + a sin)."""
    half = v.shape[-1] // 2
    a, b = v[..., :half], v[..., half:]
    c = cos.astype(v.dtype)
    s = sin.astype(v.dtype)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, n: int) -> np.ndarray:
    """Softmax attention of one query row over cached rows 0..n-1.

    q [D]; K, V [S, D] (only the first n rows are valid).  Scale 1/sqrt(D);
    the Audio8-ASR report states no sliding window, so every cached row is
    visible."""
    D = q.shape[-1]
    s = K[:n] @ q / np.sqrt(np.asarray(D, dtype=q.dtype))
    s = s - np.max(s)
    e = np.exp(s)
    a = e / np.sum(e)
    return a @ V[:n]


def gqa_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, n: int) -> np.ndarray:
    """q [Hq, D]; K, V [Hkv, S, D].  Query head h reads KV head h // (Hq/Hkv)
    (the ncnn port broadcasts 8 KV heads to 16 query heads)."""
    hq, hkv = q.shape[0], K.shape[0]
    r = hq // hkv
    return np.stack([attention(q[h], K[h // r], V[h // r], n) for h in range(hq)])


# --------------------------------------------------------------------------
# KV cache of one stream
# --------------------------------------------------------------------------

class Cache:
    """Per-layer K and V buffers [Hkv, S, D] of one stream, plus the next
    write position.  Layout as in the Audio8-ASR report ([heads, Smax,
    head_dim], written in place)."""

    def __init__(self, model: Model, capacity: int):
        shp = (model.n_kv_heads, capacity, model.head_dim)
        self.K = [np.zeros(shp, model.dtype) for _ in range(model.n_layers)]
        self.V = [np.zeros(shp, model.dtype) for _ in range(model.n_layers)]
        self.pos = 0

    @property
    def capacity(self) -> int:
        return self.K[0].shape[1]

    def grow(self, capacity: int) -> None:
        """Bucket growth (Audio8-ASR report, dynamic window mechanism): copy the
        valid rows [:, :pos, :] of every layer into larger buffers; the write
        position (token and RoPE position) stays where it was."""
        if capacity <= self.pos:
            raise ValueError("new capacity must exceed the valid length")
        for l in range(len(self.K)):
            for buf in (self.K, self.V):
                old = buf[l]
                new = np.zeros((old.shape[0], capacity, old.shape[2]), old.dtype)
                new[:, :self.pos] = old[:, :self.pos]
                buf[l] = new


# --------------------------------------------------------------------------
# one token through the stack
# --------------------------------------------------------------------------

def _store_kv(model: Model, a: np.ndarray) -> np.ndarray:
    return bf16_round(a) if model.kv_bf16 else a


def _qkv(model: Model, L: dict, u: np.ndarray):
    """Projections, QK norm and bias; u is [..., h]."""
    q = u @ L["wq"].T
    k = u @ L["wk"].T
    v = u @ L["wv"].T
    if L["bq"] is not None:
        q = q + L["bq"]
        k = k + L["bk"]
        v = v + L["bv"]
    hq, hkv, D = model.n_q_heads, model.n_kv_heads, model.head_dim
    q = q.reshape(q.shape[:-1] + (hq, D))
    k = k.reshape(k.shape[:-1] + (hkv, D))
    v = v.reshape(v.shape[:-1] + (hkv, D))
    if model.qk_norm:
        q = rms_norm(q, L["q_norm"], model.rms_eps)
        k = rms_norm(k, L["k_norm"], model.rms_eps)
    return q, k, v


def _mlp(model: Model, L: dict, x: np.ndarray) -> np.ndarray:
    w = rms_norm(x, L["mlp_norm"], model.rms_eps)
    a = silu(w @ L["w_gate"].T) * (w @ L["w_up"].T)
    return x + a @ L["w_down"].T


def embed(model: Model, toks: Sequence[int], table_ids: Sequence[int],
          extra: Optional[np.ndarray] = None) -> np.ndarray:
    """Step input: sum over g of tables[table_ids[g]][toks[g]], plus extra.
    For the Talker frame this is the 16 code embeddings plus the text
    embedding (ncnn port, two-level generation).  Rows are input_dim wide."""
    x = np.zeros(model.input_dim, model.dtype)
    for t, g in zip(toks, table_ids):
        x = x + model.tables[g][t]
    if extra is not None:
        x = x + np.asarray(extra, model.dtype)
    return x


def project_input(model: Model, x: np.ndarray) -> np.ndarray:
    """Input rows into the stack's width: x W_in^T + b_in when the stack has
    an input projection (the qwen3-tts-hip log's Code Predictor stages
    "prefix projection" and "remaining projection": the Code Predictor's
    inputs come in the Talker's width), else x."""
    x = np.asarray(x, model.dtype)
    if model.in_proj is None:
        return x
    y = x @ model.in_proj.T
    return y + model.in_proj_bias if model.in_proj_bias is not None else y


def head_out(model: Model, x: np.ndarray, head: int):
    """Final RMSNorm (the hidden state y) and LM head logits z = W_head y."""
    y = rms_norm(x, model.final_norm, model.rms_eps)
    return y, y @ model.heads[head].T


def step(model: Model, cache: Cache, x: np.ndarray, head: int = 0,
         rope_pos: Optional[Sequence[int]] = None):
    """One decode step of one stream at position cache.pos; returns (y, z)
    and advances the position by one.  Per layer: input RMSNorm, q/k/v
    projections (+bias), QK norm, RoPE at p, cache append, attention over rows
    0..p, output projection + residual, post norm, SwiGLU MLP + residual.
    rope_pos = (t, h, w) rotates by those positions (mrope_cos_sin) instead of
    p; the row is still cached at p."""
    p = cache.pos
    if p >= cache.capacity:
        raise ValueError("KV cache full")
    x = project_input(model, x)
    if rope_pos is None:
        cos, sin = rope_cos_sin(p, model.head_dim, model.rope_theta)
    else:
        cos, sin = mrope_cos_sin(rope_pos, model.head_dim, model.rope_theta,
                                 model.mrope_sections)
    for l, L in enumerate(model.layers):
        u = rms_norm(x, L["attn_norm"], model.rms_eps)
        q, k, v = _qkv(model, L, u)
        q = rope(q, cos, sin)
        k = rope(k, cos, sin)
        cache.K[l][:, p] = _store_kv(model, k)
        cache.V[l][:, p] = _store_kv(model, v)
        o = gqa_attention(q, cache.K[l], cache.V[l], p + 1)
        x = x + o.reshape(-1) @ L["wo"].T
        x = _mlp(model, L, x)
    cache.pos = p + 1
    return head_out(model, x, head)


def prefill(model: Model, cache: Cache, X: np.ndarray, head: int = 0,
            rope_pos: Optional[np.ndarray] = None):
    """T rows at positions 0..T-1 (the cache is reset first), written as
    whole-block matrix products with a causal mask: row t attends to rows
    0..t.  Returns (y, z) of the last row.  rope_pos [T, 3]: the rotary
    positions (t, h, w) of each row in place of its index."""
    X = project_input(model, X)
    T = X.shape[0]
    if T == 0 or T > cache.capacity:
        raise ValueError("prefill length out of range")
    cache.pos = 0
    if rope_pos is None:
        cs = [rope_cos_sin(t, model.head_dim, model.rope_theta) for t in range(T)]
    else:
        cs = [mrope_cos_sin(rope_pos[t], model.head_dim, model.rope_theta, model.mrope_sections)
              for t in range(T)]
    cos = np.stack([c for c, _ in cs])[:, None, :]
    sin = np.stack([s for _, s in cs])[:, None, :]
    hq, hkv = model.n_q_heads, model.n_kv_heads
    r = hq // hkv
    scale = 1.0 / np.sqrt(np.asarray(model.head_dim, model.dtype))
    mask = np.tril(np.ones((T, T), bool))
    x = X
    for l, L in enumerate(model.layers):
        u = rms_norm(x, L["attn_norm"], model.rms_eps)
        q, k, v = _qkv(model, L, u)           # [T, H, D]
        q = rope(q, cos, sin)
        k = rope(k, cos, sin)
        cache.K[l][:, :T] = _store_kv(model, k).transpose(1, 0, 2)
        cache.V[l][:, :T] = _store_kv(model, v).transpose(1, 0, 2)
        o = np.empty((T, hq, model.head_dim), model.dtype)
        for h in range(hq):
            Kh, Vh = cache.K[l][h // r, :T], cache.V[l][h // r, :T]
            s = (q[:, h] @ Kh.T) * scale
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            o[:, h] = (e / e.sum(axis=1, keepdims=True)) @ Vh
        x = x + o.reshape(T, -1) @ L["wo"].T
        x = _mlp(model, L, x)
    cache.pos = T
    return head_out(model, x[-1], head)


# --------------------------------------------------------------------------
# greedy choice with repetition penalty
# --------------------------------------------------------------------------

def penalized_logits(z: np.ndarray, seen: Optional[np.ndarray], rho: float) -> np.ndarray:
    """Repetition penalty on the tokens already generated (seen[t] True):
    positive logits are divided by rho, the others multiplied by it.  The
    qwen3-tts-hip log makes this a generation option (default 1.05) and the
    ncnn port applies it to the Talker's main token."""
    z = np.array(z, dtype=np.float32, copy=True)
    if seen is None or rho == 1.0:
        return z
    r = np.float32(rho)
    idx = np.nonzero(seen)[0]
    zs = z[idx]
    z[idx] = np.where(zs > 0, zs / r, zs * r).astype(np.float32)
    return z


def penalized_argmax(z: np.ndarray, seen: Optional[np.ndarray], rho: float):
    """Greedy token after the penalty: the lowest index among the maxima.
    Returns (token, margin) where margin = best - second best (0 on a tie).
    Marks the token in ``seen`` when given.  Arithmetic in float32, the
    precision the kernel takes the same decision in."""
    zp = penalized_logits(z, seen, rho)
    tok = int(np.argmax(zp))          # numpy returns the first maximum
    best = zp[tok]
    rest = np.delete(zp, tok)
    margin = float(best - rest.max()) if rest.size else float("inf")
    if seen is not None:
        seen[tok] = True
    return tok, margin


# --------------------------------------------------------------------------
# sampled choice: repetition penalty, temperature, top-k, top-p, one uniform
# --------------------------------------------------------------------------

class SampleDraw(NamedTuple):
    """One sampled token and how far the draw sat from a different outcome.

    pos:     the token's place in the kept candidates (0 = largest logit);
    gap:     distance of u from the nearest interior boundary of the
             cumulative distribution (inf with one candidate);
    cut_gap: distance of top_p from the nearest cumulative probability of the
             top-k candidates (inf when top_p >= 1);
    kmargin: k-th largest penalized logit minus the (k+1)-th (inf when k = V).
    """
    tok: int
    pos: int
    gap: float
    cut_gap: float
    kmargin: float

    def robustness(self, k: int) -> float:
        """Smallest change (of a probability, or of a logit at the top-k cut)
        that could alter the token: the gap and the top-p cut always; the
        k-th / (k+1)-th margin only when the token is the k-th candidate (a
        swap at the cut elsewhere moves the other boundaries by a fraction of
        that candidate's small probability)."""
        r = min(self.gap, self.cut_gap)
        return min(r, self.kmargin) if self.pos == k - 1 else r


def topk_candidates(zp: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest penalized logits, in descending order of
    value, equal values by ascending index (the total order that makes the
    top-k set unique)."""
    order = np.lexsort((np.arange(zp.size), -zp.astype(np.float64)))
    return order[:k]


def sampling_distribution(z: np.ndarray, seen: Optional[np.ndarray], rho: float, k: int,
                          temperature: float, top_p: float = 1.0):
    """The distribution a sampled step draws from (qwen3-tts-hip
    OPTIMIZATION_LOG, GenerateOptions defaults and device-sampler entries:
    repetition penalty, temperature, top-k up to 256, top-p).

    Order of the steps: the penalty on the seen tokens (float32, as in
    penalized_logits); the top-k set of the penalized logits; softmax of
    (logit / temperature) over that set; top-p keeps the shortest prefix, in
    descending order, whose probability reaches top_p.  The temperature is a
    positive scale, so taking the top-k set before or after it gives the same
    set.  Returns (tokens in descending order of logit, probabilities that sum
    to one, cumulative probabilities of the full top-k set, penalized
    logits)."""
    zp = penalized_logits(z, seen, rho)
    cand = topk_candidates(zp, k)
    v = zp[cand].astype(np.float64)
    w = np.exp((v - v[0]) / float(temperature))
    cum_k = np.cumsum(w) / np.sum(w)
    m = len(cand)
    if top_p < 1.0:
        m = int(np.searchsorted(cum_k, top_p, side="left")) + 1   # first cum >= top_p
        m = min(m, len(cand))
    p = w[:m] / np.sum(w[:m])
    return cand[:m], p, cum_k, zp


def sample_topk(z: np.ndarray, seen: Optional[np.ndarray], rho: float, k: int,
                temperature: float, top_p: float, u: float) -> SampleDraw:
    """Sampled token by inversion of the cumulative distribution: the
    candidates in descending order of logit, the first whose cumulative
    probability exceeds the uniform u in [0, 1).  With k = 1 this is
    penalized_argmax.  Marks the token in ``seen`` when given.  Float64
    arithmetic after the float32 penalty."""
    toks, p, cum_k, zp = sampling_distribution(z, seen, rho, k, temperature, top_p)
    cdf = np.cumsum(p)
    i = min(int(np.searchsorted(cdf, u, side="right")), len(toks) - 1)
    tok = int(toks[i])
    gap = float(np.min(np.abs(cdf[:-1] - u))) if len(toks) > 1 else math.inf
    cut_gap = float(np.min(np.abs(cum_k - top_p))) if top_p < 1.0 else math.inf
    if k < zp.size:
        order = topk_candidates(zp, k + 1)
        kmargin = float(zp[order[k - 1]]) - float(zp[order[k]])
    else:
        kmargin = math.inf
    if seen is not None:
        seen[tok] = True
    return SampleDraw(tok, i, gap, cut_gap, kmargin)


# --------------------------------------------------------------------------
# loops
# --------------------------------------------------------------------------

def bucket_for(pos: int, capacity: int) -> int:
    """Capacity after growth: double until the row about to be written
    (index pos) fits (Audio8-ASR report: grow when the write position reaches
    the limit)."""
    while pos >= capacity:
        capacity *= 2
    return capacity


def run_lm(model: Model, X0: np.ndarray, n_steps: int, s_init: int,
           forced: Optional[Sequence[int]] = None, head: int = 0,
           rho: float = 1.0, on_step=None, sampling=None, controls: Optional[Controls] = None):
    """Plain LM loop: prefill X0 (token 1 comes from its last row), then
    n_steps steps, step k consuming token k.  Buckets grow before a write at
    position == capacity.  With ``forced`` the fed tokens are taken from it
    (teacher forcing) instead of the chosen ones.  Choices are greedy, or
    with ``sampling`` = (k, temperature, top_p, u[n_steps + 1]) the choice
    after the prefill (index 0) and after step k draws with u[k].  Returns
    per-step lists of (y, z, tok, margin), index 0 being the prefill.  With
    ``controls`` every choice goes through choose_controlled (the steps after
    a stop still run, fed eos)."""
    cache = Cache(model, s_init)
    seen = np.zeros(model.heads[head].shape[0], bool) if rho != 1.0 else None

    def pick(z, k):
        if controls is None:
            return choose(z, seen, rho, sampling, k)
        return choose_controlled(z, seen, rho, controls, sampling, k)

    y, z = prefill(model, cache, X0, head)
    tok, margin = pick(z, 0)
    out = [(y, z, tok, margin)]
    if on_step:
        on_step(0, cache)
    for k in range(1, n_steps + 1):
        fed = forced[k - 1] if forced is not None else out[-1][2]
        cap = bucket_for(cache.pos, cache.capacity)
        if cap != cache.capacity:
            cache.grow(cap)
        x = embed(model, [fed], [0])
        y, z = step(model, cache, x, head)
        tok, margin = pick(z, k)
        out.append((y, z, tok, margin))
        if on_step:
            on_step(k, cache)
    return out, cache


class Controls:
    """Generation controls of one sequence (ncnn port, Talker section: the
    codes only matched once suppress and min_new_tokens were applied; ASR
    report: decoding runs to EOS).  suppress: bool [V] of tokens never chosen
    (or None); eos: end token or -1; min_new: choices with index below it
    cannot be eos.  State: ``count`` choices made so far (the index of the
    next one) and ``eos_step``, the index of the choice that gave eos (-1
    before); after it every choice returns eos without touching ``seen``."""

    def __init__(self, suppress=None, eos: int = -1, min_new: int = 0, first_index: int = 0):
        self.suppress = suppress
        self.eos = eos
        self.min_new = min_new
        self.count = first_index
        self.eos_step = -1

    def mask(self, z: np.ndarray) -> np.ndarray:
        """Logits with the suppressed tokens (and eos before min_new) at -inf;
        the penalty leaves -inf in place, so masking before it is the same."""
        z = np.array(z, dtype=np.float32, copy=True)
        if self.suppress is not None:
            z[np.asarray(self.suppress, bool)] = -np.inf
        if self.eos >= 0 and self.count < self.min_new:
            z[self.eos] = -np.inf
        return z


def choose_controlled(z: np.ndarray, seen: Optional[np.ndarray], rho: float, ctl: Controls,
                      sampling=None, i: int = 0) -> Tuple[int, float]:
    """One choice under the controls: after a stop, eos; otherwise the greedy
    or sampled choice (``choose``) on the masked logits, and a stop when it
    is eos.  Returns (token, robustness)."""
    if ctl.eos_step >= 0:
        ctl.count += 1
        return ctl.eos, math.inf
    tok, r = choose(ctl.mask(z), seen, rho, sampling, i)
    if ctl.eos >= 0 and tok == ctl.eos:
        ctl.eos_step = ctl.count
    ctl.count += 1
    return tok, r


def choose(z: np.ndarray, seen: Optional[np.ndarray], rho: float, sampling=None,
           i: int = 0) -> Tuple[int, float]:
    """Greedy (sampling None) or sampled choice of one token.  ``sampling`` =
    (k, temperature, top_p, uniforms) and the draw uses uniforms[i].  Returns
    (token, robustness): the greedy top-2 margin, or SampleDraw.robustness
    of the draw (a decision that a small change of the logits cannot flip has
    it well above zero)."""
    if sampling is None:
        return penalized_argmax(z, seen, rho)
    k, t, top_p, u = sampling
    d = sample_topk(z, seen, rho, k, t, top_p, float(u[i]))
    return d.tok, d.robustness(k)


def code_predictor_frame(cp: Model, y_talker: np.ndarray, c0: int,
                         cp_capacity: int = 16, forced: Optional[Sequence[int]] = None,
                         sampling=None):
    """Code Predictor pass of one frame (ncnn port, two-level generation;
    qwen3-tts-hip CodePredictor sub-stages: prefill, first logits/token, then
    the remaining groups as decode steps).  The cache starts empty each frame.
    Prefill rows: the Talker hidden state y and the Talker embedding of c0, at
    positions 0 and 1; head 0 gives c1.  Step j (1..14) feeds E_cp[j][c_j]
    at position j+1 and head j gives c_{j+1}.  No penalty; greedy, or with
    ``sampling`` = (k, temperature, top_p, u[15]) the choice of c_{j+1} draws
    with u[j] (the log's subtalker sampling options).
    Returns codes [c1..c15] and per-pass (y, z, margin)."""
    cache = Cache(cp, cp_capacity)
    X = np.stack([np.asarray(y_talker, cp.dtype), cp.tables[0][c0]])
    yy, z = prefill(cp, cache, X, head=0)
    c, m = choose(z, None, 1.0, sampling, 0)
    codes, trace = [c], [(yy, z, m)]
    n_groups = len(cp.heads)
    for j in range(1, n_groups):
        fed = forced[j - 1] if forced is not None else codes[-1]
        x = embed(cp, [fed], [j])
        yy, z = step(cp, cache, x, head=j)
        c, m = choose(z, None, 1.0, sampling, j)
        codes.append(c)
        trace.append((yy, z, m))
    return codes, trace


def run_talker(talker: Model, cp: Model, X0: np.ndarray, text: np.ndarray,
               n_frames: int, s_init: int, rho: float = 1.05,
               cp_capacity: int = 16, forced: Optional[Sequence[Sequence[int]]] = None,
               tk_sampling=None, cp_sampling=None, tk_controls: Optional[Controls] = None):
    """Two-level Talker frame loop (ncnn port, Talker section).

    Prefill X0 gives (y_0, z_0) and the main code c0_0 (penalty rho over the
    main codes generated so far).  Frame f: the Code Predictor turns (y_f,
    c0_f) into c1..c15; the next Talker input is E_tk[c0_f] + sum_j
    E_cp[j][c_j] + text[f+1]; a Talker step gives (y_{f+1}, z_{f+1}) and
    c0_{f+1}.  ``forced[f]`` (16 codes) replaces frame f's generated codes
    when teacher forcing.  Sampled choices: tk_sampling = (k, temperature,
    top_p, u[n_frames]) draws c0_f with u[f]; cp_sampling = (k, temperature,
    top_p, u[n_frames, 15]) draws frame f's c_{j+1} with u[f, j].  With
    ``tk_controls`` every c0 goes through choose_controlled (the prefill's
    choice first).  Returns per-frame dicts."""
    cache = Cache(talker, s_init)
    seen = np.zeros(talker.heads[0].shape[0], bool)

    def pick(z, f):
        if tk_controls is None:
            return choose(z, seen, rho, tk_sampling, f)
        return choose_controlled(z, seen, rho, tk_controls, tk_sampling, f)

    y, z = prefill(talker, cache, X0, 0)
    c0, m0 = pick(z, 0)
    frames = []
    for f in range(n_frames):
        if forced is not None:
            c0_used = forced[f][0]
            cp_forced = forced[f][1:]
        else:
            c0_used, cp_forced = c0, None
        cps = None
        if cp_sampling is not None:
            cps = cp_sampling[:3] + (np.asarray(cp_sampling[3])[f],)
        codes, cp_trace = code_predictor_frame(cp, y, c0_used, cp_capacity, cp_forced, cps)
        used = [c0_used] + (list(cp_forced) if cp_forced is not None else codes)
        frames.append(dict(y=y, z=z, c0=c0, margin=m0, codes=codes, cp=cp_trace))
        if f == n_frames - 1:
            break
        x = embed(talker, used, list(range(16)), text[f + 1])
        if forced is not None:
            seen[:] = False
            for g in range(f + 1):
                seen[forced[g][0]] = True
        y, z = step(talker, cache, x, 0)
        c0, m0 = pick(z, f + 1)
    return frames, cache
