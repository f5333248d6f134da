"""Loop-only float64 recompute of the whole sequence, for tiny shapes.

A second form of the same definition as ``decoder``, kept deliberately
different in structure: no KV cache (every prefix is recomputed from its
first row), scalar Python loops instead of array products, the rotation
written per channel pair, bf16 rounding done with frexp/round-half-even
instead of bit manipulation.  Agreement of the cached oracle with this form at
every step pins the cache logic (append position, visible length, bucket
copies, reset) -- the "stepwise decode equals full recompute" check of the
RKNN sidecar page and the ncnn port's KV-cache section.

Only for tiny models: cost grows as T^2 * L * h * (Hq*D) in pure Python.
"""

from __future__ import annotations

import math
import struct
from typing import List, Sequence


def _bf16(x: float) -> float:
    """Nearest bf16 value (8 significant bits), ties to even."""
    if x == 0.0 or math.isinf(x) or math.isnan(x):
        return x
    m, e = math.frexp(x)              # x = m * 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256.0), e - 8)   # round(): half to even


def _dot(a: Sequence[float], b: Sequence[float]) -> float:
    s = 0.0
    for i in range(len(a)):
        s += float(a[i]) * float(b[i])
    return s


def _matvec(W, x) -> List[float]:
    return [_dot(W[n], x) for n in range(len(W))]


def _rms(x: Sequence[float], g, eps: float) -> List[float]:
    ms = 0.0
    for v in x:
        ms += v * v
    inv = 1.0 / math.sqrt(ms / len(x) + eps)
    return [x[i] * inv * float(g[i]) for i in range(len(x))]


def _f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def _freq_positions(pos, half: int, sections) -> List[int]:
    """Position of each rotary frequency: pos itself (an int), or for
    (t, h, w) positions under interleaved sections, frequency i in group
    i // 3 takes h at offset 1 while that group is below s_h, w at offset 2
    while below s_w, and t otherwise."""
    if isinstance(pos, int):
        return [pos] * half
    t, h, w = pos
    s_h, s_w = (0, 0) if sections is None else (sections[1], sections[2])
    out = []
    for i in range(half):
        grp, off = divmod(i, 3)
        if off == 1 and grp < s_h:
            out.append(h)
        elif off == 2 and grp < s_w:
            out.append(w)
        else:
            out.append(t)
    return out


def _rotate(v: List[float], pos, theta: float, sections=None) -> List[float]:
    """Rotate channel pairs (i, i + D/2) by p_i * theta^(-2i/D) with p_i the
    frequency's position (_freq_positions); the cosine and sine are taken at
    float32 precision, as the definition fixes."""
    D = len(v)
    half = D // 2
    ps = _freq_positions(pos, half, sections)
    out = list(v)
    for i in range(half):
        ang = ps[i] * theta ** (-2.0 * i / D)
        c, s = _f32(math.cos(ang)), _f32(math.sin(ang))
        a, b = v[i], v[i + half]
        out[i] = a * c - b * s
        out[i + half] = b * c + a * s
    return out


def forward_rows(model, rows: Sequence[Sequence[float]], rope_pos=None) -> List[List[float]]:
    """Residual stream after the last layer for every row, rows at positions
    0..T-1, row t attending to rows 0..t (recomputed, no cache).  rope_pos:
    per row (t, h, w) rotary positions in place of the row index."""
    hq, hkv, D = model.n_q_heads, model.n_kv_heads, model.head_dim
    grp = hq // hkv
    eps = model.rms_eps
    xs = [[float(v) for v in r] for r in rows]
    if getattr(model, "in_proj", None) is not None:     # input projection
        b = model.in_proj_bias
        xs = [[_dot(model.in_proj[i], x) + (float(b[i]) if b is not None else 0.0)
               for i in range(len(model.in_proj))] for x in xs]
    T = len(xs)
    for L in model.layers:
        Q, K, Vv = [], [], []
        for t in range(T):
            u = _rms(xs[t], L["attn_norm"], eps)
            q = _matvec(L["wq"], u)
            k = _matvec(L["wk"], u)
            v = _matvec(L["wv"], u)
            if L["bq"] is not None:
                q = [q[i] + float(L["bq"][i]) for i in range(len(q))]
                k = [k[i] + float(L["bk"][i]) for i in range(len(k))]
                v = [v[i] + float(L["bv"][i]) for i in range(len(v))]
            qh = [q[h * D:(h + 1) * D] for h in range(hq)]
            kh = [k[h * D:(h + 1) * D] for h in range(hkv)]
            vh = [v[h * D:(h + 1) * D] for h in range(hkv)]
            if model.qk_norm:
                qh = [_rms(a, L["q_norm"], eps) for a in qh]
                kh = [_rms(a, L["k_norm"], eps) for a in kh]
            rp = t if rope_pos is None else tuple(int(c) for c in rope_pos[t])
            sec = getattr(model, "mrope_sections", None)
            qh = [_rotate(a, rp, model.rope_theta, sec) for a in qh]
            kh = [_rotate(a, rp, model.rope_theta, sec) for a in kh]
            if model.kv_bf16:
                kh = [[_bf16(c) for c in a] for a in kh]
                vh = [[_bf16(c) for c in a] for a in vh]
            Q.append(qh)
            K.append(kh)
            Vv.append(vh)
        new = []
        for t in range(T):
            o = []
            for h in range(hq):
                g = h // grp
                sc = [_dot(Q[t][h], K[j][g]) / math.sqrt(D) for j in range(t + 1)]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                tot = sum(w)
                for d in range(D):
                    acc = 0.0
                    for j in range(t + 1):
                        acc += w[j] / tot * Vv[j][g][d]
                    o.append(acc)
            x = [xs[t][i] + v for i, v in enumerate(_matvec(L["wo"], o))]
            wv = _rms(x, L["mlp_norm"], eps)
            gt = _matvec(L["w_gate"], wv)
            up = _matvec(L["w_up"], wv)
            a = [gt[i] / (1.0 + math.exp(-gt[i])) * up[i] for i in range(len(gt))]
            x = [x[i] + v for i, v in enumerate(_matvec(L["w_down"], a))]
            new.append(x)
        xs = new
    return xs


def last_outputs(model, rows, head: int = 0, rope_pos=None):
    """(y, z) of the last row: final RMSNorm and LM head."""
    x = forward_rows(model, rows, rope_pos)[-1]
    y = _rms(x, model.final_norm, model.rms_eps)
    return y, _matvec(model.heads[head], y)
