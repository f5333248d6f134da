"""Helpers shared by the tests: build oracle models.

Tiny random models for the oracle pins are drawn here directly; full-size
models come from the package's seeded input module and are converted into
the oracle's plain container."""

from __future__ import annotations

import numpy as np

from oracle import decoder as od
from oracle import quant as oq


def tiny_model(L=2, h=16, hq=4, hkv=2, D=4, F=24, V=40, qk_norm=True,
               bias=True, kv_bf16=False, n_heads=1, tables=(40,), seed=1,
               scale=0.3, theta=1.0e4, gains_random=True, dtype=np.float64):
    rng = np.random.default_rng(seed)

    def w(*shape):
        return rng.standard_normal(shape) * scale

    def g(n):
        return (1.0 + 0.2 * rng.standard_normal(n)) if gains_random else np.ones(n)

    layers = []
    for _ in range(L):
        layers.append(dict(
            attn_norm=g(h), wq=w(hq * D, h), wk=w(hkv * D, h), wv=w(hkv * D, h),
            bq=w(hq * D) if bias else None, bk=w(hkv * D) if bias else None,
            bv=w(hkv * D) if bias else None,
            q_norm=g(D) if qk_norm else None, k_norm=g(D) if qk_norm else None,
            wo=w(h, hq * D), mlp_norm=g(h), w_gate=w(F, h), w_up=w(F, h),
            w_down=w(h, F)))
    hp = dict(n_layers=L, hidden=h, n_q_heads=hq, n_kv_heads=hkv, head_dim=D,
              ffn=F, rope_theta=theta, rms_eps=1e-6, qk_norm=qk_norm,
              kv_bf16=kv_bf16)
    heads = [w(V, h) for _ in range(n_heads)]
    tabs = [w(v, h) for v in tables]
    return od.make_model(hp, layers, g(h), heads, tabs, dtype=dtype)


_LINEARS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def oracle_from_weights(mw, dtype=np.float64, quant=None):
    """inputs.ModelWeights -> oracle Model (float values of the stored data).
    With ``quant`` ("q8" / "q4") the seven per-layer matrices are replaced by
    the oracle quantizer's read-back of them."""
    s = mw.shape
    hp = dict(n_layers=s.n_layers, hidden=s.hidden, n_q_heads=s.n_q_heads,
              n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, ffn=s.ffn,
              rope_theta=s.rope_theta, rms_eps=s.rms_eps, qk_norm=s.qk_norm,
              kv_bf16=(s.kv_dtype == "bf16"), mrope_sections=s.mrope_sections)
    layers = []
    for Lw in mw.layers:
        layers.append(dict(
            attn_norm=Lw.attn_norm, wq=Lw.wq.values, wk=Lw.wk.values,
            wv=Lw.wv.values, bq=Lw.bq, bk=Lw.bk, bv=Lw.bv, q_norm=Lw.q_norm,
            k_norm=Lw.k_norm, wo=Lw.wo.values, mlp_norm=Lw.mlp_norm,
            w_gate=Lw.w_gate.values, w_up=Lw.w_up.values,
            w_down=Lw.w_down.values))
        if quant is not None:
            L = layers[-1]
            for name in _LINEARS:
                v = np.asarray(L[name], np.float32)
                codes, scales = oq.quantize(v, quant)
                L[name] = oq.dequantize(codes, scales, quant, v.shape[1])
    return od.make_model(hp, layers, mw.final_norm,
                         [t.values for t in mw.heads],
                         [t.values for t in mw.tables], dtype=dtype,
                         in_proj=mw.in_proj.values if mw.in_proj is not None else None,
                         in_proj_bias=mw.in_proj_bias)


def normwise_rel(got, ref) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i|  (per vector)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))
