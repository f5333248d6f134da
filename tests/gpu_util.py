"""Helpers of the GPU parity tests: drive the C ABI through the device module
and compare with the oracle."""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

from autoregressive_transformer_decode_amd import device as dv
from autoregressive_transformer_decode_amd import inputs
from oracle import decoder as od
from tests._models import normwise_rel, oracle_from_weights

TOL = 2e-3          # normwise max relative error on y and logits
MARGIN = 1e-2       # tokens must agree where the oracle's top-2 margin exceeds this
# every GPU parity model draws its norm gains as 1 + GAIN_SD * N(0, 1), a separate draw
# per gain vector, so applying a gain, and which vector each kernel reads, is checked
# (the tiny workload keeps its configured unit gains)
GAIN_SD = 0.1


def small_shape(name, L, h, hq, hkv, D, F, V, dtype, qk_norm, bias, tables=None, n_heads=1,
                theta=1e6, kv_dtype=None):
    return inputs.ModelShape(name=name, n_layers=L, hidden=h, n_q_heads=hq, n_kv_heads=hkv,
                             head_dim=D, ffn=F, vocab=V, n_lm_heads=n_heads, qk_norm=qk_norm,
                             qkv_bias=bias, rope_theta=theta, rms_eps=1e-6, dtype=dtype,
                             table_vocabs=tuple(tables or [V]),
                             kv_dtype=kv_dtype if kv_dtype is not None else dtype)


@dataclasses.dataclass
class StepCheck:
    worst: float = 0.0
    n: int = 0
    tokens_checked: int = 0

    def add(self, y_gpu, z_gpu, y_ref, z_ref, what=""):
        e = max(normwise_rel(y_gpu, y_ref), normwise_rel(z_gpu, z_ref))
        self.worst = max(self.worst, e)
        self.n += 1
        assert e <= TOL, f"{what}: normwise error {e:.3e} > {TOL}"


def lm_parity(mw, X0, n_steps, s_init, grow_to=None, seed_check=True, oracle_dtype=np.float64,
              rho=1.0, quant=None):
    """Prefill X0, then n_steps teacher-forced steps with the oracle's tokens
    (bucket growth as the oracle does it).  With ``quant`` the GPU holds the
    seven per-layer matrices block-quantized and the oracle runs on its own
    quantizer's read-back of them.  Returns (StepCheck, oracle trace, GPU
    logits of every step as numpy)."""
    om = oracle_from_weights(mw, dtype=oracle_dtype, quant=quant)
    ref, _ = od.run_lm(om, X0, n_steps, s_init, rho=rho)
    s = mw.shape
    dm = dv.DeviceModel(mw, quant=quant)
    max_ctx = X0.shape[0] + n_steps
    cap_final = od.bucket_for(max_ctx - 1, s_init)
    dec = dv.Decoder(dm, max_slots=1, max_rows=X0.shape[0], max_ctx=max(cap_final, max_ctx))
    dec.grow(0, s_init)
    h, V = s.hidden, s.vocab
    chk = StepCheck()
    y = torch.empty(1, h, device="cuda")
    z = torch.empty(1, V, device="cuda")
    dec.prefill(torch.from_numpy(np.asarray(X0, np.float32)).cuda(), y_out=y[0], logits_out=z[0])
    zs = []
    tok = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    gtok = torch.zeros(1, dtype=torch.int32, device="cuda")
    margin = torch.zeros(1, device="cuda")
    seen = torch.zeros(1, dv.seen_words(V), dtype=torch.int32, device="cuda")
    for k in range(0, n_steps + 1):
        if k > 0:
            pos, cap = dec.position(0)
            if pos >= cap:
                dec.grow(0, od.bucket_for(pos, cap))
            tok.fill_(ref[k - 1][2])
            dec.step(tok, [0], y_out=y, logits_out=z)
        dv.greedy_argmax(z[0], seen if rho != 1.0 else None, rho, gtok, margin)
        torch.cuda.synchronize()
        zn = z[0].cpu().numpy()
        chk.add(y[0].cpu().numpy(), zn, ref[k][0], ref[k][1], f"step {k}")
        zs.append(zn)
        if ref[k][3] > MARGIN:
            assert int(gtok.item()) == ref[k][2], f"step {k}: token {gtok.item()} != {ref[k][2]}"
            chk.tokens_checked += 1
        if rho != 1.0:   # keep the GPU's seen set equal to the oracle's fed tokens
            seen.zero_()
            for j in range(k + 1):
                t = ref[j][2]
                seen[0, t // 32] |= (1 << (t % 32)) if t % 32 < 31 else -(1 << 31)
    dec.close()
    return chk, ref, zs
