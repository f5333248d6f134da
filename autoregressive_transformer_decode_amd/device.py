"""Device-memory plumbing around the C ABI (torch allocates, the library
computes).

``DeviceModel`` uploads generated weights to HBM and builds the
``atd_weights`` pointer structs; ``Decoder`` owns a decoder handle plus the
KV buckets it attaches, and forwards each call to the binding with tensor
data pointers and the current torch stream."""

from __future__ import annotations

import ctypes as C
import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import binding as B
from . import inputs
from .inputs import BF16, ModelShape, ModelWeights


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _to_dev(arr: np.ndarray, device) -> torch.Tensor:
    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, np.float32))
    return t.to(device, non_blocking=False).contiguous()


QUANT_FORMATS = {None: B.ATD_WFMT_DENSE, "q8": B.ATD_WFMT_Q8, "q4": B.ATD_WFMT_Q4}
_LINEARS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def quantize_blocks(w: torch.Tensor, fmt: str):
    """(codes, scales) of a dense [N, K] device matrix in the block format
    ``fmt`` ("q8" or "q4"), from the library's quantizer."""
    n, k = w.shape
    code_bytes = n * k if fmt == "q8" else n * k // 2
    codes = torch.empty(code_bytes, dtype=torch.uint8, device=w.device)
    scales = torch.empty(n, k // B.ATD_QBLOCK, dtype=torch.int16, device=w.device)
    B.quantize_blocks(w.data_ptr(), B.ATD_BF16 if w.dtype == torch.bfloat16 else B.ATD_F32, n, k,
                      QUANT_FORMATS[fmt], codes.data_ptr(), scales.data_ptr(), _stream())
    return codes, scales


class DeviceModel:
    """Weights of one stack in HBM.  ``tables`` may be shared with another
    stack (the Talker and the Code Predictor use the same code embeddings).
    ``quant`` ("q8" / "q4") stores the seven per-layer matrices block-quantized
    by the library's quantizer (the dense copies are released)."""

    def __init__(self, mw: ModelWeights, device="cuda",
                 tables: Optional[List[torch.Tensor]] = None, quant: Optional[str] = None):
        s = mw.shape
        self.shape = s
        self.quant = quant
        self.weight_format = QUANT_FORMATS[quant]
        self.keep: List[torch.Tensor] = []

        def up(a):
            if a is None:
                return None
            t = _to_dev(a, device)
            self.keep.append(t)
            return t

        self.layers = []
        for Lw in mw.layers:
            self.layers.append(dict(
                attn_norm=up(Lw.attn_norm), wq=up(Lw.wq.storage), wk=up(Lw.wk.storage),
                wv=up(Lw.wv.storage), bq=up(Lw.bq), bk=up(Lw.bk), bv=up(Lw.bv),
                q_norm=up(Lw.q_norm), k_norm=up(Lw.k_norm), wo=up(Lw.wo.storage),
                mlp_norm=up(Lw.mlp_norm), w_gate=up(Lw.w_gate.storage),
                w_up=up(Lw.w_up.storage), w_down=up(Lw.w_down.storage)))
            if quant is not None:
                L = self.layers[-1]
                for name in _LINEARS:
                    codes, scales = quantize_blocks(L[name], quant)
                    L[name + "_scale"] = scales
                    self.keep.extend([codes, scales])
                    dense, L[name] = L[name], codes
                    self.keep = [t for t in self.keep if t is not dense]
                torch.cuda.current_stream().synchronize()
        self.final_norm = up(mw.final_norm)
        self.in_proj = up(mw.in_proj.storage) if mw.in_proj is not None else None
        self.in_proj_bias = up(mw.in_proj_bias) if mw.in_proj_bias is not None else None
        self.heads = [up(h.storage) for h in mw.heads]
        if tables is None:
            tables = [up(t.storage) for t in mw.tables]
        else:
            self.keep.extend(tables)
        self.tables = tables
        self.table_vocab = [int(t.shape[0]) for t in tables]
        self._build_structs()

    def _build_structs(self):
        n = len(self.layers)
        self._layers = (B.atd_layer_weights * n)()
        for i, L in enumerate(self.layers):
            for k, v in L.items():
                setattr(self._layers[i], k, v.data_ptr() if v is not None else None)
        self._heads = (C.c_void_p * len(self.heads))(*[h.data_ptr() for h in self.heads])
        self._tables = (C.c_void_p * len(self.tables))(*[t.data_ptr() for t in self.tables])
        self._vocab = (C.c_int32 * len(self.tables))(*self.table_vocab)
        self.weights = B.atd_weights(
            layers=C.cast(self._layers, C.POINTER(B.atd_layer_weights)),
            final_norm=self.final_norm.data_ptr(),
            lm_heads=C.cast(self._heads, C.POINTER(C.c_void_p)),
            tables=C.cast(self._tables, C.POINTER(C.c_void_p)),
            table_vocab=C.cast(self._vocab, C.POINTER(C.c_int32)),
            in_proj=self.in_proj.data_ptr() if self.in_proj is not None else None,
            in_proj_bias=self.in_proj_bias.data_ptr() if self.in_proj_bias is not None else None)


def make_config(s: ModelShape, max_slots: int, max_rows: int, max_ctx: int,
                n_tables: Optional[int] = None, flags: int = 0,
                weight_format: int = B.ATD_WFMT_DENSE) -> B.atd_config:
    return B.atd_config(
        n_layers=s.n_layers, hidden=s.hidden, n_q_heads=s.n_q_heads, n_kv_heads=s.n_kv_heads,
        head_dim=s.head_dim, ffn=s.ffn, vocab=s.vocab, n_lm_heads=s.n_lm_heads,
        n_tables=n_tables if n_tables is not None else len(s.table_vocabs),
        qk_norm=int(s.qk_norm), qkv_bias=int(s.qkv_bias),
        dtype=B.ATD_BF16 if s.dtype == BF16 else B.ATD_F32,
        kv_dtype=B.ATD_BF16 if s.kv_dtype == BF16 else B.ATD_F32,
        rope_theta=s.rope_theta, rms_eps=s.rms_eps,
        max_slots=max_slots, max_rows=max_rows, max_ctx=max_ctx, flags=flags,
        weight_format=weight_format, input_dim=s.input_dim,
        mrope_sections=(C.c_int32 * 3)(*(s.mrope_sections or (0, 0, 0))))


class Decoder:
    """A decoder handle plus the KV buckets it holds for each slot."""

    def __init__(self, model: DeviceModel, max_slots: int = 1, max_rows: int = 1,
                 max_ctx: int = 4096, mfma: bool = True, kv_dtype: Optional[str] = None,
                 l2_prefetch: bool = True):
        self.model = model
        s = model.shape
        if kv_dtype is not None and kv_dtype != s.kv_dtype:
            s = dataclasses.replace(s, kv_dtype=kv_dtype)
        self.shape = s
        self.cfg = make_config(s, max_slots, max_rows, max_ctx,
                               flags=(0 if mfma else B.ATD_FLAG_NO_MFMA) |
                               (0 if l2_prefetch else B.ATD_FLAG_NO_L2_PREFETCH),
                               weight_format=model.weight_format)
        self.handle = B.decoder_create(self.cfg, model.weights)
        self.kv = {}   # slot -> (list of K tensors, list of V tensors)
        self.kv_dtype = torch.bfloat16 if s.kv_dtype == BF16 else torch.float32

    def close(self):
        if self.handle:
            B.decoder_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- KV buckets
    def alloc_kv(self, capacity: int, device="cuda"):
        s = self.shape
        shp = (s.n_kv_heads, capacity, s.head_dim)
        ks = [torch.zeros(shp, dtype=self.kv_dtype, device=device) for _ in range(s.n_layers)]
        vs = [torch.zeros(shp, dtype=self.kv_dtype, device=device) for _ in range(s.n_layers)]
        return ks, vs

    def grow(self, slot: int, capacity: int, kv=None):
        """Attach a new bucket (allocated here unless given); the old one is
        dropped after the stream passes the copy."""
        ks, vs = kv if kv is not None else self.alloc_kv(capacity)
        B.kv_bucket_grow(self.handle, slot, [k.data_ptr() for k in ks],
                         [v.data_ptr() for v in vs], capacity, _stream())
        old = self.kv.get(slot)
        self.kv[slot] = (ks, vs)
        if old is not None:
            torch.cuda.current_stream().synchronize()
        return ks, vs

    def position(self, slot: int = 0):
        return B.decoder_get_position(self.handle, slot)

    def set_position(self, slot: int, pos: int):
        B.decoder_set_position(self.handle, slot, pos, _stream())

    # -- compute
    def prefill(self, x: torch.Tensor, slot: int = 0, head: int = 0,
                y_out: Optional[torch.Tensor] = None, logits_out: Optional[torch.Tensor] = None,
                rope_pos: Optional[torch.Tensor] = None):
        """rope_pos: device int32 [T, 3] rotary (t, h, w) positions of the rows
        (decoder_prefill_mrope), or None (positions 0..T-1)."""
        T = int(x.shape[0])
        if logits_out is None:
            logits_out = torch.empty(self.shape.vocab, device=x.device, dtype=torch.float32)
        y = y_out.data_ptr() if y_out is not None else None
        if rope_pos is None:
            B.decoder_prefill(self.handle, slot, x.data_ptr(), T, head, y, logits_out.data_ptr(),
                              _stream())
        else:
            assert rope_pos.dtype == torch.int32 and tuple(rope_pos.shape) == (T, 3)
            B.decoder_prefill_mrope(self.handle, slot, x.data_ptr(), T,
                                    rope_pos.contiguous().data_ptr(), head, y,
                                    logits_out.data_ptr(), _stream())
        return y_out, logits_out

    def step(self, tok: Optional[torch.Tensor], table_ids: Sequence[int], slot0: int = 0,
             nrows: int = 1, extra: Optional[torch.Tensor] = None, head: int = 0,
             y_out: Optional[torch.Tensor] = None, logits_out: Optional[torch.Tensor] = None,
             rope_pos: Optional[torch.Tensor] = None, slots: Optional[Sequence[int]] = None):
        """rope_pos: device int32 [nrows, 3] rotary (t, h, w) positions
        (decoder_step_mrope), or None (each slot's cache position).  slots: the
        slot of each row (decoder_step_slots), or None for slot0 .. slot0 +
        nrows - 1."""
        G = len(table_ids)
        if slots is not None:
            nrows = len(slots)
        if logits_out is None:
            logits_out = torch.empty(nrows, self.shape.vocab, device="cuda", dtype=torch.float32)
        tp = tok.data_ptr() if tok is not None else None
        ex = extra.data_ptr() if extra is not None else None
        y = y_out.data_ptr() if y_out is not None else None
        if slots is not None:
            assert rope_pos is None, "decoder_step_slots takes cache positions"
            B.decoder_step_slots(self.handle, nrows, list(slots), tp, G, table_ids, ex, head, y,
                                 logits_out.data_ptr(), _stream())
        elif rope_pos is None:
            B.decoder_step(self.handle, slot0, nrows, tp, G, table_ids, ex, head, y,
                           logits_out.data_ptr(), _stream())
        else:
            assert rope_pos.dtype == torch.int32 and tuple(rope_pos.shape) == (nrows, 3)
            B.decoder_step_mrope(self.handle, slot0, nrows, tp, G, table_ids, ex,
                                 rope_pos.contiguous().data_ptr(), head, y,
                                 logits_out.data_ptr(), _stream())
        return y_out, logits_out

    def generate(self, n_steps: int, tok_io: torch.Tensor, table_ids: Sequence[int] = (0,),
                 slot: int = 0, extra: Optional[torch.Tensor] = None, head: int = 0,
                 seen: Optional[torch.Tensor] = None, penalty: float = 1.0,
                 tokens_out: Optional[torch.Tensor] = None, y_out: Optional[torch.Tensor] = None,
                 logits_out: Optional[torch.Tensor] = None,
                 sampling: Optional["Sampling"] = None, controls: Optional["Controls"] = None):
        """n_steps steps on the device (graph-replayed step + token choice):
        greedy, or sampled with ``sampling`` (its uniforms: one per step);
        ``controls``: suppress / eos / min_new_tokens / stop."""
        if logits_out is None:
            logits_out = torch.empty(self.shape.vocab, device="cuda", dtype=torch.float32)
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        B.decoder_generate(self.handle, slot, n_steps, tok_io.data_ptr(), len(table_ids),
                           table_ids, ptr(extra), head, ptr(seen), float(penalty),
                           _c_sampling(sampling), ptr(tokens_out), ptr(y_out),
                           logits_out.data_ptr(), _stream(), controls=_c_controls(controls))
        return logits_out

    def time_stage(self, stage: int, slot0: int = 0, nrows: int = 1, reps: int = 8) -> float:
        """Mean microseconds per layer of one decode stage over nrows slots."""
        return B.decoder_time_stage(self.handle, stage, slot0, nrows, reps, _stream())

    def embed(self, tok: Optional[torch.Tensor], table_ids: Sequence[int], x_out: torch.Tensor,
              nrows: int = 1, extra: Optional[torch.Tensor] = None):
        B.decoder_embed(self.handle, nrows, tok.data_ptr() if tok is not None else None,
                        len(table_ids), table_ids,
                        extra.data_ptr() if extra is not None else None, x_out.data_ptr(),
                        _stream())
        return x_out


def talker_frames(tk: "Decoder", cp: "Decoder", n_frames: int, codes_io: torch.Tensor,
                  y_io: torch.Tensor, text: Optional[torch.Tensor], seen: torch.Tensor,
                  penalty: float, codes_out: Optional[torch.Tensor] = None,
                  tk_logits: Optional[torch.Tensor] = None, cp_logits: Optional[torch.Tensor] = None,
                  tk_slot: int = 0, cp_slot: int = 0, tk_sampling: Optional["Sampling"] = None,
                  cp_sampling: Optional["Sampling"] = None,
                  tk_controls: Optional["Controls"] = None):
    """n_frames frames of the Talker / Code Predictor loop on the device
    (talker_generate_frames); greedy, or sampled with tk_sampling (uniforms
    [n_frames]) / cp_sampling (uniforms [n_frames, 15]); returns (tk_logits,
    cp_logits)."""
    if tk_logits is None:
        tk_logits = torch.empty(tk.shape.vocab, device="cuda", dtype=torch.float32)
    if cp_logits is None:
        cp_logits = torch.empty(cp.shape.vocab, device="cuda", dtype=torch.float32)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    B.talker_generate_frames(tk.handle, tk_slot, cp.handle, cp_slot, n_frames, codes_io.data_ptr(),
                             y_io.data_ptr(), ptr(text), seen.data_ptr(), float(penalty),
                             _c_sampling(tk_sampling), _c_sampling(cp_sampling), ptr(codes_out),
                             tk_logits.data_ptr(), cp_logits.data_ptr(), _stream(),
                             tk_controls=_c_controls(tk_controls))
    return tk_logits, cp_logits


@dataclasses.dataclass
class Sampling:
    """Sampled-choice settings (atd_sampling) with their device uniforms."""
    top_k: int
    temperature: float
    top_p: float
    uniforms: torch.Tensor    # float32 on the device, values in [0, 1)


def _c_sampling(sp: Optional[Sampling]):
    if sp is None:
        return None
    assert sp.uniforms.dtype == torch.float32 and sp.uniforms.is_cuda and sp.uniforms.is_contiguous()
    return B.atd_sampling(int(sp.top_k), float(sp.temperature), float(sp.top_p),
                          sp.uniforms.data_ptr())


def sample_topk(logits: torch.Tensor, seen: Optional[torch.Tensor], penalty: float,
                sampling: Sampling, tok_out: torch.Tensor, controls: Optional["Controls"] = None):
    """Sampled token per row of logits ([V] or [B, V]); row b draws
    sampling.uniforms[b]."""
    Bn, V = (1, logits.shape[0]) if logits.dim() == 1 else logits.shape
    B.sample_topk(logits.data_ptr(), Bn, V, seen.data_ptr() if seen is not None else None,
                  float(penalty), _c_sampling(sampling), tok_out.data_ptr(), _stream(),
                  controls=_c_controls(controls))
    return tok_out


@dataclasses.dataclass
class Controls:
    """Generation controls (atd_controls): suppress bits (device int32
    [B, ceil(V/32)] or None), eos (-1: none), min_new_tokens, first_index,
    eos_step (device int32 [B], -1 while running, or None)."""
    suppress: Optional[torch.Tensor] = None
    eos: int = -1
    min_new_tokens: int = 0
    first_index: int = 0
    eos_step: Optional[torch.Tensor] = None


def _c_controls(c: Optional[Controls]):
    if c is None:
        return None
    return B.atd_controls(c.suppress.data_ptr() if c.suppress is not None else None, int(c.eos),
                          int(c.min_new_tokens), int(c.first_index),
                          c.eos_step.data_ptr() if c.eos_step is not None else None)


def greedy_argmax(logits: torch.Tensor, seen: Optional[torch.Tensor], penalty: float,
                  tok_out: torch.Tensor, margin_out: Optional[torch.Tensor] = None,
                  controls: Optional[Controls] = None):
    Bn, V = (1, logits.shape[0]) if logits.dim() == 1 else logits.shape
    B.greedy_argmax(logits.data_ptr(), Bn, V, seen.data_ptr() if seen is not None else None,
                    float(penalty), tok_out.data_ptr(),
                    margin_out.data_ptr() if margin_out is not None else None, _stream(),
                    controls=_c_controls(controls))
    return tok_out


def seen_words(vocab: int) -> int:
    return (vocab + 31) // 32


def fill_batched_caches(dec: "Decoder", lens: Sequence[int], seed: int = 0) -> None:
    """Load the batched workload's synthetic caches: slot b gets its seeded
    window of each layer's pool (inputs.batched_kv) in rows [0, lens[b]) and
    its write position set to lens[b].  Buckets must be attached already."""
    s = dec.shape
    for l in range(s.n_layers):
        pool = inputs.batched_kv_pool(s, l, seed=seed)
        pk = torch.from_numpy(pool[0].view(np.int16)).cuda().view(torch.bfloat16)
        pv = torch.from_numpy(pool[1].view(np.int16)).cuda().view(torch.bfloat16)
        for b, n in enumerate(lens):
            o, n = inputs.batched_kv_offset(b, int(n)), int(n)
            dec.kv[b][0][l][:, :n].copy_(pk[:, o:o + n])
            dec.kv[b][1][l][:, :n].copy_(pv[:, o:o + n])
    for b, n in enumerate(lens):
        dec.set_position(b, int(n))



def conv1d_causal(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor],
                  dilation: int = 1, y: Optional[torch.Tensor] = None,
                  accumulate: bool = False) -> torch.Tensor:
    """Causal dilated 1-D convolution (codec_conv1d_causal): x [Cin, T],
    w [Cout, Cin, K] float32 on the device -> [Cout, T] (added to y when
    accumulate)."""
    cin, T = x.shape
    cout, _, K = w.shape
    if y is None:
        y = torch.empty(cout, T, device=x.device, dtype=torch.float32)
    B.codec_conv1d_causal(x.data_ptr(), w.data_ptr(), bias.data_ptr() if bias is not None else None,
                          cin, cout, T, K, dilation, int(accumulate), y.data_ptr(), _stream())
    return y


def transconv1d_pack(w: torch.Tensor, stride: int) -> torch.Tensor:
    """Phase-packed weights of a transposed convolution w [Cin, Cout, 2s]."""
    cin, cout, K = w.shape
    assert K == 2 * stride
    packed = torch.empty(stride, cout, cin * 2, device=w.device, dtype=torch.float32)
    B.codec_transconv1d_pack(w.data_ptr(), cin, cout, stride, packed.data_ptr(), _stream())
    return packed


def transconv1d(x: torch.Tensor, packed: torch.Tensor, bias: Optional[torch.Tensor], stride: int,
                y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Transposed 1-D convolution by phases (codec_transconv1d): x [Cin, T]
    -> [Cout, T * stride]."""
    cin, T = x.shape
    cout = packed.shape[1]
    if y is None:
        y = torch.empty(cout, T * stride, device=x.device, dtype=torch.float32)
    B.codec_transconv1d(x.data_ptr(), packed.data_ptr(), bias.data_ptr() if bias is not None else None,
                        cin, cout, T, stride, y.data_ptr(), _stream())
    return y
