"""Model shapes, workloads and seeded synthetic inputs.

This module describes *what* is decoded (layer counts, widths, step counts)
and draws the synthetic weights and inputs.  It holds none of the decode
arithmetic: both the GPU path and the CPU oracle receive the arrays made
here and nothing else.

Random draws follow one fixed recipe so that any consumer can regenerate the
same values: every tensor has an integer id; its elements are drawn in blocks
of ``BLOCK`` values, block ``b`` from ``numpy.random.default_rng([seed,
model_id, tensor_id, b])`` as float32 standard normals times the scale.  For
bf16 models the float32 draw is rounded to bf16 (round to nearest even).
Norm gains are 1 (the workloads' configuration); with ``gain_sd`` > 0 every
gain vector is 1 + gain_sd * N(0, 1) instead, each drawn under its own tensor
id (so a kernel that reads the wrong gain vector shows).  Block seeding makes
the values independent of how many threads draw them.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 1 << 20
WEIGHT_SCALE = 0.02

F32 = "f32"
BF16 = "bf16"

# tensor ids inside a layer (layer l uses ids 1000*(l+1) + k)
_T_WQ, _T_WK, _T_WV, _T_BQ, _T_BK, _T_BV, _T_WO, _T_WG, _T_WU, _T_WD = range(1, 11)
_T_HEAD = 90_000
_T_TABLE = 80_000
_T_PREFILL = 70_000
_T_TEXT = 70_001
_T_TOKENS = 70_002
_T_KV = 60_000
_T_INPROJ = 91_000
# gains: per layer base + 11..14 (input, q, k, post-attention); final 92_000
_T_G_ATTN, _T_G_Q, _T_G_K, _T_G_MLP = range(11, 15)
_T_G_FINAL = 92_000


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Shape of one decoder stack (Qwen2/Qwen3 style)."""

    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int            # vocab of every LM head of this stack
    n_lm_heads: int       # 1, or 15 for the code predictor
    qk_norm: bool
    qkv_bias: bool
    rope_theta: float
    rms_eps: float
    dtype: str            # weight and embedding storage: F32 or BF16
    table_vocabs: Tuple[int, ...]   # vocab of each embedding table
    model_id: int = 0     # separates the random streams of two stacks
    kv_dtype: str = F32   # KV-cache storage: F32 or BF16
    input_dim: int = 0    # width of the input rows when projected (0: hidden)
    mrope_sections: Optional[Tuple[int, int, int]] = None   # interleaved t/h/w sections

    @property
    def in_width(self) -> int:
        """Width of the input rows: tables, extra and prefill rows."""
        return self.input_dim or self.hidden

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def weight_elems(self, with_head: bool = True) -> int:
        h, q, kv, f = self.hidden, self.q_dim, self.kv_dim, self.ffn
        per_layer = h * q + 2 * h * kv + q * h + 3 * h * f
        n = per_layer * self.n_layers
        if with_head:
            n += self.vocab * h
        if self.input_dim:
            n += h * self.input_dim    # the input projection
        return n


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batch: int
    prefill: int
    steps: int
    s_init: int                      # initial KV capacity (bucket)
    s_max: int                       # largest KV capacity used
    cp: Optional[ModelShape] = None  # code predictor (Talker frames)
    frames: int = 0
    penalty: float = 1.0
    prefill_kind: str = "embeddings"  # or "tokens"
    len_range: Tuple[int, int] = (0, 0)  # batched: per-stream KV length range


def _shape(name, L, h, hq, hkv, d, f, v, dtype, qk_norm, qkv_bias, tables,
           n_heads=1, model_id=0, kv_dtype=F32):
    return ModelShape(name=name, n_layers=L, hidden=h, n_q_heads=hq,
                      n_kv_heads=hkv, head_dim=d, ffn=f, vocab=v,
                      n_lm_heads=n_heads, qk_norm=qk_norm, qkv_bias=qkv_bias,
                      rope_theta=1.0e6, rms_eps=1.0e-6, dtype=dtype,
                      table_vocabs=tuple(tables), model_id=model_id,
                      kv_dtype=kv_dtype)


TINY = _shape("tiny", 2, 512, 8, 4, 64, 1536, 2048, F32, True, False, [2048])
ASR = _shape("asr", 8, 512, 8, 8, 64, 2048, 151936, BF16, False, True, [151936])
TALKER06 = _shape("talker0.6b", 28, 1024, 16, 8, 128, 3072, 3072, BF16, True,
                  False, [3072] + [2048] * 15)
CP06 = _shape("code_predictor", 5, 1024, 16, 8, 128, 3072, 2048, BF16, True,
              False, [3072] + [2048] * 15, n_heads=15, model_id=1)
TALKER17 = _shape("talker1.7b", 28, 2048, 16, 8, 128, 6144, 3072, BF16, True,
                  False, [3072])
# the Talkers rotate with interleaved mRoPE, t/h/w sections [24, 20, 20]
TALKER06 = dataclasses.replace(TALKER06, mrope_sections=(24, 20, 20))
TALKER17 = dataclasses.replace(TALKER17, mrope_sections=(24, 20, 20))
# the 1.7B Talker in the frame loop (16 code tables) and its Code Predictor,
# whose inputs come in the Talker's width through an input projection
TALKER17F = dataclasses.replace(TALKER17, name="talker1.7b-frames",
                                table_vocabs=tuple([3072] + [2048] * 15))
CP17 = dataclasses.replace(CP06, name="code_predictor-1.7b", input_dim=2048)
# the batched workload states bf16 for the KV cache as well as the weights
TALKER17_KVBF16 = dataclasses.replace(TALKER17, name="talker1.7b-kvbf16", kv_dtype=BF16)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, batch=1, prefill=16, steps=16, s_init=128,
                     s_max=128, prefill_kind="tokens"),
    "asr": Workload("asr", ASR, batch=1, prefill=110, steps=400, s_init=128,
                    s_max=512),
    "talker0.6b": Workload("talker0.6b", TALKER06, batch=1, prefill=64,
                           steps=74, s_init=256, s_max=256, cp=CP06,
                           frames=75, penalty=1.05),
    "talker1.7b": Workload("talker1.7b", TALKER17, batch=1, prefill=512,
                           steps=1536, s_init=2048, s_max=2048),
    "talker1.7b-frames": Workload("talker1.7b-frames", TALKER17F, batch=1, prefill=64,
                                  steps=74, s_init=256, s_max=256, cp=CP17,
                                  frames=75, penalty=1.05),
    "batched64": Workload("batched64", TALKER17_KVBF16, batch=64, prefill=0,
                          steps=32, s_init=4096 + 64, s_max=4096 + 64,
                          len_range=(256, 4096)),
}

# code-predictor cache: 2 prefill rows + 14 steps
CP_CAPACITY = 16


# --------------------------------------------------------------------------
# drawing
# --------------------------------------------------------------------------

def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def normal(seed: int, model_id: int, tensor_id: int, shape: Sequence[int],
           scale: float = WEIGHT_SCALE) -> np.ndarray:
    """float32 N(0,1)*scale, block-seeded (see module docstring)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, np.float32)
    nb = (n + BLOCK - 1) // BLOCK

    def fill(b):
        lo, hi = b * BLOCK, min(n, (b + 1) * BLOCK)
        rng = np.random.default_rng([seed, model_id, tensor_id, b])
        rng.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        out[lo:hi] *= np.float32(scale)

    if nb > 2:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nb)))
    else:
        for b in range(nb):
            fill(b)
    return out.reshape(shape)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Storage conversion of generated inputs (NaN never occurs here)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A generated tensor: float32 values, plus bf16 bits when stored as bf16."""

    values: np.ndarray
    bits: Optional[np.ndarray] = None

    @property
    def storage(self) -> np.ndarray:
        return self.bits if self.bits is not None else self.values


def _stored(values: np.ndarray, dtype: str) -> Tensor:
    if dtype == BF16:
        bits = to_bf16_bits(values)
        return Tensor(bf16_bits_to_f32(bits).reshape(values.shape),
                      bits.reshape(values.shape))
    return Tensor(np.ascontiguousarray(values, np.float32))


@dataclasses.dataclass
class LayerWeights:
    attn_norm: np.ndarray           # [h] f32
    wq: Tensor                      # [Hq*D, h]
    wk: Tensor                      # [Hkv*D, h]
    wv: Tensor                      # [Hkv*D, h]
    bq: Optional[np.ndarray]        # [Hq*D] f32 or None
    bk: Optional[np.ndarray]
    bv: Optional[np.ndarray]
    q_norm: Optional[np.ndarray]    # [D] f32 or None
    k_norm: Optional[np.ndarray]
    wo: Tensor                      # [h, Hq*D]
    mlp_norm: np.ndarray            # [h]
    w_gate: Tensor                  # [F, h]
    w_up: Tensor                    # [F, h]
    w_down: Tensor                  # [h, F]


@dataclasses.dataclass
class ModelWeights:
    shape: ModelShape
    layers: List[LayerWeights]
    final_norm: np.ndarray          # [h]
    heads: List[Tensor]             # n_lm_heads x [V, h]
    tables: List[Tensor]            # embedding tables [V_g, in_width]
    in_proj: Optional[Tensor] = None          # [h, input_dim] when projected
    in_proj_bias: Optional[np.ndarray] = None  # [h]


def make_tables(shape: ModelShape, seed: int = 0) -> List[Tensor]:
    """Embedding tables.  Drawn with model_id 0 so stacks can share them."""
    return [_stored(normal(seed, 0, _T_TABLE + g, (v, shape.in_width)), shape.dtype)
            for g, v in enumerate(shape.table_vocabs)]


def make_weights(shape: ModelShape, seed: int = 0,
                 tables: Optional[List[Tensor]] = None, gain_sd: float = 0.0) -> ModelWeights:
    """All weights of a stack.  Gains are 1, or with gain_sd > 0 drawn as
    1 + gain_sd * N(0, 1) (float32), a separate draw per gain vector."""
    h, q, kv, f, d = shape.hidden, shape.q_dim, shape.kv_dim, shape.ffn, shape.head_dim
    mid = shape.model_id

    def gain(tid, n):
        if gain_sd <= 0.0:
            return np.ones(n, np.float32)
        return (np.float32(1.0) + normal(seed, mid, tid, (n,), scale=gain_sd)).astype(np.float32)

    layers = []
    for l in range(shape.n_layers):
        base = 1000 * (l + 1)

        def w(k, shp):
            return _stored(normal(seed, mid, base + k, shp), shape.dtype)

        def b(k, n):
            return normal(seed, mid, base + k, (n,)) if shape.qkv_bias else None

        layers.append(LayerWeights(
            attn_norm=gain(base + _T_G_ATTN, h),
            wq=w(_T_WQ, (q, h)), wk=w(_T_WK, (kv, h)), wv=w(_T_WV, (kv, h)),
            bq=b(_T_BQ, q), bk=b(_T_BK, kv), bv=b(_T_BV, kv),
            q_norm=gain(base + _T_G_Q, d) if shape.qk_norm else None,
            k_norm=gain(base + _T_G_K, d) if shape.qk_norm else None,
            wo=w(_T_WO, (h, q)), mlp_norm=gain(base + _T_G_MLP, h),
            w_gate=w(_T_WG, (f, h)), w_up=w(_T_WU, (f, h)), w_down=w(_T_WD, (h, f)),
        ))
    heads = [_stored(normal(seed, mid, _T_HEAD + j, (shape.vocab, h)), shape.dtype)
             for j in range(shape.n_lm_heads)]
    if tables is None:
        tables = make_tables(shape, seed)
    in_proj = in_bias = None
    if shape.input_dim:
        in_proj = _stored(normal(seed, mid, _T_INPROJ, (h, shape.input_dim)), shape.dtype)
        in_bias = normal(seed, mid, _T_INPROJ + 1, (h,))
    return ModelWeights(shape, layers, gain(_T_G_FINAL, h), heads, tables, in_proj, in_bias)


def prefill_embeddings(wl: Workload, seed: int = 0) -> np.ndarray:
    """[T, h] float32 N(0, 0.02) prefill inputs ("random embeddings")."""
    return normal(seed, 2, _T_PREFILL, (wl.prefill, wl.model.hidden))


def prefill_tokens(wl: Workload, seed: int = 0) -> np.ndarray:
    """[T] int32 token ids uniform in [0, V) (token prefill workloads)."""
    rng = np.random.default_rng([seed, 2, _T_TOKENS])
    return rng.integers(0, wl.model.table_vocabs[0], wl.prefill).astype(np.int32)


def text_embeddings(wl: Workload, seed: int = 0) -> np.ndarray:
    """[frames+1, h] float32 per-frame text embeddings N(0, 0.02)."""
    return normal(seed, 2, _T_TEXT, (wl.frames + 1, wl.model.hidden))


def batched_lengths(wl: Workload, seed: int = 0) -> np.ndarray:
    """Per-stream KV lengths, uniform in [lo, hi] inclusive."""
    lo, hi = wl.len_range
    return np.random.default_rng(seed).integers(lo, hi + 1, wl.batch).astype(np.int32)


def batched_first_inputs(wl: Workload, seed: int = 0) -> np.ndarray:
    """[B, h] float32 first-step inputs for the batched workload."""
    return normal(seed, 2, _T_PREFILL + 1, (wl.batch, wl.model.hidden))


KV_POOL_ROWS = 8192


def batched_kv_pool(shape: ModelShape, layer: int, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Synthetic cache rows of one layer for the batched workload: K, V
    [Hkv, KV_POOL_ROWS, D] as bf16 bit patterns of N(0, 1) values."""
    kvshape = (shape.n_kv_heads, KV_POOL_ROWS, shape.head_dim)
    tid = _T_KV + 2 * layer
    k = to_bf16_bits(normal(seed, 3, tid, kvshape, scale=1.0))
    v = to_bf16_bits(normal(seed, 3, tid + 1, kvshape, scale=1.0))
    return k.reshape(kvshape), v.reshape(kvshape)


def batched_kv_offset(stream: int, length: int) -> int:
    """First pool row of a stream's cache window (windows of different
    streams start at different rows)."""
    return (stream * 1237) % (KV_POOL_ROWS - length + 1)


def batched_kv(shape: ModelShape, stream: int, length: int, layer: int,
               seed: int = 0, pool=None) -> Tuple[np.ndarray, np.ndarray]:
    """Cache contents of one stream and layer: K, V [Hkv, length, D] bf16 bit
    patterns, a window of the layer's pool."""
    k, v = pool if pool is not None else batched_kv_pool(shape, layer, seed)
    o = batched_kv_offset(stream, length)
    return k[:, o:o + length], v[:, o:o + length]


_T_UNIFORM = 70_003


def uniforms(seed: int, stream: int, n) -> np.ndarray:
    """Uniform draws in [0, 1) (float32) for sampled token choices, one per
    choice: ``numpy.random.default_rng([seed, 2, _T_UNIFORM, stream])``.
    ``n`` may be a shape."""
    rng = np.random.default_rng([seed, 2, _T_UNIFORM, stream])
    return rng.random(n, dtype=np.float32)



@dataclasses.dataclass(frozen=True)
class CodecShape:
    """Convolution stack of a codec decoder: an input convolution, stages of
    (transposed convolution with kernel 2s, then residual units of a dilated
    convolution and a 1-tap convolution added back), an output convolution.
    Channel-major [channels, frames] float32."""
    name: str
    frames: int                      # input frames of the stack
    channels: Tuple[int, ...]        # width before the first stage, after each stage
    strides: Tuple[int, ...]
    kernel: int = 7
    dilations: Tuple[int, ...] = (1, 3, 9)
    out_channels: int = 1


_CODEC_ID = 12   # model id of the codec stack's random streams

# 6 s of audio: 300 frames of the convolution stack's input, x 480 -> 144000 samples
CODEC = CodecShape("codec", frames=300, channels=(1024, 512, 256, 128, 64), strides=(8, 5, 4, 3))


def codec_layers(c: CodecShape):
    """The stack in order: ("conv", cin, cout, K, dilation, T, residual) and
    ("trans", cin, cout, stride, T_in) entries."""
    T, ch = c.frames, c.channels
    out = [("conv", ch[0], ch[0], c.kernel, 1, T, False)]
    for i, s_ in enumerate(c.strides):
        out.append(("trans", ch[i], ch[i + 1], s_, T))
        T *= s_
        for d in c.dilations:
            out.append(("conv", ch[i + 1], ch[i + 1], c.kernel, d, T, False))
            out.append(("conv", ch[i + 1], ch[i + 1], 1, 1, T, True))
    out.append(("conv", ch[-1], c.out_channels, c.kernel, 1, T, False))
    return out


def codec_flops(c: CodecShape) -> float:
    f = 0.0
    for L in codec_layers(c):
        if L[0] == "conv":
            _, cin, cout, K, _, T, _ = L
            f += 2.0 * cin * cout * K * T
        else:
            _, cin, cout, s_, T = L
            f += 2.0 * cin * cout * 2 * T * s_
    return f


def make_codec_weights(c: CodecShape, seed: int = 0):
    """Per layer (weights, bias): conv [cout, cin, K], transposed [cin, cout, 2s];
    N(0, 1/fan_in) weights (0.09/fan_in for a residual branch's 1-tap
    convolution) and N(0, 0.01) biases."""
    ws = []
    for i, L in enumerate(codec_layers(c)):
        if L[0] == "conv":
            _, cin, cout, K, _, _, res = L
            # a residual branch's last convolution is drawn smaller, so that
            # twelve residual additions keep the activations O(1)
            sc = (0.3 if res else 1.0) / math.sqrt(cin * K)
            w = normal(seed, _CODEC_ID, 2 * i, (cout, cin, K), scale=sc)
        else:
            _, cin, cout, s_, _ = L
            w = normal(seed, _CODEC_ID, 2 * i, (cin, cout, 2 * s_), scale=1.0 / math.sqrt(2 * cin))
        ws.append((w, normal(seed, _CODEC_ID, 2 * i + 1, (L[2],), scale=0.1)))
    return ws


def codec_input(c: CodecShape, seed: int = 0) -> np.ndarray:
    """[channels[0], frames] N(0, 1) input of the stack."""
    return normal(seed, _CODEC_ID, 9999, (c.channels[0], c.frames), scale=1.0)
