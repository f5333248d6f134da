"""C-ABI tests that need no GPU: the library loads, exports every entry point
declared in include/atd.h, and the host validation layer refuses bad
arguments with the documented status codes (dry-run decoders never touch
HIP)."""

import ctypes as C
import os
import re

import pytest

from autoregressive_transformer_decode_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "atd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^(?:int|const char\*)\s+(\w+)\s*\(", src, flags=re.M)


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(B.lib, n), n


def _cfg(**kw):
    base = dict(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=128,
                vocab=100, n_lm_heads=2, n_tables=2, qk_norm=1, qkv_bias=0, dtype=B.ATD_BF16,
                kv_dtype=B.ATD_BF16,
                rope_theta=1e6, rms_eps=1e-6, max_slots=4, max_rows=8, max_ctx=64,
                flags=B.ATD_FLAG_DRY_RUN)
    base.update(kw)
    return B.atd_config(**base)


class FakeWeights:
    """Aligned, never-dereferenced pointer values for dry-run decoders."""

    def __init__(self, cfg, bias=False, qk=True, misalign=None, scales=False):
        self.next = 0x10000
        self.layers = (B.atd_layer_weights * cfg.n_layers)()
        for l in range(cfg.n_layers):
            for f in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up",
                      "w_down"):
                setattr(self.layers[l], f, self._p())
            if scales:
                for f in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
                    setattr(self.layers[l], f + "_scale", self._p())
            if bias:
                for f in ("bq", "bk", "bv"):
                    setattr(self.layers[l], f, self._p())
            if qk:
                for f in ("q_norm", "k_norm"):
                    setattr(self.layers[l], f, self._p())
        if misalign:
            setattr(self.layers[0], misalign, getattr(self.layers[0], misalign) + 4)
        self.heads = (C.c_void_p * cfg.n_lm_heads)(*[self._p() for _ in range(cfg.n_lm_heads)])
        self.tables = (C.c_void_p * cfg.n_tables)(*[self._p() for _ in range(cfg.n_tables)])
        self.vocab = (C.c_int32 * cfg.n_tables)(*([100] * cfg.n_tables))
        self.w = B.atd_weights(layers=C.cast(self.layers, C.POINTER(B.atd_layer_weights)),
                               final_norm=self._p(),
                               lm_heads=C.cast(self.heads, C.POINTER(C.c_void_p)),
                               tables=C.cast(self.tables, C.POINTER(C.c_void_p)),
                               table_vocab=C.cast(self.vocab, C.POINTER(C.c_int32)))

    def _p(self):
        self.next += 0x1000
        return self.next


def _create(cfg, fw=None):
    fw = fw or FakeWeights(cfg, bias=bool(cfg.qkv_bias), qk=bool(cfg.qk_norm))
    return B.decoder_create(cfg, fw.w), fw


@pytest.mark.parametrize("kw,code,needle", [
    (dict(head_dim=96), B.ATD_ERR_UNSUPPORTED, "head_dim 96"),
    (dict(dtype=7), B.ATD_ERR_DTYPE, "dtype 7"),
    (dict(kv_dtype=2), B.ATD_ERR_DTYPE, "kv_dtype 2"),
    (dict(n_q_heads=6, n_kv_heads=4), B.ATD_ERR_SHAPE, "n_q_heads 6"),
    (dict(n_q_heads=6, n_kv_heads=2), B.ATD_ERR_UNSUPPORTED, "= 3"),
    (dict(hidden=60), B.ATD_ERR_UNSUPPORTED, "hidden 60"),
    (dict(ffn=16384), B.ATD_ERR_UNSUPPORTED, "ffn 16384"),
    (dict(vocab=1), B.ATD_ERR_SHAPE, "vocab 1"),
    (dict(n_tables=17), B.ATD_ERR_UNSUPPORTED, "n_tables 17"),
    (dict(max_rows=0), B.ATD_ERR_CAPACITY, "max_rows 0"),
    (dict(rope_theta=-1.0), B.ATD_ERR_INVALID_ARG, "rope_theta"),
    (dict(flags=8), B.ATD_ERR_INVALID_ARG, "flags"),
])
def test_create_rejects_config(kw, code, needle):
    cfg = _cfg(**kw)
    fw = FakeWeights(_cfg())
    with pytest.raises(B.AtdError) as ei:
        B.decoder_create(cfg, fw.w)
    assert ei.value.code == code
    assert needle in str(ei.value)


def test_create_accepts_documented_flags():
    """Every flag atd.h documents is accepted; the next bit is not."""
    for f in (B.ATD_FLAG_NO_MFMA, B.ATD_FLAG_NO_L2_PREFETCH,
              B.ATD_FLAG_NO_MFMA | B.ATD_FLAG_NO_L2_PREFETCH):
        cfg = _cfg(flags=B.ATD_FLAG_DRY_RUN | f)
        h = B.decoder_create(cfg, FakeWeights(cfg).w)
        B.decoder_destroy(h)
    with pytest.raises(B.AtdError):
        cfg = _cfg(flags=B.ATD_FLAG_DRY_RUN | 8)
        B.decoder_create(cfg, FakeWeights(cfg).w)


def test_create_rejects_weights():
    cfg = _cfg()
    with pytest.raises(B.AtdError) as ei:
        B.decoder_create(cfg, FakeWeights(cfg, misalign="wk").w)
    assert ei.value.code == B.ATD_ERR_INVALID_ARG and "layers[0].wk" in str(ei.value)
    fw = FakeWeights(cfg)
    fw.layers[1].w_up = None
    with pytest.raises(B.AtdError) as ei:
        B.decoder_create(cfg, fw.w)
    assert "layers[1].w_up is NULL" in str(ei.value)
    with pytest.raises(B.AtdError) as ei:     # bias given without qkv_bias
        B.decoder_create(cfg, FakeWeights(cfg, bias=True).w)
    assert "qkv_bias = 0" in str(ei.value)
    with pytest.raises(B.AtdError) as ei:     # qk-norm gains required
        B.decoder_create(cfg, FakeWeights(cfg, qk=False).w)
    assert "q_norm is NULL" in str(ei.value)


def test_dry_run_schedule_and_kv_full():
    cfg = _cfg()
    h, fw = _create(cfg)
    try:
        kv = [0x900000 + 0x1000 * i for i in range(cfg.n_layers)]
        vv = [0xA00000 + 0x1000 * i for i in range(cfg.n_layers)]
        # nothing attached yet
        with pytest.raises(B.AtdError) as ei:
            B.decoder_prefill(h, 0, 0x5000, 4, 0, None, 0x6000, 0)
        assert "no KV buffers" in str(ei.value)
        B.kv_bucket_grow(h, 0, kv, vv, 4, 0)
        assert B.decoder_get_position(h, 0) == (0, 4)
        with pytest.raises(B.AtdError) as ei:
            B.decoder_prefill(h, 0, 0x5000, 5, 0, None, 0x6000, 0)
        assert ei.value.code == B.ATD_ERR_KV_FULL
        B.decoder_prefill(h, 0, 0x5000, 3, 1, None, 0x6000, 0)
        assert B.decoder_get_position(h, 0) == (3, 4)
        B.decoder_step(h, 0, 1, 0x7000, 1, [0], None, 0, None, 0x6000, 0)
        assert B.decoder_get_position(h, 0) == (4, 4)
        with pytest.raises(B.AtdError) as ei:       # position == capacity
            B.decoder_step(h, 0, 1, 0x7000, 1, [0], None, 0, None, 0x6000, 0)
        assert ei.value.code == B.ATD_ERR_KV_FULL and "position 4, capacity 4" in str(ei.value)
        assert B.decoder_get_position(h, 0) == (4, 4)   # refused call changed nothing
        with pytest.raises(B.AtdError) as ei:       # bucket must exceed the valid rows
            B.kv_bucket_grow(h, 0, [p + 0x400000 for p in kv], [p + 0x400000 for p in vv], 4, 0)
        assert ei.value.code == B.ATD_ERR_CAPACITY
        with pytest.raises(B.AtdError) as ei:       # aliasing the buffers in use
            B.kv_bucket_grow(h, 0, kv, [p + 0x400000 for p in vv], 8, 0)
        assert "aliases" in str(ei.value)
        B.kv_bucket_grow(h, 0, [p + 0x400000 for p in kv], [p + 0x400000 for p in vv], 8, 0)
        assert B.decoder_get_position(h, 0) == (4, 8)   # same position after growth
        B.decoder_step(h, 0, 1, 0x7000, 1, [0], None, 0, None, 0x6000, 0)
        assert B.decoder_get_position(h, 0) == (5, 8)
        with pytest.raises(B.AtdError) as ei:
            B.kv_bucket_grow(h, 0, kv, vv, 65, 0)   # beyond max_ctx
        assert ei.value.code == B.ATD_ERR_CAPACITY
    finally:
        B.decoder_destroy(h)


def test_dry_run_step_argument_checks():
    cfg = _cfg()
    h, fw = _create(cfg)
    try:
        for s in range(2):
            B.kv_bucket_grow(h, s, [0x900000 + 0x1000 * (i + 8 * s) for i in range(2)],
                             [0xA00000 + 0x1000 * (i + 8 * s) for i in range(2)], 16, 0)
        cases = [
            (dict(B=9), B.ATD_ERR_CAPACITY, "max_rows 8"),
            (dict(slot0=3, B=2), B.ATD_ERR_INVALID_ARG, "slots [3, 5)"),
            (dict(B=3), B.ATD_ERR_INVALID_ARG, "slot 2 has no KV"),
            (dict(head=2), B.ATD_ERR_INVALID_ARG, "head 2"),
            (dict(table_ids=[2]), B.ATD_ERR_INVALID_ARG, "table_ids[0] = 2"),
            (dict(G=0, table_ids=[]), B.ATD_ERR_INVALID_ARG, "G = 0 needs extra"),
            (dict(logits=None), B.ATD_ERR_INVALID_ARG, "logits_out is NULL"),
            (dict(y=0x6004), B.ATD_ERR_INVALID_ARG, "not 16-byte aligned"),
        ]
        for kw, code, needle in cases:
            a = dict(slot0=0, B=1, tok=0x7000, G=1, table_ids=[0], extra=None, head=0, y=None,
                     logits=0x6000)
            a.update(kw)
            with pytest.raises(B.AtdError) as ei:
                B.decoder_step(h, a["slot0"], a["B"], a["tok"], a["G"], a["table_ids"],
                               a["extra"], a["head"], a["y"], a["logits"], 0)
            assert ei.value.code == code, (kw, ei.value)
            assert needle in str(ei.value), (kw, str(ei.value))
        assert B.decoder_get_position(h, 0) == (0, 16)
        B.decoder_step(h, 0, 2, 0x7000, 2, [0, 1], 0x8000, 1, 0x6000, 0x6000, 0)
        assert B.decoder_get_position(h, 1) == (1, 16)
        B.decoder_set_position(h, 1, 16, 0)
        with pytest.raises(B.AtdError) as ei:
            B.decoder_step(h, 0, 2, 0x7000, 1, [0], None, 0, None, 0x6000, 0)
        assert ei.value.code == B.ATD_ERR_KV_FULL and "slot 1" in str(ei.value)
        with pytest.raises(B.AtdError):
            B.decoder_set_position(h, 1, 17, 0)
    finally:
        B.decoder_destroy(h)


def test_dry_run_step_slots():
    """decoder_step_slots: the listed slots (any subset, any order) advance and
    no other; a bad list is refused before anything changes."""
    cfg = _cfg()
    h, fw = _create(cfg)
    try:
        for s in range(4):
            B.kv_bucket_grow(h, s, [0x900000 + 0x1000 * (i + 8 * s) for i in range(2)],
                             [0xA00000 + 0x1000 * (i + 8 * s) for i in range(2)], 4, 0)
        B.decoder_step_slots(h, 2, [3, 1], 0x7000, 1, [0], None, 0, None, 0x6000, 0)
        assert [B.decoder_get_position(h, s)[0] for s in range(4)] == [0, 1, 0, 1]
        B.decoder_step_slots(h, 3, [1, 0, 3], 0x7000, 1, [0], None, 0, None, 0x6000, 0)
        assert [B.decoder_get_position(h, s)[0] for s in range(4)] == [1, 2, 0, 2]
        cases = [
            ([2, 2], B.ATD_ERR_INVALID_ARG, "appears twice"),
            ([0, 4], B.ATD_ERR_INVALID_ARG, "slots[1] = 4 outside [0, 4)"),
            ([-1], B.ATD_ERR_INVALID_ARG, "slots[0] = -1"),
        ]
        for slots, code, needle in cases:
            with pytest.raises(B.AtdError) as ei:
                B.decoder_step_slots(h, len(slots), slots, 0x7000, 1, [0], None, 0, None,
                                     0x6000, 0)
            assert ei.value.code == code and needle in str(ei.value), (slots, ei.value)
        with pytest.raises(B.AtdError) as ei:
            B.decoder_step_slots(h, 9, list(range(9)), 0x7000, 1, [0], None, 0, None, 0x6000, 0)
        assert ei.value.code == B.ATD_ERR_CAPACITY
        B.decoder_set_position(h, 3, 4, 0)
        with pytest.raises(B.AtdError) as ei:      # slot 3 full: nothing advances
            B.decoder_step_slots(h, 2, [2, 3], 0x7000, 1, [0], None, 0, None, 0x6000, 0)
        assert ei.value.code == B.ATD_ERR_KV_FULL and "slot 3" in str(ei.value)
        assert [B.decoder_get_position(h, s)[0] for s in range(4)] == [1, 2, 0, 4]
        rc = B.lib.decoder_step_slots(h, 1, None, 0x7000, 1, B._i32_array([0]), None, 0, None,
                                      0x6000, 0)
        assert rc == B.ATD_ERR_INVALID_ARG and "slots is NULL" in B.decoder_last_error(h)
    finally:
        B.decoder_destroy(h)


def test_workspace_bytes():
    """atd_workspace_bytes: what decoder_create allocates; grows with the
    rows, slots and context the decoder is sized for; 0 for a dry run; config
    errors as decoder_create."""
    base = dict(flags=0)
    small = B.atd_workspace_bytes(_cfg(**base), 0)
    assert small > 0 and small % 256 == 0
    assert B.atd_workspace_bytes(_cfg(max_rows=64, **base), 0) > small
    assert B.atd_workspace_bytes(_cfg(max_ctx=4096, **base), 0) > small
    assert B.atd_workspace_bytes(_cfg(max_slots=64, **base), 0) > small
    assert B.atd_workspace_bytes(_cfg(input_dim=128, **base), 1) > small
    assert B.atd_workspace_bytes(_cfg(), 0) == 0
    with pytest.raises(B.AtdError) as ei:
        B.atd_workspace_bytes(_cfg(head_dim=96, **base), 0)
    assert ei.value.code == B.ATD_ERR_UNSUPPORTED


def test_greedy_argmax_argument_checks():
    for args, needle in [((0, 1, 10, None, 1.0, 0x100, None, 0), "NULL"),
                         ((0x100, 0, 10, None, 1.0, 0x100, None, 0), "B = 0"),
                         ((0x100, 1, 1, None, 1.0, 0x100, None, 0), "V = 1"),
                         ((0x100, 1, 10, None, 0.0, 0x100, None, 0), "penalty"),
                         ((0x100, 1, 10, None, float("nan"), 0x100, None, 0), "penalty")]:
        with pytest.raises(B.AtdError) as ei:
            B.greedy_argmax(*args)
        assert ei.value.code == B.ATD_ERR_INVALID_ARG and needle in str(ei.value)


def test_create_without_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    cfg = _cfg(flags=0)
    fw = FakeWeights(cfg)
    with pytest.raises(B.AtdError) as ei:
        B.decoder_create(cfg, fw.w)
    assert ei.value.code == B.ATD_ERR_DEVICE


def test_dry_run_talker_frames():
    """talker_generate_frames: shape/slot/capacity checks, and the positions
    it leaves (Talker + n_frames - 1 rows, Code Predictor at 16)."""
    tk, tfw = _create(_cfg(n_tables=16, n_lm_heads=1))
    cp, cfw = _create(_cfg(n_tables=16, n_lm_heads=15))
    small, sfw = _create(_cfg(n_tables=16, n_lm_heads=4))
    L = 2
    try:
        kv = lambda base: ([base + 0x1000 * i for i in range(L)], [base + 0x80000 + 0x1000 * i for i in range(L)])  # noqa: E731
        B.kv_bucket_grow(tk, 0, *kv(0x900000), 40, 0)
        B.decoder_prefill(tk, 0, 0x5000, 8, 0, None, 0x6000, 0)
        args = lambda n, cpd=cp, ts=None, cs=None: (  # noqa: E731
            tk, 0, cpd, 0, n, 0x7000, 0x8000, 0x9000, 0xA000, 1.05, ts, cs, None, 0xB000, 0xC000, 0)
        with pytest.raises(B.AtdError) as ei:          # Code Predictor slot not attached
            B.talker_generate_frames(*args(4))
        assert "Code Predictor slot 0" in str(ei.value)
        B.kv_bucket_grow(cp, 0, *kv(0xD00000), 12, 0)
        with pytest.raises(B.AtdError) as ei:          # a pass needs 16 rows
            B.talker_generate_frames(*args(4))
        assert ei.value.code == B.ATD_ERR_KV_FULL
        B.kv_bucket_grow(cp, 0, *kv(0xE00000), 16, 0)
        B.kv_bucket_grow(small, 0, *kv(0xF00000), 16, 0)
        with pytest.raises(B.AtdError) as ei:          # too few LM heads
            B.talker_generate_frames(*args(4, small))
        assert ei.value.code == B.ATD_ERR_SHAPE
        with pytest.raises(B.AtdError) as ei:          # 33 more rows do not fit 40 from 8
            B.talker_generate_frames(*args(34))
        assert ei.value.code == B.ATD_ERR_KV_FULL
        assert B.decoder_get_position(tk, 0) == (8, 40)
        B.talker_generate_frames(*args(5))
        assert B.decoder_get_position(tk, 0) == (12, 40)
        assert B.decoder_get_position(cp, 0) == (16, 16)
        B.talker_generate_frames(*args(1))             # one frame: no Talker step
        assert B.decoder_get_position(tk, 0) == (12, 40)
        with pytest.raises(B.AtdError):
            B.talker_generate_frames(*args(0))
        ok = B.atd_sampling(50, 0.9, 1.0, 0x10000)
        B.talker_generate_frames(*args(3, cp, ok, ok))  # sampled: same positions
        assert B.decoder_get_position(tk, 0) == (14, 40)
        for bad in (B.atd_sampling(101, 0.9, 1.0, 0x10000),      # top_k > V = 100
                    B.atd_sampling(50, 0.9, 1.0, None)):         # no uniforms
            with pytest.raises(B.AtdError) as ei:
                B.talker_generate_frames(*args(2, cp, None, bad))
            assert ei.value.code == B.ATD_ERR_INVALID_ARG
        assert B.decoder_get_position(tk, 0) == (14, 40)
    finally:
        for h in (tk, cp, small):
            B.decoder_destroy(h)


def test_sample_topk_argument_checks():
    """sample_topk and the sampling settings: every refusal happens in host
    code before any device call."""
    ok = dict(top_k=50, temperature=0.9, top_p=1.0, uniforms=0x300)
    cases = [
        (dict(ok, top_k=0), "top_k", B.ATD_ERR_INVALID_ARG),
        (dict(ok, top_k=257), "top_k", B.ATD_ERR_INVALID_ARG),
        (dict(ok, top_k=1001), "top_k", B.ATD_ERR_INVALID_ARG),      # > V
        (dict(ok, temperature=0.0), "temperature", B.ATD_ERR_INVALID_ARG),
        (dict(ok, temperature=float("inf")), "temperature", B.ATD_ERR_INVALID_ARG),
        (dict(ok, temperature=float("nan")), "temperature", B.ATD_ERR_INVALID_ARG),
        (dict(ok, top_p=0.0), "top_p", B.ATD_ERR_INVALID_ARG),
        (dict(ok, top_p=1.5), "top_p", B.ATD_ERR_INVALID_ARG),
        (dict(ok, top_p=float("nan")), "top_p", B.ATD_ERR_INVALID_ARG),
        (dict(ok, uniforms=None), "uniforms", B.ATD_ERR_INVALID_ARG),
    ]
    for kw, needle, code in cases:
        with pytest.raises(B.AtdError) as ei:
            B.sample_topk(0x100, 2, 1000, None, 1.0, B.atd_sampling(**kw), 0x200, 0)
        assert ei.value.code == code and needle in str(ei.value), (kw, str(ei.value))
    # 300000 logits in 37 chunks keep 37 * 256 candidates: more than one
    # workgroup selects from
    with pytest.raises(B.AtdError) as ei:
        B.sample_topk(0x100, 1, 300000, None, 1.0, B.atd_sampling(**dict(ok, top_k=256)),
                      0x200, 0)
    assert ei.value.code == B.ATD_ERR_UNSUPPORTED
    with pytest.raises(B.AtdError) as ei:
        B.sample_topk(0x100, 1, 1000, None, 0.0, B.atd_sampling(**ok), 0x200, 0)
    assert "penalty" in str(ei.value)
    with pytest.raises(B.AtdError):
        B.sample_topk(None, 1, 1000, None, 1.0, B.atd_sampling(**ok), 0x200, 0)


def test_dry_run_generate_sampling():
    """decoder_generate takes sampling settings (checked against the vocab)
    and advances the position like the greedy form."""
    h, fw = _create(_cfg())
    try:
        L = 2
        B.kv_bucket_grow(h, 0, [0x1000 * (i + 1) for i in range(L)],
                         [0x80000 + 0x1000 * i for i in range(L)], 32, 0)
        B.decoder_prefill(h, 0, 0x5000, 4, 0, None, 0x6000, 0)
        sp = B.atd_sampling(50, 0.9, 1.0, 0x7000)
        B.decoder_generate(h, 0, 5, 0x8000, 1, [0], None, 0, None, 1.0, sp, None, None,
                           0x6000, 0)
        assert B.decoder_get_position(h, 0) == (9, 32)
        with pytest.raises(B.AtdError) as ei:
            B.decoder_generate(h, 0, 5, 0x8000, 1, [0], None, 0, None, 1.0,
                               B.atd_sampling(101, 0.9, 1.0, 0x7000), None, None, 0x6000, 0)
        assert ei.value.code == B.ATD_ERR_INVALID_ARG and "top_k" in str(ei.value)
        B.decoder_generate(h, 0, 5, 0x8000, 1, [0], None, 0, None, 1.0, None, None, None,
                           0x6000, 0)
        assert B.decoder_get_position(h, 0) == (14, 32)
    finally:
        B.decoder_destroy(h)


def test_quantized_config_checks():
    """weight_format: unknown value, shapes that are not whole blocks, and
    scale pointers missing (quantized) or present (dense) are refused; a
    quantized dry-run decoder steps like a dense one."""
    with pytest.raises(B.AtdError) as ei:
        B.decoder_create(_cfg(weight_format=7), FakeWeights(_cfg(), scales=True).w)
    assert ei.value.code == B.ATD_ERR_DTYPE
    with pytest.raises(B.AtdError) as ei:
        B.decoder_create(_cfg(weight_format=B.ATD_WFMT_Q8, ffn=136),
                         FakeWeights(_cfg(), scales=True).w)
    assert ei.value.code == B.ATD_ERR_SHAPE and "ffn 136" in str(ei.value)
    with pytest.raises(B.AtdError) as ei:
        B.decoder_create(_cfg(weight_format=B.ATD_WFMT_Q4), FakeWeights(_cfg()).w)
    assert ei.value.code == B.ATD_ERR_INVALID_ARG and "wq_scale" in str(ei.value)
    with pytest.raises(B.AtdError) as ei:
        B.decoder_create(_cfg(), FakeWeights(_cfg(), scales=True).w)
    assert ei.value.code == B.ATD_ERR_INVALID_ARG and "dense" in str(ei.value)
    cfg = _cfg(weight_format=B.ATD_WFMT_Q4)
    fw = FakeWeights(cfg, scales=True)
    h = B.decoder_create(cfg, fw.w)
    try:
        B.kv_bucket_grow(h, 0, [0x1000, 0x2000], [0x3000, 0x4000], 16, 0)
        B.decoder_prefill(h, 0, 0x5000, 4, 0, None, 0x6000, 0)
        assert B.decoder_get_position(h, 0) == (4, 16)
    finally:
        B.decoder_destroy(h)


def test_quantize_blocks_argument_checks():
    ok = (0x1000, B.ATD_BF16, 4, 64, B.ATD_WFMT_Q8, 0x2000, 0x3000, 0)
    cases = [
        ((None,) + ok[1:], B.ATD_ERR_INVALID_ARG, "NULL"),
        (ok[:5] + (0x2008,) + ok[6:], B.ATD_ERR_INVALID_ARG, "aligned"),
        (ok[:6] + (0x3001,) + ok[7:], B.ATD_ERR_INVALID_ARG, "aligned"),
        ((0x1000, 5) + ok[2:], B.ATD_ERR_DTYPE, "dtype 5"),
        (ok[:4] + (B.ATD_WFMT_DENSE,) + ok[5:], B.ATD_ERR_DTYPE, "format 0"),
        (ok[:3] + (48,) + ok[4:], B.ATD_ERR_SHAPE, "cols 48"),
        (ok[:2] + (0,) + ok[3:], B.ATD_ERR_SHAPE, "rows 0"),
    ]
    for args, code, needle in cases:
        with pytest.raises(B.AtdError) as ei:
            B.quantize_blocks(*args)
        assert ei.value.code == code and needle in str(ei.value), (args, str(ei.value))


def test_controls_argument_checks():
    """atd_controls: eos outside [-1, V), negative counts and misaligned
    pointers are refused before any device call."""
    for ctl, needle in [(B.atd_controls(None, 10, 0, 0, None), "eos 10"),
                        (B.atd_controls(None, -2, 0, 0, None), "eos -2"),
                        (B.atd_controls(None, 3, -1, 0, None), "min_new_tokens"),
                        (B.atd_controls(None, 3, 0, -4, None), "first_index"),
                        (B.atd_controls(0x102, 3, 0, 0, None), "aligned"),
                        (B.atd_controls(None, 3, 0, 0, 0x203), "aligned")]:
        with pytest.raises(B.AtdError) as ei:
            B.greedy_argmax(0x100, 1, 10, None, 1.0, 0x200, None, 0, controls=ctl)
        assert ei.value.code == B.ATD_ERR_INVALID_ARG and needle in str(ei.value), str(ei.value)
        with pytest.raises(B.AtdError):
            B.sample_topk(0x100, 1, 10, None, 1.0, B.atd_sampling(5, 1.0, 1.0, 0x300), 0x200, 0,
                          controls=ctl)
    h, fw = _create(_cfg())
    try:
        B.kv_bucket_grow(h, 0, [0x1000, 0x2000], [0x3000, 0x4000], 32, 0)
        B.decoder_prefill(h, 0, 0x5000, 4, 0, None, 0x6000, 0)
        good = B.atd_controls(0x7000, 5, 3, 1, 0x8000)
        B.decoder_generate(h, 0, 6, 0x9000, 1, [0], None, 0, None, 1.0, None, None, None, 0x6000,
                           0, controls=good)
        assert B.decoder_get_position(h, 0) == (10, 32)
        with pytest.raises(B.AtdError):
            B.decoder_generate(h, 0, 6, 0x9000, 1, [0], None, 0, None, 1.0, None, None, None,
                               0x6000, 0, controls=B.atd_controls(None, 100, 0, 0, None))
    finally:
        B.decoder_destroy(h)


def test_codec_argument_checks():
    """The codec convolutions refuse NULL / misaligned pointers and sizes
    below 1 before any device call."""
    with pytest.raises(B.AtdError) as ei:
        B.codec_conv1d_causal(None, 0x100, None, 4, 4, 8, 3, 1, 0, 0x200, 0)
    assert ei.value.code == B.ATD_ERR_INVALID_ARG
    with pytest.raises(B.AtdError) as ei:
        B.codec_conv1d_causal(0x102, 0x100, None, 4, 4, 8, 3, 1, 0, 0x200, 0)
    assert "aligned" in str(ei.value)
    for args in [(0, 4, 8, 3, 1), (4, 4, 8, 0, 1), (4, 4, 8, 3, 0), (4, 4, 0, 3, 1)]:
        with pytest.raises(B.AtdError) as ei:
            B.codec_conv1d_causal(0x100, 0x200, None, *args, 0, 0x300, 0)
        assert ei.value.code == B.ATD_ERR_INVALID_ARG
    with pytest.raises(B.AtdError):
        B.codec_conv1d_causal(0x100, 0x200, 0x301, 4, 4, 8, 3, 1, 0, 0x300, 0)
    with pytest.raises(B.AtdError):
        B.codec_transconv1d(0x100, 0x200, None, 4, 4, 8, 0, 0x300, 0)
    with pytest.raises(B.AtdError):
        B.codec_transconv1d_pack(0x100, 4, 0, 2, 0x200, 0)
    with pytest.raises(B.AtdError) as ei:
        B.codec_conv1d_causal(0x100, 0x200, None, 1 << 16, 4, 1 << 16, 3, 1, 0, 0x300, 0)
    assert "2^31" in str(ei.value)


@pytest.mark.parametrize("sec,ok", [((0, 0, 0), True), ((24, 20, 20), True), ((64, 0, 0), True),
                                    ((22, 21, 21), True), ((24, 20, 21), False),
                                    ((-4, 34, 34), False), ((4, 30, 30), False)])
def test_mrope_sections_and_entry_checks(sec, ok):
    """mrope_sections must cover D/2 = 64 frequencies with 3 max(s_h, s_w) <=
    64; the *_mrope entry points refuse a NULL rope_pos and otherwise follow
    the plain entry points' schedule."""
    cfg = _cfg(head_dim=128, n_q_heads=4, n_kv_heads=2)
    cfg.mrope_sections = (C.c_int32 * 3)(*sec)
    if not ok:
        with pytest.raises(B.AtdError) as ei:
            B.decoder_create(cfg, FakeWeights(cfg).w)
        assert ei.value.code == B.ATD_ERR_INVALID_ARG and "mrope_sections" in str(ei.value)
        return
    h, fw = _create(cfg)
    try:
        B.kv_bucket_grow(h, 0, [0x900000 + 0x1000 * i for i in range(cfg.n_layers)],
                         [0xA00000 + 0x1000 * i for i in range(cfg.n_layers)], 16, 0)
        with pytest.raises(B.AtdError) as ei:
            B.decoder_prefill_mrope(h, 0, 0x5000, 3, None, 0, None, 0x6000, 0)
        assert "rope_pos is NULL" in str(ei.value)
        with pytest.raises(B.AtdError) as ei:
            B.decoder_prefill_mrope(h, 0, 0x5000, 17, 0x7100, 0, None, 0x6000, 0)
        assert ei.value.code == B.ATD_ERR_CAPACITY
        B.decoder_prefill_mrope(h, 0, 0x5000, 3, 0x7100, 0, None, 0x6000, 0)
        assert B.decoder_get_position(h, 0) == (3, 16)
        with pytest.raises(B.AtdError) as ei:
            B.decoder_step_mrope(h, 0, 1, 0x7000, 1, [0], None, None, 0, None, 0x6000, 0)
        assert "rope_pos is NULL" in str(ei.value)
        B.decoder_step_mrope(h, 0, 1, 0x7000, 1, [0], None, 0x7100, 0, None, 0x6000, 0)
        assert B.decoder_get_position(h, 0) == (4, 16)
    finally:
        B.decoder_destroy(h)
