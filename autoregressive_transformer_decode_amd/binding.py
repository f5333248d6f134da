"""ctypes binding of libatd.so: one Python function per C entry point, same
names and argument order (pointers as integers, the stream as an integer
hipStream_t).  Marshalling and error translation only: every computation
runs in the library's HIP kernels.  Importing this module fails loudly if the
library has not been built."""

from __future__ import annotations

import ctypes as C
import os

# One HIP runtime per process: torch ships its own libamdhip64 with the same
# soname as the system one.  Loading torch first makes the library bind to the
# runtime that torch's allocator and streams live in; loading the library
# first would bring in a second runtime.
import torch  # noqa: F401  (imported for its HIP runtime)

HERE = os.path.dirname(os.path.abspath(__file__))
# ATD_LIBRARY names another build of the same library (e.g. the host-sanitized
# one that build.py makes with --sanitize); the default is the in-tree build.
LIB_PATH = os.environ.get("ATD_LIBRARY") or os.path.join(HERE, "libatd.so")

ATD_OK = 0
ATD_ERR_INVALID_ARG = -1
ATD_ERR_SHAPE = -2
ATD_ERR_DTYPE = -3
ATD_ERR_KV_FULL = -4
ATD_ERR_CAPACITY = -5
ATD_ERR_DEVICE = -6
ATD_ERR_UNSUPPORTED = -7
ATD_F32 = 0
ATD_BF16 = 1
ATD_FLAG_DRY_RUN = 1
ATD_FLAG_NO_MFMA = 2
ATD_FLAG_NO_L2_PREFETCH = 4
ATD_WFMT_DENSE, ATD_WFMT_Q8, ATD_WFMT_Q4 = 0, 1, 2
ATD_QBLOCK = 32

STATUS_NAMES = {0: "OK", -1: "INVALID_ARG", -2: "SHAPE", -3: "DTYPE", -4: "KV_FULL",
                -5: "CAPACITY", -6: "DEVICE", -7: "UNSUPPORTED"}

EXPORTS = ("decoder_create", "decoder_destroy", "decoder_last_error", "kv_bucket_grow",
           "decoder_set_position", "decoder_get_position", "decoder_prefill",
           "decoder_step", "decoder_step_slots", "atd_workspace_bytes", "decoder_prefill_mrope", "decoder_step_mrope", "decoder_embed", "greedy_argmax", "greedy_argmax_noalloc", "sample_topk", "decoder_generate",
           "talker_generate_frames", "quantize_blocks", "codec_conv1d_causal",
           "codec_transconv1d_pack", "codec_transconv1d", "decoder_time_stage", "atd_read_stream")

ATD_STAGE_QKV, ATD_STAGE_ROPE, ATD_STAGE_ATTN, ATD_STAGE_OPROJ, ATD_STAGE_GATEUP, \
    ATD_STAGE_DOWN, ATD_STAGE_HEAD = range(7)


class AtdError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


class atd_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("n_lm_heads", C.c_int32), ("n_tables", C.c_int32),
                ("qk_norm", C.c_int32), ("qkv_bias", C.c_int32), ("dtype", C.c_int32),
                ("kv_dtype", C.c_int32),
                ("rope_theta", C.c_double), ("rms_eps", C.c_float),
                ("max_slots", C.c_int32), ("max_rows", C.c_int32), ("max_ctx", C.c_int32),
                ("flags", C.c_int32), ("weight_format", C.c_int32), ("input_dim", C.c_int32),
                ("mrope_sections", C.c_int32 * 3)]


ATD_TOPK_MAX = 256


class atd_sampling(C.Structure):
    _fields_ = [("top_k", C.c_int32), ("temperature", C.c_float), ("top_p", C.c_float),
                ("uniforms", C.c_void_p)]


class atd_controls(C.Structure):
    _fields_ = [("suppress", C.c_void_p), ("eos", C.c_int32), ("min_new_tokens", C.c_int32),
                ("first_index", C.c_int32), ("eos_step", C.c_void_p)]


class atd_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "q_norm", "k_norm", "wo",
        "mlp_norm", "w_gate", "w_up", "w_down", "wq_scale", "wk_scale", "wv_scale", "wo_scale",
        "w_gate_scale", "w_up_scale", "w_down_scale")]


class atd_weights(C.Structure):
    _fields_ = [("layers", C.POINTER(atd_layer_weights)), ("final_norm", C.c_void_p),
                ("lm_heads", C.POINTER(C.c_void_p)), ("tables", C.POINTER(C.c_void_p)),
                ("table_vocab", C.POINTER(C.c_int32)), ("in_proj", C.c_void_p),
                ("in_proj_bias", C.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m autoregressive_transformer_decode_amd.build` (there is no fallback)")
    lib = C.CDLL(LIB_PATH)
    vp, i32, f32 = C.c_void_p, C.c_int32, C.c_float
    sig = {
        "decoder_create": ([C.POINTER(atd_config), C.POINTER(atd_weights), C.POINTER(vp)], C.c_int),
        "decoder_destroy": ([vp], C.c_int),
        "decoder_last_error": ([vp], C.c_char_p),
        "kv_bucket_grow": ([vp, i32, C.POINTER(vp), C.POINTER(vp), i32, vp], C.c_int),
        "decoder_set_position": ([vp, i32, i32, vp], C.c_int),
        "decoder_get_position": ([vp, i32, C.POINTER(i32), C.POINTER(i32)], C.c_int),
        "decoder_prefill": ([vp, i32, vp, i32, i32, vp, vp, vp], C.c_int),
        "decoder_step": ([vp, i32, i32, vp, i32, C.POINTER(i32), vp, i32, vp, vp, vp], C.c_int),
        "decoder_step_slots": ([vp, i32, C.POINTER(i32), vp, i32, C.POINTER(i32), vp, i32, vp,
                                vp, vp], C.c_int),
        "atd_workspace_bytes": ([C.POINTER(atd_config), i32, C.POINTER(C.c_size_t)], C.c_int),
        "decoder_prefill_mrope": ([vp, i32, vp, i32, vp, i32, vp, vp, vp], C.c_int),
        "decoder_step_mrope": ([vp, i32, i32, vp, i32, C.POINTER(i32), vp, vp, i32, vp, vp, vp],
                               C.c_int),
        "decoder_embed": ([vp, i32, vp, i32, C.POINTER(i32), vp, vp, vp], C.c_int),
        "greedy_argmax": ([vp, i32, i32, vp, f32, C.POINTER(atd_controls), vp, vp, vp], C.c_int),
        "greedy_argmax_noalloc": ([vp, i32, i32, vp, f32, C.POINTER(atd_controls), vp, vp, vp],
                                  C.c_int),
        "sample_topk": ([vp, i32, i32, vp, f32, C.POINTER(atd_sampling), C.POINTER(atd_controls),
                         vp, vp], C.c_int),
        "decoder_generate": ([vp, i32, i32, vp, i32, C.POINTER(i32), vp, i32, vp, f32,
                              C.POINTER(atd_sampling), C.POINTER(atd_controls), vp, vp, vp, vp],
                             C.c_int),
        "talker_generate_frames": ([vp, i32, vp, i32, i32, vp, vp, vp, vp, f32,
                                    C.POINTER(atd_sampling), C.POINTER(atd_sampling),
                                    C.POINTER(atd_controls), vp, vp, vp, vp], C.c_int),
        "quantize_blocks": ([vp, i32, C.c_int64, i32, i32, vp, vp, vp], C.c_int),
        "codec_conv1d_causal": ([vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp], C.c_int),
        "codec_transconv1d_pack": ([vp, i32, i32, i32, vp, vp], C.c_int),
        "codec_transconv1d": ([vp, vp, vp, i32, i32, i32, i32, vp, vp], C.c_int),
        "decoder_time_stage": ([vp, i32, i32, i32, i32, vp, C.POINTER(C.c_double)], C.c_int),
        "atd_read_stream": ([vp, C.c_size_t, i32, vp, vp, C.POINTER(C.c_double)], C.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def _check(rc: int, handle=None):
    if rc != ATD_OK:
        msg = lib.decoder_last_error(handle).decode(errors="replace")
        raise AtdError(rc, msg)
    return rc


def _i32_array(vals):
    arr = (C.c_int32 * max(1, len(vals)))(*vals)
    return arr


def _ptr_array(vals):
    return (C.c_void_p * max(1, len(vals)))(*vals)


# ----------------------------------------------------------------- entry points

def decoder_create(cfg: atd_config, weights: atd_weights) -> int:
    out = C.c_void_p()
    _check(lib.decoder_create(C.byref(cfg), C.byref(weights), C.byref(out)))
    return out.value


def decoder_destroy(handle: int) -> None:
    _check(lib.decoder_destroy(handle))


def decoder_last_error(handle) -> str:
    return lib.decoder_last_error(handle).decode(errors="replace")


def kv_bucket_grow(handle: int, slot: int, k_new, v_new, s_new: int, stream: int) -> None:
    _check(lib.kv_bucket_grow(handle, slot, _ptr_array(k_new), _ptr_array(v_new), s_new,
                              stream), handle)


def decoder_set_position(handle: int, slot: int, pos: int, stream: int) -> None:
    _check(lib.decoder_set_position(handle, slot, pos, stream), handle)


def decoder_get_position(handle: int, slot: int):
    p, c = C.c_int32(), C.c_int32()
    _check(lib.decoder_get_position(handle, slot, C.byref(p), C.byref(c)), handle)
    return p.value, c.value


def decoder_prefill(handle: int, slot: int, x: int, T: int, head: int, y_out, logits_out: int,
                    stream: int) -> None:
    _check(lib.decoder_prefill(handle, slot, x, T, head, y_out, logits_out, stream), handle)


def decoder_step(handle: int, slot0: int, B: int, tok, G: int, table_ids, extra, head: int,
                 y_out, logits_out: int, stream: int) -> None:
    _check(lib.decoder_step(handle, slot0, B, tok, G, _i32_array(list(table_ids)), extra, head,
                            y_out, logits_out, stream), handle)


def decoder_step_slots(handle: int, B: int, slots, tok, G: int, table_ids, extra, head: int,
                       y_out, logits_out: int, stream: int) -> None:
    _check(lib.decoder_step_slots(handle, B, _i32_array(list(slots)), tok, G,
                                  _i32_array(list(table_ids)), extra, head, y_out, logits_out,
                                  stream), handle)


def atd_workspace_bytes(cfg: atd_config, input_projection: int) -> int:
    out = C.c_size_t(0)
    _check(lib.atd_workspace_bytes(C.byref(cfg), input_projection, C.byref(out)))
    return out.value


def decoder_prefill_mrope(handle: int, slot: int, x: int, T: int, rope_pos, head: int, y_out,
                          logits_out: int, stream: int) -> None:
    _check(lib.decoder_prefill_mrope(handle, slot, x, T, rope_pos, head, y_out, logits_out,
                                     stream), handle)


def decoder_step_mrope(handle: int, slot0: int, B: int, tok, G: int, table_ids, extra,
                       rope_pos, head: int, y_out, logits_out: int, stream: int) -> None:
    _check(lib.decoder_step_mrope(handle, slot0, B, tok, G, _i32_array(list(table_ids)), extra,
                                  rope_pos, head, y_out, logits_out, stream), handle)


def decoder_embed(handle: int, B: int, tok, G: int, table_ids, extra, x_out: int,
                  stream: int) -> None:
    _check(lib.decoder_embed(handle, B, tok, G, _i32_array(list(table_ids)), extra, x_out,
                             stream), handle)


def greedy_argmax(logits: int, B: int, V: int, seen, penalty: float, tok_out: int, margin_out,
                  stream: int, controls=None) -> None:
    _check(lib.greedy_argmax(logits, B, V, seen, penalty, _byref(controls), tok_out, margin_out,
                             stream))


def greedy_argmax_noalloc(logits: int, B: int, V: int, seen, penalty: float, tok_out: int,
                          margin_out, stream: int, controls=None) -> None:
    _check(lib.greedy_argmax_noalloc(logits, B, V, seen, penalty, _byref(controls), tok_out,
                                     margin_out, stream))


def _byref(st):
    """None, or a ctypes struct passed by reference."""
    return None if st is None else C.byref(st)


def sample_topk(logits: int, B: int, V: int, seen, penalty: float, sampling: atd_sampling,
                tok_out: int, stream: int, controls=None) -> None:
    _check(lib.sample_topk(logits, B, V, seen, penalty, C.byref(sampling), _byref(controls),
                           tok_out, stream))


def decoder_generate(handle: int, slot: int, n_steps: int, tok_io: int, G: int, table_ids,
                     extra, head: int, seen, penalty: float, sampling, tokens_out, y_out,
                     logits_out: int, stream: int, controls=None) -> None:
    _check(lib.decoder_generate(handle, slot, n_steps, tok_io, G, _i32_array(list(table_ids)),
                                extra, head, seen, penalty, _byref(sampling), _byref(controls),
                                tokens_out, y_out, logits_out, stream), handle)


def talker_generate_frames(tk: int, tk_slot: int, cp: int, cp_slot: int, n_frames: int,
                           codes_io: int, y_io: int, text, seen: int, penalty: float,
                           tk_sampling, cp_sampling, codes_out, tk_logits: int, cp_logits: int,
                           stream: int, tk_controls=None) -> None:
    _check(lib.talker_generate_frames(tk, tk_slot, cp, cp_slot, n_frames, codes_io, y_io, text,
                                      seen, penalty, _byref(tk_sampling), _byref(cp_sampling),
                                      _byref(tk_controls), codes_out, tk_logits, cp_logits,
                                      stream), tk)


def quantize_blocks(w: int, dtype: int, rows: int, cols: int, fmt: int, codes: int, scales: int,
                    stream: int) -> None:
    _check(lib.quantize_blocks(w, dtype, rows, cols, fmt, codes, scales, stream))


def codec_conv1d_causal(x: int, w: int, bias, cin: int, cout: int, T: int, K: int,
                        dilation: int, accumulate: int, y: int, stream: int) -> None:
    _check(lib.codec_conv1d_causal(x, w, bias, cin, cout, T, K, dilation, accumulate, y, stream))


def codec_transconv1d_pack(w: int, cin: int, cout: int, stride: int, packed: int,
                           stream: int) -> None:
    _check(lib.codec_transconv1d_pack(w, cin, cout, stride, packed, stream))


def codec_transconv1d(x: int, packed: int, bias, cin: int, cout: int, T: int, stride: int,
                      y: int, stream: int) -> None:
    _check(lib.codec_transconv1d(x, packed, bias, cin, cout, T, stride, y, stream))


def decoder_time_stage(handle: int, stage: int, slot0: int, B: int, reps: int,
                       stream: int) -> float:
    us = C.c_double(0.0)
    _check(lib.decoder_time_stage(handle, stage, slot0, B, reps, stream, C.byref(us)), handle)
    return us.value


def atd_read_stream(buf: int, nbytes: int, reps: int, sink: int, stream: int) -> float:
    us = C.c_double(0.0)
    _check(lib.atd_read_stream(buf, nbytes, reps, sink, stream, C.byref(us)))
    return us.value
