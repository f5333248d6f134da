#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload talker1.7b]

A step is one decode step of the whole stack (embedding, every layer, final
norm, LM head, penalized greedy argmax feeding the next step) on synthetic
seeded weights and inputs already resident in HBM.  The default workload is
the 1.7B Talker shape at batch 1: a 512-row prefill (untimed), then K greedy
steps replayed from a HIP graph on the device (K = 1536 runs the context to
2048; with fewer steps, untimed steps first move the context so that the
timed ones sit around the workload's mean context, 1280, and config.context
names the timed range).  The same run then times the batched workload on the
same weights (64 streams, seeded cache lengths in [256, 4096], bf16 cache, 32
iterations of one step per stream) and reports it under "batch64", with its
own CPU oracle baseline.  Prints one JSON line.

Also measured in the same run:
  roofline      the dominant kernel (RMSNorm + gate/up + SwiGLU GEMV): its
                algorithmic bytes per launch over its average duration; the
                library enqueues that kernel for every layer in turn (each
                layer's weights once, as in a step) between two HIP events on
                this stream; HBM traffic per launch from the committed
                rocprofv3 counter summary when it matches the kernel source.
  cpu_baseline  the CPU oracle on this host's cores, on a bounded sample of
                the same workload (decode steps after the same prefill).
  hbm_attainable  the device's attainable read bandwidth: the library's
                streaming read kernel over 4 GiB (past the 256 MB memory-side
                cache); step_hbm.frac_of_attainable is the step against it.
  sampled       the same K steps with the Qwen TTS sampling defaults (top-k
                50, temperature 0.9, top-p 1, repetition penalty 1.05) drawn
                on the device by sample_topk inside the step graph.
  token_choice_us  microseconds per call of greedy_argmax and sample_topk on
                one row of the vocabulary.
  prefill       the 512-row prefill alone (MFMA, layer by layer), best of three.
  mrope         eager steps through decoder_step_mrope (distinct t/h/w rotary
                positions) against eager decoder_step on the same schedule.
  quantized     the same K greedy steps with the seven per-layer matrices
                block-quantized by the library (int8 and 4-bit codes with one
                fp16 scale per 32 weights): tokens/s, step bytes and the gate/up
                kernel's GB/s.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/sec at batch 1 and 64; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "autoregressive_transformer_decode_amd", "csrc", "kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gateup_gemv_talker1.7b_traffic.json")
ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_split_batched64_traffic.json")
GEMM_COUNTER_FILE = os.path.join(ROOT, "profiles", "gemm_mfma_counters.json")
QUANT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gateup_gemv_{}_talker1.7b_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """Hash of the source of the roofline kernel (the GEMV template and its
    launch shape), so that stored counters stay valid while other kernels in
    the file change."""
    return _source_hash(("template <typename WT, int MR, int KS, int KI, int EPI, bool NORM, int RW>",
                         "static void gemv_shape(", "static int gemv_rw(",
                         "static void gemv_dispatch_shape(", "hipError_t launch_gemv("))


# bytes per weight of the block-quantized formats: the code and 2 bytes of
# fp16 scale per 32 weights
QUANT_BPW = {"q8": 1.0 + 2.0 / 32, "q4": 0.5 + 2.0 / 32}


def weight_elems_layers(shape) -> int:
    """Weights of the per-layer matrices (no LM head, no input projection)."""
    h, q, kv, f = shape.hidden, shape.q_dim, shape.kv_dim, shape.ffn
    return (h * q + 2 * h * kv + q * h + 3 * h * f) * shape.n_layers


def weight_bytes(shape, quant=None) -> int:
    """Bytes of every matrix a step reads once: the layers' seven matrices
    (block-quantized with ``quant``) and one LM head (in the stack dtype)."""
    wb = 2 if shape.dtype == "bf16" else 4
    if quant is None:
        return shape.weight_elems(with_head=True) * wb
    head = shape.vocab * shape.hidden
    body = shape.weight_elems(with_head=True) - head
    return int(body * QUANT_BPW[quant] + head * wb)


def kv_row_bytes(shape) -> int:
    return 2 * shape.n_layers * shape.kv_dim * (2 if shape.kv_dtype == "bf16" else 4)


def gateup_bytes(shape, quant=None) -> int:
    """Algorithmic bytes of one gate/up launch: both [F, h] matrices once
    (codes and scales when quantized), the input row in and the [F]
    activation out (float32)."""
    wb = (2 if shape.dtype == "bf16" else 4) if quant is None else QUANT_BPW[quant]
    return int(2 * shape.ffn * shape.hidden * wb) + 4 * shape.hidden + 4 * shape.ffn


def oracle_model(mw, dtype):
    from oracle import decoder as od
    s = mw.shape
    hp = dict(n_layers=s.n_layers, hidden=s.hidden, n_q_heads=s.n_q_heads,
              n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, ffn=s.ffn,
              rope_theta=s.rope_theta, rms_eps=s.rms_eps, qk_norm=s.qk_norm,
              kv_bf16=(s.kv_dtype == "bf16"))
    layers = [dict(attn_norm=L.attn_norm, wq=L.wq.values, wk=L.wk.values, wv=L.wv.values,
                   bq=L.bq, bk=L.bk, bv=L.bv, q_norm=L.q_norm, k_norm=L.k_norm,
                   wo=L.wo.values, mlp_norm=L.mlp_norm, w_gate=L.w_gate.values,
                   w_up=L.w_up.values, w_down=L.w_down.values) for L in mw.layers]
    return od.make_model(hp, layers, mw.final_norm, [h.values for h in mw.heads],
                         [t.values for t in mw.tables], dtype=dtype)


def cpu_baseline(mw, X0, s_init, budget_s, max_steps):
    """The oracle (float32, as it stands) on the host: prefill, then greedy
    steps until the time budget is spent; tokens/s over the timed steps."""
    import numpy as np
    from oracle import decoder as od
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    om = oracle_model(mw, np.float32)
    cache = od.Cache(om, max(s_init, X0.shape[0] + max_steps + 1))
    _, z = od.prefill(om, cache, X0, 0)
    tok = int(np.argmax(z))
    n, t0 = 0, time.perf_counter()
    while n < max_steps:
        _, z = od.step(om, cache, om.tables[0][tok], 0)
        tok = int(np.argmax(z))
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=n / dt, unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"{n} greedy decode steps after the {X0.shape[0]}-row prefill "
                       f"(context {X0.shape[0] + 1}..{X0.shape[0] + n}), float32 numpy, "
                       f"prefill untimed")


def cpu_baseline_batched(mw, wl, budget_s):
    """The oracle (float32, as it stands) on the batched workload: streams in a
    seeded order, each with its synthetic cache (the seeded bf16 window of
    every layer, upcast to float32 outside the timing) stepped twice, as two
    iterations (the first from its input row, the second from its greedy
    token), until the time budget is spent.  Streams are independent, so
    tokens/s over the sampled stream-steps is the rate of whole iterations."""
    import numpy as np
    from autoregressive_transformer_decode_amd import inputs
    from oracle import decoder as od
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    s = wl.model
    om = oracle_model(mw, np.float32)
    lens = inputs.batched_lengths(wl, seed=0)
    X1 = inputs.batched_first_inputs(wl, seed=0)
    pools = [inputs.batched_kv_pool(s, l, seed=0) for l in range(s.n_layers)]
    order = np.random.default_rng(1).permutation(wl.batch)
    spent, n_tok, used = 0.0, 0, []
    for b in order:
        b, n = int(b), int(lens[b])
        cache = od.Cache(om, n + 2)
        for l in range(s.n_layers):
            k, v = inputs.batched_kv(s, b, n, l, pool=pools[l])
            cache.K[l][:, :n] = inputs.bf16_bits_to_f32(k)
            cache.V[l][:, :n] = inputs.bf16_bits_to_f32(v)
        cache.pos = n
        t0 = time.perf_counter()
        _, z = od.step(om, cache, X1[b].astype(np.float32), 0)
        _, z = od.step(om, cache, om.tables[0][int(np.argmax(z))], 0)
        spent += time.perf_counter() - t0
        n_tok += 2
        used.append(b)
        del cache
        if spent > budget_s and len(used) >= 2:
            break
    return dict(value=n_tok / spent, unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"{len(used)} of {wl.batch} streams (cache lengths "
                       f"{int(lens[used].min())}..{int(lens[used].max())}), two steps each as "
                       f"two iterations, float32 numpy; caches upcast from the seeded bf16 "
                       f"pool outside the timing; {spent:.1f} s timed")


def _source_hash(starts) -> str:
    with open(KERNEL_SRC) as f:
        src = f.read()
    parts = []
    for start in starts:
        i = src.find(start)
        if i < 0:
            return "missing"
        parts.append(src[i:src.find("\n}\n", i) + 3])
    return hashlib.sha256("".join(parts).encode()).hexdigest()[:16]


def attn_kernel_hash() -> str:
    """Hash of the split-K attention kernels' sources (split, state merge) and
    their launch shape."""
    return _source_hash(("template <int D, int R, bool COH>",
                         "template <typename KT, int D, int R, int LPK, int U, bool DEFER>",
                         "template <int D, int R>\n__global__ __launch_bounds__(256) void k_attn_merge(",
                         "static void attn_dispatch_r(", "hipError_t launch_attention("))


def gemm_kernel_hash() -> str:
    """Hash of the matrix-core GEMM kernels' sources (64-row decode GEMM,
    128 x 128 prefill tiles)."""
    return _source_hash(("template <int NKS, int EPI, int CB>\n__global__ __launch_bounds__(512) void k_gemm_dec(",
                         "template <int NST>\n__global__ __launch_bounds__(256) void k_gemm_tile("))


def gemm_counters(role, rows):
    """Matrix-core counters of one GEMM from the committed summary (busy share
    of the launch, fetched bytes over weight bytes), or None when the GEMM
    kernels changed since the counters were taken."""
    try:
        with open(GEMM_COUNTER_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != gemm_kernel_hash():
        return None
    for r in t.get("kernels", []):
        if r["role"] == role and r["rows"] == rows:
            return dict(kernel=r["kernel"], mfma_busy_frac=r["mfma_busy_over_duration"],
                        fetch_over_weights=r["fetch_mib"] / r["weight_mib"],
                        lds_bank_conflicts=r["lds_bank_conflicts"])
    return None


def traffic_per_launch(algo, path=None, hashfn=None):
    """HBM bytes per launch from a committed counter summary, or None when the
    kernel's source changed since the counters were taken or the summary is of
    another shape (its algorithmic bytes per launch differ from ``algo``)."""
    try:
        with open(path or TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != (hashfn or kernel_hash)():
        return None
    if t.get("algorithmic_bytes_per_launch") != algo:
        return None
    return t.get("bytes_per_launch")


def read_stream_gbs(nbytes=4 << 30, reps=5):
    """Attainable read bandwidth: the library's streaming read kernel over a
    4 GiB buffer (well past the 256 MB memory-side cache), mean of `reps`
    full reads after a warm-up read."""
    import torch
    from autoregressive_transformer_decode_amd import binding as B
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    us = B.atd_read_stream(buf.data_ptr(), nbytes, reps, sink.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    del buf
    torch.cuda.empty_cache()
    return dict(gbs=nbytes / (us / 1e6) / 1e9, bytes=nbytes, us_per_read=us, reads=reps,
                kernel="k_read_stream (grid-stride 16-byte loads, 4096 workgroups)")


def bench_lm(args, wl):
    import numpy as np
    import torch
    from autoregressive_transformer_decode_amd import binding as B
    from autoregressive_transformer_decode_amd import device as dv
    from autoregressive_transformer_decode_amd import inputs

    s = wl.model
    t = time.perf_counter()
    mw = inputs.make_weights(s, seed=0)
    X0 = inputs.prefill_embeddings(wl, seed=0)
    log(f"weights generated in {time.perf_counter() - t:.1f}s")
    dm = dv.DeviceModel(mw)
    dec = dv.Decoder(dm, max_slots=1, max_rows=wl.prefill, max_ctx=wl.s_max,
                     l2_prefetch=not args.no_l2_prefetch)
    if args.roofline_only:
        # the roofline kernel alone, as measured for the bench line: its
        # launches for every layer's weights in turn between two HIP events
        reps = 16
        dec.grow(0, wl.s_init)   # time_stage steps an attached slot
        dec.time_stage(B.ATD_STAGE_GATEUP, 0, 1, 4)
        avg_s = dec.time_stage(B.ATD_STAGE_GATEUP, 0, 1, reps) / 1e6
        per_launch = gateup_bytes(s)
        dec.close()
        return dict(roofline_only=True, workload=wl.name, launches_timed=reps * s.n_layers,
                    kernel="k_gemv (RMSNorm + gate/up + SwiGLU), bf16 weights",
                    avg_launch_us=avg_s * 1e6, bytes_per_launch=per_launch,
                    achieved_gbs=per_launch / avg_s / 1e9,
                    frac=per_launch / avg_s / 1e9 / HBM_PEAK_GBS)
    P0 = wl.prefill
    K = args.steps if args.steps is not None else wl.steps
    W = args.warmup
    if P0 + max(K, W) > wl.s_max:
        raise SystemExit(f"--steps/--warmup beyond the {wl.s_max}-row context of {wl.name}")
    # fewer timed steps than the workload's: fast-forward (untimed) so that the
    # timed steps sit around the workload's mean context ((P0 + 1 + s_max) / 2)
    skip = max(0, int(round((P0 + 1 + wl.s_max) / 2.0 - P0 - (K + 1) / 2.0)))
    skip = 0 if args.no_fast_forward else min(skip, wl.s_max - P0 - max(K, W))
    # bucket ladder: the cache doubles before a write at its capacity (ASR report's
    # dynamic window); the buckets are allocated up front, outside the timing
    caps = [wl.s_init]
    while caps[-1] < P0 + skip + max(K, W):
        caps.append(min(2 * caps[-1], wl.s_max))
    buckets = [dec.alloc_kv(c) for c in caps]
    dec.grow(0, caps[0], kv=buckets[0])
    cur = dict(dec=dec, buckets=buckets)
    X0_d = torch.from_numpy(X0).cuda()
    z = torch.empty(s.vocab, device="cuda")
    y = torch.empty(s.hidden, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")

    seen = torch.zeros(dv.seen_words(s.vocab), dtype=torch.int32, device="cuda")
    uni = torch.from_numpy(inputs.uniforms(0, 0, skip + max(K, W) + 1)).cuda()

    def schedule(n, sampled=False):
        """Rewind to the first bucket, prefill (untimed), `skip` untimed steps,
        then n timed steps from the step graph (greedy, or the sampling
        defaults with the penalty), growing the bucket where the context
        reaches it; returns the seconds of the timed steps."""
        dec, buckets = cur["dec"], cur["buckets"]
        dec.set_position(0, 0)
        if dec.position(0)[1] != caps[0]:
            dec.grow(0, caps[0], kv=buckets[0])
        dec.prefill(X0_d, logits_out=z)
        seen.zero_()
        if sampled:
            dv.sample_topk(z, seen, SAMPLING_PENALTY, dv.Sampling(*SAMPLING, uni[0:1]), tok)
        else:
            dv.greedy_argmax(z, None, 1.0, tok)
        state = dict(done=0, b=0)

        def run(n_steps):
            end = state["done"] + n_steps
            while state["done"] < end:
                done = state["done"]
                pos, cap = dec.position(0)
                if pos >= cap:
                    state["b"] += 1
                    dec.grow(0, caps[state["b"]], kv=buckets[state["b"]])
                    continue
                k = min(end - done, cap - pos)
                if sampled:
                    dec.generate(k, tok, y_out=y, logits_out=z, seen=seen,
                                 penalty=SAMPLING_PENALTY,
                                 sampling=dv.Sampling(*SAMPLING, uni[1 + done:1 + done + k]))
                else:
                    dec.generate(k, tok, y_out=y, logits_out=z)
                state["done"] = done + k

        run(skip)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(n)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # warmup (captures the step graph of every bucket the timed run visits)
    W = K if len(caps) > 1 else W
    if W:
        schedule(W)
    # the prefill alone (MFMA GEMMs over all its rows, layer by layer): the
    # faster of three runs
    pf = float("inf")
    for _ in range(3):
        dec.set_position(0, 0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dec.prefill(X0_d, logits_out=z)
        torch.cuda.synchronize()
        pf = min(pf, time.perf_counter() - t0)
    # 2 flops per weight and row for the layers (the LM head runs on the last row),
    # plus the causal attention products (q.k and p.v over the rows before each row)
    pf_flops = 2.0 * P0 * weight_elems_layers(s) + 2.0 * s.hidden * s.vocab + \
        2.0 * 2 * s.n_layers * s.n_q_heads * s.head_dim * (P0 * (P0 + 1) / 2)
    dt = schedule(K)
    log(f"timed {K} steps (context {P0 + skip + 1}..{P0 + skip + K}): {dt * 1e3:.1f} ms "
        f"(buckets {caps})")
    # the same run with the sampling defaults (graphs captured by a warmup)
    dt_s = None
    if not args.no_sampled:
        schedule(K if len(caps) > 1 else min(W, K), sampled=True)
        dt_s = schedule(K, sampled=True)
        log(f"timed {K} sampled steps: {dt_s * 1e3:.1f} ms")

    # interleaved mRoPE: eager steps through decoder_step_mrope with distinct
    # rotary positions against eager decoder_step, same schedule, alternating
    mrope = None
    if s.mrope_sections is not None and not args.no_sampled:
        n_m = min(256, K)
        rp = torch.tensor([[P0 + k, 7 + k % 5, 11 + k % 3] for k in range(n_m)],
                          dtype=torch.int32, device="cuda")
        tk2 = tok.view(1, 1)
        z2, y2 = z.view(1, -1), y.view(1, -1)

        def eager(use):
            dec.set_position(0, 0)
            if dec.position(0)[1] != caps[0]:
                dec.grow(0, caps[0], kv=buckets[0])
            dec.prefill(X0_d, logits_out=z)
            dv.greedy_argmax(z, None, 1.0, tok)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for k in range(n_m):
                dec.step(tk2, [0], y_out=y2, logits_out=z2, rope_pos=rp[k:k + 1] if use else None)
                dv.greedy_argmax(z, None, 1.0, tok)
            torch.cuda.synchronize()
            return time.perf_counter() - t0

        eager(True)
        tm = dict(plain=float("inf"), mrope=float("inf"))
        for _ in range(2):
            tm["plain"] = min(tm["plain"], eager(False))
            tm["mrope"] = min(tm["mrope"], eager(True))
        mrope = dict(sections=list(s.mrope_sections), steps=n_m,
                     value=n_m / tm["mrope"], unit="tokens/s",
                     plain_eager_tokens_per_s=n_m / tm["plain"],
                     overhead=tm["mrope"] / tm["plain"] - 1.0,
                     step="eager decoder_step_mrope + greedy_argmax per token, rotary positions "
                          "(t, h, w) distinct; against eager decoder_step on the same schedule "
                          "(each leg the faster of two alternating runs)")
        log(f"mrope eager: {mrope['value']:.1f} tokens/s vs plain {mrope['plain_eager_tokens_per_s']:.1f}")

    # roofline: the dominant kernel's launches, every layer's weights in turn
    # as in a step, timed with HIP events on this stream
    reps = 16
    avg_s = dec.time_stage(B.ATD_STAGE_GATEUP, 0, 1, reps) / 1e6
    launches = reps * s.n_layers
    per_launch = gateup_bytes(s)
    achieved = per_launch / avg_s / 1e9
    traffic = traffic_per_launch(per_launch)

    attainable = read_stream_gbs()
    mean_ctx = P0 + skip + (K + 1) / 2.0
    step_bytes = weight_bytes(s) + kv_row_bytes(s) * mean_ctx
    ms_step = dt * 1e3 / K
    out = dict(
        metric=METRIC, value=K / dt, unit="tokens/s", n_gpus=1, steps=K, warmup=W,
        ms_per_step=ms_step, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16" if s.dtype == "bf16" else "f32", data="synthetic",
        config=dict(workload=wl.name, batch=1, prefill=P0,
                    context=[P0 + skip + 1, P0 + skip + K],
                    layers=s.n_layers, hidden=s.hidden, heads=[s.n_q_heads, s.n_kv_heads],
                    head_dim=s.head_dim, ffn=s.ffn, vocab=s.vocab,
                    step="graph-replayed decode step + greedy argmax on device",
                    kv_buckets=caps, l2_prefetch=not args.no_l2_prefetch),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=traffic,
                      kernel="k_gemv (RMSNorm + gate/up + SwiGLU), bf16 weights",
                      bytes_per_launch=per_launch, avg_launch_us=avg_s * 1e6,
                      launches_timed=launches),
        step_hbm=dict(algorithmic_bytes=step_bytes, achieved_gbs=step_bytes / (ms_step / 1e3) / 1e9,
                      frac=step_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
                      frac_of_attainable=step_bytes / (ms_step / 1e3) / 1e9 / attainable["gbs"]),
        hbm_attainable=attainable,
        sampled=None if dt_s is None else dict(
            value=K / dt_s, unit="tokens/s", ms_per_step=dt_s * 1e3 / K,
            settings=dict(zip(("top_k", "temperature", "top_p"), SAMPLING),
                          penalty=SAMPLING_PENALTY)),
        token_choice_us=None if args.no_sampled else time_choice(s.vocab),
        mrope=mrope,
        prefill=dict(rows=P0, ms=pf * 1e3, tokens_per_s=P0 / pf, tflops=pf_flops / pf / 1e12,
                     mfma_peak_tflops=2500.0, gate_up_counters=gemm_counters("gate/up", P0),
                     note="bf16 MFMA with float32 activations as bf16 hi + lo operands (two "
                          "products per weight); rows layer by layer in chunks of up to 512, "
                          "GEMMs over 128 x 128 output tiles (64-row tiles where those leave "
                          "compute units idle), causal flash attention on the float32 "
                          "matrix cores"),
    )
    dec.close()
    # the same greedy run with the seven per-layer matrices block-quantized
    # (int8 / 4-bit codes, fp16 scale per 32 weights, dequantized in the GEMV)
    if s.dtype == "bf16" and not args.no_quantized:
        out["quantized"] = {}
        for fmt in ("q8", "q4"):
            qdm = dv.DeviceModel(mw, quant=fmt)
            qdec = dv.Decoder(qdm, max_slots=1, max_rows=wl.prefill, max_ctx=wl.s_max,
                              l2_prefetch=not args.no_l2_prefetch)
            qbuckets = [qdec.alloc_kv(c) for c in caps]
            qdec.grow(0, caps[0], kv=qbuckets[0])
            cur.update(dec=qdec, buckets=qbuckets)
            schedule(W)
            dt_q = schedule(K)
            qg = qdec.time_stage(B.ATD_STAGE_GATEUP, 0, 1, reps) / 1e6
            qb = weight_bytes(s, fmt) + kv_row_bytes(s) * mean_ctx
            log(f"timed {K} steps, {fmt} weights: {dt_q * 1e3:.1f} ms")
            out["quantized"][fmt] = dict(
                value=K / dt_q, unit="tokens/s", ms_per_step=dt_q * 1e3 / K,
                weight_bytes_per_step=weight_bytes(s, fmt),
                step_hbm=dict(algorithmic_bytes=qb, achieved_gbs=qb / (dt_q / K) / 1e9,
                              frac=qb / (dt_q / K) / 1e9 / HBM_PEAK_GBS),
                gate_up=dict(avg_launch_us=qg * 1e6, bytes_per_launch=gateup_bytes(s, fmt),
                             achieved_gbs=gateup_bytes(s, fmt) / qg / 1e9,
                             traffic=traffic_per_launch(gateup_bytes(s, fmt),
                                                        QUANT_TRAFFIC_FILE.format(fmt))))
            qdec.close()
            del qdec, qbuckets, qdm
            torch.cuda.empty_cache()
    # the batched workload is the same stack (same weights) with a bf16 cache
    bwl = inputs.WORKLOADS["batched64"]
    import dataclasses
    same_stack = dataclasses.replace(bwl.model, name=s.name, kv_dtype=s.kv_dtype) == s
    if not args.no_batched and same_stack:
        log("batched64 ...")
        out["batch64"] = bench_batched(args, bwl, dm=dm, mw=mw, steps=bwl.steps, warmup=4)
    del dm
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(mw, X0, wl.s_init, args.cpu_seconds, 64)
    else:
        out["cpu_baseline"] = None
    return out


def attn_stage_bytes(shape, lens) -> int:
    """Algorithmic bytes of one layer's attention stage over a batch of decode
    rows at cache lengths `lens`: every valid K and V row once, the new row
    written, the step's q/k/v row in and the attention output out (float32)."""
    kvb = 2 if shape.kv_dtype == "bf16" else 4
    per_row = 2 * shape.kv_dim * kvb
    B = len(lens)
    qkv = shape.q_dim + 2 * shape.kv_dim
    return int(sum(int(l) for l in lens)) * per_row + B * per_row + B * (qkv + shape.q_dim) * 4


def bench_batched(args, wl, dm=None, mw=None, steps=None, warmup=None):
    """The batched workload: 64 streams, one decode step each per iteration,
    seeded cache lengths, tokens fed back by the on-device greedy argmax."""
    import numpy as np
    import torch
    from autoregressive_transformer_decode_amd import binding as B
    from autoregressive_transformer_decode_amd import device as dv
    from autoregressive_transformer_decode_amd import inputs

    s = wl.model
    Bn = wl.batch
    K = steps if steps is not None else wl.steps
    W = warmup if warmup is not None else 4
    if mw is None:
        mw = inputs.make_weights(s, seed=0)
    if dm is None:
        dm = dv.DeviceModel(mw)
    lens = inputs.batched_lengths(wl, seed=0)
    X1 = torch.from_numpy(inputs.batched_first_inputs(wl, seed=0)).cuda()
    dec = dv.Decoder(dm, max_slots=Bn, max_rows=Bn, max_ctx=wl.s_max, kv_dtype=s.kv_dtype)
    for b in range(Bn):
        dec.grow(b, int(lens[b]) + max(K, W) + 1)
    t = time.perf_counter()
    dv.fill_batched_caches(dec, lens, seed=0)
    torch.cuda.synchronize()
    log(f"batched: {Bn} caches filled in {time.perf_counter() - t:.1f}s "
        f"(lengths {int(lens.min())}..{int(lens.max())}, mean {float(lens.mean()):.0f})")
    y = torch.empty(Bn, s.hidden, device="cuda")
    z = torch.empty(Bn, s.vocab, device="cuda")
    tok = torch.zeros(Bn, 1, dtype=torch.int32, device="cuda")

    def iterations(n):
        for it in range(n):
            if it == 0:
                dec.step(None, [], nrows=Bn, extra=X1, y_out=y, logits_out=z)
            else:
                dec.step(tok, [0], nrows=Bn, y_out=y, logits_out=z)
            dv.greedy_argmax(z, None, 1.0, tok.view(Bn))

    def rewind():
        for b in range(Bn):
            dec.set_position(b, int(lens[b]))

    iterations(W)
    rewind()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    iterations(K)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"batched: timed {K} iterations x {Bn} streams: {dt * 1e3:.1f} ms")
    rewind()
    torch.cuda.synchronize()
    reps = 4
    st = {name: dec.time_stage(code, 0, Bn, reps)
          for name, code in (("qkv", B.ATD_STAGE_QKV), ("attention", B.ATD_STAGE_ATTN),
                             ("o_proj", B.ATD_STAGE_OPROJ), ("gate_up", B.ATD_STAGE_GATEUP),
                             ("down", B.ATD_STAGE_DOWN))}
    dec.close()
    a_bytes = attn_stage_bytes(s, lens)
    a_gbs = a_bytes / (st["attention"] / 1e6) / 1e9
    gu_flops = 2.0 * Bn * 2 * s.ffn * s.hidden
    gu_w = 2 * s.ffn * s.hidden * (2 if s.dtype == "bf16" else 4)
    mean_ctx = float(lens.mean()) + (K + 1) / 2.0
    step_bytes = weight_bytes(s) + kv_row_bytes(s) * mean_ctx * Bn
    ms_it = dt * 1e3 / K
    cpu = None
    if not args.no_cpu_baseline:
        log("batched cpu baseline (oracle) ...")
        cpu = cpu_baseline_batched(mw, wl, args.cpu_seconds)
    return dict(
        cpu_baseline=cpu,
        value=Bn * K / dt, unit="tokens/s", streams=Bn, iterations=K, warmup=W,
        ms_per_iteration=ms_it,
        config=dict(workload=wl.name, batch=Bn, kv_lengths=[int(lens.min()), int(lens.max())],
                    kv_length_mean=float(lens.mean()), kv_dtype=s.kv_dtype,
                    layers=s.n_layers, hidden=s.hidden, ffn=s.ffn, vocab=s.vocab),
        roofline=dict(bound="hbm", achieved=a_gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=a_gbs / HBM_PEAK_GBS,
                      traffic=traffic_per_launch(a_bytes, ATTN_TRAFFIC_FILE, attn_kernel_hash),
                      traffic_kernel="k_attn_split + k_attn_merge (counters of the stage's two launches)",
                      kernel="attention stage (k_attn_split, then k_attn_merge for the blocks' states), 64 rows",
                      bytes_per_launch=a_bytes, avg_launch_us=st["attention"],
                      launches_timed=reps * s.n_layers),
        gemm_gate_up=dict(us=st["gate_up"], tflops=gu_flops / (st["gate_up"] / 1e6) / 1e12,
                          mfma_peak_tflops=2500.0,
                          weight_gbs=gu_w / (st["gate_up"] / 1e6) / 1e9,
                          counters=gemm_counters("gate/up", Bn)),
        stage_us_per_layer=st,
        step_hbm=dict(algorithmic_bytes=step_bytes,
                      achieved_gbs=step_bytes / (ms_it / 1e3) / 1e9,
                      frac=step_bytes / (ms_it / 1e3) / 1e9 / HBM_PEAK_GBS),
    )


# the Qwen TTS generation defaults: top-k 50, temperature 0.9, top-p 1.0,
# repetition penalty 1.05
SAMPLING = (50, 0.9, 1.0)
SAMPLING_PENALTY = 1.05


def time_choice(V, reps=100):
    """Microseconds per call of the token-choice kernels on one row of V
    logits: `reps` calls captured in one graph, replayed between two events
    (the launch cost inside a replayed step, not the host's): greedy_argmax,
    and sample_topk with the sampling defaults."""
    import torch
    from autoregressive_transformer_decode_amd import device as dv
    from autoregressive_transformer_decode_amd import inputs
    z = torch.from_numpy(inputs.normal(0, 9, 0, (V,), scale=3.0)).cuda()
    seen = torch.zeros(dv.seen_words(V), dtype=torch.int32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    uni = torch.from_numpy(inputs.uniforms(0, 9, reps)).cuda()
    out = {}
    for name in ("greedy_argmax", "sample_topk"):
        def call(i):
            if name == "greedy_argmax":
                dv.greedy_argmax(z, seen, SAMPLING_PENALTY, tok)
            else:
                dv.sample_topk(z, seen, SAMPLING_PENALTY, dv.Sampling(*SAMPLING, uni[i:i + 1]), tok)
        call(0)   # first call sets up the library's scratch outside the capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(reps):
                call(i)
        graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1e3 / reps
        del graph
    out["vocab"] = V
    return out


def bench_frames(args, wl):
    """The Talker frame loop (0.6B shape): 64-row prefill, then frames of one
    Talker step and one Code Predictor pass (2-row prefill + 14 steps),
    replayed from graphs on the device (talker_generate_frames)."""
    import numpy as np
    import torch
    from autoregressive_transformer_decode_amd import device as dv
    from autoregressive_transformer_decode_amd import inputs

    s, c = wl.model, wl.cp
    n = args.steps if args.steps is not None else wl.frames
    tmw = inputs.make_weights(s, seed=0)
    cmw = inputs.make_weights(c, seed=0, tables=tmw.tables)
    tdm = dv.DeviceModel(tmw)
    cdm = dv.DeviceModel(cmw, tables=tdm.tables)
    tdec = dv.Decoder(tdm, max_slots=1, max_rows=wl.prefill, max_ctx=wl.s_init,
                      l2_prefetch=not args.no_l2_prefetch)
    cdec = dv.Decoder(cdm, max_slots=1, max_rows=2, max_ctx=inputs.CP_CAPACITY,
                      l2_prefetch=not args.no_l2_prefetch)
    tdec.grow(0, wl.s_init)
    cdec.grow(0, inputs.CP_CAPACITY)
    if wl.prefill + n - 1 > wl.s_init:
        raise SystemExit(f"--steps beyond the {wl.s_init}-row Talker cache")
    X0 = torch.from_numpy(inputs.prefill_embeddings(wl, seed=0)).cuda()
    text = torch.from_numpy(inputs.text_embeddings(wl, seed=0)).cuda()
    if text.shape[0] < n:
        text = torch.cat([text, text[1:2].expand(n - text.shape[0], -1)])
    y = torch.empty(s.hidden, device="cuda")
    zt = torch.empty(s.vocab, device="cuda")
    codes = torch.zeros(16, dtype=torch.int32, device="cuda")
    seen = torch.zeros(dv.seen_words(s.vocab), dtype=torch.int32, device="cuda")
    out = torch.zeros(n, 16, dtype=torch.int32, device="cuda")

    ut = torch.from_numpy(inputs.uniforms(0, 1, n)).cuda()
    uc = torch.from_numpy(inputs.uniforms(0, 2, (n, 15))).cuda()

    def run(frames, sampled):
        """Prefill and the first code (untimed), then `frames` frames; returns
        the seconds of the frame loop."""
        seen.zero_()
        tdec.prefill(X0, y_out=y, logits_out=zt)
        ts = cs = None
        if sampled:
            ts, cs = dv.Sampling(*SAMPLING, ut), dv.Sampling(*SAMPLING, uc)
            dv.sample_topk(zt, seen, wl.penalty, dv.Sampling(*SAMPLING, ut[0:1]), codes[0:1])
        else:
            dv.greedy_argmax(zt, seen, wl.penalty, codes[0:1])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dv.talker_frames(tdec, cdec, frames, codes, y, text, seen, wl.penalty, codes_out=out,
                         tk_sampling=ts, cp_sampling=cs)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    run(min(n, 4), False)   # warm-up runs of the loop (capture the frame graphs)
    run(min(n, 4), True)
    # the two legs alternate, twice; each reports its faster run
    dt, dt_s = float("inf"), float("inf")
    for _ in range(2):
        dt = min(dt, run(n, False))
        dt_s = min(dt_s, run(n, True))
    tdec.close()
    cdec.close()
    fps = n / dt
    kv_row = lambda sh: 2 * sh.n_layers * sh.kv_dim * (2 if sh.kv_dtype == "bf16" else 4)  # noqa: E731
    mean_ctx = wl.prefill + (n - 1) / 2.0
    talker_b = weight_bytes(s) + kv_row(s) * mean_ctx
    # a pass: 15 forward passes (2-row prefill, 14 steps), each over every layer
    # and one LM head (weight_bytes counts one head); cache rows 2..16
    cp_b = 15 * weight_bytes(c) + kv_row(c) * sum(range(2, 17))
    frame_b = ((n - 1) * talker_b + n * cp_b) / n
    log(f"frames: {n} in {dt * 1e3:.1f} ms")
    return dict(
        metric="Talker frames/s (1 Talker step + 15 Code Predictor passes per frame)",
        value=fps, unit="frames/s", n_gpus=1, steps=n, warmup=1, ms_per_step=dt * 1e3 / n,
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload=wl.name, frames=n, prefill=wl.prefill, penalty=wl.penalty,
                    talker_layers=s.n_layers, cp_layers=c.n_layers, hidden=s.hidden,
                    step="graph-replayed frames (talker_generate_frames)",
                    l2_prefetch=not args.no_l2_prefetch,
                    timing="greedy and sampled runs of all frames alternate twice; each "
                           "leg reports its faster run"),
        codes_per_s=16 * fps, rtf_equivalent=(1.0 / fps) / 0.08,
        frame_hbm=dict(algorithmic_bytes=frame_b, achieved_gbs=frame_b * fps / 1e9,
                       frac=frame_b * fps / 1e9 / HBM_PEAK_GBS),
        sampled=dict(value=n / dt_s, unit="frames/s", ms_per_frame=dt_s * 1e3 / n,
                     rtf_equivalent=(dt_s / n) / 0.08,
                     settings=dict(zip(("top_k", "temperature", "top_p"), SAMPLING),
                                   penalty=wl.penalty, code_predictor="same, no penalty")),
        token_choice_us=dict(talker=time_choice(s.vocab), code_predictor=time_choice(c.vocab)),
        roofline=None, cpu_baseline=None)


ALU_PEAK_TFLOPS = 157.3          # fp32 vector, published (packed FP32 counted)
ALU_UNPACKED_TFLOPS = 78.6       # 256 CUs x 64 FMA lanes x 2 flops x 2.4 GHz


def codec_stack(layers, run_conv, run_trans, h):
    """Enqueue the codec stack on `h`: run_conv(h, layer_index, out, accumulate)
    and run_trans(h, layer_index) return their outputs; a dilated convolution
    followed by a residual 1-tap convolution forms a unit whose result is added
    to the stage tensor."""
    u = None
    for i, L in enumerate(layers):
        if L[0] == "trans":
            h = run_trans(h, i)
        elif L[6]:
            h = run_conv(u, i, h, True)
        elif i + 1 < len(layers) and layers[i + 1][0] == "conv" and layers[i + 1][6]:
            u = run_conv(h, i, None, False)
        else:
            h = run_conv(h, i, None, False)
    return h


def bench_codec(args, wl):
    """The codec decoder's convolution stack (26 causal convolutions, 4
    transposed) on float32 [channels, frames] tensors: each rep runs the whole
    stack; per-layer HIP events on the stream give each kernel's time."""
    import dataclasses
    import numpy as np
    import torch
    from autoregressive_transformer_decode_amd import device as dv
    from autoregressive_transformer_decode_amd import inputs

    c = wl
    layers = inputs.codec_layers(c)
    ws = inputs.make_codec_weights(c, seed=0)
    dw = []
    for L, (w, b) in zip(layers, ws):
        wd, bd = torch.from_numpy(w).cuda(), torch.from_numpy(b).cuda()
        dw.append((dv.transconv1d_pack(wd, L[3]) if L[0] == "trans" else wd, bd))
    x = torch.from_numpy(inputs.codec_input(c, seed=0)).cuda()
    # one output buffer per layer, allocated before the timed region
    bufs = []
    for L in layers:
        if L[0] == "trans":
            bufs.append(torch.empty(L[2], L[4] * L[3], device="cuda"))
        else:
            bufs.append(None if L[6] else torch.empty(L[2], L[5], device="cuda"))
    events = None

    def mark(i):
        if events is not None:
            events[i].record()

    def run_conv(h, i, out, acc):
        mark(2 * i)
        w, b = dw[i]
        y = dv.conv1d_causal(h, w, b, layers[i][4], y=out if acc else bufs[i], accumulate=acc)
        mark(2 * i + 1)
        return y

    def run_trans(h, i):
        mark(2 * i)
        y = dv.transconv1d(h, dw[i][0], dw[i][1], layers[i][3], y=bufs[i])
        mark(2 * i + 1)
        return y

    reps = args.steps if args.steps is not None else 10
    warm = max(1, min(args.warmup, 3))
    for _ in range(warm):
        out = codec_stack(layers, run_conv, run_trans, x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        out = codec_stack(layers, run_conv, run_trans, x)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    # per-layer times from events around each launch (separate reps)
    events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(layers))]
    per = np.zeros(len(layers))
    for _ in range(reps):
        codec_stack(layers, run_conv, run_trans, x)
        torch.cuda.synchronize()
        per += [events[2 * i].elapsed_time(events[2 * i + 1]) for i in range(len(layers))]
    per = per / reps * 1e-3
    events = None
    flops = []
    for L in layers:
        if L[0] == "conv":
            flops.append(2.0 * L[1] * L[2] * L[3] * L[5])
        else:
            flops.append(2.0 * L[1] * L[2] * 2 * L[4] * L[3])
    flops = np.array(flops)
    conv = np.array([L[0] == "conv" for L in layers])
    total = float(flops.sum())
    samples = out.shape[1]
    conv_t, conv_f = float(per[conv].sum()), float(flops[conv].sum())
    tr_t, tr_f = float(per[~conv].sum()), float(flops[~conv].sum())
    # the roofline kernel is k_conv1d, which runs both kinds of layer
    achieved = total / float(per.sum()) / 1e12
    log(f"codec stack: {dt * 1e3:.2f} ms ({total / dt / 1e12:.1f} TFLOP/s); causal conv "
        f"{conv_t * 1e3:.2f} ms at {conv_f / conv_t / 1e12:.1f} TFLOP/s, transposed {tr_t * 1e3:.2f} ms at "
        f"{tr_f / tr_t / 1e12:.1f} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = codec_cpu_baseline(c, args.cpu_seconds)
    return dict(
        metric="codec decoder convolution stack: output samples/s", value=samples / dt,
        unit="samples/s", n_gpus=1, steps=reps, warmup=warm, ms_per_step=dt * 1e3,
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload="codec", frames=c.frames, channels=list(c.channels),
                    strides=list(c.strides), kernel=c.kernel, dilations=list(c.dilations),
                    causal_convs=int(conv.sum()), transposed_convs=int((~conv).sum()),
                    output_samples=int(samples),
                    step="the whole stack, one launch per layer (codec_conv1d_causal, "
                         "codec_transconv1d), weights prepacked before timing"),
        tflops=total / dt / 1e12, gflop_per_step=total / 1e9,
        audio_s_per_s=samples / 24000.0 / dt,
        per_layer_ms=[round(t * 1e3, 4) for t in per],
        transconv=dict(ms=tr_t * 1e3, tflops=tr_f / tr_t / 1e12),
        causal_conv=dict(ms=conv_t * 1e3, tflops=conv_f / conv_t / 1e12),
        roofline=dict(bound="alu", achieved=achieved, peak=ALU_PEAK_TFLOPS, unit="TFLOP/s",
                      frac=achieved / ALU_PEAK_TFLOPS, traffic=None,
                      kernel="k_conv1d (causal and phase-split transposed convolutions), "
                             "all 30 launches of a stack",
                      flops_per_launch=total / len(layers),
                      avg_launch_us=float(per.sum()) / len(layers) * 1e6,
                      unpacked_fp32_peak=ALU_UNPACKED_TFLOPS),
        cpu_baseline=cpu)


def codec_cpu_baseline(c, budget_s):
    """The oracle's stack (float64 numpy) on the first input frames of the same
    workload: every layer, at reduced length (the cost per output sample of a
    convolution stack does not depend on the length)."""
    import dataclasses
    import numpy as np
    from autoregressive_transformer_decode_amd import inputs
    from oracle import codec as oc

    frames = max(1, min(c.frames, int(round(c.frames * budget_s / 75.0))))
    cs = dataclasses.replace(c, frames=frames)
    layers = inputs.codec_layers(cs)
    ws = inputs.make_codec_weights(cs, seed=0)
    h = inputs.codec_input(c, seed=0)[:, :frames].astype(np.float64)

    def run_conv(h, i, out, acc):
        w, b = ws[i]
        y = oc.conv1d_causal(h, w, b, layers[i][4])
        return out + y if acc else y

    def run_trans(h, i):
        return oc.transconv1d(h, ws[i][0], ws[i][1], layers[i][3])

    t0, c0 = time.perf_counter(), time.process_time()
    out = codec_stack(layers, run_conv, run_trans, h)
    dt, cpu_s = time.perf_counter() - t0, time.process_time() - c0
    # threads actually used: process CPU time over wall time
    return dict(value=out.shape[1] / dt, unit="samples/s", cores=max(1, round(cpu_s / dt)),
                kind="oracle",
                sample=f"the whole stack on the first {frames} of {c.frames} input frames "
                       f"({out.shape[1]} output samples) in {dt:.1f} s, float64 numpy")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="talker1.7b",
                    choices=["talker1.7b", "asr", "tiny", "batched64", "talker0.6b",
                             "talker1.7b-frames", "codec"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batched", action="store_true",
                    help="skip the 64-stream leg of the default (1.7B) run")
    ap.add_argument("--no-sampled", action="store_true",
                    help="skip the sampled leg and the token-choice timing (counter runs)")
    ap.add_argument("--no-fast-forward", action="store_true",
                    help="time the steps right after the prefill instead of centring them on "
                         "the workload's mean context (short counter runs)")
    ap.add_argument("--no-quantized", action="store_true",
                    help="skip the int8 / 4-bit weight legs (short counter runs)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the stand-alone timing of the roofline kernel (for its kernel trace)")
    ap.add_argument("--no-l2-prefetch", action="store_true",
                    help="decoders without the step attention's L2 weight prefetch "
                         "(ATD_FLAG_NO_L2_PREFETCH; counter runs of the stand-alone gate/up GEMV)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 8 plain device copies of 256 MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if args.copy_calibration:
        # a copy kernel of known size: each launch reads and writes 256 MiB
        src = torch.ones(64 << 20, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": src.numel() * 4, "launches": 8}))
        return
    from autoregressive_transformer_decode_amd import inputs
    if args.workload == "codec":
        print(json.dumps(bench_codec(args, inputs.CODEC)), flush=True)
        return
    wl = inputs.WORKLOADS[args.workload]
    if wl.cp is not None:
        out = bench_frames(args, wl)
    elif wl.batch > 1:
        r = bench_batched(args, wl, steps=args.steps, warmup=args.warmup)
        out = dict(metric=METRIC, value=r["value"], unit="tokens/s", n_gpus=1, steps=r["iterations"],
                   warmup=r["warmup"], ms_per_step=r["ms_per_iteration"], higher_is_better=True,
                   scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
                   config=r["config"], roofline=r["roofline"], gemm_gate_up=r["gemm_gate_up"],
                   stage_us_per_layer=r["stage_us_per_layer"], step_hbm=r["step_hbm"],
                   cpu_baseline=r["cpu_baseline"])
    else:
        out = bench_lm(args, wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
