#!/usr/bin/env python3
"""Benchmark the GatedDeltaNet layer on one MI355X.

One step = the whole layer path over one packed row: the gates (g, beta from
a, b, A_log, dt_bias), conv1d+SiLU+L2, the chunked gated delta rule,
RMSNormGated, and (for the training workload) the backward of all of them
(--fused-gates: the gates computed inside the chunk kernels instead).  Default workload: the training step, 8 sequences x
8192 tokens packed in one row, 16 q/k heads, 32 v heads, d = 128, bf16.

Prints ONE JSON line with the throughput (tokens/s), the roofline of the
dominant kernel, and the CPU oracle timed on a bounded sample of the same
workload (all sequences, --cpu-heads of the q/k heads).  Two timed regions of
--steps steps each, after --warmup untimed ones: the step launched eagerly with
the library's per-kernel HIP events on (the per-kernel durations and the
roofline; reported under "eager"), then the same step recorded once into a HIP
graph and replayed (the throughput and ms_per_step; --graph 0 reports the eager
figures instead).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    "train": "training step: fwd+bwd, 8 x 8192 packed varlen row, 16 qk / 32 v heads, d=128, bf16",
    "dense": "forward: 4 x 2048 dense batch as one packed row, 16 qk / 32 v heads, d=128, bf16",
    "varlen": "forward: 20 log-uniform lengths packed into 32768 tokens, h0 in / ht out, d=128, bf16",
    "long": "forward: one 65536-token sequence, 16 qk / 32 v heads, d=128, bf16",
    "tiny": "forward: 64 tokens, 2 heads, d=16, chunk 16, fp32",
    "decode": "decode: 256 sequences advance one token each from their states and conv windows, "
              "16 qk / 32 v heads, d=128, bf16",
}


def csrc_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(HERE, "gated_delta_rule_conv1d_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_bytes(cfg, n_chunks: int, has_h0: bool) -> dict:
    """Algorithmic bytes per launch of each kernel: every input it must read
    once and every output it must write once, workspace tensors included at
    the precision they are stored in (a q/k tile shared by the G v-heads of a
    k-head counts once).  Slot = (chunk, v-head); k-slot = (chunk, k-head)."""
    T, N, Hk, Hv, D, C = cfg.T, cfg.N, cfg.h_qk, cfg.h_v, cfg.d_k, cfg.chunk
    es = 2 if cfg.dtype == "bf16" else 4
    lo = 2 if cfg.dtype == "bf16" else 1        # hi + lo parts of split bf16 operands
    Cch = 2 * Hk * D + Hv * D
    W = cfg.width
    S, SK = n_chunks * Hv, n_chunks * Hk
    tile_e, tile_f = C * D * es, C * D * 4    # [C][D] tile in the element type / in fp32
    cc_f, row_f = C * C * 4, C * 4            # [C][C] fp32 tile / one fp32 row of C
    dd_f = D * D * 4                          # [D][D] fp32 state
    qk_in = SK * 2 * tile_e                   # q and k of each k-slot
    v_in = S * tile_e
    gb_in = 2 * T * Hv * 4                    # g and beta
    st = N * Hv * dd_f                        # one state per (sequence, v-head)
    # K^T (and the reverse pass's K rows) as the state passes read them: plain
    # bf16 K at d = 128, chunk 64 (the decay goes onto W's / K dH's rows
    # there), else K~ in hi + lo parts
    kt = 1 if (cfg.dtype == "bf16" and D == 128 and C == 64) else lo
    # the plain K^T is the same for the G v-heads of a k-head: written once per
    # k-slot; the inference forward's 16-column state pass (at most 64 chains)
    # also reads q from a copy the preparation writes in its load order
    kt_out = SK * tile_e if kt == 1 else S * kt * tile_e
    q_frag = kt == 1 and N * Hv * 4 <= 256
    prep_out = S * (tile_e + tile_f + cc_f + row_f) + kt_out   # Wk, U, P, gamma; K^T
    # what the preparation adds for the reverse pass: T and Wk^T (hi + lo); for the tiled
    # reverse pass also P^T, the K rows and (Gamma q)^T (the whole-state pass, kt == 1,
    # forms those from P, k and q)
    prep_bwd_out = S * (cc_f + lo * tile_e) + (0 if kt == 1 else S * (cc_f + (kt + lo) * tile_e))
    # the reverse pass: P (or P^T), K rows, Wk^T, (Gamma q)^T (or q), gamma, dO in; dH_n and
    # dW^T out (the tiled pass also writes dW rows)
    if kt == 1:
        state_bwd = SK * 2 * tile_e + S * (cc_f + lo * tile_e + row_f + tile_e) + S * (dd_f + tile_f)
    else:
        state_bwd = S * (cc_f + (kt + 2 * lo) * tile_e + row_f + tile_e) + S * (dd_f + 2 * tile_f)
    return {
        # decode: the state is read and written once per (sequence, v-head)
        "recurrent_step": 2 * N * Hv * dd_f + N * (2 * Hk * D + 2 * Hv * D) * es + 2 * N * Hv * 4,
        "conv_step": (2 * (W - 1) + 2) * N * Cch * es + Cch * W * es,
        "gates_fwd": 4 * T * Hv * 4 + 2 * Hv * 4,    # a, b in; g, beta out
        "gates_bwd": 6 * T * Hv * 4 + 2 * Hv * 4,    # a, b, dg, dbeta in; da, db out
        "conv_fwd": 2 * T * Cch * es + Cch * W * es,
        "conv_bwd": 3 * T * Cch * es + Cch * W * es,
        "norm_fwd": 3 * T * Hv * D * es + D * es,
        "norm_bwd": 5 * T * Hv * D * es + D * es,
        "chunk_prep": qk_in + v_in + gb_in + prep_out + (SK * tile_e if q_frag else 0),
        # + what the reverse pass reads from the preparation (prep_bwd_out above)
        "chunk_prep_bwd": qk_in + v_in + gb_in + prep_out + prep_bwd_out,
        "chunk_state_fwd": SK * tile_e + kt_out + S * (tile_e + tile_f + cc_f + row_f)
                           + S * tile_e + (st if has_h0 else 0) + st,
        # forward that also keeps the backward's products: prep_bwd's outputs, and H_c, W per slot
        "chunk_prep_save": qk_in + v_in + gb_in + prep_out + prep_bwd_out,
        "chunk_state_save": SK * tile_e + kt_out + S * (tile_e + tile_f + cc_f + row_f)
                            + S * tile_e + (st if has_h0 else 0) + st + S * (dd_f + tile_f),
        "chunk_state_store": kt_out + S * (tile_e + tile_f + row_f) + (st if has_h0 else 0)
                             + S * (dd_f + tile_f),
        "chunk_state_bwd": state_bwd,
        "chunk_grad_a": SK * tile_e + S * (2 * dd_f + 2 * tile_f + 2 * tile_e + 2 * row_f)
                        + S * (3 * tile_f + 2 * cc_f + 4),
        "chunk_grad_b": qk_in + S * (4 * tile_f + 4 * cc_f + tile_e + 2 * row_f + 4)
                        + S * (tile_e + 2 * row_f) + SK * 2 * tile_e,
    }


def fused_minimum_bytes(cfg) -> int:
    """What one step must move through HBM at the least, whatever the kernel
    split: every input read once and every output written once, nothing in
    between.  Per token, forward: the pre-conv q, k, v row, z, g and beta
    (fp32), the norm output (o when there is no norm); backward adds the
    re-read of those inputs, dy in and dq, dk, dv, dz, dg, dbeta out.  Per
    sequence: its initial state read (when given) and its final state written
    (fp32 [Hv][dk][dv]); a decode step also reads and writes its conv window."""
    Hk, Hv, dk, dv = cfg.h_qk, cfg.h_v, cfg.d_k, cfg.d_v
    es = 2 if cfg.dtype == "bf16" else 4
    row = (2 * Hk * dk + Hv * dv) * es          # conv input, or its gradient
    vh = Hv * dv * es                           # z, y, dy or dz
    gb = 2 * Hv * 4                             # g and beta, or their gradients
    fwd = row + gb + vh * (2 if cfg.norm else 1)
    bwd = (row + gb + vh) + vh + (row + gb + vh) if cfg.bwd else 0   # re-read, dy, gradients
    state = Hv * dk * dv * 4
    per_seq = state * (2 if cfg.h0 else 1)
    if cfg.decode:
        per_seq += 2 * (cfg.width - 1) * (2 * Hk * dk + Hv * dv) * es
    return (fwd + bwd) * cfg.T + per_seq * cfg.N


def kernel_flops(cfg, n_chunks: int) -> dict:
    """Algorithmic flops per launch: the method's contractions, triangular
    factors counted once (no split-precision extra products)."""
    Hv, Hk, D, C = cfg.h_v, cfg.h_qk, cfg.d_k, cfg.chunk
    S, SK = n_chunks * Hv, n_chunks * Hk
    tri = C * (C + 1) // 2                     # entries of a lower-inclusive C x C factor
    cd2 = 2 * C * D * D                        # one [C][D] x [D][D] product
    return {
        "chunk_prep": SK * 2 * 2 * tri * D + S * (C ** 3 // 3 + 2 * 2 * tri * D),
        "chunk_prep_save": SK * 2 * 2 * tri * D + S * (C ** 3 // 3 + 2 * 2 * tri * D),
        "chunk_state_save": S * (3 * cd2 + 2 * tri * D),
        "chunk_prep_bwd": SK * 2 * 2 * tri * D + S * (C ** 3 // 3 + 2 * 2 * tri * D),
        "chunk_state_fwd": S * (3 * cd2 + 2 * tri * D),
        "chunk_state_store": S * 2 * cd2,
        "chunk_state_bwd": S * (3 * cd2 + 2 * tri * D),
        "chunk_grad_a": S * (3 * cd2 + 2 * 2 * C * C * D + 2 * tri * D),
        "chunk_grad_b": SK * 2 * tri * D + S * (2 * 2 * tri * D + 2 * C ** 3 + 3 * 2 * tri * D + 2 * C * C * D),
    }


def load_traffic(kernel: str, workload: str, n_launch_units: float):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(HERE, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for ln in f:
            if ln.startswith("#") or "=" not in ln:
                continue
            k, v = ln.split("=", 1)
            rec[k.strip()] = v.strip()
    if rec.get("csrc_hash") != csrc_hash():
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, inp, kheads: int):
    """The CPU oracle, as it stands, on all sequences of the workload restricted
    to `kheads` q/k heads (with their v-heads); scaled to whole-layer tokens/s."""
    import oracle
    sub_cfg, sub, _, _ = oracle.subset(cfg, inp, list(range(cfg.N)), list(range(kheads)))
    sub = {k: (v.astype("float64") if v.dtype.kind == "f" else v) for k, v in sub.items()}
    hv = kheads * cfg.h_v // cfg.h_qk
    gate_in = [inp["a"][:, :hv], inp["b"][:, :hv], inp["A_log"][:hv], inp["dt_bias"][:hv]]
    t0 = time.perf_counter()
    g, beta = oracle.gates(*gate_in)
    fwd = oracle.layer_fwd(sub_cfg, sub)
    if cfg.bwd:
        r = oracle.layer_bwd(sub_cfg, sub, fwd, sub["dy"])
        oracle.gates_bwd(*gate_in, r["dg"], r["dbeta"])
    dt = time.perf_counter() - t0
    tokens_equiv = cfg.T * kheads / cfg.h_qk
    single = single_thread_oracle()
    return {"value": tokens_equiv / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "single_thread": single,
            "sample": ("one-token sequences from the same states, conv from zero history: " if cfg.decode else "") +
                      f"all {cfg.N} sequences ({cfg.T} tokens) x {kheads} of {cfg.h_qk} q/k heads "
                      f"({hv} v-heads), gates + layer, fp64 {'fwd+bwd' if cfg.bwd else 'fwd'}; "
                      f"{dt:.1f} s scaled to whole-layer tokens/s",
            "seconds": dt}


def single_thread_oracle() -> dict:
    """The oracle on one thread, forward: the whole tiny workload, and the
    dense 4 x 2048 workload on 1 of its 16 q/k heads (scaled to whole-layer
    tokens/s)."""
    import oracle
    import synth
    full = oracle.threads()
    oracle.set_threads(1)
    res = {}
    try:
        for name, kheads in (("tiny", None), ("dense", 1)):
            cfg = synth.config(name)
            inp = synth.make_inputs(cfg)
            if kheads:
                cfg, inp, _, _ = oracle.subset(cfg, inp, list(range(cfg.N)), list(range(kheads)))
            t0 = time.perf_counter()
            oracle.layer_fwd(cfg, inp)
            dt = time.perf_counter() - t0
            scale = synth.config(name).h_qk / cfg.h_qk
            res[name] = {"tokens_per_s": round(cfg.T / scale / dt, 1), "seconds": round(dt, 3),
                         "sample": f"{cfg.T} tokens x {cfg.h_qk} of {synth.config(name).h_qk} q/k heads, fwd"}
    finally:
        oracle.set_threads(full)
    return res


def achievable_peaks(gdn, torch) -> dict:
    """What this chip reaches, beside the published peaks every kernel is
    priced against: a 16-byte-per-lane streaming copy of 2 GiB (read + write
    bytes / time) and a loop of independent bf16 matrix-core products on 16
    waves per compute unit; each the best of 5 runs timed with HIP events."""
    n = 2 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    out = torch.empty(1024 * 256, dtype=torch.float32, device="cuda:0")

    def best(fn, reps=5):
        fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)

    t_copy = best(lambda: gdn.probe_copy(src, dst))
    t_tcopy = best(lambda: dst.copy_(src))
    flops = 1024 * 4 * 8 * 20000 * 16384      # the same for both shapes (4 chains of twice the work)
    t_16 = best(lambda: gdn.probe_mfma(out, 1024, 20000, 0))
    t_32 = best(lambda: gdn.probe_mfma(out, 1024, 20000, 1))
    del src, dst
    gbs = 2 * n / min(t_copy, t_tcopy) / 1e9
    tf16, tf32 = flops / t_16 / 1e12, flops / t_32 / 1e12
    return {"copy_GBps": round(gbs, 1), "copy_frac_of_peak": round(gbs / HBM_PEAK_GBS, 3),
            "copy_GBps_probe_kernel": round(2 * n / t_copy / 1e9, 1),
            "copy_GBps_torch": round(2 * n / t_tcopy / 1e9, 1),
            "mfma_bf16_16x16x32_TFLOPs": round(tf16, 1), "mfma_bf16_32x32x16_TFLOPs": round(tf32, 1),
            "mfma_frac_of_peak": round(max(tf16, tf32) / MFMA_BF16_PEAK_TFLOPS, 3),
            "method": "copy: gdn_probe_copy and torch copy_ of 2 GiB (read + write bytes); mfma: gdn_probe_mfma, "
                      "1024 x 256 threads, 20000 rounds of independent v_mfma_f32_16x16x32_bf16 (8 chains) or "
                      "v_mfma_f32_32x32x16_bf16 (4 chains); best of 5, HIP events"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="train", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-heads", type=int, default=8, help="q/k heads in the CPU-oracle sample (0: skip)")
    ap.add_argument("--peaks", type=int, default=1, help="also time the achievable-peak probes (0: skip)")
    ap.add_argument("--fused-gates", action="store_true",
                    help="compute the gates inside the chunk kernels (gdn_chunk_*_gated) instead of with "
                         "gdn_gates / gdn_gates_bwd (measured slightly slower: the default is the separate kernels)")
    ap.add_argument("--graph", type=int, default=1,
                    help="1: the reported throughput times the step replayed from a HIP graph (per-kernel "
                         "durations still come from the eager timed steps); 0: eager launches only")
    ap.add_argument("--max-tokens", type=int, default=0, metavar="N",
                    help="bounded-memory training step: the chunk calls run per token segment of at most N "
                         "tokens and the backward recomputes the forward's chunk products (0: the whole row, "
                         "the forward keeping its products for the backward)")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the reference for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters of rocprofv3) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calib:
        src = torch.empty(args.copy_calib << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_calib << 20, "repeats": 3}))
        return

    import gated_delta_rule_conv1d_amd as gdn
    import synth

    cfg = synth.config(args.workload)
    t_gen = time.perf_counter()
    inp = synth.make_inputs(cfg, keep_raw=True)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    bf = cfg.dtype == "bf16"

    def to_dev(key):
        if bf and key + "_bits" in inp:
            return torch.from_numpy(inp[key + "_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(inp[key], dtype=np.float32)).to(dev)

    x, w = to_dev("x"), to_dev("w_conv")
    ga, gb, A_log, dt_bias = (to_dev(k) for k in ("a", "b", "A_log", "dt_bias"))
    cu = torch.from_numpy(inp["cu"]).to(dev)
    z = to_dev("z") if cfg.norm else None
    wn = to_dev("w_norm") if cfg.norm else None
    h0 = to_dev("h0") if cfg.h0 else None
    dy = to_dev("dy") if cfg.bwd else None
    shape = gdn.Shape(cfg.N, cfg.T, cfg.h_qk, cfg.h_v, cfg.d_k, cfg.d_v, cfg.chunk,
                      gdn.BF16 if bf else gdn.F32, 1.0)
    layer = gdn.GatedDeltaNetLayer(shape, cfg.width, dev, norm=cfg.norm)

    if cfg.decode:
        window = to_dev("window")
        state = h0  # advanced in place, step after step

        def step():
            g, beta = layer.gates(ga, gb, A_log, dt_bias)
            yc = gdn.conv1d_step(x, w, window, shape)
            q, k, v = layer.split(yc)
            o, _ = gdn.recurrent_step(q, k, v, g, beta, shape, state_in=state, state_out=state)
            gdn.norm_gate(o, z, wn, shape)
    elif args.fused_gates:
        gates = (ga, gb, A_log, dt_bias)

        def step():
            # the chunk kernels compute g and beta from the raw gate inputs (and,
            # backward, their gradients); a training step keeps the forward's
            # chunk products for the backward
            f = layer.forward(x, w, None, None, cu, z, wn, h0, for_backward=cfg.bwd, gates=gates)
            if cfg.bwd:
                layer.backward(dy, x, w, None, None, cu, f, z, wn, h0, gates=gates)
    elif args.max_tokens:
        def step():
            g, beta = layer.gates(ga, gb, A_log, dt_bias)
            f = layer.forward(x, w, g, beta, cu, z, wn, h0, max_tokens=args.max_tokens)
            if cfg.bwd:
                r = layer.backward(dy, x, w, g, beta, cu, f, z, wn, h0)
                layer.gates_backward(ga, gb, A_log, dt_bias, r["dg"], r["dbeta"])
    else:
        def step():
            g, beta = layer.gates(ga, gb, A_log, dt_bias)
            # a training step keeps the forward's chunk products for the backward
            f = layer.forward(x, w, g, beta, cu, z, wn, h0, for_backward=cfg.bwd)
            if cfg.bwd:
                r = layer.backward(dy, x, w, g, beta, cu, f, z, wn, h0)
                layer.gates_backward(ga, gb, A_log, dt_bias, r["dg"], r["dbeta"])

    # Per-kernel durations come from HIP events that the library records around
    # each launch on the stream it launches on, during the eager timed steps
    # themselves.  Warm-up runs with recording on too, so that the timed steps
    # reuse pooled events instead of creating them.
    gdn.profile_enable(True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    gdn.profile_enable(True)  # clears the warm-up records
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    rep = gdn.profile_report()
    gdn.profile_enable(False)
    eager = {"ms_per_step": round(elapsed * 1e3 / args.steps, 4), "value": round(cfg.T * args.steps / elapsed, 1)}

    # The same step recorded once into a HIP graph and replayed: every kernel of
    # the step runs on every replay, without the per-launch host work.  The
    # bounded-memory mode reads cu_seqlens on the host and is not capturable.
    graph_info = None
    if args.graph and not args.max_tokens:
        try:
            graph, _ = gdn.capture(step)
            for _ in range(args.warmup):
                graph.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                graph.replay()
            torch.cuda.synchronize()
            elapsed = time.perf_counter() - t0
            del graph
            graph_info = "hip graph replay"
        except Exception as e:  # report the eager figure rather than none
            torch.cuda.synchronize()
            graph_info = f"eager (graph capture failed: {type(e).__name__}: {e})"
    ms_per_step = elapsed * 1e3 / args.steps
    value = cfg.T * args.steps / elapsed

    peaks = achievable_peaks(gdn, torch) if args.peaks else None

    import oracle
    n_chunks = len(oracle.chunk_table(inp["cu"], cfg.chunk)[0])
    kb = kernel_bytes(cfg, n_chunks, cfg.h0)
    kf = kernel_flops(cfg, n_chunks)
    if args.max_tokens:
        # the chunk kernels launch once per token segment: each launch covers that
        # segment's share of the row (equal shares at the training workload)
        nseg = len(gdn.token_segments([int(c) for c in inp["cu"]], cfg.chunk, args.max_tokens))
        for d in (kb, kf):
            for key in list(d):
                if key.startswith("chunk_") and key != "chunk_index":
                    d[key] = d[key] / nseg
    kernels = {}
    base = lambda name: name.split(":", 1)[0]   # state-pass records carry their variant after a colon
    for name, (cnt, tot) in rep.items():
        avg_ms = tot / cnt
        kernels[name] = {"launches": cnt, "avg_us": round(avg_ms * 1e3, 2),
                         "share": round(tot / sum(t for _, t in rep.values()), 4)}
        if base(name) in kb:
            gbs = kb[base(name)] / (avg_ms * 1e-3) / 1e9
            kernels[name]["GBps"] = round(gbs, 1)
            kernels[name]["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 3)
        if base(name) in kf:
            tfs = kf[base(name)] / (avg_ms * 1e-3) / 1e12
            kernels[name]["TFLOPs"] = round(tfs, 2)
            kernels[name]["mfma_frac"] = round(tfs / MFMA_BF16_PEAK_TFLOPS, 4)
    dom = max(rep, key=lambda k: rep[k][1])
    cnt, tot = rep[dom]
    avg_s = tot / cnt * 1e-3
    t_hbm = kb.get(base(dom), 0) / (HBM_PEAK_GBS * 1e9)
    t_mfma = kf.get(base(dom), 0) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_mfma > t_hbm:
        achieved = kf[base(dom)] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = kb.get(base(dom), 0) / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = dom
    roof["avg_us"] = round(avg_s * 1e6, 2)
    roof["algorithmic_bytes"] = kb.get(base(dom))
    # the committed counters cover the whole-row launches of the standard step:
    # not the per-segment launches of --max-tokens, nor the fused-gate kernels
    roof["traffic"] = None if (args.max_tokens or args.fused_gates) else load_traffic(base(dom), args.workload, 1)

    # whole-step roofline of the path (fused algorithmic minimum)
    step_bytes = fused_minimum_bytes(cfg) if args.workload != "tiny" else None

    cpu = None
    if args.cpu_heads > 0:
        cpu = cpu_baseline(cfg, inp, min(args.cpu_heads, cfg.h_qk))

    out = {
        "metric": ("GatedDeltaNet fwd+bwd tokens/s, packed varlen H=32 d=128 bf16; % roofline" if cfg.bwd else
                   "GatedDeltaNet decode tokens/s (one token per sequence); % roofline" if cfg.decode else
                   "GatedDeltaNet fwd tokens/s, packed varlen; % roofline"),
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "launch": graph_info or "eager",
        "eager": eager,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOADS[args.workload]}", "tokens": cfg.T,
                   "n_seqs": cfg.N, "h_qk": cfg.h_qk, "h_v": cfg.h_v, "d": cfg.d_k, "chunk": cfg.chunk,
                   "gates": ("g, beta computed from a, b, A_log, dt_bias inside the chunk kernels"
                             if args.fused_gates and not cfg.decode else
                             "g, beta computed from a, b, A_log, dt_bias in the step (gate kernels)"),
                   "parallelism": "single GPU",
                   "chunk_workspace_gib": round(sum(t.numel() for t in layer._ws.values()) / 2 ** 30, 3),
                   "max_tokens": args.max_tokens or None},
        "roofline": roof,
        "step_fraction_of_fused_minimum": (round(step_bytes / (HBM_PEAK_GBS * 1e9) / (ms_per_step * 1e-3), 4)
                                           if step_bytes else None),
        "kernels": kernels,
        "achievable_peaks": peaks,
        "cpu_baseline": cpu,
        "input_generation_s": round(t_gen, 2),
        "csrc_hash": csrc_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
