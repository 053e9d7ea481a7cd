"""Benchmark of the HSTU attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS] [--no-cpu-baseline] [--extended]
    python bench.py --only {layers,cached,attn_bwd,layer_bwd,layer_bwd_call,softmax}

A step is one hstu_attn_fwd call (QK^T, bias, SiLU, mask and AV of every allowed pair) over the
L = 8192 workload: 8 sequences of 8192 events, 4 heads x 128, P = Tb = 256 bias buckets, causal,
bf16 with fp32 accumulation; inputs are resident in HBM before the timed region.  The FLOP count
covers allowed (causal, non-padded) pairs only: sum_b H * n_b (n_b + 1) / 2 * 4 * Dh.

Before the W warm-up steps, untimed calls run for --settle-ms (300 ms by default) so that the chip has
reached its sustained clock when the K timed steps start; `clock_settle` in the output says how many.

Prints one JSON line.  `roofline` compares the kernel's average duration (HIP events on the stream
it runs on) with the MI355X dense bf16 MFMA peak; `cpu_baseline` times the float64 oracle on a
bounded sample of the same workload on the host cores.  --extended also prints, to stderr, the
timings of the other workloads (layer, stack and candidate-masked forwards, cached-history scoring,
attention backward, layer backward); --only runs one of those legs alone.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0          # MI355X dense bf16 MFMA (no sparsity)
HBM_PEAK_GBS = 8000.0
METRIC = "HSTU attn fwd TFLOP/s (causal, jagged) at L=8192 bf16; % MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_L8192_traffic.json")
# every source the attention forward kernel is compiled from (its traffic figure is void once any changes)
KERNEL_SOURCES = [os.path.join(ROOT, "hstu_sequential_transduction_attn_amd", "csrc", f)
                  for f in ("attn_fwd.hip", "attn_common.hpp", "device_common.hpp", "row_ids.hpp", "work_order.hpp", "kernels.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source (else None)."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _oracle_unit(task):
    """One worker of the CPU baseline: the float64 oracle on 128-row query blocks of one (sequence, head),
    in the given order, until its time budget is spent.  Returns (FLOP, blocks done, seconds)."""
    q, k, v, tau, wp, wt, blocks, budget_s = task
    from oracle import hstu_oracle as O
    n, dh = q.shape
    jag = dict(seq_offsets=np.array([0, n], np.int64), timestamps=tau, mask=0, num_candidates=None, attn_scale=None)
    flop, done, t0 = 0, 0, time.perf_counter()
    for r0 in blocks:
        rows = np.arange(r0, min(r0 + 128, n))
        O.attn_fwd(jag, q[:, None], k[:, None], v[:, None], wp, wt, row_sample={0: rows})
        flop += int((rows + 1).sum()) * 4 * dh
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    return flop, done, time.perf_counter() - t0


def cpu_baseline(case, budget_s: float = 15.0):
    """Time the float64 oracle on the host: one single-threaded process per core (up to 16) over the
    (sequence, head) units of the workload, each unit's 128-row query blocks in an order spread over the
    sequence (bit-reversed block index), every block against all its causal keys; each unit stops after
    its share of about budget_s, so a host too slow for the whole workload times a spread sample of it."""
    import multiprocessing as mp
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    j = case.jagged
    offs = j.seq_offsets.astype(np.int64)
    units = [(b, h) for b in range(j.num_seqs) for h in range(case.num_heads)]
    per_unit_s = budget_s / -(-len(units) // cores)
    tasks = []
    for b, h in units:
        o0, o1 = int(offs[b]), int(offs[b + 1])
        nblk = (o1 - o0 + 127) // 128
        bits = max(1, (nblk - 1).bit_length())
        order = sorted(range(nblk), key=lambda x: int(format(x, f"0{bits}b")[::-1], 2))
        sl = slice(o0, o1)
        tasks.append((case.q.values[sl, h], case.k.values[sl, h], case.v.values[sl, h], j.timestamps[sl],
                      case.rab.pos_bias, case.rab.time_bias, [128 * x for x in order], per_unit_s))
    env = {k_: os.environ.get(k_) for k_ in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k_ in env:
        os.environ[k_] = "1"    # each worker is one core
    try:
        t0 = time.perf_counter()
        with mp.get_context("spawn").Pool(cores) as pool:
            t1 = time.perf_counter()
            res = pool.map(_oracle_unit, tasks, chunksize=1)
            wall = time.perf_counter() - t1
        total = time.perf_counter() - t0
    finally:
        for k_, v_ in env.items():
            if v_ is None:
                os.environ.pop(k_, None)
            else:
                os.environ[k_] = v_
    flop = sum(r[0] for r in res)
    blocks = sum(r[1] for r in res)
    nblk = sum((int(offs[b + 1] - offs[b]) + 127) // 128 for b, _ in units)
    return {"value": flop / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 oracle in {cores} single-threaded processes (one per host core, "
                      f"{len(os.sched_getaffinity(0))} available) over the {len(units)} (sequence, head) units: "
                      f"{blocks} of the workload's {nblk} query blocks of 128 rows, spread over each sequence, "
                      f"each against all its causal keys ({flop:.3e} FLOP in {wall:.1f} s; {total:.1f} s with "
                      f"process start-up)"}


def run(args):
    import torch
    from hstu_sequential_transduction_attn_amd import configs as C
    from hstu_sequential_transduction_attn_amd import _lib as ops

    ops.load_library()  # fails loudly without the HIP library
    dev = torch.device("cuda:0")
    case = C.attn_L8192()
    j = case.jagged

    def t(x):
        if x.dtype == "bf16":
            return torch.from_numpy(x.bits.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x.values).to(dev)
    q, k, v = t(case.q), t(case.k), t(case.v)
    offs = torch.from_numpy(j.seq_offsets.astype(np.int32)).to(dev)
    tau = torch.from_numpy(j.timestamps).to(dev)
    wp = torch.from_numpy(case.rab.pos_bias).to(dev)
    wt = torch.from_numpy(case.rab.time_bias).to(dev)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    ws = torch.empty(max(ops.attn_workspace_bytes(offs, tau, q, wp, wt, max_seq_len=j.max_seq_len), 1),
                     dtype=torch.uint8, device=dev)

    def step():
        ops.attn_fwd(offs, tau, q, k, v, wp, wt, max_seq_len=j.max_seq_len, out=out, workspace=ws, stream=stream)

    # The chip's power management needs on the order of 100 ms of sustained load to reach its sustained
    # clock; a timed region of a few milliseconds right after a few calls from idle measures that ramp
    # (about 12% slower), not the kernel.  So untimed calls run for settle_ms first, then the W warm-up
    # steps, then exactly K timed steps.
    settle_calls, t_settle = 0, time.perf_counter()
    while args.settle_ms > 0 and (time.perf_counter() - t_settle) * 1e3 < args.settle_ms and settle_calls < 5000:
        for _ in range(25):
            step()
        torch.cuda.synchronize()
        settle_calls += 25
    settle_ms = (time.perf_counter() - t_settle) * 1e3 if settle_calls else 0.0
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps

    flop = case.flops()
    tflops = flop * args.steps / wall / 1e12
    achieved = flop / (kernel_ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attn_L8192: hstu_attn_fwd, 8 jagged sequences x 8192 events, H=4, Dh=128, "
                               "P=Tb=256, causal, bf16 in/out, fp32 accumulation",
                   "global_batch": j.num_seqs, "seq_len": j.max_seq_len, "tokens": j.total_tokens,
                   "flop_per_step": flop, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(), "kernel_ms": round(kernel_ms, 4)},
        "clock_settle": {"calls": settle_calls, "ms": round(settle_ms, 1),
                         "note": "untimed calls before the warm-up steps, so the timed steps run at the sustained clock"},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(rec), flush=True)
    if args.extended:
        extended(args, dev)


def steady_ms(fn, warm_ms: float = 100.0, timed_ms: float = 60.0) -> float:
    """Milliseconds per call of fn on the current stream at the chip's steady clock: untimed calls for
    about warm_ms of sustained load first (at least 2), then at least 5 timed calls (about timed_ms)."""
    import torch
    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    est = max((time.perf_counter() - t0) * 1e3, 1e-3)
    for _ in range(max(2, min(400, int(warm_ms / est)))):
        fn()
    reps = max(5, min(200, int(timed_ms / est)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def extended(args, dev, layers_only=False):
    """Layer workloads (stderr, informational): layer_bf16, stack8_bf16 and mfalcon_bf16 with every input
    and weight resident on the device; one forward = gather (when the workload stages its input from an
    embedding table) + every layer.  Timed with HIP events on the stream the kernels run on."""
    import torch
    from hstu_sequential_transduction_attn_amd import configs as C
    from hstu_sequential_transduction_attn_amd import inputs as I
    from hstu_sequential_transduction_attn_amd import _lib as ops

    def t(x, dtype=None):
        if isinstance(x, I.Tensor):
            if x.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(x.bits).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(x.values)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    for name, mk, residual_f32, act_split in [("layer_bf16", C.layer_bf16, False, False),
                                              ("stack8_bf16", C.stack8_bf16, True, True),
                                              ("mfalcon_bf16", C.mfalcon_bf16, True, False)]:
        case = mk()
        j = case.jagged
        offs, tau = t(j.seq_offsets.astype(np.int32)), t(j.timestamps.astype(np.int64))
        ncand = None if j.num_candidates is None else t(j.num_candidates.astype(np.int32))
        layers = [dict(w1=t(L.w_uvqk), w2=t(L.w_out), wp=t(L.rab.pos_bias), wt=t(L.rab.time_bias), eps=L.ln_eps)
                  for L in case.layers]
        if case.table_rows:
            table = torch.zeros((case.table_rows, case.d_model), dtype=torch.bfloat16, device=dev)
            table.index_copy_(0, t(case.table_touched.astype(np.int64)), t(case.table_values))
            ids = t(case.ids.astype(np.int64))
            x0 = None
        else:
            table = ids = None
            x0 = t(case.x)
        H, Dh = case.num_heads, case.head_dim
        probe = x0 if x0 is not None else torch.empty((j.total_tokens, case.d_model), dtype=torch.bfloat16, device=dev)
        nws = ops.layer_workspace_bytes(probe, offs, tau, layers[0]["w1"], layers[0]["w2"], layers[0]["wp"],
                                        layers[0]["wt"], H, Dh, max_seq_len=j.max_seq_len, ln_output=True,
                                        mask=j.mask, act_split=act_split)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        ydt = torch.float32 if residual_f32 else None

        def forward():
            x = ops.gather_rows(table, ids) if table is not None else x0
            for li, L in enumerate(layers):
                x = ops.layer_fwd(x, offs, tau, L["w1"], L["w2"], L["wp"], L["wt"], H, Dh,
                                  max_seq_len=j.max_seq_len, ln_eps=L["eps"], ln_output=li < len(layers) - 1,
                                  mask=j.mask, num_candidates=ncand, y_dtype=ydt, act_split=act_split, workspace=ws)
            return x
        ms = steady_ms(forward)
        T, D, HD = j.total_tokens, case.d_model, H * Dh
        pairs = I.allowed_pairs(j)
        flop = len(layers) * (2 * T * D * 4 * HD + pairs * H * 4 * Dh + 2 * T * HD * D)
        print(f"[extended] {name}: {ms:.3f} ms per forward ({len(layers)} layers, T={T}, D={D}, H={H}x{Dh}); "
              f"{flop:.3e} algorithmic FLOP -> {flop / ms / 1e9:.1f} TFLOP/s", file=sys.stderr, flush=True)
        if table is not None:
            # the same forward as one hstu_stack_fwd call: gather and inter-layer LayerNorms fused into the GEMMs
            sl = [dict(w_uvqk=L["w1"], w_out=L["w2"], pos_bias=L["wp"], time_bias=L["wt"], ln_eps=L["eps"])
                  for L in layers]
            y32 = torch.empty((j.total_tokens, case.d_model), dtype=torch.float32, device=dev)
            nsws = ops.stack_workspace_bytes(table, offs, tau, sl, H, Dh, max_seq_len=j.max_seq_len, mask=j.mask,
                                             num_candidates=ncand)
            sws = torch.empty(max(nsws, 1), dtype=torch.uint8, device=dev)

            def stacked():
                return ops.stack_fwd(table, ids, offs, tau, sl, H, Dh, max_seq_len=j.max_seq_len, mask=j.mask,
                                     num_candidates=ncand, act_split=act_split, y=y32, workspace=sws)
            ms2 = steady_ms(stacked)
            print(f"[extended] {name} (hstu_stack_fwd, gather and LayerNorms fused): {ms2:.3f} ms per forward; "
                  f"{flop / ms2 / 1e9:.1f} TFLOP/s", file=sys.stderr, flush=True)
            del sws, y32
        del table, ws
    if layers_only:
        return
    cached_scoring(dev)
    attn_backward(dev)
    layer_backward(dev)
    softmax_context(dev)


def layer_backward(dev, train_step: bool = True):
    """Layer backward (stderr, informational): hstu_layer_bwd on one layer of layer_bf16 (bf16 stream,
    no output LayerNorm) and of stack8_bf16 (its first layer: fp32 activations and gradients, output
    LayerNorm, split activations), for a random upstream gradient.  One call recomputes the forward
    (nothing is saved) and forms dx and every parameter gradient.  Algorithmic FLOP: the forward's
    GEMMs and attention, plus dg, dW2, dx, dW1 (2 T D HD each for the H*Dh-wide ones, 2 T D 4HD for the
    projection's) and 2.5x the attention's pair products.  With train_step, also one layer's forward +
    backward, recomputing the forward and from saved activations."""
    import torch
    from hstu_sequential_transduction_attn_amd import configs as C
    from hstu_sequential_transduction_attn_amd import inputs as I
    from hstu_sequential_transduction_attn_amd import _lib as ops

    def t(x, f32=False):
        if isinstance(x, I.Tensor):
            if x.dtype == "bf16" and not f32:
                return torch.from_numpy(np.ascontiguousarray(x.bits).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(x.values)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    for name, mk, stream32, ln_output in [("layer_bf16", C.layer_bf16, False, False),
                                          ("stack8_bf16 layer 0", lambda: C.stack8_bf16(num_layers=1), True, True)]:
        case = mk()
        j = case.jagged
        L = case.layers[0]
        offs, tau = t(j.seq_offsets.astype(np.int32)), t(j.timestamps.astype(np.int64))
        T, D, H, Dh = j.total_tokens, case.d_model, case.num_heads, case.head_dim
        gen = torch.Generator(device=dev).manual_seed(7)
        dt = torch.float32 if stream32 else torch.bfloat16
        x = torch.randn((T, D), device=dev, generator=gen).to(dt)
        dy = torch.randn((T, D), device=dev, generator=gen).to(dt)
        w1, w2, wp, wt = t(L.w_uvqk), t(L.w_out), t(L.rab.pos_bias), t(L.rab.time_bias)
        nws = ops.layer_bwd_workspace_bytes(x, offs, tau, w1, w2, wp, wt, H, Dh, max_seq_len=j.max_seq_len,
                                            ln_output=ln_output, mask=j.mask)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        dx = torch.empty_like(dy)
        f32 = dict(dtype=torch.float32, device=dev)
        grads = dict(d_w_uvqk=torch.empty(w1.shape, **f32), d_b_uvqk=torch.empty(w1.shape[0], **f32),
                     d_w_out=torch.empty(w2.shape, **f32), d_b_out=torch.empty(D, **f32),
                     d_pos_bias=torch.empty(wp.shape, **f32), d_time_bias=torch.empty(wt.shape, **f32))

        def run():
            ops.layer_bwd(x, dy, offs, tau, w1, w2, wp, wt, H, Dh, max_seq_len=j.max_seq_len, ln_eps=L.ln_eps,
                          ln_output=ln_output, mask=j.mask, act_split=stream32, workspace=ws, dx=dx, grads=grads)

        ms = steady_ms(run)
        HD = H * Dh
        pairs = I.allowed_pairs(j)
        attn = pairs * H * 4 * Dh
        fwd = 2 * T * D * 4 * HD + attn + (2 * T * HD * D if ln_output else 0)
        bwd = 2 * (2 * T * D * HD) + 2 * (2 * T * D * 4 * HD) + 2.5 * attn
        flop = fwd + bwd
        print(f"[extended] layer_bwd {name}: {ms:.3f} ms per backward (T={T}, D={D}, H={H}x{Dh}, forward "
              f"recomputed); {flop:.3e} algorithmic FLOP ({bwd:.3e} backward + {fwd:.3e} recompute) -> "
              f"{flop / ms / 1e9:.1f} TFLOP/s", file=sys.stderr, flush=True)

        if not train_step:
            del ws, x, dy, dx, grads
            continue
        # one layer's training step both ways: forward + backward that recomputes the forward, and
        # forward that keeps its activations + backward that reads them
        fkw = dict(max_seq_len=j.max_seq_len, ln_eps=L.ln_eps, ln_output=ln_output, mask=j.mask, act_split=stream32)
        y = torch.empty_like(x)
        fws = torch.empty(max(ops.layer_workspace_bytes(x, offs, tau, w1, w2, wp, wt, H, Dh, max_seq_len=j.max_seq_len,
                                                        ln_output=ln_output, mask=j.mask, act_split=stream32), 1),
                          dtype=torch.uint8, device=dev)
        nsv = ops.layer_saved_bytes(x, offs, tau, w1, w2, wp, wt, H, Dh, max_seq_len=j.max_seq_len,
                                    ln_output=ln_output, mask=j.mask)
        saved = torch.empty(nsv, dtype=torch.uint8, device=dev)

        def step_recompute():
            ops.layer_fwd(x, offs, tau, w1, w2, wp, wt, H, Dh, workspace=fws, y=y, **fkw)
            run()

        def step_saved():
            ops.layer_fwd(x, offs, tau, w1, w2, wp, wt, H, Dh, y=y, saved=saved, **fkw)
            ops.layer_bwd(x, dy, offs, tau, w1, w2, wp, wt, H, Dh, workspace=ws, dx=dx, grads=grads, saved=saved,
                          **fkw)

        res = {}
        for label, fn in (("recompute", step_recompute), ("saved", step_saved)):
            res[label] = steady_ms(fn)
        print(f"[extended] layer_train_step {name}: forward + backward {res['recompute']:.3f} ms recomputing the "
              f"forward, {res['saved']:.3f} ms from saved activations ({nsv / 1e9:.2f} GB kept)",
              file=sys.stderr, flush=True)
        del ws, x, dy, dx, grads, saved, fws, y


def attn_backward(dev):
    """Attention backward on the attn_L8192 shapes (stderr, informational): hstu_attn_bwd (dq, dk, dv and
    both bias-table gradients) for a random upstream gradient.  Algorithmic FLOP: five pair products per
    allowed pair (the score recompute, dP = dO v, dv, dq, dk), i.e. 2.5x the forward's."""
    import torch
    from hstu_sequential_transduction_attn_amd import configs as C
    from hstu_sequential_transduction_attn_amd import inputs as I
    from hstu_sequential_transduction_attn_amd import _lib as ops

    case = C.attn_L8192()
    j = case.jagged

    def t(x):
        if isinstance(x, I.Tensor):
            return torch.from_numpy(np.ascontiguousarray(x.bits).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    offs, tau = t(j.seq_offsets.astype(np.int32)), t(j.timestamps.astype(np.int64))
    q, k, v = t(case.q), t(case.k), t(case.v)
    g = torch.randn(q.shape, device=dev).to(torch.bfloat16)
    wp, wt = t(case.rab.pos_bias), t(case.rab.time_bias)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)

    def run():
        ops.attn_bwd(offs, tau, q, k, v, g, wp, wt, max_seq_len=j.max_seq_len, workspace=ws)

    ms = steady_ms(run)
    flop = 2.5 * case.flops()
    print(f"[extended] attn_bwd_L8192: {ms:.3f} ms per backward (dq, dk, dv, bias tables); {flop:.3e} algorithmic "
          f"FLOP -> {flop / ms / 1e9:.1f} TFLOP/s ({flop / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS * 100:.1f}% of dense bf16 peak)",
          file=sys.stderr, flush=True)


def cached_scoring(dev):
    """Candidates against a cached history (stderr, informational).  16 users with the mfalcon_bf16
    history lengths U{1024..8192}, 1024 candidates each, H = 4 x 128, P = Tb = 128, bf16.  The same
    request is scored (a) in one pass: hstu_attn_fwd with the candidate mask over history + candidates,
    and (b) as 4 micro-batches of 256 candidates per user against the history's K, V and timestamps
    (hstu_attn_fwd_cached, c_b of the one pass), and as one micro-batch of 1024.  Inputs resident; HIP
    events on the kernels' stream."""
    import torch
    from hstu_sequential_transduction_attn_amd import inputs as I
    from hstu_sequential_transduction_attn_amd import _lib as ops

    def t(x):
        if isinstance(x, I.Tensor):
            return torch.from_numpy(np.ascontiguousarray(x.bits).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    users, m, mb = 16, 1024, 256
    hist = [int(v) for v in I.rng_for(5, 0).integers(1024, 8193, size=users)]
    full = I.attn_case("mfalcon_cached", 5, [h + m for h in hist], H=4, Dh=128, P=128, Tb=128, dtype="bf16",
                       num_candidates=[m] * users, with_u=False)
    cc = I.split_candidates(full)
    j = full.jagged
    offs, tau, ncand = t(j.seq_offsets.astype(np.int32)), t(j.timestamps.astype(np.int64)), t(j.num_candidates)
    q, k, v = t(full.q), t(full.k), t(full.v)
    wp, wt = t(full.rab.pos_bias), t(full.rab.time_bias)
    h_offs, h_tau = t(cc.hist_offsets.astype(np.int32)), t(cc.hist_timestamps.astype(np.int64))
    kh, vh = t(cc.k_hist), t(cc.v_hist)
    scale = t((1.0 / cc.one_pass_lengths).astype(np.float32))
    co = cc.cand_offsets.astype(np.int64)

    def one_pass():
        ops.attn_fwd(offs, tau, q, k, v, wp, wt, max_seq_len=j.max_seq_len, mask=ops.MASK_CAUSAL_CANDIDATES,
                     num_candidates=ncand)

    def micro_batches(mb):
        batches = []
        for s in range(m // mb):
            idx = np.concatenate([np.arange(co[b] + s * mb, co[b] + (s + 1) * mb) for b in range(users)])
            ti = torch.from_numpy(idx).to(dev)
            batches.append(dict(offs=t(I.offsets_of([mb] * users)), tau=t(cc.cand_timestamps[idx]),
                                q=t(cc.q)[ti].contiguous(), k=t(cc.k)[ti].contiguous(), v=t(cc.v)[ti].contiguous()))
        b0 = batches[0]
        nws = ops.attn_cached_workspace_bytes(h_offs, h_tau, b0["offs"], b0["tau"], 4, 128, wp, wt,
                                              max_candidates=mb, max_history=max(hist))
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)

        def run():
            for bt in batches:
                ops.attn_fwd_cached(h_offs, h_tau, kh, vh, bt["offs"], bt["tau"], bt["q"], bt["k"], bt["v"], wp, wt,
                                    max_candidates=mb, max_history=max(hist), attn_scale=scale, workspace=ws)
        return run

    timed = steady_ms

    per_pair = 4 * 4 * 128
    pairs_cached = sum(m * (h + 1) for h in hist)
    t_one = timed(one_pass)
    line = (f"[extended] mfalcon_cached: one pass (history + {m} candidates) {t_one:.3f} ms, "
            f"{I.allowed_pairs(j) * per_pair / t_one / 1e9:.1f} TFLOP/s")
    for mb in (256, 1024):
        tc = timed(micro_batches(mb))
        line += (f"; cached history, {m // mb} micro-batch(es) of {mb}: {tc:.3f} ms, "
                 f"{pairs_cached * per_pair / tc / 1e9:.1f} TFLOP/s, {t_one / tc:.2f}x faster")
    print(line, file=sys.stderr, flush=True)


def softmax_context(dev):
    """Context for the HSTU abstract's speed claim against FlashAttention2-based Transformers at length
    8192 (stderr): the self-written causal softmax attention on the attn_L8192 inputs beside
    hstu_attn_fwd, both timed at the steady clock.  Same causal FLOP count for both (QK^T and AV)."""
    import torch
    from hstu_sequential_transduction_attn_amd import configs as C
    from hstu_sequential_transduction_attn_amd import _lib as ops
    case = C.attn_L8192()
    j = case.jagged

    def t(x):
        return torch.from_numpy(x.bits.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = t(case.q), t(case.k), t(case.v)
    offs = torch.from_numpy(j.seq_offsets.astype(np.int32)).to(dev)
    tau = torch.from_numpy(j.timestamps).to(dev)
    wp = torch.from_numpy(case.rab.pos_bias).to(dev)
    wt = torch.from_numpy(case.rab.time_bias).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(max(ops.attn_workspace_bytes(offs, tau, q, wp, wt, max_seq_len=j.max_seq_len), 1),
                     dtype=torch.uint8, device=dev)
    flop = case.flops()
    ms_h = steady_ms(lambda: ops.attn_fwd(offs, tau, q, k, v, wp, wt, max_seq_len=j.max_seq_len, out=out,
                                          workspace=ws))
    ms_s = steady_ms(lambda: ops.softmax_attn_fwd(offs, q, k, v, max_seq_len=j.max_seq_len, out=out))
    print(f"[extended] softmax vs pointwise attention, attn_L8192 shapes: hstu_attn_fwd {ms_h:.3f} ms "
          f"({flop / ms_h / 1e9:.1f} TFLOP/s), causal softmax attention {ms_s:.3f} ms "
          f"({flop / ms_s / 1e9:.1f} TFLOP/s); ratio {ms_s / ms_h:.2f}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed calls for about this long before the warm-up steps (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extended", action="store_true")
    ap.add_argument("--only", choices=["layers", "cached", "attn_bwd", "layer_bwd", "layer_bwd_call", "softmax"],
                    help="run only this informational leg of --extended (stderr), without the metric line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy (torch copy_) five times, to scale "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE against a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the attention forward of one GPU's share is the measured "
              f"unit (--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.only:
        import torch
        from hstu_sequential_transduction_attn_amd import _lib as ops
        ops.load_library()
        dev = torch.device("cuda:0")
        {"layers": lambda: extended(args, dev, layers_only=True), "cached": lambda: cached_scoring(dev),
         "attn_bwd": lambda: attn_backward(dev), "layer_bwd": lambda: layer_backward(dev),
         "layer_bwd_call": lambda: layer_backward(dev, train_step=False),
         "softmax": lambda: softmax_context(dev)}[args.only]()
        return
    run(args)


def calibrate_copy(nbytes: int = 256 << 20):
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 5}), flush=True)


if __name__ == "__main__":
    main()
