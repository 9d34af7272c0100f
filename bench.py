"""Decode-step benchmark: latent-KV decode attention on one MI355X.

A step is one pass of the hot path over the whole batch of one layer: the
latent append of the new token (h = x A into row len-1 of both caches),
then decode attention over the len rows (query absorption when applicable,
the context-split kernel, the split merge with the B_v up-projection), on one
stream. By default (--step combined) the step's work before the decode call
is one palu_latent_append_prepare call: the cache write, with the query
absorption as extra workgroups of the same launch (the query-side operands
do not depend on the cache); --step apart makes the append call and then a
decode call that forms its own operands; --step overlap forms them on a
second stream beside the append (palu_decode_attn_prepare), whose per-step
fork and join measured more than they hide.

Default workload: Llama-3-8B-shaped GQA (B=8, Hq=32, Hkv=8, d=128, 2 groups of
4 KV heads at rank 256, 32768 tokens of context, bf16 latents), absorbed-key
mode (no RoPE). The reconstruct+RoPE mode of the same shape is timed too and
reported beside it. Inputs are seeded synthetic tensors resident in HBM before
timing starts; several copies of the cache are rotated so that the 256 MB
Infinity Cache cannot serve the latents.

Prints ONE JSON line. Timing: W warm-up steps, then K steps between
torch.cuda.synchronize() calls, timed with events on the launch stream; each
timed loop follows untimed calls of the same work (at least W, about 40 ms of
GPU time: on this part the clocks take about 25 ms of continuous work to
settle). The main kernel is also timed alone with HIP events the library
records around it (palu_profile_begin/end), which gives the roofline
figure.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode steps/s + latent HBM GB/s (% peak), Llama-3-8B shape, 32K ctx"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
ROTATE_BYTES = 1.5 * 2 ** 30   # total size of the rotated cache copies


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--mode", default="absorbed", choices=["absorbed", "reconstruct"])
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip timing the other key mode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="rough CPU time budget of the oracle sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration runs)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="skip the second timed loop with events around the main kernel")
    ap.add_argument("--no-full-rank", action="store_true",
                    help="skip the uncompressed baseline (full bf16 K and V)")
    ap.add_argument("--step", default="combined", choices=["combined", "apart", "overlap"],
                    help="combined: palu_latent_append_prepare then the decode call; apart: "
                         "the append call, then a decode call forming its own operands; "
                         "overlap: the operands on a second stream beside the append")
    ap.add_argument("--a-layout", default="out_in", choices=["out_in", "in_out"],
                    help="memory layout of the dtype-cache step's projections a_k, a_v: "
                         "out_in = [G*r, d_model] (the nn.Linear weight layout, one-pass cache "
                         "write), in_out = [d_model, G*r]; the quantised steps take in_out")
    ap.add_argument("--no-quant", action="store_true",
                    help="skip the int8- and int4-latent absorbed steps")
    ap.add_argument("--profile-calls", type=int, default=0,
                    help="profiling run: copy 1 GiB on the device (the counters' "
                         "calibration), make this many decode calls of --config in --mode "
                         "(default split plan, no cache rotation) and exit; for rocprofv3 "
                         "counter passes")
    ap.add_argument("--profile-bits", type=int, default=0, choices=[0, 8, 4],
                    help="with --profile-calls: the int8 (8) or int4 (4) latent cache "
                         "(absorbed keys) instead of the dtype cache")
    ap.add_argument("--profile-hadamard", action="store_true",
                    help="with --profile-bits: a Hadamard-rotated cache")
    ap.add_argument("--profile-groups", type=int, default=0, choices=[0, 1, 2, 4, 8],
                    help="with --profile-calls: the head-grouping sweep's workload with "
                         "this many KV heads per group (the --config shape at 75%% key "
                         "compression) instead of --config itself")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the HBM read-stream probe")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the rebuilt-key rows of the other workloads (2, 4, 5)")
    ap.add_argument("--no-oracle-configs", action="store_true",
                    help="skip timing the oracle per workload and key mode")
    ap.add_argument("--no-sweep", dest="sweep", action="store_false",
                    help="skip the head-grouping sweep (s = 1, 2, 4, 8 KV heads per "
                         "group at 75%% key compression) and add it to the JSON line")
    return ap.parse_args()


def _r(x, n):
    """round, with None for a figure that was not measured"""
    return round(x, n) if math.isfinite(x) else None


def dev(torch, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


STEP = "combined"   # set by --step

WARM_MS = 40.0   # GPU work enqueued ahead of each timed loop


def warm_ahead(torch, stream, fn, n_min):
    """Enqueue untimed calls fn(i) on `stream` ahead of a timed loop, without
    waiting for them: at least n_min and about WARM_MS of GPU time (the
    per-call time is taken from three calls first). The GPU's clocks settle
    while it runs them (on this part a kernel reaches its steady rate after
    about 25 ms of continuous work), and meanwhile the host queues the timed
    calls, so the timed loop's events see back-to-back GPU execution rather
    than the host's first submissions."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(3):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    per_ms = max(1e-3, a.elapsed_time(b) / 3)
    for i in range(int(min(4000, max(n_min, math.ceil(WARM_MS / per_ms))))):
        fn(i)


def host_us(fn, n):
    """Host time of n calls of fn(i) (queued, not waited for), per call."""
    t0 = time.perf_counter()
    for i in range(n):
        fn(i)
    return (time.perf_counter() - t0) / max(1, n) * 1e6


def step_setup(torch, P, desc):
    """The prepared copy of a descriptor (decode calls after the query-side
    operands were formed) and, for --step overlap, the second stream."""
    pdesc = P.AttnDesc.from_buffer_copy(desc)
    pdesc.prepared = 1
    return pdesc, (torch.cuda.Stream() if STEP == "overlap" else None)


def time_mode(torch, P, W, cfg, t, mode, args, n_copies):
    """Returns dict with ms/step, kernel ms, and the output of the first step."""
    theta = cfg.rope_theta if mode == "reconstruct" else 0.0
    q, bk, bv = dev(torch, t["q"]), dev(torch, t["b_k"]), dev(torch, t["b_v"])
    lens = dev(torch, t["lens"])
    x, ak, av = dev(torch, t["x"]), dev(torch, t["a_k"]), dev(torch, t["a_v"])
    a_layout = P.PALU_A_OUT_IN if args.a_layout == "out_in" else P.PALU_A_IN_OUT
    if a_layout == P.PALU_A_OUT_IN:
        ak, av = ak.t().contiguous(), av.t().contiguous()
    pos = (lens - 1).to(torch.int32).contiguous()
    hk0, hv0 = dev(torch, t["h_k"]), dev(torch, t["h_v"])
    caches = [(hk0, hv0)] + [(hk0.clone(), hv0.clone()) for _ in range(n_copies - 1)]
    desc = P.attn_desc(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       head_dim=cfg.head_dim, n_groups=cfg.n_groups, rank=cfg.rank,
                       max_ctx=cfg.max_ctx, dtype=P.PALU_BF16 if cfg.dtype == "bf16" else P.PALU_F32,
                       mode=mode, rope_theta=theta, split_tokens=args.split_tokens)
    adesc = P.append_desc(batch=cfg.batch, d_model=cfg.d_model, n_groups=cfg.n_groups,
                          rank=cfg.rank, max_ctx=cfg.max_ctx, dtype=desc.dtype,
                          a_layout=a_layout)
    ws = torch.empty(P.palu_decode_attn_workspace(desc), dtype=torch.uint8, device="cuda")
    aws = torch.zeros(P.palu_latent_append_workspace(adesc), dtype=torch.uint8, device="cuda")
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device="cuda")
    n_split, split_tokens, kname = P.palu_decode_attn_plan(desc)
    stream = torch.cuda.current_stream()
    pdesc, side = step_setup(torch, P, desc)
    bkp = None if mode == "full_rank" else bk

    def step(i):
        hk, hv = caches[i % n_copies]
        if STEP == "apart":
            P.palu_latent_append(adesc, x, ak, av, hk, hv, pos, aws, stream)
            P.palu_decode_attn(desc, q, hk, hv, bk, bv, lens, out, ws, stream)
            return
        if STEP == "combined":
            P.palu_latent_append_prepare(adesc, 0, x, ak, av, hk, hv, None, None, pos, aws,
                                         desc, q, bkp, ws, stream)
            P.palu_decode_attn(pdesc, q, hk, hv, bk, bv, lens, out, ws, stream)
            return
        # the query-side operands on a second stream, under the cache write
        side.wait_stream(stream)
        P.palu_decode_attn_prepare(pdesc, q, bkp, ws, side)
        P.palu_latent_append(adesc, x, ak, av, hk, hv, pos, aws, stream)
        stream.wait_stream(side)
        P.palu_decode_attn(pdesc, q, hk, hv, bk, bv, lens, out, ws, stream)

    # the first step's output is kept for the sampled parity check (the append
    # has written row len-1 of copy 0)
    def decode(i):
        hk, hv = caches[i % n_copies]
        P.palu_decode_attn(desc, q, hk, hv, bk, bv, lens, out, ws, stream)

    step(0)
    torch.cuda.synchronize()
    first_out = out.clone()
    step_host = host_us(lambda i: step(i + 1), max(1, args.warmup))
    torch.cuda.synchronize()
    # timed loop 1: the steps alone (the throughput figure), behind the
    # warm-up work
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm_ahead(torch, stream, step, args.warmup)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    # timed loop 1b: the decode call alone (no cache write), the quantity the
    # pages compare with the uncompressed baseline
    call_host = host_us(decode, max(1, args.warmup))
    torch.cuda.synchronize()
    warm_ahead(torch, stream, decode, args.warmup)
    e0.record(stream)
    for i in range(args.steps):
        decode(i)
    e1.record(stream)
    torch.cuda.synchronize()
    decode_ms = e0.elapsed_time(e1)
    # timed loop 1c: each decode call between its own events, for the spread
    # (mean, median, p10, p90 of single calls)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    warm_ahead(torch, stream, decode, args.warmup)
    for i, (a, b_) in enumerate(ev):
        hk, hv = caches[i % n_copies]
        a.record(stream)
        P.palu_decode_attn(desc, q, hk, hv, bk, bv, lens, out, ws, stream)
        b_.record(stream)
    torch.cuda.synchronize()
    calls_us = np.array([a.elapsed_time(b_) * 1e3 for a, b_ in ev])
    # timed loop 2: the same steps with HIP events recorded by the library
    # around the main kernel on its launch stream (the roofline figure); the
    # event packets add a few microseconds between kernels, so this loop does
    # not give the step rate
    kern_ms, kern_n = float("nan"), 0
    if not args.no_kernel_events:
        warm_ahead(torch, stream, step, args.warmup)
        P.palu_profile_begin(args.steps)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        kern_ms, kern_n = P.palu_profile_end()
    return dict(ms_per_step=total_ms / args.steps, kernel_ms=kern_ms / max(1, kern_n),
                decode_ms=decode_ms / args.steps, calls_us=calls_us,
                host_us_per_step=step_host, host_us_per_call=call_host,
                kernel=kname, n_split=n_split, split_tokens=split_tokens,
                out=first_out.cpu().numpy())


def time_quant(torch, P, W, cfg, t, args, bits, rot=False):
    """The absorbed step over an int8 (bits 8) or int4 (bits 4) latent cache
    (codes plus one fp32 scale per row; rows Hadamard-rotated with rot):
    quantised append, then decode. Same shape, same timing loops."""
    ti = W.generate(cfg, parts=(f"i{bits}",))
    sfx = "" if bits == 8 else "_i4"
    q, bk, bv = dev(torch, t["q"]), dev(torch, t["b_k"]), dev(torch, t["b_v"])
    lens = dev(torch, t["lens"])
    x, ak, av = dev(torch, t["x"]), dev(torch, t["a_k"]), dev(torch, t["a_v"])
    pos = (lens - 1).to(torch.int32).contiguous()
    from rank_compressed_kv_amd.layout import pack_i4_cache, pack_i8_cache
    pack = pack_i8_cache if bits == 8 else pack_i4_cache
    bufs0 = [dev(torch, pack(ti[f"k_i{bits}"], "k")), dev(torch, pack(ti[f"v_i{bits}"], "v")),
             dev(torch, ti["sk" + sfx]), dev(torch, ti["sv" + sfx])]
    per_copy = sum(b.numel() * b.element_size() for b in bufs0)
    n_copies = min(16, max(1, int(math.ceil(ROTATE_BYTES / per_copy))))
    caches = [bufs0] + [[b.clone() for b in bufs0] for _ in range(n_copies - 1)]
    desc = P.attn_desc(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       head_dim=cfg.head_dim, n_groups=cfg.n_groups, rank=cfg.rank,
                       max_ctx=cfg.max_ctx, dtype=P.PALU_BF16, mode="absorbed",
                       split_tokens=args.split_tokens, hadamard=rot)
    adesc = P.append_desc(batch=cfg.batch, d_model=cfg.d_model, n_groups=cfg.n_groups,
                          rank=cfg.rank, max_ctx=cfg.max_ctx, dtype=P.PALU_BF16, hadamard=rot)
    ws = torch.empty(P.palu_decode_attn_workspace(desc), dtype=torch.uint8, device="cuda")
    append_ws = (P.palu_latent_append_i8_workspace if bits == 8
                 else P.palu_latent_append_i4_workspace)
    decode_fn = P.palu_decode_attn_i8 if bits == 8 else P.palu_decode_attn_i4
    append_fn = P.palu_latent_append_i8 if bits == 8 else P.palu_latent_append_i4
    aws = torch.zeros(append_ws(adesc), dtype=torch.uint8, device="cuda")
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    pdesc, side = step_setup(torch, P, desc)

    def decode(i):
        hk, hv, sk, sv = caches[i % n_copies]
        decode_fn(desc, q, hk, hv, sk, sv, bk, bv, lens, out, ws, stream)

    def step(i):
        hk, hv, sk, sv = caches[i % n_copies]
        if STEP == "apart":
            append_fn(adesc, x, ak, av, hk, hv, sk, sv, pos, aws, stream)
            decode(i)
            return
        if STEP == "combined":
            P.palu_latent_append_prepare(adesc, bits, x, ak, av, hk, hv, sk, sv, pos, aws, desc,
                                         q, bk, ws, stream)
            decode_fn(pdesc, q, hk, hv, sk, sv, bk, bv, lens, out, ws, stream)
            return
        side.wait_stream(stream)
        P.palu_decode_attn_prepare(pdesc, q, bk, ws, side)
        append_fn(adesc, x, ak, av, hk, hv, sk, sv, pos, aws, stream)
        stream.wait_stream(side)
        decode_fn(pdesc, q, hk, hv, sk, sv, bk, bv, lens, out, ws, stream)

    step(0)
    torch.cuda.synchronize()
    first = out.clone()
    for i in range(args.warmup):
        step(i + 1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn in (("step", step), ("decode", decode)):
        warm_ahead(torch, stream, fn, args.warmup)
        e0.record(stream)
        for i in range(args.steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / args.steps
    kern_ms, kern_n = float("nan"), 0
    if not args.no_kernel_events:
        warm_ahead(torch, stream, step, args.warmup)
        P.palu_profile_begin(args.steps)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        kern_ms, kern_n = P.palu_profile_end()
    del caches
    return dict(ms_per_step=res["step"], decode_ms=res["decode"],
                kernel_ms=kern_ms / max(1, kern_n), out=first.cpu().numpy(), ti=ti)


def time_full_rank(torch, P, W, cfg, t, args):
    """The uncompressed baseline at the same shape: full bf16 K and V
    [B, Hkv, L, d], keys cached rotated, one decode call per step."""
    tf = W.generate(cfg, parts=("full",))
    q, lens = dev(torch, t["q"]), dev(torch, t["lens"])
    k0, v0 = dev(torch, tf["k_full"]), dev(torch, tf["v_full"])
    kv_bytes = 2 * k0.numel() * k0.element_size()
    n_copies = max(1, int(math.ceil(ROTATE_BYTES / kv_bytes)))
    caches = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(n_copies - 1)]
    desc = P.attn_desc(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       head_dim=cfg.head_dim, n_groups=cfg.n_kv_heads, rank=cfg.head_dim,
                       max_ctx=cfg.max_ctx, dtype=P.PALU_BF16, mode="full_rank",
                       split_tokens=0)
    ws = torch.empty(P.palu_decode_attn_workspace(desc), dtype=torch.uint8, device="cuda")
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(i):
        k, v = caches[i % n_copies]
        P.palu_decode_attn(desc, q, k, v, None, None, lens, out, ws, stream)

    call(0)
    torch.cuda.synchronize()
    first = out.clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    warm_ahead(torch, stream, call, args.warmup)
    e0.record(stream)
    for i in range(args.steps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    warm_ahead(torch, stream, call, args.warmup)
    P.palu_profile_begin(args.steps)
    for i in range(args.steps):
        call(i)
    torch.cuda.synchronize()
    kern_ms, kern_n = P.palu_profile_end()
    bytes_ = 2 * int(np.sum(t["lens"], dtype=np.int64)) * cfg.n_kv_heads * cfg.head_dim * 2
    del caches
    return dict(ms=ms, kernel_ms=kern_ms / max(1, kern_n), bytes=bytes_, out=first.cpu().numpy(),
                k=tf["k_full"], v=tf["v_full"])


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16, published


def roofline(cfg, t, mode, res, lat_bytes, kern_gbs, traffic):
    """The main kernel against its bound: HBM for the absorbed keys (16 FLOP
    per latent byte); for rebuilt keys whichever of the latent bytes at 8 TB/s
    and the key-rebuild FLOPs (2 r D_g per token and group) at the dense bf16
    MFMA peak takes longer."""
    kus = res["kernel_ms"] * 1e3
    rec = {"bound": "hbm", "achieved": _r(kern_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": _r(kern_gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": res["kernel"],
           "kernel_us": _r(kus, 2), "algorithmic_bytes": lat_bytes,
           # the estimated times of the pages' roofline table: bytes at peak HBM
           # bandwidth (and, rebuilding keys, FLOPs at the dense MFMA peak)
           "ideal_us_hbm": _r(lat_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2)}
    if mode == "reconstruct":
        tokens = int(np.sum(t["lens"], dtype=np.int64))
        flops = 2.0 * tokens * cfg.n_groups * cfg.rank * cfg.group_dim
        rec["algorithmic_flops"] = flops
        rec["ideal_us_mfma"] = _r(flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6, 2)
        if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > lat_bytes / (HBM_PEAK_GBS * 1e9):
            tf = flops / (kus * 1e-6) / 1e12
            rec.update({"bound": "mfma", "achieved": _r(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": _r(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
    return rec


def reconstruct_configs(torch, P, W, O, args, which=(2, 4, 5)):
    """The rebuilt-key decode call at the other workloads' full sizes (MHA
    Llama-2-7B, the 128K-token outlier context, the ragged J-LRD batch): call
    time behind warm-up work, kernel time from the library's events, each
    against its roofline, and two sampled (b, h) outputs against the oracle.
    Caches are rotated over enough copies to defeat the Infinity Cache."""
    rows = {}
    for c in which:
        cfg = W.CONFIGS[c]
        t = W.generate(cfg, parts=("decode",))
        lat_bytes = W.latent_bytes(cfg, t["lens"])
        tokens = int(np.sum(t["lens"], dtype=np.int64))
        flops = 2.0 * tokens * cfg.n_groups * cfg.rank * cfg.group_dim
        n_copies = min(16, max(1, int(math.ceil(ROTATE_BYTES / lat_bytes))))
        q, bk, bv, lens = (dev(torch, t[k]) for k in ("q", "b_k", "b_v", "lens"))
        hk0, hv0 = dev(torch, t["h_k"]), dev(torch, t["h_v"])
        caches = [(hk0, hv0)] + [(hk0.clone(), hv0.clone()) for _ in range(n_copies - 1)]
        desc = P.attn_desc(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                           head_dim=cfg.head_dim, n_groups=cfg.n_groups, rank=cfg.rank,
                           max_ctx=cfg.max_ctx, dtype=P.PALU_BF16, mode="reconstruct",
                           rope_theta=cfg.rope_theta)
        ws = torch.empty(P.palu_decode_attn_workspace(desc), dtype=torch.uint8, device="cuda")
        out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32,
                          device="cuda")
        n_split, split_tokens, kname = P.palu_decode_attn_plan(desc)
        stream = torch.cuda.current_stream()

        def call(i):
            hk, hv = caches[i % n_copies]
            P.palu_decode_attn(desc, q, hk, hv, bk, bv, lens, out, ws, stream)

        call(0)
        torch.cuda.synchronize()
        first = out.cpu().numpy()
        n = max(5, args.steps // 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        warm_ahead(torch, stream, call, 3)
        e0.record(stream)
        for i in range(n):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        call_us = e0.elapsed_time(e1) / n * 1e3
        warm_ahead(torch, stream, call, 3)
        P.palu_profile_begin(n)
        for i in range(n):
            call(i)
        torch.cuda.synchronize()
        kms, kn = P.palu_profile_end()
        kus = kms / max(1, kn) * 1e3
        del caches, hk0, hv0
        torch.cuda.empty_cache()
        rng = np.random.default_rng(c)
        pairs = [(int(rng.integers(cfg.batch)), int(rng.integers(cfg.n_q_heads)))
                 for _ in range(2)]
        want = O.decode_attention(t["q"], t["h_k"], t["h_v"], t["b_k"], t["b_v"], t["lens"],
                                  rope_theta=cfg.rope_theta, select=pairs)
        idx = tuple(np.array(pairs).T)
        d = first.astype(np.float64)[idx] - want[idx]
        tf = flops / (kus * 1e-6) / 1e12
        gbs = lat_bytes / (kus * 1e-6) / 1e9
        mfma_bound = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > lat_bytes / (HBM_PEAK_GBS * 1e9)
        rows[f"cfg{c}"] = {
            "workload": f"{cfg.name}: B={cfg.batch} Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} "
                        f"d={cfg.head_dim} G={cfg.n_groups} r={cfg.rank} ctx={cfg.max_ctx}"
                        + (" ragged" if cfg.ragged else ""),
            "kernel": kname, "n_split": n_split, "split_tokens": split_tokens,
            "us_per_decode_call": round(call_us, 2), "kernel_us": round(kus, 2),
            "latent_bytes": lat_bytes, "rebuild_flops": flops,
            "ideal_us_hbm": round(lat_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
            "ideal_us_mfma": round(flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6, 2),
            "latent_GBps_kernel": round(gbs, 1), "rebuild_TFLOPs": round(tf, 1),
            "roofline": {"bound": "mfma" if mfma_bound else "hbm",
                         "frac": round(tf / MFMA_BF16_PEAK_TFLOPS if mfma_bound
                                       else gbs / HBM_PEAK_GBS, 4),
                         "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                         "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)},
            "sampled_parity_max_abs": float(np.abs(d).max()),
            "sampled_parity_rel_l2": float(np.linalg.norm(d) / np.linalg.norm(want[idx]))}
        print(f"[bench] cfg{c} reconstruct: {call_us:.1f} us/call, kernel {kname} {kus:.1f} us",
              file=sys.stderr, flush=True)
        del t
    return rows


def oracle_per_config(O, W, budget_s):
    """The oracle timed on the host per (workload, key mode): one (b, head
    group) pair at full context per configuration, scaled to a whole step;
    plus the whole of the tiny workload with one BLAS thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threadpool_limits, cores = None, os.cpu_count() or 1
    rows = {}
    for c, cfg in W.CONFIGS.items():
        # one sequence is enough: the oracle works pair by pair
        small = cfg.scaled(batch=1)
        t = W.generate(small, parts=("decode",))
        hpg = cfg.n_q_heads // cfg.n_groups
        for mode in cfg.modes:
            theta = cfg.rope_theta if mode == "reconstruct" else 0.0
            sel = [(0, i) for i in range(hpg)]
            t0 = time.perf_counter()
            O.decode_attention(t["q"], t["h_k"], t["h_v"], t["b_k"], t["b_v"], t["lens"],
                               rope_theta=theta, select=sel)
            el = time.perf_counter() - t0
            # a ragged workload's pairs cost in proportion to their length:
            # scale the sampled pair to the mean length of the range
            n0 = int(t["lens"][0])
            mean_len = (cfg.ragged[0] + cfg.ragged[1]) / 2 if cfg.ragged else n0
            pairs = cfg.batch * cfg.n_groups
            per_step = el * pairs * mean_len / max(1, n0)
            rows[f"cfg{c}_{mode}"] = {"s_per_pair": round(el, 4), "pair_len": n0,
                                      "pairs_per_step": pairs,
                                      "steps_per_s": round(1.0 / per_step, 6)}
            if el > budget_s:
                break
    one = None
    if threadpool_limits is not None:
        cfg = W.CONFIGS[1]
        t = W.generate(cfg)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            for mode in cfg.modes:
                O.decode_attention(t["q"], t["h_k"], t["h_v"], t["b_k"], t["b_v"], t["lens"],
                                   rope_theta=0.0)
            el = time.perf_counter() - t0
        one = {"cores": 1, "s_per_step_both_modes": round(el, 4),
               "steps_per_s_per_mode": round(len(cfg.modes) / el, 2)}
    return {"cores": int(cores), "kind": "oracle", "per_config": rows, "tiny_one_thread": one,
            "what": "one (batch, head-group) pair at full context per workload and key mode, "
                    "fp64 NumPy; steps/s = 1 / (seconds per pair x pairs per step)"}


def granularity_sweep(torch, P, W, cfg, args):
    """Decode-call time per head grouping at 75% key compression (r = D_g / 4):
    M-LRD s = 1 ... J-LRD s = Hkv, same total latent bytes; key-rebuild FLOPs
    grow with s. Both key modes; the reconstruct mode carries RoPE."""
    rows = []
    for s in (1, 2, 4, 8):
        if cfg.n_kv_heads % s:
            continue
        c = sweep_config(cfg, s)
        t = W.generate(c)
        lat_bytes = W.latent_bytes(c, t["lens"])
        tokens = int(np.sum(t["lens"], dtype=np.int64))
        flops = 2.0 * tokens * c.n_groups * c.rank * c.group_dim      # key rebuild
        q, bk, bv, lens = (dev(torch, t[k]) for k in ("q", "b_k", "b_v", "lens"))
        hk, hv = dev(torch, t["h_k"]), dev(torch, t["h_v"])
        del t
        row = {"s": s, "groups": c.n_groups, "rank": c.rank, "latent_bytes": lat_bytes,
               "rebuild_gflop": round(flops / 1e9, 2),
               "rebuild_flop_per_byte": round(flops / lat_bytes, 1),
               "ideal_us_hbm": round(lat_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
               "ideal_us_mfma_rebuild": round(flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6, 2)}
        for mode in ("absorbed", "reconstruct"):
            theta = c.rope_theta if mode == "reconstruct" else 0.0
            desc = P.attn_desc(batch=c.batch, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads,
                               head_dim=c.head_dim, n_groups=c.n_groups, rank=c.rank,
                               max_ctx=c.max_ctx, dtype=P.PALU_BF16, mode=mode, rope_theta=theta)
            ws = torch.empty(P.palu_decode_attn_workspace(desc), dtype=torch.uint8, device="cuda")
            out = torch.empty(c.batch, c.n_q_heads, c.head_dim, dtype=torch.float32, device="cuda")
            _, _, kname = P.palu_decode_attn_plan(desc)
            stream = torch.cuda.current_stream()
            n = max(5, args.steps // 4)
            warm_ahead(torch, stream, lambda i: P.palu_decode_attn(desc, q, hk, hv, bk, bv, lens,
                                                                   out, ws, stream), 3)
            P.palu_profile_begin(n)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                P.palu_decode_attn(desc, q, hk, hv, bk, bv, lens, out, ws, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            kms, kn = P.palu_profile_end()
            kus = kms / max(1, kn) * 1e3
            call_us = e0.elapsed_time(e1) / n * 1e3
            entry = {"kernel": kname, "call_us": round(call_us, 2), "kernel_us": round(kus, 2),
                     "latent_GBps_kernel": round(lat_bytes / (kus * 1e-6) / 1e9, 1)}
            if mode == "reconstruct":
                tf = flops / (kus * 1e-6) / 1e12
                entry["rebuild_TFLOPs"] = round(tf, 1)
                ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
                entry["roofline_bound"] = "mfma" if flops / lat_bytes > ridge else "hbm"
            row[mode] = entry
        rows.append(row)
        print(f"[sweep] s={s} r={c.rank}: absorbed {row['absorbed']['kernel_us']} us, "
              f"reconstruct {row['reconstruct']['kernel_us']} us", file=sys.stderr, flush=True)
        del q, bk, bv, lens, hk, hv
        torch.cuda.empty_cache()
    return rows


def sweep_config(cfg, s):
    """The head-grouping sweep's workload: cfg's shape with s KV heads a group
    and rank s * d / 4 (75% key compression at every grouping)."""
    return cfg.scaled(n_groups=cfg.n_kv_heads // s, rank=s * cfg.head_dim // 4, seed=60 + s)


def profile_calls(torch, P, W, cfg, args):
    """The decode call of one workload, made --profile-calls times on one
    cache (for counter passes: every call of the main kernel is the same
    work), after a 1 GiB device copy that calibrates the HBM byte counters;
    prints the plan."""
    src = torch.empty(2 ** 28, dtype=torch.float32, device="cuda").fill_(1.0)
    torch.empty_like(src).copy_(src)
    torch.cuda.synchronize()
    del src
    bits = args.profile_bits
    mode = "absorbed" if bits else args.mode
    t = W.generate(cfg, parts=("decode",) + ((f"i{bits}",) if bits else ()))
    theta = cfg.rope_theta if mode == "reconstruct" else 0.0
    q, bk, bv, lens = (dev(torch, t[k]) for k in ("q", "b_k", "b_v", "lens"))
    desc = P.attn_desc(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       head_dim=cfg.head_dim, n_groups=cfg.n_groups, rank=cfg.rank,
                       max_ctx=cfg.max_ctx, dtype=P.PALU_BF16 if cfg.dtype == "bf16" else P.PALU_F32,
                       mode=mode, rope_theta=theta, split_tokens=args.split_tokens,
                       hadamard=bool(bits and args.profile_hadamard))
    ws = torch.empty(P.palu_decode_attn_workspace(desc), dtype=torch.uint8, device="cuda")
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device="cuda")
    if bits:
        from rank_compressed_kv_amd.layout import pack_i4_cache, pack_i8_cache
        pack = pack_i8_cache if bits == 8 else pack_i4_cache
        sfx = "" if bits == 8 else "_i4"
        hk, hv = dev(torch, pack(t[f"k_i{bits}"], "k")), dev(torch, pack(t[f"v_i{bits}"], "v"))
        sk, sv = dev(torch, t["sk" + sfx]), dev(torch, t["sv" + sfx])
        fn = P.palu_decode_attn_i8 if bits == 8 else P.palu_decode_attn_i4
        call = lambda: fn(desc, q, hk, hv, sk, sv, bk, bv, lens, out, ws)
    else:
        hk, hv = dev(torch, t["h_k"]), dev(torch, t["h_v"])
        call = lambda: P.palu_decode_attn(desc, q, hk, hv, bk, bv, lens, out, ws)
    for _ in range(args.profile_calls):
        call()
    torch.cuda.synchronize()
    ns, st, kname = P.palu_decode_attn_plan(desc)
    what = f"int{bits}{' hadamard' if args.profile_hadamard else ''}" if bits else cfg.dtype
    print(f"[profile] cfg{args.config} {cfg.name} {mode} {what}: {args.profile_calls} calls, "
          f"n_split {ns}, split_tokens {st}, latent bytes {W.latent_bytes(cfg, t['lens'])}",
          flush=True)


def read_stream_probe(torch):
    """The HBM read rate a plain streaming kernel reaches here (libpalu_probe:
    16-byte non-temporal loads, one contiguous chunk per workgroup): the best
    of a few launch shapes over a 1 GiB buffer, ten launches each."""
    import ctypes
    path = os.path.join(ROOT, "rank_compressed_kv_amd", "libpalu_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.palu_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p]
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    out = torch.empty(65536, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = None
    for grid in (256, 512, 1024, 2048):
        for threads in (256, 512):
            for inflight in (4, 8, 16):
                call = lambda: lib.palu_probe_read_stream(buf.data_ptr(), nbytes, out.data_ptr(),
                                                          grid, threads, inflight,
                                                          stream.cuda_stream)
                if call() != 0:
                    continue
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(10):
                    call()
                e1.record(stream)
                torch.cuda.synchronize()
                gbs = 10 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
                if best is None or gbs > best["GBps"]:
                    best = {"GBps": round(gbs, 1), "grid": grid, "threads": threads,
                            "loads_in_flight_per_thread": inflight}
    del buf, out
    torch.cuda.empty_cache()
    if best:
        best["frac_of_published_peak"] = round(best["GBps"] / HBM_PEAK_GBS, 4)
        best["what"] = ("1 GiB read once per launch with 16-byte non-temporal loads, "
                        "best launch shape of 24")
    return best


def oracle_appended(O, cfg, t, caches, rot=False, bits=8):
    """The caches as the oracle has them after one step's append: row len-1 of
    each sequence replaced by the oracle's own cache write of x A (bf16: the
    exact row rounded to fp32, then to bf16; int8 / int4 (bits): its
    quantisation, of the Hadamard-rotated row with rot)."""
    if bits == 8:
        quant = O.append_rows_i8_hadamard if rot else O.append_rows_i8
    else:
        quant = O.append_rows_i4_hadamard if rot else O.append_rows_i4
    B, G, r = cfg.batch, cfg.n_groups, cfg.rank
    out = []
    for cache, a in zip(caches, ("a_k", "a_v")):
        h64 = O.latent_project(t["x"], t[a]).reshape(B, G, r)
        if isinstance(cache, tuple):                    # (codes, scales)
            codes, scales = cache[0].copy(), cache[1].copy()
            for b in range(B):
                p = int(t["lens"][b]) - 1
                if p >= 0:
                    codes[b, :, p], scales[b, :, p] = quant(h64[b])
            out.append((codes, scales))
            continue
        c = cache.copy()
        for b in range(B):
            p = int(t["lens"][b]) - 1
            if p >= 0:
                c[b, :, p] = (O.append_rows_bf16(h64[b]) if cfg.dtype == "bf16"
                              else h64[b].astype(np.float32))
        out.append(c)
    return out


def sampled_parity(O, cfg, t, res, mode, pairs):
    """Compare sampled (b, h) outputs of the first timed step with the oracle
    on the cache after its own append of the step's token."""
    theta = cfg.rope_theta if mode == "reconstruct" else 0.0
    hk, hv = oracle_appended(O, cfg, t, (t["h_k"], t["h_v"]))
    want = O.decode_attention(t["q"], hk, hv, t["b_k"], t["b_v"], t["lens"], rope_theta=theta,
                              select=pairs)
    got = res["out"].astype(np.float64)
    idx = tuple(np.array(pairs).T)
    d = got[idx] - want[idx]
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(want[idx]))


def cpu_baseline(O, cfg, t, mode, budget_s):
    """Time the oracle on the host cores on a bounded sample of the workload:
    whole (b, g) pairs (all their query heads) in order, over repeated steps
    when one step takes less than the budget, until the budget is spent."""
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    theta = cfg.rope_theta if mode == "reconstruct" else 0.0
    heads_per_group = cfg.n_q_heads // cfg.n_groups
    pairs_total = cfg.batch * cfg.n_groups
    done, t0 = 0, time.perf_counter()
    while True:
        b, g = divmod(done % pairs_total, cfg.n_groups)
        sel = [(b, g * heads_per_group + i) for i in range(heads_per_group)]
        O.decode_attention(t["q"], t["h_k"], t["h_v"], t["b_k"], t["b_v"], t["lens"],
                           rope_theta=theta, select=sel)
        done += 1
        el = time.perf_counter() - t0
        if el > budget_s:
            break
    steps = done / pairs_total
    return {"value": steps / el, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} (batch, head-group) pairs, {pairs_total} to a step "
                      f"({steps:.2f} steps; {heads_per_group} query heads a pair), "
                      f"fp64 NumPy, {el:.1f} s; steps/s = steps / seconds"}


def load_traffic(kernel: str, args_suffix: str = "", label: str = ""):
    """HBM bytes (read + write) per launch of a kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE passes (scaled by a 1 GiB copy measured in
    the same runs; rank_compressed_kv_amd.profiling writes the record). The
    records are keyed by kernel name with template arguments: the one whose
    name is `kernel`, whose arguments end with args_suffix and whose label
    (the variant a pass ran, e.g. "hadamard"; none for the plain one) is
    `label` is taken. None
    when there is no single such record or when the kernel's sources have
    changed since its counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        hits = [v for key, v in rec["kernels"].items()
                for name, lab in [key.split(" | ") if " | " in key else (key, "")]
                if name.split("<")[0] == kernel and name.endswith(args_suffix) and lab == label]
        if len(hits) != 1 or not hits[0].get("sources"):
            return None
        h = hashlib.sha256()
        for rel in hits[0]["sources"]:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != hits[0]["sources_sha256"]:
            return None
        return round(hits[0]["bytes"])
    except Exception:
        return None


def main():
    global STEP
    args = parse()
    STEP = args.step
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the library has no multi-GPU path); "
              f"got --gpus {args.gpus}", file=sys.stderr)
        sys.exit(2)
    import torch
    import rank_compressed_kv_amd as P
    import workloads as W
    if not os.path.exists(P.library_path()):
        from rank_compressed_kv_amd import build
        build.build()
    P.library()
    torch.cuda.set_device(0)

    cfg = W.CONFIGS[args.config]
    if args.profile_calls:
        if args.profile_groups:
            cfg = sweep_config(cfg, args.profile_groups)
        profile_calls(torch, P, W, cfg, args)
        return
    t = W.generate(cfg, parts=("decode", "append"))
    # the append writes row len-1, so the step attends over exactly len rows
    lat_bytes = W.latent_bytes(cfg, t["lens"])
    # enough copies to defeat the 256 MB Infinity Cache (at most 16: a tiny
    # workload is launch-bound whatever the cache holds)
    n_copies = min(16, max(1, int(math.ceil(ROTATE_BYTES / lat_bytes))))
    print(f"[bench] cfg{args.config} {cfg.name}: latent bytes/step {lat_bytes}, "
          f"{n_copies} cache copies", file=sys.stderr, flush=True)

    if args.copy_probe:
        src = torch.empty(2 ** 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    modes = [args.mode]
    if not args.no_secondary:
        modes += [m for m in cfg.modes if m != args.mode]
    results = {}
    for mode in modes:
        res = time_mode(torch, P, W, cfg, t, mode, args, n_copies)
        results[mode] = res
        print(f"[bench] {mode}: {res['ms_per_step'] * 1e3:.1f} us/step, main kernel "
              f"{res['kernel']} {res['kernel_ms'] * 1e3:.1f} us", file=sys.stderr, flush=True)

    from oracle import palu_oracle as O
    rng = np.random.default_rng(0)
    pairs = [(int(rng.integers(cfg.batch)), int(rng.integers(cfg.n_q_heads))) for _ in range(4)]
    parity = {}
    for mode in modes:
        parity[mode] = sampled_parity(O, cfg, t, results[mode], mode, pairs)
    main_res = results[args.mode]
    full = None
    if not args.no_full_rank and cfg.dtype == "bf16":
        fr = time_full_rank(torch, P, W, cfg, t, args)
        want = O.full_rank_attention(t["q"], fr["k"], fr["v"], t["lens"], select=pairs)
        idx = tuple(np.array(pairs).T)
        dd = fr["out"].astype(np.float64)[idx] - want[idx]
        dec_ms = results["absorbed"]["decode_ms"] if "absorbed" in results else None
        full = {"us_per_call": round(fr["ms"] * 1e3, 2),
                "kernel_us": _r(fr["kernel_ms"] * 1e3, 2),
                "kv_bytes": fr["bytes"],
                "GBps_kernel": _r(fr["bytes"] / (fr["kernel_ms"] * 1e-3) / 1e9, 1),
                "sampled_parity_max_abs": float(np.abs(dd).max()),
                "palu_absorbed_speedup_decode_call": (round(fr["ms"] / dec_ms, 3)
                                                      if dec_ms else None)}
        print(f"[bench] full-rank baseline: {fr['ms'] * 1e3:.1f} us/call, kernel "
              f"{fr['kernel_ms'] * 1e3:.1f} us", file=sys.stderr, flush=True)

    quant = None
    if not args.no_quant and cfg.dtype == "bf16" and "absorbed" in results and \
            cfg.rank in (64, 128, 256) and cfg.max_ctx % 32 == 0:
        quant = {}
        ntok = int(np.sum(t["lens"], dtype=np.int64))
        for bits in (8, 4):
            # codes of both matrices plus the two fp32 scales of every row
            qbytes = ntok * cfg.n_groups * (2 * cfg.rank * bits // 8 + 8)
            entry = {"algorithmic_bytes": qbytes}
            sfx = "" if bits == 8 else "_i4"
            for rot in (False, True):
                ri = time_quant(torch, P, W, cfg, t, args, bits, rot)
                ti = ri.pop("ti")
                (ck, sk), (cv, sv) = oracle_appended(
                    O, cfg, t, ((ti[f"k_i{bits}"], ti["sk" + sfx]),
                                (ti[f"v_i{bits}"], ti["sv" + sfx])), rot, bits)
                deq = O.dequantize_rows_i8_hadamard if rot else O.dequantize_rows_i8
                # the oracle dequantises only the sampled sequences
                dmax, num, den = 0.0, 0.0, 0.0
                for b, h in pairs:
                    w = O.decode_attention(t["q"][b:b + 1], deq(ck[b:b + 1], sk[b:b + 1]),
                                           deq(cv[b:b + 1], sv[b:b + 1]), t["b_k"], t["b_v"],
                                           t["lens"][b:b + 1], select=[(0, h)])[0, h]
                    dd = ri["out"][b, h].astype(np.float64) - w
                    dmax = max(dmax, float(np.abs(dd).max()))
                    num, den = num + float(dd @ dd), den + float(w @ w)
                kus = ri["kernel_ms"] * 1e3
                entry["hadamard" if rot else "plain"] = {
                    "us_per_step": round(ri["ms_per_step"] * 1e3, 2),
                    "us_per_decode_call": round(ri["decode_ms"] * 1e3, 2),
                    "kernel_us": _r(kus, 2),
                    "GBps_kernel": _r(qbytes / (kus * 1e-6) / 1e9, 1),
                    "frac_hbm_kernel": _r(qbytes / (kus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "step_speedup_vs_bf16": round(results["absorbed"]["ms_per_step"]
                                                  / ri["ms_per_step"], 3),
                    "traffic": load_traffic("split_absorbed_int_kernel", f", {bits}>",
                                            "hadamard" if rot else ""),
                    "sampled_parity_max_abs": dmax,
                    "sampled_parity_rel_l2": math.sqrt(num / den) if den > 0 else None}
                print(f"[bench] int{bits} absorbed{' hadamard' if rot else ''}: "
                      f"{ri['ms_per_step'] * 1e3:.1f} us/step, kernel {kus:.1f} us",
                      file=sys.stderr, flush=True)
            quant[f"int{bits}"] = entry

    ms = main_res["ms_per_step"]
    steps_s = 1e3 / ms
    gbs_step = lat_bytes / (ms * 1e-3) / 1e9
    kern_gbs = lat_bytes / (main_res["kernel_ms"] * 1e-3) / 1e9
    traffic = load_traffic(main_res["kernel"])
    line = {
        "metric": METRIC,
        "value": round(steps_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) bf16 latents, B ~ N(0,1/r)), no weights",
        "config": {"workload": f"{cfg.name} {args.mode}: B={cfg.batch} Hq={cfg.n_q_heads} "
                               f"Hkv={cfg.n_kv_heads} d={cfg.head_dim} G={cfg.n_groups} "
                               f"r={cfg.rank} ctx={cfg.max_ctx}",
                   "global_batch": cfg.batch, "seq_len": cfg.max_ctx, "parallelism": "none (1 GPU)",
                   "step": {"combined": "cache write with the query-side operands in the "
                                        "same call (palu_latent_append_prepare), then the "
                                        "decode call",
                            "apart": "cache write, then the decode call (one stream)",
                            "overlap": "cache write, with the query-side operands formed on a "
                                       "second stream beside it, then the decode call"}[STEP]
                           + ("; a_k, a_v stored [G*r, d_model]" if args.a_layout == "out_in"
                              else "; a_k, a_v stored [d_model, G*r]"),
                   "mode": args.mode, "n_split": main_res["n_split"],
                   "split_tokens": main_res["split_tokens"]},
        "latent_GBps": round(gbs_step, 1),
        "latent_pct_hbm_peak": round(100 * gbs_step / HBM_PEAK_GBS, 2),
        "roofline": roofline(cfg, t, args.mode, main_res, lat_bytes, kern_gbs, traffic),
        "full_rank_baseline": full,
        "quantised_latents": quant,
        "timing": "each timed loop (and each kernel-event loop) follows untimed calls of "
                  "the same work, at least W and about 40 ms of GPU time, enqueued without "
                  "waiting: the clocks settle during them and the host queues the timed "
                  "calls meanwhile, so the events time back-to-back GPU execution at the "
                  "steady clock rate; host_us_* is the binding's submission time per step "
                  "or call",
        "modes": {m: {"us_per_step": round(r["ms_per_step"] * 1e3, 2),
                      "us_per_decode_call": round(r["decode_ms"] * 1e3, 2),
                      "host_us_per_step": round(r["host_us_per_step"], 1),
                      "host_us_per_decode_call": round(r["host_us_per_call"], 1),
                      "decode_call_us_spread": {
                          "mean": round(float(np.mean(r["calls_us"])), 2),
                          "median": round(float(np.median(r["calls_us"])), 2),
                          "p10": round(float(np.percentile(r["calls_us"], 10)), 2),
                          "p90": round(float(np.percentile(r["calls_us"], 90)), 2)},
                      "kernel_us": _r(r["kernel_ms"] * 1e3, 2), "kernel": r["kernel"],
                      "latent_GBps_kernel": _r(lat_bytes / (r["kernel_ms"] * 1e-3) / 1e9, 1),
                      "sampled_parity_max_abs": parity[m][0],
                      "sampled_parity_rel_l2": parity[m][1]}
                  for m, r in results.items()},
    }
    if not args.no_probe:
        probe = read_stream_probe(torch)
        if probe:
            probe["main_kernel_frac_of_probe"] = round(kern_gbs / probe["GBps"], 4)
        line["read_stream_probe"] = probe
    if not args.no_configs:
        line["reconstruct_other_workloads"] = reconstruct_configs(torch, P, W, O, args)
    if args.sweep:
        line["granularity_sweep"] = granularity_sweep(torch, P, W, cfg, args)
    if not args.no_cpu_baseline and not args.no_oracle_configs:
        line["oracle_per_workload"] = oracle_per_config(O, W, args.cpu_seconds)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(O, cfg, t, args.mode, args.cpu_seconds)
        line["gpu_over_cpu_baseline"] = round(line["value"] / line["cpu_baseline"]["value"], 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
