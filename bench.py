#!/usr/bin/env python3
"""Benchmark of the KV coder hot path on one MI355X.

One step = kvc_encode then kvc_decode of the whole Qwen3-8B-shaped bf16 KV
cache (36 layers x {K,V} x batch 4 x 8 KV heads x 4096 tokens x 128
channels = 1.21G scalars, 2.42 GB) under the pages' three-part mixture, with
sigma calibrated per (layer, kv, head, channel) from 128 x 1024 held-out
tokens and p_hat from 2^20 samples.  Inputs are resident in HBM when timing
starts; generation, calibration and the marginal are not timed.

Prints one JSON line.  value = raw-KV GB/s of the round trip
(2 bytes x scalars / (encode + decode time)); encode and decode GB/s,
bits/scalar three ways, the dominant kernel's HBM roofline fraction and the
CPU oracle's rate on a bounded sample are reported beside it.
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["entropy_coding_amd/csrc/kvc_kernels.hip", "entropy_coding_amd/csrc/kvc_device.hpp",
                  "entropy_coding_amd/csrc/kvc_internal.hpp"]
TRAFFIC_FILE = "profiles/traffic_qwen3-8b_bf16.txt"
VALU_FILE = "profiles/valu_k_encode_k_decode_qwen3-8b_bf16.md"
# plain-ALU peak: one wave64 vector instruction per CU per cycle
# (4 SIMD16 units, 4 cycles each) at 2.4 GHz on 256 CUs, in lane-ops/s
ALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of each coding kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE passes, each scaled by what the same
    counter reads for a copy of known size), or {} when the summary is
    missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return {}
    out, sha = {}, None
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and parts[0] == "kernel_sources_sha256":
                sha = parts[1]
            elif len(parts) >= 3 and parts[0] == "traffic":
                kv = dict(p.split("=", 1) for p in parts[2:])
                out[parts[1]] = {k: float(v) for k, v in kv.items()}
    return out if sha == kernel_sources_sha256() else {}


def measured_valu():
    """VALU instructions per wave step (one token of one 64-lane chunk) of
    each coding kernel from the committed counter summary, or {} when it is
    missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, VALU_FILE)
    if not os.path.exists(path):
        return {}
    out, sha = {}, None
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and parts[0] == "kernel_sources_sha256":
                sha = parts[1]
            elif len(parts) == 3 and parts[0] == "valu":
                out[parts[1]] = float(parts[2].split("=", 1)[1])
    return out if sha == kernel_sources_sha256() else {}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# CPU oracle baseline (runs before the GPU is touched; plain fork pool)
# ---------------------------------------------------------------------------
def _oracle_worker(args):
    """One worker's share: half the planes of one layer at the workload's
    full token count and chunk length, drawn on the host with the same
    recipe; returns (encode s, decode s, scalars, stream bytes)."""
    import numpy as np
    import torch
    import oracle as O
    from entropy_coding_amd import workloads as W
    wid, layer, half, tc = args
    torch.set_num_threads(1)
    w = W.WORKLOADS[wid]
    kv, mu = W.layer_data(w, layer, device="cpu")
    sig = W.layer_sigma_true(w, layer, device="cpu")
    pref = O.build_marginal(W.to_numpy_bits(W.marginal_samples(w, device="cpu")), O.BF16,
                            w.w_narrow_bp, w.w_wide_bp)
    g = kv.shape[0] // 2
    sel = slice(half * g, (half + 1) * g)
    kvn, mun, sgn = W.to_numpy_bits(kv[sel]), W.to_numpy_bits(mu[sel]), sig[sel].numpy()
    del kv, mu
    t0 = time.perf_counter()
    st = O.encode(kvn, mun, sgn, pref, O.BF16, O.BF16, w.w_narrow_bp, w.w_wide_bp, tc)
    t1 = time.perf_counter()
    out = O.decode(st, mun, sgn, pref)
    t2 = time.perf_counter()
    assert np.array_equal(out, kvn)
    return t1 - t0, t2 - t1, kvn.size, len(st)


def cpu_baseline(workload, workers: int = 0):
    """The oracle, as it stands, on a bounded sample of the same workload:
    each worker codes and decodes half the planes of one layer (32 planes of
    4096 tokens x 128 channels, 448 chunks of the workload's chunk length,
    coded by the oracle in one batch), one worker per host core.  The rate
    is the sample's raw bytes over the slowest worker's encode and decode
    time (the pool's parallel time; the host-side data generation in each
    worker is not timed)."""
    cores = len(os.sched_getaffinity(0))
    n_workers = workers or cores
    jobs = [(workload.cid, i // 2 % workload.layers, i % 2, workload.chunk_tokens) for i in range(n_workers)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(n_workers) as pool:
        res = pool.map(_oracle_worker, jobs)
    wall = time.perf_counter() - t0
    n = sum(r[2] for r in res)
    enc = max(r[0] for r in res)
    dec = max(r[1] for r in res)
    rt = max(r[0] + r[1] for r in res)
    raw = 2.0 * n
    per = res[0][2] // (workload.tokens * workload.channels)
    return {
        "value": raw / rt / 1e9, "unit": "GB/s", "cores": n_workers, "kind": "oracle",
        "sample": f"{n} scalars: {n_workers} workers, each {per} planes x {workload.tokens} tokens x "
                  f"{workload.channels} channels of one layer (same recipe drawn on the host), "
                  f"{workload.chunk_tokens}-token chunks coded in one batch; encode+decode round trip, "
                  f"slowest worker {rt:.2f} s (pool wall {wall:.2f} s)",
        "encode_gbps": raw / enc / 1e9, "decode_gbps": raw / dec / 1e9,
    }


# ---------------------------------------------------------------------------
# GPU run
# ---------------------------------------------------------------------------
def prepare(workload, dev, calib_reps: int, sigma_block: int = 0, sigma_fit: str = "rms", narrow_dof: int = 0,
            channel_split: bool = False):
    import torch
    from entropy_coding_amd import kvc
    from entropy_coding_amd import workloads as W

    w = workload
    G, T, D = w.planes, w.tokens, w.channels
    kv = torch.empty((G, T, D), dtype=torch.bfloat16 if w.kv_dtype == W.BF16 else torch.uint8, device=dev)
    mu = torch.empty((G, T, D), dtype=torch.bfloat16 if w.mu_dtype == W.BF16 else torch.float32, device=dev)
    if sigma_block and w.calib_tokens < T:
        raise SystemExit("sigma blocks need calibration data over every position (calib_tokens = tokens)")
    sigma = torch.empty(kvc.sigma_shape(G, T, D, sigma_block), dtype=torch.float32, device=dev)
    split = torch.empty((G, D), dtype=torch.int32, device=dev) if channel_split else None
    ppl = w.planes_per_layer
    t0 = time.perf_counter()
    prefix = kvc.kvc_build_marginal(W.marginal_samples(w, device=dev), (w.w_narrow_bp, w.w_wide_bp))
    for l in range(w.layers):
        k_l, m_l = W.layer_data(w, l, device=dev)
        kv[l * ppl:(l + 1) * ppl] = k_l
        mu[l * ppl:(l + 1) * ppl] = m_l
        del k_l, m_l
        ck, cm = W.layer_calibration(w, l, reps=calib_reps, device=dev)
        if sigma_fit == "rate":
            s_kvh = kvc.kvc_calibrate_sigma_rate(ck, cm, prefix, (w.w_narrow_bp, w.w_wide_bp), block_tokens=sigma_block,
                                                 narrow_dof=narrow_dof)
        else:
            s_kvh = kvc.kvc_calibrate_sigma(ck, cm, block_tokens=sigma_block)
        sigma[l * ppl:(l + 1) * ppl] = W.expand_sigma(w, s_kvh)
        if split is not None:
            # each (kv, head, channel)'s narrow weight, fitted under that sigma
            w_kvh = kvc.kvc_calibrate_split(ck, cm, s_kvh, prefix, (w.w_narrow_bp, w.w_wide_bp),
                                            block_tokens=sigma_block, narrow_dof=narrow_dof)
            split[l * ppl:(l + 1) * ppl] = W.expand_sigma(w, w_kvh)
        del ck, cm
    torch.cuda.synchronize()
    log(f"[bench] generated {w.name}: {w.n_scalars} scalars, sigma ({sigma_fit}) from {calib_reps}x{w.calib_tokens} "
        f"tokens per layer{', per-channel weights' if split is not None else ''}, in {time.perf_counter() - t0:.1f} s")
    return kv, mu, sigma, prefix, split


def offload_reload(w, kv, mu, side, prefix, kvc, enc, parts, dws, steps: int):
    """Host-offload reload, one layer per call: every layer's stream sits in
    pinned host memory; the copy of layer l+1 to the device (its own stream)
    overlaps the decode of layer l.  Compared with copying the raw layers."""
    import torch
    dev = kv.device
    streams = []
    for i, sl in enumerate(parts):
        streams.append(enc(kv[sl], mu[sl], side[i], prefix).cpu())
    sizes = [s.numel() for s in streams]
    offs = [0]
    for n in sizes:
        offs.append(offs[-1] + n)
    host = torch.empty(offs[-1], dtype=torch.uint8, pin_memory=True)
    for s, o in zip(streams, offs):
        host[o:o + s.numel()].copy_(s)
    del streams
    out = torch.empty_like(kv, dtype=torch.int16 if kv.dtype == torch.bfloat16 else torch.uint8)
    layers = [host[o:o + n] for o, n in zip(offs[:-1], sizes)]
    g = parts[0].stop - parts[0].start
    mu_l = mu.view(len(parts), g, *mu.shape[1:])
    sig_l = torch.stack(side)                         # each layer's side buffer (sigma, weights)
    out_l = out.view(len(parts), g, *out.shape[1:])
    half = (max(sizes) + 511) // 256 * 256
    staging = torch.empty(2 * half, dtype=torch.uint8, device=dev)
    rws = torch.empty(len(parts) * kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    copy_stream = torch.cuda.Stream(device=dev)

    def reload():
        # the library's pipeline: H2D copies on copy_stream overlapping the
        # decode of the layer before
        rc, failed = kvc.kvc_reload(layers, mu_l, sig_l, prefix, out_l, staging, rws, copy_stream=copy_stream)
        if rc != kvc.KVC_OK:
            raise kvc.KvcError(rc, f"kvc_reload (layer {failed})")

    reload()
    t0 = time.perf_counter()
    for _ in range(steps):
        reload()
    t_comp = (time.perf_counter() - t0) / steps
    if not torch.equal(out, kv.view(out.dtype)):
        raise SystemExit("offload reload decoded wrong KV")
    # the same layers moved raw: one pinned layer copied per layer
    raw_layer = kv[parts[0]].numel() * kv.element_size()
    host_raw = torch.empty(raw_layer, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(raw_layer, dtype=torch.uint8, device=dev)
    dst.copy_(host_raw, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for _l in parts:
            dst.copy_(host_raw, non_blocking=True)
        torch.cuda.synchronize()
    t_raw = (time.perf_counter() - t0) / steps
    raw_total = float(raw_layer) * len(parts)
    return {
        "metric": f"host-offload reload of {w.name}, one layer per call: GB/s of raw KV delivered to HBM",
        "value": raw_total / t_comp / 1e9, "unit": "GB/s", "steps": steps,
        "compressed_ms": t_comp * 1e3, "raw_copy_ms": t_raw * 1e3, "raw_copy_gbps": raw_total / t_raw / 1e9,
        "speedup_vs_raw_copy": t_raw / t_comp, "stream_bytes": offs[-1], "raw_bytes": raw_total,
        "bits_per_scalar": 8.0 * offs[-1] / w.n_scalars,
        "pipeline": "kvc_reload: pinned host streams -> H2D copies on their own stream, each overlapping the decode "
                    "of the layer before",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2,
                    help="workload id: 2 = the bench line; 1 and 3 code the whole cache in one call, 4 one layer per call")
    ap.add_argument("--calib-reps", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=0, help="oracle workers (0 = one per host core)")
    ap.add_argument("--chunk-tokens", type=int, default=None, help="override the workload's chunk length")
    ap.add_argument("--offload", action="store_true",
                    help="(per-layer workload 4) also time the host-offload reload: pinned streams, copies overlapped with decode")
    ap.add_argument("--sigma-block", type=int, default=0,
                    help="position-aware sigma: one sigma per block of this many tokens (0 = per plane)")
    ap.add_argument("--sigma-fit", choices=["rms", "rate"], default="rms",
                    help="sigma calibration: the RMS of the residual, or the scale fitted to the code length")
    ap.add_argument("--streams", type=int, default=2,
                    help="(per-layer workload 4) HIP streams the asynchronous one-layer encode calls are spread "
                         "over; 1 = synchronous calls one after another")
    ap.add_argument("--decode-streams", type=int, default=3,
                    help="(per-layer workload 4) HIP streams the asynchronous one-layer decode calls are spread over")
    ap.add_argument("--narrow-dof", type=int, default=0,
                    help="narrow part of the mixture: 0 = the pages' Gaussian, nu = Student's t with nu degrees of freedom")
    ap.add_argument("--channel-split", action="store_true",
                    help="per-(plane, channel) narrow weights calibrated to the code length (kvc_calibrate_split)")
    ap.add_argument("--paged", type=int, default=0,
                    help="decode straight into a paged KV cache with pages of this many tokens (shuffled table)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="after the timed steps, copy 1 GiB once (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from entropy_coding_amd import workloads as W
    w = W.WORKLOADS[args.workload]
    if args.workload == 0:
        raise SystemExit("workload 0 is a parity case (1M scalars), not a bench line")
    per_layer = args.workload == 4            # streamed one layer per call

    cpu = None
    if not args.no_cpu_baseline and w.kv_dtype == W.BF16:
        log("[bench] cpu_baseline: oracle on a host sample ...")
        cpu = cpu_baseline(w, args.cpu_workers)
        log(f"[bench] cpu_baseline {cpu['value']:.4f} GB/s on {cpu['cores']} cores")

    import torch
    from entropy_coding_amd import kvc   # fails loudly if libkvc.so is missing

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    reps = args.calib_reps if args.calib_reps is not None else w.calib_reps
    kv, mu, sigma, prefix, split = prepare(w, dev, reps, args.sigma_block, args.sigma_fit, args.narrow_dof,
                                           args.channel_split)
    n = w.n_scalars
    weights = (w.w_narrow_bp, w.w_wide_bp)
    # with sigma blocks the library's default picks a divisor of the block length
    tc = args.chunk_tokens if args.chunk_tokens else (0 if args.sigma_block else w.chunk_tokens)
    kv_code = kvc.KVC_BF16 if w.kv_dtype == W.BF16 else kvc.KVC_E4M3
    mu_code = kvc.KVC_BF16 if w.mu_dtype == W.BF16 else kvc.KVC_F32
    kv_size = 2 if w.kv_dtype == W.BF16 else 1
    mu_size = 2 if w.mu_dtype == W.BF16 else 4
    # one call over the whole cache, or one call per layer
    parts = ([slice(l * w.planes_per_layer, (l + 1) * w.planes_per_layer) for l in range(w.layers)]
             if per_layer else [slice(0, w.planes)])
    g_part = parts[0].stop - parts[0].start
    p = kvc.make_params(kv_code, mu_code, g_part, w.tokens, w.channels, weights, tc, args.sigma_block, args.narrow_dof,
                        1 if split is not None else 0)
    # the side buffer of each call: sigma, then (per-channel weights) the weights
    side = [sigma[sl] if split is None else kvc.side_info(sigma[sl], split[sl]) for sl in parts]
    enc = kvc.Encoder(p, dev)
    if tc == 0:
        tc = kvc.kvc_stream_info(enc(kv[parts[0]], mu[parts[0]], side[0], prefix)[:128].cpu().numpy())[0] \
            .chunk_tokens
    kv_out = torch.empty((w.planes, w.tokens, w.channels), dtype=torch.int16 if kv_size == 2 else torch.uint8,
                         device=dev)
    dws = torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    log(f"[bench] buffers: stream capacity {enc.capacity / 1e9:.2f} GB, workspace {enc.workspace.numel() / 1e9:.2f} GB,"
        f" {len(parts)} call(s) per step")

    fallback = [0]
    stream_total = [0]
    paged = None
    if args.paged:
        if per_layer or w.kv_dtype != W.BF16:
            raise SystemExit("--paged is defined on the one-call bf16 workloads")
        pt = args.paged
        max_pages = -(-w.tokens // pt)
        num_pages = w.batch * max_pages
        gen = torch.Generator(device="cpu").manual_seed(11)
        table = torch.randperm(num_pages, generator=gen).to(torch.int32).reshape(w.batch, max_pages).to(dev)
        pools = [torch.empty((num_pages, pt, w.heads, w.channels), dtype=torch.int16, device=dev)
                 for _ in range(2 * w.layers)]
        paged = kvc.PagedKV(pools, table, pt)
        log(f"[bench] paged output: {len(pools)} pools of {num_pages} x {pt}-token pages, shuffled table")

    def step(stats=None):
        e_ms, d_ms = [0.0] * kvc.ENCODE_STAGES, [0.0] * kvc.DECODE_STAGES
        fb, nbytes = 0, 0
        for i, sl in enumerate(parts):
            ei, di = {}, {}
            st = enc(kv[sl], mu[sl], side[i], prefix, info=ei)
            if paged is not None:
                rc = kvc.kvc_decode_paged(st, mu[sl], side[i], prefix, paged, dws, info=di, header=enc.header)
            else:
                rc = kvc.kvc_decode_into(st, mu[sl], side[i], prefix, kv_out[sl], dws, info=di, header=enc.header)
            if rc != kvc.KVC_OK:
                raise kvc.KvcError(rc, "kvc_decode")
            e_ms = [a + b for a, b in zip(e_ms, ei["stage_ms"])]
            d_ms = [a + b for a, b in zip(d_ms, di["stage_ms"])]
            fb += di["fallback_symbols"]
            nbytes += st.numel()
        fallback[0], stream_total[0] = fb, nbytes
        if stats is not None:
            stats.append((e_ms, d_ms))

    pipelined = per_layer and args.streams > 1 and paged is None
    if pipelined:
        # every layer's encode queued without waiting (one encoder per layer,
        # its outcome read after the pass), spread over `streams` HIP streams
        # so that two one-layer calls (half the chip each) run at once; then
        # every decode the same way
        encs = [enc] + [kvc.Encoder(p, dev) for _ in parts[1:]]
        dwss = [dws] + [torch.empty(kvc.DECODE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev) for _ in parts[1:]]
        qs = [torch.cuda.Stream(device=dev) for _ in range(max(args.streams, args.decode_streams))]
        es, ds = args.streams, args.decode_streams
        log(f"[bench] pipelined: {len(parts)} one-layer calls queued asynchronously, encode over {es} and decode "
            f"over {ds} streams")

        def step(stats=None):
            main = torch.cuda.current_stream(dev)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record(main)
            for q in qs:
                q.wait_stream(main)
            for l, sl in enumerate(parts):
                encs[l].enqueue(kv[sl], mu[sl], side[l], prefix, stream=qs[l % es])
            for q in qs:
                main.wait_stream(q)
            ev[1].record(main)
            sts = [encs[l].result(stream=qs[l % es]) for l in range(len(parts))]
            ev[2].record(main)
            for q in qs:
                q.wait_stream(main)
            for l, sl in enumerate(parts):
                rc = kvc.kvc_decode_async(sts[l], mu[sl], side[l], prefix, kv_out[sl], dwss[l], encs[l].header.copy(),
                                          stream=qs[l % ds])
                if rc != kvc.KVC_OK:
                    raise kvc.KvcError(rc, "kvc_decode_async")
            for q in qs:
                main.wait_stream(q)
            ev[3].record(main)
            fb = 0
            for l in range(len(parts)):
                di = {}
                rc = kvc.kvc_decode_result(dwss[l], stream=qs[l % ds], info=di)
                if rc != kvc.KVC_OK:
                    raise kvc.KvcError(rc, "kvc_decode_result")
                fb += di["fallback_symbols"]
            torch.cuda.synchronize()
            fallback[0], stream_total[0] = fb, sum(st.numel() for st in sts)
            if stats is not None:
                # no per-kernel stage times for queued calls: the whole pass
                e, d = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
                stats.append(([0.0, e], [0.0, d]))

    for i in range(args.warmup):
        step()
        log(f"[bench] warmup {i + 1}/{args.warmup}")
    torch.cuda.synchronize()
    stats = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(stats)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {elapsed:.3f} s")
    if args.traffic_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] traffic probe: copied 1 GiB")
    scatter_ms = None
    if paged is not None:
        # read the pages back through the table into the contiguous layout
        tl = paged.block_table.long()
        bh = w.batch * w.heads
        for lk, pool in enumerate(paged.pools):
            kv_out[lk * bh:(lk + 1) * bh] = pool[tl].reshape(w.batch, -1, w.heads, w.channels)[:, :w.tokens] \
                .permute(0, 2, 1, 3).reshape(bh, w.tokens, w.channels)
        # the unfused alternative needs a second pass over the decoded KV
        # (read and write every byte once): at least one device copy of it
        dst = torch.empty_like(kv_out)
        dst.copy_(kv_out)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(3):
            dst.copy_(kv_out)
        ev1.record()
        torch.cuda.synchronize()
        scatter_ms = ev0.elapsed_time(ev1) / 3
        del dst
    ok = torch.equal(kv_out, kv.view(torch.int16) if kv_size == 2 else kv)
    if not ok:
        raise SystemExit("decoded KV differs from the input")
    stream_bytes = stream_total[0]
    bits_int, bits_float = 0.0, 0.0
    for sl in parts:
        bi, bf = kvc.kvc_estimate_bits(kv[sl], mu[sl], sigma[sl], prefix, weights,
                                       sigma_block_tokens=args.sigma_block, chunk_tokens=tc, narrow_dof=args.narrow_dof,
                                       channel_split=None if split is None else split[sl])
        frac = (sl.stop - sl.start) / w.planes
        bits_int += bi * frac
        bits_float += bf * frac

    def median(xs):
        # of the timed calls: robust to one slow call
        import statistics
        return statistics.median(xs)

    enc_kernel = median([s[0][1] for s in stats])
    enc_total = median([sum(s[0]) for s in stats])
    dec_kernel = median([s[1][1] for s in stats])
    dec_total = median([sum(s[1]) for s in stats])
    ms_per_step = elapsed / args.steps * 1e3
    raw = float(kv_size) * n
    # algorithmic bytes of the coding kernels: KV and mu in, words and states
    # out (encode); words and states and mu in, KV out (decode)
    alg = float(kv_size + mu_size) * n + stream_bytes
    traffic = measured_traffic() if args.workload == 2 and tc == w.chunk_tokens and not args.paged \
        and not args.sigma_block and args.sigma_fit == "rms" and not args.narrow_dof and not args.channel_split else {}

    def roofline(kernel, avg_ms):
        a = alg / (avg_ms * 1e-3) / 1e9
        t = traffic.get(kernel, {}).get("total")
        return {"bound": "hbm", "kernel": kernel, "achieved": a, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBPS, "traffic": t, "algorithmic_bytes": alg, "avg_ms": avg_ms}

    rl = {"k_encode": roofline("k_encode", enc_kernel), "k_decode": roofline("k_decode", dec_kernel)}
    # the ALU view of the same kernels (their bound): vector lane-operations
    # per second from the counted instructions per wave step, against one
    # wave64 instruction per CU-cycle
    valu = measured_valu() if traffic else {}
    alu = {}
    for k, ms in (("k_encode", enc_kernel), ("k_decode", dec_kernel)):
        if k in valu:
            a = valu[k] * 64.0 * (n / 64.0) / (ms * 1e-3) / 1e12
            alu[k] = {"bound": "alu", "kernel": k, "achieved": a, "peak": ALU_PEAK_TOPS, "unit": "T lane-ops/s",
                      "frac": a / ALU_PEAK_TOPS, "valu_per_wave_step": valu[k]}
    # the same algorithmic bytes over each whole call (per-call tables,
    # checksum and launches included): what a caller of kvc_encode /
    # kvc_decode gets
    call_rl = {k: {"ms": ms, "achieved": alg / (ms * 1e-3) / 1e9,
                   "frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
               for k, ms in (("encode", enc_total), ("decode", dec_total))}
    dominant = "k_decode" if dec_kernel >= enc_kernel else "k_encode"
    res = {
        "metric": "encode/decode GB/s of raw KV + bits/scalar, Qwen3-8B-shaped bf16 KV" if args.workload == 2
                  else f"encode/decode GB/s of raw KV + bits/scalar, {w.name}",
        "value": raw / (ms_per_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if kv_size == 2 else "e4m3",
        "data": "synthetic",
        "config": {
            "workload": w.name, "shape": [w.layers, 2, w.batch, w.heads, w.tokens, w.channels],
            "scalars": n, "mixture_bp": list(weights), "chunk_tokens": tc, "sigma_block_tokens": args.sigma_block,
            "sigma_calibration": f"{args.sigma_fit}, {reps}x{w.calib_tokens} tokens per layer",
            "narrow_part": "gaussian" if args.narrow_dof == 0 else f"student-t, {args.narrow_dof} dof",
            "mixture_weights": "per (plane, channel), calibrated to the code length" if args.channel_split
                               else "the call's, every channel",
            "mu_dtype": "bf16" if mu_size == 2 else "fp32", "calls_per_step": len(parts),
            "decode_output": f"paged, {args.paged}-token pages" if args.paged else "contiguous",
            "calls": (f"asynchronous, encode on {args.streams} and decode on {args.decode_streams} streams "
                      "(times: whole passes)" if pipelined
                      else "synchronous, one after another"),
            "second_pass_copy_ms": scatter_ms,
        },
        "encode_gbps": raw / (enc_total * 1e-3) / 1e9,
        "decode_gbps": raw / (dec_total * 1e-3) / 1e9,
        "encode_ms": enc_total, "decode_ms": dec_total,
        "encode_stage_ms": {k: median([s[0][i] for s in stats]) for i, k in
                            enumerate(["prologue", "encode_kernel"])},
        "decode_stage_ms": {k: median([s[1][i] for s in stats]) for i, k in enumerate(["prologue", "decode_kernel"])},
        "bits_per_scalar": {"coded": 8.0 * stream_bytes / n, "integer_model": bits_int, "float_model": bits_float,
                            # what the stream spends beyond the model: the 64 final states of every chunk (the
                            # price of the chunk length), the header and directory, renormalisation and padding
                            "chunk_overhead": 8.0 * stream_bytes / n - bits_int,
                            "header_and_directory": 8.0 * sum(
                                128 + 8 * ((sl.stop - sl.start) * -(-w.tokens // tc) * (w.channels // 64) + 1)
                                for sl in parts) / n},
        "stream_bytes": stream_bytes,
        "decode_fallback_share": fallback[0] / n,
        "roundtrip_exact": ok,
        "roofline": rl[dominant],
        "rooflines": rl,
        "call_rooflines": call_rl,
        "alu_rooflines": alu or None,
        "cpu_baseline": cpu,
        "pages_context": {"bits_per_scalar_qwen3_0.6B_to_32B": [6.74, 5.92],
                          "fp8_bits_per_element": [2.05, 2.59]},
    }
    print(json.dumps(res))
    if args.offload:
        if not per_layer:
            raise SystemExit("--offload is defined on the per-layer workload (4)")
        print(json.dumps(offload_reload(w, kv, mu, side, prefix, kvc, enc, parts, dws, max(1, args.steps))))


if __name__ == "__main__":
    main()
