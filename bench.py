"""Benchmark of the block-sparse masked attention forward on one MI355X.

A step is one pass of the whole path over one batch of synthetic inputs that
are already resident in HBM: the block metadata build followed by the
attention forward (for a dense-mask workload, whose metadata is built once on
the host, the forward alone). The default workload is causal MHA, B=2, H=32,
S=8192, D=128, bf16, 128x128 blocks. Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload c3h] [--no-cpu-baseline]

Throughput counts 4*bq*bkv*D FLOPs per non-empty (b, h, i, j) block (the
QKᵀ and P·V products of every block that is not skipped). The element-exact
count, 4*D per allowed (q, k) pair, is reported beside it
(config.element_flops, config.element_tflops).
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix peak: 256 CU x 4096 FLOP/clk x 2.4 GHz
# fp32 vector peak for the instructions the fp32 kernel can issue: packed
# fp32 (two FMAs per lane) is disabled in this build, so one FMA per lane per
# clock: 256 CU x 4 SIMD x 16 lanes x 2 FLOP x 2.4 GHz (AMD's 157.3 counts
# packed FMAs)
PEAK_F32_TFLOPS = 78.6
METRIC = "splash fwd TFLOP/s (unmasked FLOPs) + % bf16 MFMA peak, causal S=8192"
# the backward workloads report the same kind of figure for the backward pass
BWD_METRIC = "splash bwd TFLOP/s (unmasked FLOPs, 5 products per block) + % bf16 MFMA peak"
# the sources each direction's kernels are built from: a counter summary stays
# valid while these are unchanged
KERNEL_SOURCES = {
    False: ["splash_fwd_bf16.hip", "splash_fwd_rows64.hip", "splash_fwd_f32.hip", "cdna4.h", "internal.h"],
    True: ["splash_bwd_bf16.hip", "splash_bwd_f32.hip", "softmax_delta.hip", "cdna4.h", "internal.h"],
}


def kernel_source_hash(backward: bool = False) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[backward]:
        with open(os.path.join(ROOT, "block_sparse_masked_splash_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, backward: bool = False):
    """HBM bytes per timed call from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"splash_{'bwd' if backward else 'fwd'}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != kernel_source_hash(backward):
        return None
    return t.get("bytes_per_launch")


def allowed_pairs(w, gen) -> int:
    """Allowed (query, key) pairs summed over every (batch, head), counted row
    by row, for the element-exact FLOP count (4 * D per pair).

    A head mask is a band lo <= k - q <= hi (causal: hi <= 0), so query q
    keeps the keys [max(0, q + lo), min(S - 1, q + hi)]; packed documents
    (segment ids that are runs of equal values, as the workloads draw them)
    clip that interval to q's document. A dense mask is counted from its bits,
    ANDed with the band."""
    import numpy as np

    S = w.S
    q = np.arange(S, dtype=np.int64)
    big = 1 << 40

    def band(head):
        causal, wl_, wr = (int(x) for x in head)
        lo = -wl_ if wl_ >= 0 else -big
        hi = wr if wr >= 0 else big
        return lo, (min(hi, 0) if causal else hi)

    heads = [w.head_masks[0] if len(w.head_masks) == 1 else w.head_masks[h] for h in range(w.H)]
    if gen.get("dense") is not None:
        d = gen["dense"].numpy().astype(bool)
        k = np.arange(S, dtype=np.int64)[None, :]
        total = 0
        for head in heads:
            lo, hi = band(head)
            dd = (k - q[:, None] >= lo) & (k - q[:, None] <= hi)
            total += int((d & dd).sum())
        return w.B * total
    seg = gen.get("q_segment_ids")
    total = 0
    for b in range(w.B if seg is not None else 1):
        a0, e0 = np.zeros(S, dtype=np.int64), np.full(S, S - 1, dtype=np.int64)
        if seg is not None:
            ids = seg[b].numpy()
            change = np.flatnonzero(np.diff(ids)) + 1
            starts = np.concatenate([[0], change])
            ends = np.concatenate([change - 1, [S - 1]])
            run = np.repeat(np.arange(starts.size), ends - starts + 1)
            a0, e0 = starts[run], ends[run]
        for head in heads:
            lo, hi = band(head)
            a = np.maximum(a0, q + lo)
            e = np.minimum(e0, q + hi)
            total += int(np.maximum(e - a + 1, 0).sum())
    return total * (1 if seg is not None else w.B)


_BLAS_LIMIT = None


def _cpu_worker_init():
    # one BLAS thread per worker process (the pool's processes are the
    # cores); set before numpy loads its BLAS, and enforced once it has
    global _BLAS_LIMIT
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy  # noqa: F401  (imported before timing starts)
    import oracle  # noqa: F401
    try:
        from threadpoolctl import threadpool_limits
        _BLAS_LIMIT = threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _cpu_ready(_):
    return os.getpid()


def _cpu_task(task):
    """One oracle task of the CPU baseline: some query blocks of one (batch,
    head), forward (or backward) rows formed by the fp64 oracle. Returns the
    block FLOPs it covered."""
    import numpy as np
    import oracle

    (S, bq, bkv, D, scale, head, pointwise, backward, blocks, q, k, v, do, qs, dense) = task
    k64, v64 = k.astype(np.float64), v.astype(np.float64)
    flops = 0
    for n, i in enumerate(blocks):
        rows = np.arange(i * bq, min(S, (i + 1) * bq))
        m = oracle.element_mask(S, S, head, qs, qs, rows=rows, dense=dense)
        q64 = q[n].astype(np.float64)
        if backward:
            do64 = do[n].astype(np.float64)
            if pointwise:
                oracle.pointwise_attention_bwd_rows(q64, k64, v64, do64, scale, m, S)
            else:
                oracle.softmax_attention_bwd_rows(q64, k64, v64, do64, scale, m)
        elif pointwise:
            oracle.pointwise_attention_rows(q64, k64, v64, scale, m, S)
        else:
            oracle.softmax_attention_rows(q64, k64, v64, scale, m)
        cls, _ = oracle.mask_info_row(S, S, bq, bkv, head, i, qs, qs, dense=dense)
        flops += int(np.count_nonzero(cls)) * (10 if backward else 4) * bq * bkv * D
    return flops


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(w, gen, budget_s: float = 12.0, single_s: float = 5.0):
    """The oracle, as it is, on a bounded sample of the same workload: tasks of
    a few whole query blocks of one random (b, h), run by a process pool with
    one worker per core of this process's CPU share (at most 16) and one BLAS
    thread per worker, for about ``budget_s`` seconds; then the same kind of
    sample in one process on one core for about ``single_s`` seconds. Runs
    before anything touches the GPU (the pool's processes are started fresh,
    not forked)."""
    import multiprocessing as mp

    import numpy as np

    try:
        share = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        share = os.cpu_count() or 1
    workers = max(1, min(share, os.cpu_count() or 1, 16))
    rng = np.random.default_rng(12345)
    S, bq, bkv, D = w.S, w.block_q, w.block_kv, w.D
    nq = -(-S // bq)
    per_task = 1 if w.backward else 4
    qs_all = gen["q_segment_ids"]
    dense = None if gen["dense"] is None else gen["dense"].numpy()

    def tasks():
        while True:
            b, h = int(rng.integers(w.B)), int(rng.integers(w.H))
            hk = h // (w.H // w.n_kv_heads)
            blocks = sorted(int(x) for x in rng.integers(nq, size=per_task))
            head = w.head_masks[0] if len(w.head_masks) == 1 else w.head_masks[h]
            q = [gen["q"][b, h, i * bq:min(S, (i + 1) * bq)].float().numpy() for i in blocks]
            do = None
            if w.backward:
                do = [gen["d_o"][b, h, i * bq:min(S, (i + 1) * bq)].float().numpy() for i in blocks]
            yield (S, bq, bkv, D, w.scale, head, w.pointwise, w.backward, blocks, q,
                   gen["k"][b, hk].float().numpy(), gen["v"][b, hk].float().numpy(), do,
                   None if qs_all is None else qs_all[b].numpy(), dense)

    def run(pool, n_workers, budget):
        # every worker started and initialised before the clock starts
        pool.map(_cpu_ready, range(4 * n_workers), chunksize=1)
        it = tasks()
        pending, flops, done = [], 0, 0
        t0 = time.perf_counter()
        while True:
            while len(pending) < 2 * n_workers and (time.perf_counter() - t0 < budget or done + len(pending) < 2):
                pending.append(pool.apply_async(_cpu_task, (next(it),)))
            if not pending:
                break
            flops += pending.pop(0).get()
            done += 1
        return flops, done, time.perf_counter() - t0

    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        flops, done, dt = run(pool, workers, budget_s)
    with ctx.Pool(1, initializer=_cpu_worker_init) as pool:
        f1, d1, t1 = run(pool, 1, single_s)
    blocks_desc = "one query block" if per_task == 1 else f"{per_task} query blocks"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": (f"{done} tasks ({blocks_desc} of {bq} rows of one random (b, h) each), fp64 numpy oracle, "
                       f"{workers} worker processes x 1 BLAS thread, {dt:.1f} s wall"),
            "single_core": {"value": f1 / t1 / 1e12, "tasks": d1, "seconds": round(t1, 1)},
            "cpu_count": os.cpu_count(), "cpu_share": share, "cpu_model": _cpu_model(),
            "blas_threads_per_worker": 1}


def gemm_reference(dev, n: int = 8192, reps: int = 10) -> float:
    """TFLOP/s of torch's bf16 GEMM (n x n x n) on N(0, 1) operands on this GPU:
    what the matrix cores sustain on random data, as context for the roofline
    fraction (the published peak is not reachable with such operands)."""
    import torch
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed warm-up steps: after the GPU has been idle its clock control
    # overshoots for about fifteen calls (B=2 H=32 S=8192 D=128: 1.04 -> 1.40
    # -> 1.04 ms per call); 100 steps also cover the shorter workloads, whose
    # calls are ten times shorter
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="c3h")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run N copies of a 1 GiB buffer (counter calibration)")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the dense bf16 GEMM reference measurement")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the work shards by (batch, head) with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_masked_splash_amd as sp
    from block_sparse_masked_splash_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    gen = wl.generate(w)
    pairs = allowed_pairs(w, gen)
    # the oracle's CPU baseline runs first, before anything touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, gen)
    dev = torch.device("cuda:0")
    q, k, v = (gen[n].to(dev) for n in ("q", "k", "v"))
    seg = None if gen["q_segment_ids"] is None else gen["q_segment_ids"].to(dev)
    fwd = sp.pointwise_fwd if w.pointwise else sp.splash_fwd
    out = torch.empty_like(q)

    dense = gen["dense"]
    if dense is not None:
        # a dense mask's metadata is built once, on the host (as for a mask
        # fixed ahead of time); the step is then the forward alone
        info = sp.dense_mask_info_build(w.B, w.H, dense, w.head_masks, w.block_q, w.block_kv, device=dev)
    else:
        info = sp.mask_info_build(w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, seg, seg, device=dev)
    torch.cuda.synchronize()
    nonempty = (info.block_mask != 0).sum(dim=(2, 3)).to(torch.int64)  # [Bm, Hm]
    Bm, Hm = info.block_mask.shape[:2]
    per_bh = nonempty.expand(w.B if Bm == 1 else Bm, w.H if Hm == 1 else Hm)
    blocks = int(per_bh.sum().item())
    # forward: Q Kᵀ and P V per non-empty block; backward: Q Kᵀ, dO Vᵀ, P'ᵀ dO,
    # dS'ᵀ Q and dS' K (the five products of the page's backward kernel)
    flops = blocks * (10 if w.backward else 4) * w.block_q * w.block_kv * w.D

    if w.backward:
        d_o = gen["d_o"].to(dev)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        info_dkv = sp.mask_info_build_dkv(w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, seg, seg,
                                          device=dev)
        if not w.pointwise:
            # the forward's output and log-sum-exp are the backward's inputs (made before timing)
            o_fwd, lse = sp.splash_fwd_lse(q, k, v, info, scale=w.scale)
            delta = torch.empty_like(lse)

    def build_metadata():
        if dense is None:
            sp.mask_info_build(w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, seg, seg, device=dev,
                               out=info)
        if w.backward:
            sp.mask_info_build_dkv(w.B, w.H, w.S, w.S, w.head_masks, w.block_q, w.block_kv, seg, seg, device=dev,
                                   out=info_dkv)

    def run_kernels():
        if w.backward and not w.pointwise:
            sp.softmax_bwd_preprocess(o_fwd, d_o, delta=delta)
            sp.softmax_bwd(q, k, v, d_o, lse, delta, info, info_dkv, scale=w.scale, out=grads)
        elif w.backward:
            sp.pointwise_bwd(q, k, v, d_o, info, info_dkv, scale=w.scale, out=grads)
        else:
            fwd(q, k, v, info, scale=w.scale, out=out)

    def step():
        build_metadata()
        run_kernels()

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    # No garbage-collection pass inside the timed steps (a full pass over the
    # objects the setup left behind can stall one step's launches for tens of
    # ms), and none between the warm-up and the timed steps either: after tens
    # of ms of idle the GPU's clock control overshoots for about fifteen
    # launches (kernel traces: 1.04 -> 1.40 -> 1.04 ms per call at B=2 H=32
    # S=8192 D=128), so the warm-up runs straight into the timed steps.
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        build_metadata()
        ev[s][0].record(stream)
        run_kernels()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps

    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(args.copy_calibration):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    in_f32 = w.dtype == "f32"
    peak = PEAK_F32_TFLOPS if in_f32 else PEAK_BF16_TFLOPS
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    value = flops / (ms_per_step * 1e-3) / 1e12
    desc = {
        "c1": "tiny causal attention B=1 H=1 S=256 D=64 fp32, block 64x64",
        "c2": "causal MHA B=4 H=16 S=2048 D=128 bf16, block 128x128",
        "c3h": "causal MHA B=2 H=32 S=8192 D=128 bf16, block 128x128",
        "c3": "causal AND same-document MHA B=2 H=32 S=8192 D=128 bf16, documents 256-2048, block 128x128",
        "c4": "mixed heads B=1 H=16 S=32768 D=128 bf16: 8 causal + 8 causal window 1024, block 128x128",
        "c5": "pointwise SiLU causal B=8 H=8 S=4096 D=64 bf16, N(0,0.5^2), block 128x128",
        "g3h": "grouped-query causal B=2 H=32 (8 K/V heads) S=8192 D=128 bf16, block 128x128",
        "d3h": "dense-mask MHA B=2 H=32 S=8192 D=128 bf16, the causal pattern as an [S, S] array, block 128x128",
        "d5": "dense-mask pointwise SiLU B=8 H=8 S=4096 D=64 bf16, the causal pattern as an [S, S] array, "
              "N(0,0.5^2), block 128x128",
        "b5": "pointwise SiLU backward (dq, dk, dv) B=8 H=8 S=4096 D=64 bf16 causal, N(0,0.5^2) inputs, "
              "N(0,1) output gradient, blocks 128x128 for both walks",
        "b5h": "pointwise SiLU backward (dq, dk, dv) B=2 H=16 S=4096 D=128 bf16 causal, N(0,0.5^2) inputs, "
               "N(0,1) output gradient, blocks 128x128 for both walks",
        "s3h": "softmax backward (delta, dq, dk, dv) B=2 H=32 S=8192 D=128 bf16 causal, N(0,1) inputs and "
               "output gradient, blocks 128x128 for both walks",
    }[w.name]
    fwd_name = (("pointwise_bwd" if w.pointwise else "softmax_bwd_preprocess + softmax_bwd") if w.backward
                else ("pointwise_fwd" if w.pointwise else "splash_fwd"))
    line = {
        "metric": BWD_METRIC if w.backward else METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if in_f32 else "bf16",
        "data": "synthetic (seeded N(0, sigma^2) q, k, v)",
        "config": {"workload": f"{w.name}: {desc}", "batch": w.B, "heads": w.H, "kv_heads": w.n_kv_heads,
                   "seq_len": w.S,
                   "head_dim": w.D, "block_q": w.block_q, "block_kv": w.block_kv,
                   "nonempty_blocks": blocks, "flops_per_step": flops,
                   "allowed_pairs": pairs, "element_flops": pairs * (10 if w.backward else 4) * w.D,
                   "element_tflops": round(pairs * (10 if w.backward else 4) * w.D / (ms_per_step * 1e-3) / 1e12, 3),
                   "step": (f"{fwd_name} (dense-mask metadata built once on the host, before timing)"
                            if dense is not None else
                            "mask_info_build + mask_info_build_dkv + " + fwd_name if w.backward else
                            "mask_info_build + " + fwd_name)},
        "kernel_ms": round(kernel_ms, 5),
        "pct_of_peak": round(100 * value / peak, 2),
        "roofline": {"bound": "mfma" if not in_f32 else "alu", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_for(w.name, w.backward), "kernel_source_sha256_16": kernel_source_hash(w.backward)},
    }
    if not args.no_gemm_reference and not in_f32:
        g = gemm_reference(dev)
        line["bf16_gemm_reference"] = {"tflops": round(g, 1), "what": "torch bf16 GEMM 8192^3 on N(0,1) operands",
                                       "fwd_fraction_of_it": round(achieved / g, 4)}
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
