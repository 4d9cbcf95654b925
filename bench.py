#!/usr/bin/env python3
"""Benchmark: shared-QK LSH attention forward + backward on one MI355X.

One step is the whole hot path over one batch of synthetic input already
resident in HBM: hash, sort, per-round chunk attention (with the unsort),
logsumexp combine, and the backward (per-round query- and key-side gradients,
reduction over rounds, key normalisation).  The default workload is the
64K-token text-shaped case (B=1, H=8, L=65536, d=128, 1024 buckets, 4 hash
rounds, chunk 128, bf16).

Prints one JSON line: tokens/s (B*L per step), the roofline of the dominant
kernel (its HIP-event-timed average launch against MI355X peak), and the fp64
CPU oracle timed on the host cores on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--config text]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LSH-attention fwd+bwd tokens/s at L=64K on 1 MI355X; % MFMA / HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
WORKLOAD_NAMES = {
    "tiny": "tiny fp32 forward+backward (L=1024)",
    "mid": "mid-size (B=8, H=8, L=4096)",
    "image": "image-generation-shaped (L=12288 = 64x64x3)",
    "text": "long-text-shaped (L=65536)",
    "stress": "stress: 256-cluster Gaussian mixture (B=4, L=65536)",
}
# source file of each kernel on the bf16 matrix-core path, for matching stored
# counter measurements to the code they were taken on
KERNEL_SOURCE = {
    "hash": "hash.hip", "sort_count": "sort.hip", "sort_scatter": "sort.hip",
    "prep": "attn_generic.hip", "tiles": "attn_mfma.hip", "attn_fwd": "attn_mfma.hip",
    "combine": "attn_generic.hip", "bwd_dq": "attn_mfma.hip", "bwd_dkv": "attn_mfma.hip",
    "bwd_reduce": "attn_mfma.hip",
}


def algorithmic_work(name: str, cfg, backward_prep: bool = True) -> tuple[float, float]:
    """(flops, bytes) that one launch of kernel `name` must do for `cfg`.

    prep and tiles run twice per training step; backward_prep selects the
    backward's launch (the one a step's timing of those kernels ends on).

    Bytes count every input a kernel needs read once and every output written
    once (row gathers by position count their rows once per round; a
    per-round result is written once).  Flops count the method's dense chunk
    tiles: m x 2m query-key pairs per chunk (chunk 0 sees m keys), 2 d flops
    per product per pair.  Per-round gradient partials are bf16 on this path.
    """
    s = 2 if cfg.dtype == "bf16" else 4
    B, H, L, d, nh, nb, m = cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_hashes, cfg.n_buckets, cfg.chunk_len
    T = B * H * L
    Tr = T * nh
    S = B * H * nh
    ntiles = -(-L // 4096)                          # sort tiles per segment
    cnt_bytes = S * ntiles * nb * 2                 # 16-bit per-tile bucket counts
    pairs = (2.0 * m * L - m * m) * B * H * nh      # query-key pairs of the dense chunk tiles
    meta = 4 * nh                                   # one packed record per round
    if name == "hash":
        return 2.0 * T * nh * (nb // 2) * d, T * d * s + nh * d * (nb // 2) * s + Tr * 4
    if name == "sort_count":     # bucket ids in, per-tile counts out
        return 0.0, Tr * 4 + cnt_bytes
    if name == "sort_scatter":   # bucket ids in (again), the segment's counts, perm / inv / win_lo out
        return 0.0, Tr * 4 + cnt_bytes + Tr * 12
    qtile_row = ((320 + 128 * (nh - 1) + 255) & ~255) // 32   # stored query-tile bytes per sorted row
    ktile_row = ((128 + 64 * (nh - 1) + 255) & ~255) // 32    # stored key-tile bytes per sorted row
    if name == "prep":
        if backward_prep:   # backward on the forward's records: out and dout in, D out
            return 0.0, 2 * T * d * s + T * 4
        # forward: q for the norms, inv and win_lo in; packed records (both orders) and norms out
        return 0.0, T * d * s + Tr * 8 + Tr * 8 + T * 4
    if name == "tiles":
        if backward_prep:   # query tiles: sorted record, the row's meta, lse and D gathered; tile written
            return 0.0, Tr * (4 + meta + 8) + Tr * qtile_row
        return 0.0, Tr * (4 + meta + 4) + Tr * ktile_row
    if name == "attn_fwd":   # q, v rows; o row and lse written
        return 2.0 * 2 * d * pairs, Tr * (3 * d * s + 4 + 4 + 32)
    if name == "combine":
        return 0.0, Tr * (d * s + 4) + T * (d * s + 4)
    if name == "bwd_dq":     # q, v, dout rows; bf16 dq partial
        return 3.0 * 2 * d * pairs, Tr * (3 * d * s + 2 * d + 12 + 32)
    if name == "bwd_dkv":    # q, v, dout rows; bf16 dqk and dv partials
        return 4.0 * 2 * d * pairs, Tr * (3 * d * s + 4 * d + 12 + 64)
    if name == "bwd_reduce":  # three bf16 partials per round in; dq, dv out
        return 0.0, Tr * 3 * 2 * d + T * (2 * d * s + meta)
    raise KeyError(name)


class Hip:
    """The few HIP runtime calls the timing needs (the process's own runtime)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so.7")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        if self.h.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev

    def elapsed_ms(self, a, b, missing_ok: bool = False):
        """Milliseconds between two recorded events.  With missing_ok, None when
        they were never recorded (a kernel the problem does not launch)."""
        ms = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            self.h.hipGetLastError()   # clear the runtime's last-error state
            if missing_ok:
                return None
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.h.hipEventDestroy(ev)


def rehash_variant(prob, mod, q, v, rot, do, steps, cfg) -> dict:
    """The reversible-layer step: forward, then a backward that recomputes hashing and sorting
    (lsh_attn_bwd_rehash) instead of reading the forward's saved records."""
    import torch
    import lsh_sparse_attention_amd as lsh
    from lsh_sparse_attention_amd import _lib as L_
    ws = torch.empty(lsh.workspace_bytes(prob, L_.LSH_WS_REHASH), dtype=torch.uint8, device="cuda")
    dq, dv = torch.empty_like(mod.dq), torch.empty_like(mod.dv)

    def step():
        mod.forward(q, v, rot)
        lsh.lsh_attn_bwd_rehash(prob, q, v, rot, mod.out, do, mod.lse, dq, dv, ws)

    step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del ws
    return {"ms_per_step": ms, "value": cfg.batch * cfg.seq_len / (ms * 1e-3), "unit": "tokens/s",
            "kept_between_passes": "out, lse (no buckets, sorted order or records)"}


def set_variant(q, v, rot, do, steps, cfg, hip, causal, bucket_mask, dup_by_bucket=False) -> dict:
    """The same training step (forward and saved-records backward) on the same inputs with other
    attended sets: non-causal (encoder) sets, sets without the same-bucket condition, or the
    duplicate count over bucket membership."""
    import torch
    import lsh_sparse_attention_amd as lsh
    from lsh_sparse_attention_amd import _lib as L_
    prob = lsh.problem(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_hashes, cfg.n_buckets,
                       cfg.chunk_len, cfg.scale, cfg.dtype, causal=causal, bucket_mask=bucket_mask,
                       dup_by_bucket=dup_by_bucket)
    mod = lsh.LshAttention(prob)

    def step():
        mod.forward(q, v, rot)
        mod.backward(q, v, do)

    step()
    L = L_.lib()
    evs = [(hip.event(), hip.event()) for _ in L_.KERNELS]
    for k, (a, b) in enumerate(evs):
        L.lsh_profile_kernel(k, a, b)
    step()
    torch.cuda.synchronize()
    per_kernel = {}
    for k, (a, b) in enumerate(evs):
        ms = hip.elapsed_ms(a, b, missing_ok=True)
        if ms is not None:
            per_kernel[L_.KERNELS[k]] = round(ms * 1e3, 2)
        L.lsh_profile_kernel(k, None, None)
        hip.destroy(a)
        hip.destroy(b)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del mod
    return {"ms_per_step": ms, "value": cfg.batch * cfg.seq_len / (ms * 1e-3), "unit": "tokens/s",
            "causal": causal, "bucket_mask": bucket_mask, "dup_by_bucket": dup_by_bucket, "kernels_us": per_kernel}


def ff_variant(steps, rows) -> dict:
    """The chunked feed-forward layer of the Reformer block (the paper's ablation layer, d_model
    1024, d_ff 4096) over the same number of positions, in 8 chunks: forward plus backward (which
    recomputes the hidden activations), as one step; Gaussian inputs."""
    import numpy as np
    import torch
    import lsh_sparse_attention_amd as lsh
    from lsh_sparse_attention_amd import inputs as gen
    dm, dff, chunks = gen.FF_SHAPE["d_model"], gen.FF_SHAPE["d_ff"], 8
    d = gen.generate_ff(rows, dm, dff, seed=7, grid=False)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    x, w1, w2, dy = bf(d["x"]), bf(d["w1"]), bf(d["w2"]), bf(d["dy"])
    b1, b2 = torch.from_numpy(d["b1"]).cuda(), torch.from_numpy(d["b2"]).cuda()
    ff = lsh.ff_problem(rows, dm, dff, chunks)
    wsf = torch.empty(lsh.ff_workspace_bytes(ff, False), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(lsh.ff_workspace_bytes(ff, True), dtype=torch.uint8, device="cuda")
    y, dx = torch.empty_like(x), torch.empty_like(x)
    dw1 = torch.empty((dm, dff), dtype=torch.float32, device="cuda")
    dw2 = torch.empty((dff, dm), dtype=torch.float32, device="cuda")
    db1 = torch.empty(dff, dtype=torch.float32, device="cuda")
    db2 = torch.empty(dm, dtype=torch.float32, device="cuda")

    def step():
        lsh.lsh_ff_fwd(ff, x, w1, b1, w2, b2, y, wsf)
        lsh.lsh_ff_bwd(ff, x, w1, b1, w2, dy, dx, dw1, db1, dw2, db2, wsb)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    flops = 14.0 * rows * dm * dff     # forward 2 products, backward 5 (one recomputes h)
    return {"ms_per_step": ms, "rows": rows, "d_model": dm, "d_ff": dff, "chunks": chunks,
            "tflops": flops / (ms * 1e-3) / 1e12, "frac_of_bf16_peak": flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"],
            "value": rows / (ms * 1e-3), "unit": "tokens/s"}


def gemm_tflops(n: int = 8192) -> float:
    """Rate of a plain n^3 bf16 matrix product through torch.matmul (the vendor GEMM library), the
    practical matrix-core ceiling a compute-bound kernel is compared with beside the datasheet peak."""
    import torch
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    reps = 10
    t0 = time.perf_counter()
    for _ in range(reps):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    tf = 2.0 * n ** 3 * reps / (time.perf_counter() - t0) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return tf


def kernel_rooflines(per_kernel: dict, cfg, gemm_tf) -> dict:
    """Per kernel: one launch's duration and its algorithmic bytes and flops as rates, each
    against the HBM and matrix-core peaks (and the measured GEMM rate for the products)."""
    out = {}
    for k, us in per_kernel.items():
        flops, nbytes = algorithmic_work(k, cfg)
        t = us * 1e-6
        row = {"us": round(us, 2), "gbs": round(nbytes / t / 1e9, 1),
               "frac_hbm": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 3)}
        if flops:
            tf = flops / t / 1e12
            row.update({"tflops": round(tf, 1), "frac_mfma": round(tf / MFMA_PEAK_TFLOPS[cfg.dtype], 3)})
            if gemm_tf:
                row["frac_of_gemm"] = round(tf / gemm_tf, 3)
        out[k] = row
    return out


def copy_bandwidth_gbs() -> float:
    """HBM bandwidth of a plain device-to-device copy of 1 GiB (bytes read + written per second),
    the practical ceiling a bandwidth-bound kernel is compared with beside the 8 TB/s spec."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    gbs = 2 * 4 * n * 5 / (time.perf_counter() - t0) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def source_sha(kernel: str) -> str:
    """Digest of the sources a kernel is compiled from (its file and the shared header)."""
    h = hashlib.sha256()
    for name in (KERNEL_SOURCE[kernel], "common.hpp"):
        with open(os.path.join(ROOT, "lsh_sparse_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str, key: str = "bytes_per_launch"):
    """Bytes per launch from committed rocprofv3 counter runs (key "bytes_per_launch": calibrated
    FETCH_SIZE/WRITE_SIZE; "dram_bytes_per_launch": DRAM read and write requests), if they were
    taken on the current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    rec = table.get(f"{kernel}@{workload}")
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get(key)


def cpu_model() -> str | None:
    """The host CPU's model name from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(x, heads: int):
    from oracle import oracle as ora
    cfg = x["cfg"]
    heads = max(1, min(heads, cfg.heads))
    slices = [(0, h) for h in range(heads)]
    t0 = time.perf_counter()
    ora.run_inputs(x, slices=slices, backward=True)
    dt = time.perf_counter() - t0
    tokens = cfg.seq_len * heads / cfg.heads      # the work of all heads of that many tokens
    return {
        "value": tokens / dt, "unit": "tokens/s", "cores": ora.threads(), "cpu_model": cpu_model(), "kind": "oracle",
        "sample": (f"batch 0, heads 0..{heads - 1} of {cfg.heads} at full L={cfg.seq_len}: hash, sort, "
                   f"forward and backward in fp64; {dt:.1f} s; tokens counted as L*{heads}/{cfg.heads}"),
    }


def sweep(kind: str, steps: int, warmup: int) -> int:
    """Two sweeps on the text workload's shape (d = 128, 8 heads, m = 128), one JSON line each point.

    length: total tokens fixed (B L = 65536), L from 1024 to 65536 with B = 65536 / L and
    n_buckets = L / 64 (the text workload's rows per bucket), 4 rounds; forward + backward step.
    The pages report that LSH attention's speed stays flat as L grows at a fixed total.
    rounds: the text workload with n_hashes = 1, 2, 4, 8; forward (hash, sort, attention,
    combine) and forward + backward, since more rounds can be used at evaluation."""
    import torch
    import numpy as np
    import lsh_sparse_attention_amd as lsh
    from lsh_sparse_attention_amd import inputs as gen

    def dev(a, dtype):
        a = np.ascontiguousarray(a)
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    base = gen.CONFIGS["text"]
    if kind == "length":
        points = [base.with_(name=f"len{L}", batch=65536 // L, seq_len=L, n_buckets=L // 64)
                  for L in (1024, 2048, 4096, 8192, 16384, 32768, 65536)]
    else:
        points = [base.with_(name=f"nh{nh}", n_hashes=nh) for nh in (1, 2, 4, 8)]
    for cfg in points:
        x = gen.generate(cfg, with_grad=True)
        q, v, rot, do = (dev(x[k], cfg.dtype) for k in ("q", "v", "rot", "dout"))
        prob = lsh.problem(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_hashes, cfg.n_buckets,
                           cfg.chunk_len, cfg.scale, cfg.dtype)
        mod = lsh.LshAttention(prob)
        fwd_ms = timed(lambda: mod.forward(q, v, rot))
        step_ms = timed(lambda: (mod.forward(q, v, rot), mod.backward(q, v, do)))
        tokens = cfg.batch * cfg.seq_len
        print(json.dumps({"sweep": kind, "batch": cfg.batch, "heads": cfg.heads, "seq_len": cfg.seq_len,
                          "head_dim": cfg.head_dim, "n_buckets": cfg.n_buckets, "n_hashes": cfg.n_hashes,
                          "chunk_len": cfg.chunk_len, "fwd_ms": round(fwd_ms, 4), "step_ms": round(step_ms, 4),
                          "fwd_tokens_per_s": tokens / (fwd_ms * 1e-3),
                          "step_tokens_per_s": tokens / (step_ms * 1e-3)}), flush=True)
        del mod, q, v, rot, do
        torch.cuda.empty_cache()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="text")
    ap.add_argument("--cpu-heads", type=int, default=4, help="heads of batch 0 the oracle times (0: skip)")
    ap.add_argument("--sweep", choices=("length", "rounds"),
                    help="instead of the bench line: a length sweep at fixed total tokens, or a rounds sweep")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the rehash-backward and non-causal variant steps (profiler runs: only the main "
                         "step's launches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three device copies of 1 GiB (reference point for HBM byte counters)")
    ap.add_argument("--workloads", default="tiny,mid,image,stress",
                    help="other workloads measured after the main one, each with its own line under "
                         "'workloads' (empty: none)")
    ap.add_argument("--ff-only", action="store_true",
                    help="instead of the bench line: only the chunked feed-forward step (variants.chunked_ff) "
                         "over the workload's B * L rows")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the path is per-(batch, head) independent and is not sharded here.", file=sys.stderr)
        return 2

    if args.sweep:
        return sweep(args.sweep, args.steps, args.warmup)
    import torch
    if args.ff_only:
        from lsh_sparse_attention_amd import inputs as gen_
        c = gen_.CONFIGS[args.config]
        print(json.dumps({"chunked_ff": ff_variant(args.steps, c.batch * c.seq_len)}), flush=True)
        return 0
    if args.copy_calibration:
        n = 1 << 28                                   # 2^28 fp32 = 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read": 4 * n, "bytes_written": 4 * n, "copies": 3}}), flush=True)
        return 0
    import lsh_sparse_attention_amd as lsh
    from lsh_sparse_attention_amd import _lib
    from lsh_sparse_attention_amd import inputs as gen

    cfg = gen.CONFIGS[args.config]
    t0 = time.perf_counter()
    x = gen.generate(cfg, with_grad=True)
    print(f"[bench] generated {cfg.name} inputs in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    hip = Hip()
    gtf = gemm_tflops() if cfg.dtype == "bf16" else None   # the GEMM reference rate is a bf16 one
    main_run = measure_workload(x, args.steps, args.warmup, hip, gtf, keep=True)
    mod, (q, v, rot, do) = main_run.pop("_mod"), main_run.pop("_tensors")
    prob = mod.prob
    result = {
        "metric": METRIC, "value": main_run["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_run["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": main_run["config"],
        "roofline": main_run["roofline"],
        "kernels_us": main_run["kernels_us"],
        "variants": None,
    }
    if gtf is not None:
        result["gemm_tflops"] = gtf
    result["kernels"] = main_run["kernels"]
    if result["roofline"]["bound"] == "hbm":
        # the measured denominator beside the spec one: a plain 1 GiB device copy
        result["roofline"]["copy_gbs"] = copy_bandwidth_gbs()
        result["roofline"]["frac_of_copy"] = result["roofline"]["achieved"] / result["roofline"]["copy_gbs"]
    if not args.no_variants:
        result["variants"] = {"rehash_backward": rehash_variant(prob, mod, q, v, rot, do, args.steps, cfg)}
    del mod
    torch.cuda.empty_cache()
    if not args.no_variants:
        result["variants"]["non_causal"] = set_variant(q, v, rot, do, args.steps, cfg, hip, False, True)
        result["variants"]["no_bucket_mask"] = set_variant(q, v, rot, do, args.steps, cfg, hip, True, False)
        result["variants"]["dup_by_bucket"] = set_variant(q, v, rot, do, args.steps, cfg, hip, True, True, True)
        torch.cuda.empty_cache()
        result["variants"]["chunked_ff"] = ff_variant(args.steps, cfg.batch * cfg.seq_len)
        if "gemm_tflops" in result:
            ff = result["variants"]["chunked_ff"]
            ff["frac_of_gemm"] = ff["tflops"] / result["gemm_tflops"]
    del q, v, rot, do
    torch.cuda.empty_cache()
    if args.cpu_heads > 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(x, args.cpu_heads)
    else:
        result["cpu_baseline"] = None
    del x
    # the other workloads, each its own full training step on its own inputs (parity cases of the
    # tests; reported here for their throughput and the roofline of their dominant kernel)
    others = [w for w in (args.workloads.split(",") if args.workloads else []) if w and w != cfg.name]
    if others:
        result["workloads"] = {}
    for name in others:
        t0 = time.perf_counter()
        xw = gen.generate(gen.CONFIGS[name], with_grad=True)
        print(f"[bench] workload {name}: inputs in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
        wr = measure_workload(xw, args.steps, args.warmup, hip, gtf)
        result["workloads"][name] = {k: wr[k] for k in ("config", "ms_per_step", "value", "unit", "roofline",
                                                        "kernels")}
        del xw
        torch.cuda.empty_cache()
    print(json.dumps(result), flush=True)
    return 0


def measure_workload(x, steps: int, warmup: int, hip, gtf, keep: bool = False) -> dict:
    """One workload's training step (forward + saved-records backward) on its seeded inputs.

    1. warmup - 1 untimed steps;
    2. a profiled pass of min(steps, 10) steps with every kernel bracketed by HIP events in every
       step: the per-kernel table (average launch duration over those steps; prep and tiles
       launch twice per step and their bracket holds the backward's launch);
    3. the timed region: `steps` steps, wall clock around them (synchronised on both sides), with
       only the dominant kernel bracketed by HIP events on the stream it is launched on (the
       current torch stream); its average launch duration over the timed steps gives the roofline.
    """
    import numpy as np
    import torch
    import lsh_sparse_attention_amd as lsh
    from lsh_sparse_attention_amd import _lib
    cfg = x["cfg"]

    def dev(a):
        a = np.ascontiguousarray(a)
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    q, v, rot, do = dev(x["q"]), dev(x["v"]), dev(x["rot"]), dev(x["dout"])
    prob = lsh.problem(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.n_hashes, cfg.n_buckets,
                       cfg.chunk_len, cfg.scale, cfg.dtype)
    mod = lsh.LshAttention(prob)
    L = _lib.lib()
    nk = len(_lib.KERNELS)

    def step():
        mod.forward(q, v, rot)
        mod.backward(q, v, do)

    for _ in range(max(1, warmup - 1)):
        step()
    torch.cuda.synchronize()
    # profiled pass: every kernel bracketed in every step
    nprof = max(1, min(steps, 10))
    sums, counts = [0.0] * nk, [0] * nk
    for _ in range(nprof):
        evs = [(hip.event(), hip.event()) for _ in range(nk)]
        for k, (a, b) in enumerate(evs):
            L.lsh_profile_kernel(k, a, b)
        step()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(evs):
            ms = hip.elapsed_ms(a, b, missing_ok=True)   # kernels the problem does not launch are left out
            if ms is not None:
                sums[k] += ms * 1e3
                counts[k] += 1
            L.lsh_profile_kernel(k, None, None)
            hip.destroy(a)
            hip.destroy(b)
    per_kernel = {_lib.KERNELS[k]: sums[k] / counts[k] for k in range(nk) if counts[k]}
    dominant = max(per_kernel, key=per_kernel.get)
    dk = _lib.KERNELS.index(dominant)

    # timed region: K steps, the dominant kernel bracketed on the current torch stream
    pairs = [(hip.event(), hip.event()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in pairs:
        L.lsh_profile_kernel(dk, a, b)
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    L.lsh_profile_kernel(dk, None, None)
    kern_ms = sum(hip.elapsed_ms(a, b) for a, b in pairs) / len(pairs)
    for a, b in pairs:
        hip.destroy(a)
        hip.destroy(b)

    flops, nbytes = algorithmic_work(dominant, cfg)
    t_mfma = flops / (MFMA_PEAK_TFLOPS[cfg.dtype] * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    if t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": flops / (kern_ms * 1e-3) / 1e12, "peak": MFMA_PEAK_TFLOPS[cfg.dtype],
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": nbytes / (kern_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = stored_traffic(dominant, cfg.name)
    roof["dram_traffic"] = stored_traffic(dominant, cfg.name, key="dram_bytes_per_launch")
    roof["kernel"] = dominant
    roof["kernel_us"] = kern_ms * 1e3                     # timed region, this kernel's events
    roof["kernel_us_profiled_pass"] = per_kernel[dominant]  # the per-kernel table's figure
    roof["algorithmic"] = {"flops": flops, "bytes": nbytes}
    if flops:
        roof["mfma_frac_nominal"] = flops / (kern_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[cfg.dtype]
    out = {
        "config": {"workload": WORKLOAD_NAMES.get(cfg.name, cfg.name), "name": cfg.name, "batch": cfg.batch,
                   "heads": cfg.heads, "seq_len": cfg.seq_len, "head_dim": cfg.head_dim,
                   "n_buckets": cfg.n_buckets, "n_hashes": cfg.n_hashes, "chunk_len": cfg.chunk_len,
                   "causal": True, "clustered_inputs": cfg.clustered, "dtype": cfg.dtype},
        "ms_per_step": elapsed * 1e3 / steps,
        "value": cfg.batch * cfg.seq_len * steps / elapsed, "unit": "tokens/s",
        "roofline": roof,
        "kernels_us": {k: round(u, 2) for k, u in per_kernel.items()},
        "kernels": kernel_rooflines(per_kernel, cfg, gtf),
    }
    if keep:
        out["_mod"], out["_tensors"] = mod, (q, v, rot, do)
    else:
        del mod, q, v, rot, do
    return out


if __name__ == "__main__":
    sys.exit(main())
