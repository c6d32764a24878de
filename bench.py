#!/usr/bin/env python3
"""Throughput of the MiniMax Sparse Attention hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic inputs
already resident in HBM: msa_index_topk (index scores, block max-pool,
top-k), msa_sparse_fwd (block map, sparse attention, LSE merge) and, for the
workloads that train, msa_sparse_bwd (fused main + KL index gradients).
Default workload: B=1, N=131072, H_q=64, H_kv=8, d=128, d_idx=64, block 128,
top-16, bf16, forward + backward.

Prints ONE JSON line.  `roofline` describes the kernel with the largest time
per step, timed live with hipEvents recorded by the library around each of
its launches on the caller's stream; `cpu_baseline` times the fp64 oracle on
a bounded sample of query rows on the host cores.
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

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "MSA fwd+bwd tokens/s at N=128K; sparse-attn TFLOP/s as % of bf16 MFMA peak"

# Source file of each kernel (the measured traffic of a kernel is only
# reported while this file is unchanged since the counters were taken).
KERNEL_SOURCE = {
    "index_topk": "index_topk.hip",
    "fwd_partial": "sparse_fwd.hip",
    "fwd_merge": "sparse_fwd.hip",
    "bwd_main": "sparse_bwd.hip",
    "bwd_idx_lse": "sparse_bwd.hip",
    "bwd_prep": "sparse_bwd.hip",
    "bwd_finalize": "sparse_bwd.hip",
    "bwd_dq_merge": "sparse_bwd.hip",
    "block_map": "block_map.hip",
    "block_items": "block_map.hip",
}


def support_pairs(N: int, block: int, topk: int) -> int:
    """Sum over queries t of |S(t)|: causal, own block forced, every other
    selected block fully visible -> min(k-1, t // block) * block + t % block + 1."""
    t = np.arange(N, dtype=np.int64)
    return int((np.minimum(topk - 1, t // block) * block + t % block + 1).sum())


def valid_slots(N: int, block: int, topk: int) -> int:
    """Sum over queries t of the selected blocks that exist (causal): min(k, t // block + 1)."""
    t = np.arange(N, dtype=np.int64)
    return int(np.minimum(topk, t // block + 1).sum())


def algorithmic_work(w) -> dict:
    """Algorithmic work of one launch of each kernel (flops or bytes)."""
    pairs = support_pairs(w.N, w.block_size, w.topk) * w.B          # (t, u) pairs per group/head
    esz = 2 if w.dtype == "bf16" else 4
    vis = w.B * w.N * (w.N + 1) // 2                                # causally visible (t, u)
    slots = valid_slots(w.N, w.block_size, w.topk) * w.B            # (t, selected block) per group/head
    out = {
        "index_topk": ("flop", 2.0 * w.d_idx * vis * w.H_kv),
        "fwd_partial": ("flop", 4.0 * w.d * pairs * w.H_q),
        "bwd_main": ("flop", (10.0 * w.d * w.H_q + 6.0 * w.d_idx * w.H_kv) * pairs),
        "bwd_idx_lse": ("flop", 2.0 * w.d_idx * pairs * w.H_kv),
        # merges: read a (t, h)'s partials of its valid slots, write its row
        "fwd_merge": ("byte", float(w.H_q * (slots * (w.d * esz + 4) + w.B * w.N * (w.d * esz + 4)))),
        "bwd_dq_merge": ("byte", float(w.H_q * (slots * w.d * 2 + w.B * w.N * w.d * esz))),
    }
    return out


# Symbol of each kernel in the library (for matching counter records).
KERNEL_SYMBOL = {
    "index_topk": "index_topk_kernel",
    "fwd_partial": "sparse_fwd_kernel",
    "fwd_merge": "fwd_merge_kernel",
    "bwd_main": "bwd_main16_kernel",
    "bwd_idx_lse": "idx_lse_kernel",
}
# The calibration copy: torch.neg over fp32, one read and one write of the buffer.
COPY_SYMBOL = "neg_kernel"


def source_sha(kernel: str) -> str | None:
    """sha256 over the kernel's source file and the shared device header it
    includes (work-item mapping, MFMA helpers)."""
    f = KERNEL_SOURCE.get(kernel)
    if f is None:
        return None
    h = hashlib.sha256()
    for name in (f, "msa_internal.h"):
        h.update(open(os.path.join(ROOT, "block_sparse_attention_branch_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def _counter_per_dispatch(csv_path: str, symbol: str, counter: str) -> list[float]:
    """Values of `counter` (summed over its instances) per dispatch of the
    kernels whose name contains `symbol`, from a rocprofv3 counter CSV."""
    import csv
    per = {}
    with open(csv_path, newline="") as f:
        for r in csv.DictReader(f):
            if symbol in r["Kernel_Name"] and r["Counter_Name"] == counter:
                per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(per.values())


def write_traffic(kernel: str, workload: str, fetch_csv: str, write_csv: str, copy_mib: int, command: str):
    """HBM bytes per launch of `kernel` from two counter runs (FETCH_SIZE, then
    WRITE_SIZE, both in KiB per dispatch), each scaled by the ratio of the known
    bytes of the calibration copy to what the same counter read for it."""
    sym = KERNEL_SYMBOL[kernel]
    copy_bytes = copy_mib * 2.0 ** 20
    out = {"kernel": kernel, "workload": workload, "source_sha256": source_sha(kernel), "command": command,
           "copy_bytes": copy_bytes}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = _counter_per_dispatch(path, sym, counter)
        cal = _counter_per_dispatch(path, COPY_SYMBOL, counter)
        if not vals or not cal:
            raise SystemExit(f"{path}: no {counter} records for {sym} or the calibration copy")
        kib = float(np.mean(vals))
        factor = copy_bytes / (float(np.median(cal)) * 1024.0)
        out[counter] = {"kib_per_dispatch": kib, "dispatches": len(vals), "copy_kib": float(np.median(cal)),
                        "factor": factor, "bytes": kib * 1024.0 * factor}
        total += kib * 1024.0 * factor
    out["bytes_per_launch"] = total
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def cpu_baseline(w, x, rows_n: int, seed: int = 0) -> dict | None:
    """Time the fp64 oracle (as it is) on `rows_n` query rows of batch 0:
    index branch, forward and backward of those rows, on the host cores."""
    if rows_n <= 0:
        return None
    from threadpoolctl import threadpool_info
    from oracle import msa_oracle as O
    import torch

    rng = np.random.default_rng(seed)
    ts = np.unique(np.concatenate([[0, w.N - 1], rng.integers(0, w.N, size=rows_n)]))[:rows_n]
    rows = [(0, int(t)) for t in ts]
    bt = torch.tensor(rows, dtype=torch.long)
    f32 = lambda t: t.detach().float().cpu().numpy()
    k, v, ki = f32(x["k"]), f32(x["v"]), f32(x["k_idx"])
    q, qi = f32(x["q"][bt[:, 0], bt[:, 1]]), f32(x["q_idx"][bt[:, 0], bt[:, 1]])
    dO = f32(x["dO"][bt[:, 0], bt[:, 1]]) if "dO" in x else None
    t0 = time.perf_counter()
    sel_rows = O.index_topk(qi, ki, w.block_size, w.topk, causal=w.causal, rows=rows)
    sel = np.full((w.B, w.N, w.H_kv, w.topk), -1, dtype=np.int64)
    for i, (b, t) in enumerate(rows):
        sel[b, t] = sel_rows[i]
    O.sparse_fwd(q, k, v, sel, w.block_size, w.causal, rows=rows)
    if w.backward:
        O.sparse_bwd(q, k, v, dO, qi, ki, sel, w.block_size, w.causal, rows=rows)
    dt = time.perf_counter() - t0
    threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    # Rows are drawn uniformly, so the sample's time per row estimates the mean
    # over all rows; the whole workload's time is that rate extrapolated.
    whole_s = dt / len(rows) * w.B * w.N
    return {
        "value": len(rows) / dt,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "extrapolated": True,
        "sample": (f"measured on {len(rows)} seeded uniform query rows of batch 0 of {w.name} (every group and "
                   f"head): index scores/max-pool/top-k, sparse forward" + (" and backward" if w.backward else "") +
                   f" in fp64 NumPy, {dt:.1f} s; the rate is extrapolated to all {w.B * w.N} rows "
                   f"(about {whole_s / 3600:.0f} h for one step)"),
    }


def torch_index_topk(q_idx, k_idx, topk: int, block: int, softmax: bool = True, chunk: int = 2048,
                     score_dtype=None, pooled_out=None):
    """Index top-k the plain PyTorch way, for the comparison with the fused
    kernel: materialise the causal index scores of a chunk of queries
    (q_idx k_idx^T over the visible keys), max-pool them per block, optionally
    take the softmax over the visible blocks, force each query's own block and
    call torch.topk.  Returns block_idx [B,N,H_kv,topk] int32, ascending, -1
    padded, like msa_index_topk.  score_dtype: dtype of the score product
    (default: the inputs' dtype, as torch.matmul does).  pooled_out: optional
    fp32 [B,N,H_kv,N/block] that receives the pooled scores (-inf where
    invisible, own block not forced)."""
    import torch
    B, N, H_kv, di = q_idx.shape
    dev = q_idx.device
    out = torch.full((B, N, H_kv, topk), -1, dtype=torch.int32, device=dev)
    ar = torch.arange(N, device=dev)
    big = torch.iinfo(torch.int32).max
    for b in range(B):
        kt = k_idx[b].t().contiguous()                              # [d_idx, N]
        if score_dtype is not None:
            kt = kt.to(score_dtype)
        for c0 in range(0, N, chunk):
            c1 = min(N, c0 + chunk)
            C, nb = c1 - c0, (c1 + block - 1) // block               # blocks visible to the chunk
            U = nb * block
            q = q_idx[b, c0:c1].reshape(C * H_kv, di)
            if score_dtype is not None:
                q = q.to(score_dtype)
            r = torch.matmul(q, kt[:, :U].contiguous()).view(C, H_kv, U).float()
            r.masked_fill_(ar[:U].view(1, 1, U) > ar[c0:c1].view(C, 1, 1), float("-inf"))
            pooled = r.view(C, H_kv, nb, block).amax(-1)           # [C, H_kv, nb]; -inf where invisible
            if pooled_out is not None:
                pooled_out[b, c0:c1, :, :nb] = pooled
                pooled_out[b, c0:c1, :, nb:] = float("-inf")
            if softmax:
                pooled = torch.softmax(pooled, dim=-1)              # invisible blocks -> 0
                pooled = torch.where(torch.isfinite(r.view(C, H_kv, nb, block)[..., 0]), pooled,
                                     torch.full_like(pooled, -1.0))
            own = (ar[c0:c1] // block).view(C, 1, 1).expand(C, H_kv, 1)
            pooled.scatter_(2, own, float("inf"))
            k = min(topk, nb)
            val, idx = torch.topk(pooled, k, dim=-1)
            invisible = (val < 0) if softmax else torch.isinf(val) & (val < 0)
            idx = torch.where(invisible, torch.full_like(idx, big), idx)
            idx = torch.sort(idx, dim=-1).values
            idx = torch.where(idx == big, torch.full_like(idx, -1), idx)
            out[b, c0:c1, :, :k] = idx.to(torch.int32)
    return out


def compare_topk(args) -> int:
    """Fused index top-k against the materialise-then-torch.topk pipeline on
    the index inputs of `args.workload`: one JSON line with both times."""
    import torch
    import block_sparse_attention_branch_amd as msa
    import msa_inputs
    msa.load_library()
    w = msa_inputs.WORKLOADS[args.workload]
    x = msa_inputs.make_inputs(w, args.variant, device="cuda")
    qi, ki = x["q_idx"], x["k_idx"]

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            res = fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps, res

    ours_ms, sel = timed(lambda: msa.index_topk(qi, ki, topk=w.topk, block_size=w.block_size, causal=True), 10)
    soft_ms, ref_soft = timed(lambda: torch_index_topk(qi, ki, w.topk, w.block_size, softmax=True), 3)
    raw_ms, ref_raw = timed(lambda: torch_index_topk(qi, ki, w.topk, w.block_size, softmax=False), 3)
    agree = float((torch.sort(sel, dim=-1).values == torch.sort(ref_raw, dim=-1).values).all(-1).float().mean())
    # The top-k stage alone on materialised pooled scores (what an exp-free
    # top-k replaces): softmax over the visible blocks (or none), own block
    # forced, torch.topk.  The fused kernel above also forms the scores.
    nblk = w.N // w.block_size
    pooled = torch.empty(w.B, w.N, w.H_kv, nblk, dtype=torch.float32, device="cuda")
    torch_index_topk(qi, ki, w.topk, w.block_size, softmax=False, pooled_out=pooled)
    own = (torch.arange(w.N, device="cuda") // w.block_size).view(1, w.N, 1, 1).expand(w.B, w.N, w.H_kv, 1)

    def stage(softmax):
        p = torch.softmax(pooled, dim=-1) if softmax else pooled.clone()
        p.scatter_(3, own, 2.0 if softmax else float("inf"))
        return torch.topk(p, w.topk, dim=-1)

    stage_soft_ms, _ = timed(lambda: stage(True), 3)
    stage_raw_ms, _ = timed(lambda: stage(False), 3)
    del pooled
    line = {"metric": "index top-k ms (fused kernel vs materialise + torch.topk)", "workload": w.name,
            "config": {"B": w.B, "N": w.N, "H_kv": w.H_kv, "d_idx": w.d_idx, "block_size": w.block_size,
                       "topk": w.topk, "dtype": w.dtype},
            "fused_ms": ours_ms, "torch_softmax_topk_ms": soft_ms, "torch_topk_ms": raw_ms,
            "speedup_vs_softmax_topk": soft_ms / ours_ms, "speedup_vs_topk": raw_ms / ours_ms,
            "topk_stage_softmax_ms": stage_soft_ms, "topk_stage_ms": stage_raw_ms,
            "speedup_vs_topk_stage_softmax": stage_soft_ms / ours_ms,
            "rows_identical_to_torch_topk": agree,
            "note": "torch pipeline: bf16 score product per 2048-query chunk over the visible keys, causal mask, "
                    "block max-pool, (softmax), own block forced, torch.topk, sort; topk_stage_*: softmax (or "
                    "none) + own block + torch.topk on the materialised fp32 pooled scores [B,N,H_kv,N/128]"}
    print(json.dumps(line), flush=True)
    return 0


def index_only(args) -> int:
    """The index branch alone (msa_index_topk) on the index inputs of
    `args.workload`, with bf16 and with FP8 E4M3 inputs: one JSON line with
    each kernel's time (library hipEvents) and its rate against its dtype's
    dense MFMA peak."""
    import torch
    import block_sparse_attention_branch_amd as msa
    import msa_inputs
    msa.load_library()
    w = msa_inputs.WORKLOADS[args.workload]
    flop = algorithmic_work(w)["index_topk"][1]
    res = {}
    for name, fp8, peak in (("bf16", False, PEAK_BF16_TFLOPS), ("fp8_e4m3", True, PEAK_FP8_TFLOPS)):
        x = msa_inputs.make_inputs(w, args.variant, device="cuda", index_fp8=fp8)
        qi, ki = x["q_idx"], x["k_idx"]
        del x
        for _ in range(args.warmup):
            msa.index_topk(qi, ki, topk=w.topk, block_size=w.block_size, causal=w.causal)
        torch.cuda.synchronize()
        msa.profile_enable(True)
        msa.profile_collect()
        for _ in range(args.steps):
            msa.index_topk(qi, ki, topk=w.topk, block_size=w.block_size, causal=w.causal)
        torch.cuda.synchronize()
        launches, total_ms = msa.profile_collect()["index_topk"]
        msa.profile_enable(False)
        ms = total_ms / launches
        tf = flop / (ms * 1e-3) / 1e12
        res[name] = {"ms": ms, "achieved": tf, "unit": "TFLOP/s", "peak": peak, "frac": tf / peak}
        del qi, ki
        torch.cuda.empty_cache()
    line = {"metric": "index top-k (scores + block max-pool + top-k) ms and MFMA rate", "workload": w.name,
            "config": {"B": w.B, "N": w.N, "H_kv": w.H_kv, "d_idx": w.d_idx, "block_size": w.block_size,
                       "topk": w.topk}, "flop_per_launch": flop, "steps": args.steps, "warmup": args.warmup,
            "kernels": res, "fp8_speedup": res["bf16"]["ms"] / res["fp8_e4m3"]["ms"]}
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="fwdbwd-bf16-n128k")
    ap.add_argument("--variant", default="normal", choices=["normal", "int", "planted"])
    ap.add_argument("--cpu-rows", type=int, default=512, help="query rows for the oracle baseline (0: skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, run a plain fp32 copy (torch.neg) of this many MiB three times: "
                         "the known-size kernel that calibrates the HBM byte counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 counter CSVs (FETCH_SIZE, WRITE_SIZE) of this workload, "
                         "taken with --copy-mib, into profiles/traffic_<kernel>_<workload>.json")
    ap.add_argument("--traffic-kernel", default="bwd_main")
    ap.add_argument("--traffic-command", default="", help="the rocprofv3 command the CSVs came from (recorded)")
    ap.add_argument("--compare-topk", action="store_true",
                    help="time the fused index top-k against a materialise + torch.topk pipeline (index inputs "
                         "of --workload) and print one JSON line")
    ap.add_argument("--index-only", action="store_true",
                    help="time msa_index_topk alone with bf16 and with FP8 E4M3 index inputs of --workload")
    args = ap.parse_args()

    if args.traffic_from:
        write_traffic(args.traffic_kernel, args.workload, *args.traffic_from, args.copy_mib or 1024,
                      args.traffic_command)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: libmsa has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import block_sparse_attention_branch_amd as msa
    import msa_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.compare_topk:
        return compare_topk(args)
    if args.index_only:
        return index_only(args)
    msa.load_library()
    w = msa_inputs.WORKLOADS[args.workload]
    x = msa_inputs.make_inputs(w, args.variant, device="cuda")
    torch.cuda.synchronize()

    def step():
        sel = msa.index_topk(x["q_idx"], x["k_idx"], topk=w.topk, block_size=w.block_size, causal=w.causal)
        o, lse = msa.sparse_fwd(x["q"], x["k"], x["v"], sel, d_idx=w.d_idx, block_size=w.block_size,
                                causal=w.causal)
        if w.backward:
            msa.sparse_bwd(x["q"], x["k"], x["v"], o, x["dO"], lse, sel, x["q_idx"], x["k_idx"],
                           block_size=w.block_size, causal=w.causal)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    msa.profile_enable(True)
    msa.profile_collect()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof = msa.profile_collect()
    msa.profile_enable(False)
    if args.copy_mib > 0:
        src = torch.randn(args.copy_mib * 2 ** 18, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = w.B * w.N * args.steps / elapsed
    work = algorithmic_work(w)
    kernels = {}
    for name, (launches, total_ms) in sorted(prof.items(), key=lambda kv: -kv[1][1]):
        rec = {"ms_per_step": total_ms / args.steps, "launches_per_step": launches / args.steps}
        if name in work:
            kind, amount = work[name]
            per_launch = amount / max(1, launches // args.steps)
            avg_ms = total_ms / launches
            if kind == "flop":
                rec.update(achieved=per_launch / (avg_ms * 1e-3) / 1e12, unit="TFLOP/s")
                rec["frac"] = rec["achieved"] / PEAK_BF16_TFLOPS
            else:
                rec.update(achieved=per_launch / (avg_ms * 1e-3) / 1e9, unit="GB/s")
                rec["frac"] = rec["achieved"] / PEAK_HBM_GBS
        kernels[name] = rec
    dominant = max(prof.items(), key=lambda kv: kv[1][1])[0]
    launches, total_ms = prof[dominant]
    kind, amount = work.get(dominant, ("flop", float("nan")))
    per_launch = amount / max(1, launches // args.steps)
    avg_ms = total_ms / launches
    if kind == "flop":
        achieved, peak, unit, bound = per_launch / (avg_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = per_launch / (avg_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    roofline = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
                "traffic": measured_traffic(dominant, w.name), "kernel": dominant,
                "avg_launch_ms": avg_ms, "work_per_launch": per_launch}

    sparse_flop = work["fwd_partial"][1] + (work["bwd_main"][1] if w.backward else 0.0)
    sparse_ms = sum(prof.get(n, (0, 0.0))[1] for n in ("block_map", "block_items", "fwd_partial", "fwd_merge",
                                                        "bwd_prep", "bwd_idx_lse", "bwd_main", "bwd_dq_merge",
                                                        "bwd_finalize"))
    sparse_ms /= args.steps
    sparse_tflops = sparse_flop / (sparse_ms * 1e-3) / 1e12 if sparse_ms > 0 else None

    cpu = cpu_baseline(w, x, args.cpu_rows)

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": f"synthetic ({args.variant}, seeded)",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H_q": w.H_q, "H_kv": w.H_kv, "d": w.d,
                   "d_idx": w.d_idx, "block_size": w.block_size, "topk": w.topk, "causal": w.causal,
                   "backward": w.backward, "parallelism": "single-gpu"},
        "sparse_attn_tflops": sparse_tflops,
        "sparse_attn_frac_of_bf16_peak": (sparse_tflops / PEAK_BF16_TFLOPS) if sparse_tflops else None,
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
