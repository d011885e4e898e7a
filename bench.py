"""Throughput of the DSA hot path (lightning indexer -> top-k -> sparse MQA
attention) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_128k]
    python bench.py --copy-calibration MIB   (a plain device copy, for counters)

A step is one dsa_forward call over one batch of seeded synthetic inputs that
are already resident in HBM.  The default workload is decode at 128K context:
64 sequences, each one new query token against a 131072-token cache (FP8
indexer keys [131072,128] and bf16 latent KV [131072,576] per sequence,
8 indexer heads, k = 2048, 128 query heads, value dim 512).  Prints one JSON
line; ``value`` is query tokens per second.  The line also carries the
roofline position of the step's dominant kernel and the CPU oracle's
throughput on a bounded sample of the same workload.

Per-part times come from a second timed loop that calls the two entry points
whose kernels dsa_forward runs (indexer scores + top-k selection, then sparse
attention) one after the other with HIP events recorded between them on the
stream they are launched on, so each runs in the cache state it has inside a
step; a third loop times the standalone score and top-k kernels the same
way.  The measured HBM traffic of the dominant
kernel is read from its rocprofv3 counter summary under profiles/ when that
summary was taken on the current kernel source, else it is null.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import long_context_02_amd as dsa  # noqa: E402
from long_context_02_amd.synth import WORKLOADS, make_inputs  # noqa: E402

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0     # dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0    # dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
KERNEL_SOURCES = {"cache_append": ("cache.hip",),
                  "attn_bwd": ("attention_bwd.hip", "attn_common.h"),
                  "indexer_kl": ("kl.hip",),
                  "select": ("indexer.hip", "topk.hip", "indexer_math.h", "topk_select.h"),
                  "indexer": ("indexer.hip", "indexer_math.h", "topk_select.h"),
                  "topk": ("topk.hip", "indexer_math.h", "topk_select.h"),
                  "attention": ("attention.hip", "attn_common.h")}


def source_hash(phase):
    """sha256 over the kernel sources of a phase (in a fixed order)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[phase]:
        with open(os.path.join(ROOT, "long_context_02_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work of one step (what the method must do, not what it skips)
def work(wl):
    """Algorithmic FLOP and HBM bytes of each phase: what the method must do,
    not the dense work it avoids and not the implementation's intermediates
    (the fp32 score matrix, split partials) -- those show up in the measured
    traffic instead."""
    t = np.arange(wl.T, dtype=np.int64)
    n_cand = np.minimum(wl.N, wl.q_offset + t + 1)
    n_sel = np.minimum(wl.k, n_cand)
    idx_pairs = int(n_cand.sum()) * wl.B
    attn_pairs = int(n_sel.sum()) * wl.B
    keys_read = min(wl.N, wl.q_offset + wl.T) * wl.B
    fp8 = wl.dtype == "bf16"
    key_bytes = wl.d_I + 4 if fp8 else 4 * wl.d_I
    qrow_bytes = wl.H_I * (wl.d_I + 8) if fp8 else wl.H_I * (4 * wl.d_I + 4)
    el = 2 if fp8 else 4
    kv_row = wl.d_qk * el
    # a selected latent row is read once per query token when the tokens of a
    # sequence select disjoint rows (decode), and once per sequence when many
    # tokens share the cache-resident rows (prefill, chunk): at least the
    # smaller of the two
    gathered_rows = min(attn_pairs, keys_read)
    return {
        "indexer": {
            "flops": idx_pairs * 2 * wl.H_I * wl.d_I,
            "bytes": keys_read * key_bytes + wl.B * wl.T * qrow_bytes,
            "flop_unit": "fp8" if fp8 else "f32",
        },
        "topk": {"flops": 0, "bytes": idx_pairs * 4 + wl.B * wl.T * wl.k * 4, "flop_unit": None},
        # scores and selection as one step: the indexer's inputs in, the
        # selected indices out (the scores are an intermediate)
        "select": {
            "flops": idx_pairs * 2 * wl.H_I * wl.d_I,
            "bytes": keys_read * key_bytes + wl.B * wl.T * qrow_bytes + wl.B * wl.T * wl.k * 4,
            "flop_unit": "fp8" if fp8 else "f32",
        },
        "attention": {
            "flops": attn_pairs * 2 * wl.H * (wl.d_qk + wl.d_v),
            "bytes": gathered_rows * kv_row + wl.B * wl.T * (wl.H * (wl.d_qk + wl.d_v) * el + wl.k * 4),
            "flop_unit": "bf16" if fp8 else "f32",
        },
    }


def phase_floor(w):
    """Seconds a phase needs at the published peaks: max(FLOP / MFMA peak, bytes / HBM)."""
    peak_f = {"fp8": PEAK_FP8_TFLOPS, "bf16": PEAK_BF16_TFLOPS, "f32": PEAK_F32_TFLOPS}.get(w["flop_unit"])
    t_mem = w["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_cmp = w["flops"] / (peak_f * 1e12) if peak_f else 0.0
    return max(t_mem, t_cmp)


def roofline(phase, w, seconds):
    """Roofline position of one kernel: which roof binds, and the achieved rate."""
    peak_f = {"fp8": PEAK_FP8_TFLOPS, "bf16": PEAK_BF16_TFLOPS, "f32": PEAK_F32_TFLOPS}.get(w["flop_unit"])
    t_mem = w["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_cmp = w["flops"] / (peak_f * 1e12) if peak_f else 0.0
    if t_cmp > t_mem:
        ach = w["flops"] / seconds / 1e12
        return {"kernel": phase, "bound": "mfma", "achieved": round(ach, 2), "peak": peak_f,
                "unit": "TFLOP/s", "frac": round(ach / peak_f, 4), "algorithmic": w["flops"]}
    ach = w["bytes"] / seconds / 1e9
    return {"kernel": phase, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "algorithmic": w["bytes"]}


def measured_traffic(phase, wl):
    """HBM bytes per launch of `phase` on `wl` from the counter summary in
    profiles/ (FETCH_SIZE + WRITE_SIZE, scaled by the plain-copy calibration),
    or None when there is none or it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{phase}_{wl.name}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                key, val = ln.split("=", 1)
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != source_hash(phase) or "hbm_bytes_per_launch" not in fields:
        return None
    return int(fields["hbm_bytes_per_launch"])


def copy_calibration(mib):
    """A plain device-to-device copy of a known size, for scaling the HBM
    byte counters (each launch reads and writes mib MiB)."""
    dev = torch.device("cuda:0")
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 3}), flush=True)


# ---------------------------------------------------------------------------
def timed(fn, steps, stream):
    """Average milliseconds of fn() over `steps` launches, HIP events on `stream`."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def timed_sequence(parts, steps, warmup, stream):
    """Average milliseconds of each callable when all are called in sequence,
    `steps` times, with HIP events recorded between them on `stream`."""
    names = list(parts)
    for _ in range(warmup):
        for fn in parts.values():
            fn()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        for j, name in enumerate(names):
            parts[name]()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    return {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)]))
            for j, name in enumerate(names)}


def time_cache_append(wl, g, steps, stream):
    """dsa_cache_append of B*T new tokens at rows q_offset.. of each sequence
    (after the timed steps; it overwrites those cache rows).  HBM-bound:
    bytes = new key rows read + key codes/scales written + latent rows read
    and written + positions."""
    dev = g["kv"].device
    gen = torch.Generator(device=dev).manual_seed(1)
    k_new = torch.randn(wl.B, wl.T, wl.d_I, generator=gen, device=dev)
    kv_new = torch.randn(wl.B, wl.T, wl.d_qk, generator=gen, device=dev).to(g["kv"].dtype)
    pos = torch.full((wl.B,), wl.q_offset, dtype=torch.int32, device=dev)

    dsa.cache_append(k_new, kv_new, g["k_idx"], g["k_idx_scale"], g["kv"], pos)  # checks the arguments
    # then the entry point itself with prepared arguments, so that the host
    # keeps ahead of this short kernel
    L = dsa.lib()
    ks = g["k_idx_scale"]
    fp8 = ks is not None
    args = [ctypes.c_void_p(k_new.data_ptr()), ctypes.c_void_p(kv_new.data_ptr()),
            ctypes.c_void_p(g["k_idx"].data_ptr()), ctypes.c_void_p(ks.data_ptr()) if fp8 else None,
            ctypes.c_void_p(g["kv"].data_ptr()), ctypes.c_void_p(pos.data_ptr()),
            wl.B, wl.T, wl.N, wl.d_I, wl.d_qk, dsa.FP8_E4M3FN if fp8 else dsa.F32,
            dsa.BF16 if g["kv"].dtype == torch.bfloat16 else dsa.F32,
            ctypes.c_void_p(stream.cuda_stream)]

    def fn():
        L.dsa_cache_append(*args)

    for _ in range(3):
        fn()
    ms = timed(fn, 10 * steps, stream)
    rows = wl.B * wl.T
    kv_row = wl.d_qk * g["kv"].element_size()
    nbytes = rows * (4 * wl.d_I + ((wl.d_I + 4) if fp8 else 4 * wl.d_I) + 2 * kv_row) + 4 * wl.B
    ach = nbytes / (ms / 1e3) / 1e9
    return {"ms": round(ms, 4), "tokens": rows, "bound": "hbm", "achieved": round(ach, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
            "algorithmic": nbytes}


def time_indexer_kl(wl, scores, idx, steps, stream):
    """dsa_indexer_kl over the step's [B,T,N] score rows with a random target
    (dense: HBM-bound, I and p read over the causal candidates, the gradient
    written over whole rows), then over the k selected slots of each row."""
    dev = scores.device
    gen = torch.Generator(device=dev).manual_seed(2)
    p = torch.rand(scores.shape, generator=gen, device=dev)
    p /= p.sum(-1, keepdim=True)
    p_sel = torch.rand(idx.shape, generator=gen, device=dev)
    p_sel /= p_sel.sum(-1, keepdim=True)
    out = {}
    t = np.arange(wl.T, dtype=np.int64)
    n_cand = int(np.minimum(wl.N, wl.q_offset + t + 1).sum()) * wl.B
    rows = wl.B * wl.T
    for name, fn, nbytes in (
            ("indexer_kl_dense", lambda: dsa.indexer_kl(scores, p, wl.q_offset),
             8 * n_cand + 4 * rows * wl.N + 4 * rows),
            ("indexer_kl_sparse", lambda: dsa.indexer_kl(scores, p_sel, idx=idx),
             16 * rows * wl.k + 4 * rows)):
        for _ in range(2):
            fn()
        ms = timed(fn, steps, stream)
        ach = nbytes / (ms / 1e3) / 1e9
        out[name] = {"ms": round(ms, 4), "rows": rows, "bound": "hbm", "achieved": round(ach, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "algorithmic": nbytes}
    return out


def time_attn_bwd(wl, g, idx, steps, stream):
    """dsa_sparse_mla_attn_bwd on the step's selection with a random output
    gradient (the sparse training stage's attention backward).  Algorithmic
    work per valid slot and head: 2 x (576 + 512) FLOP to recompute the logit
    and form dP, 2 x 576 for dq, 2 x (576 + 512) for the latent gradient;
    bytes: q, out, dout and lse read, dq written, the selected latent rows
    gathered once, dkv written once."""
    dev = g["q"].device
    B, T, N = wl.B, wl.T, wl.N
    out, lse = dsa.sparse_mla_attn(g["q"], g["kv"], idx, wl.d_v, wl.sm_scale)
    gen = torch.Generator(device=dev).manual_seed(3)
    dout = torch.randn(out.shape, generator=gen, device=dev, dtype=out.dtype)
    dq = torch.empty(B, T, wl.H, wl.d_qk, dtype=torch.float32, device=dev)
    dkv = torch.empty(B, N, wl.d_qk, dtype=torch.float32, device=dev)
    ws = torch.empty(dsa.workspace_size(dsa.OP_ATTN_BWD, B, T, N, wl.H_I, wl.H, wl.d_v, wl.k),
                     dtype=torch.uint8, device=dev)

    def fn():
        dsa.sparse_mla_attn_bwd(g["q"], g["kv"], idx, out, lse, dout, wl.sm_scale, dq=dq, dkv=dkv,
                                workspace=ws)

    for _ in range(2):
        fn()
    ms = timed(fn, steps, stream)
    n_valid = int(((idx >= 0) & (idx < N)).sum().item())
    rows = B * T
    flop = 2.0 * (576 + 512 + 576 + 576 + 512) * wl.H * n_valid
    nbytes = (rows * wl.H * (2 * wl.d_qk + 2 * 2 * wl.d_v + 4 + 4 * wl.d_qk) + n_valid * 2 * wl.d_qk
              + B * N * 4 * wl.d_qk)
    ach = flop / (ms / 1e3) / 1e12
    return {"attn_bwd": {"ms": round(ms, 4), "rows": rows, "bound": "mfma", "achieved": round(ach, 1),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach / PEAK_BF16_TFLOPS, 4), "algorithmic_flop": flop,
                         "algorithmic_bytes": nbytes,
                         "hbm_floor_ms": round(nbytes / (PEAK_HBM_GBS * 1e9) * 1e3, 4),
                         "traffic": measured_traffic("attn_bwd", wl)}}


def cpu_baseline(wl, g, budget_s):
    """The CPU oracle on a bounded sample of the same workload: whole rows
    (index scores -> selection -> attention), timed on this host's cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    fp8 = wl.dtype == "bf16"
    rng = np.random.default_rng(0)
    if wl.T == 1:
        order = [(int(b), 0) for b in rng.permutation(wl.B)]
    else:
        order = [(0, int(t)) for t in rng.permutation(wl.T)]
    done, spent = 0, 0.0
    host = {}
    for (b, t) in order:
        if b not in host:  # host copies of this sequence (not timed)
            host = {b: {
                "k": g["k_idx"][b].cpu().numpy() if fp8 else g["k_idx"][b].double().cpu().numpy(),
                "ks": g["k_idx_scale"][b].double().cpu().numpy() if fp8 else None,
                "kv": g["kv"][b].float().cpu().numpy(),
            }}
        h = host[b]
        qi = g["q_idx"][b, t].cpu().numpy() if fp8 else g["q_idx"][b, t].double().cpu().numpy()
        qs = g["q_idx_scale"][b, t].double().cpu().numpy() if fp8 else None
        w = g["w"][b, t].double().cpu().numpy()
        q = g["q"][b, t].double().cpu().numpy()
        t0 = time.perf_counter()
        K = oracle.dequantize(h["k"], h["ks"]) if fp8 else h["k"]
        qrow = oracle.dequantize(qi, qs) if fp8 else qi
        n_cand = min(wl.N, wl.q_offset + t + 1)
        I = oracle.index_scores_row(qrow, w, K, n_cand)
        sel = oracle.topk_select_row(I, wl.k, n_cand)
        oracle.sparse_mqa_attention_row(q, h["kv"], sel, wl.d_v, wl.sm_scale)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    return {"value": round(done / spent, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} query tokens of {wl.name} (whole rows: index scores, top-{wl.k}, "
                      f"attention; float64), {spent:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_128k", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating {wl.name} inputs on {dev}")
    g = make_inputs(wl, seed=0, device=dev)
    B, T, N = wl.B, wl.T, wl.N
    out = torch.empty(B, T, wl.H, wl.d_v, dtype=g["q"].dtype, device=dev)
    ws = torch.empty(dsa.workspace_size(dsa.OP_FORWARD, B, T, N, wl.H_I, wl.H, wl.d_v, wl.k),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        dsa.forward(g["q_idx"], g["k_idx"], g["w"], g["q"], g["kv"], k=wl.k, q_offset=wl.q_offset,
                    d_v=wl.d_v, sm_scale=wl.sm_scale, q_idx_scale=g["q_idx_scale"],
                    k_idx_scale=g["k_idx_scale"], out=out, workspace=ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ms = timed(step, args.steps, stream)

    # the step's two parts, as dsa_forward runs them (scores + selection,
    # then attention), called in sequence through their entry points with
    # HIP events between them on the launch stream; then the standalone
    # score and top-k kernels the same way
    scores = torch.empty(B, T, N, dtype=torch.float32, device=dev)
    idx = torch.empty(B, T, wl.k, dtype=torch.int32, device=dev)
    attn_ws = torch.empty(max(1, dsa.workspace_size(dsa.OP_ATTN, B, T, N, wl.H_I, wl.H, wl.d_v, wl.k)),
                          dtype=torch.uint8, device=dev)
    sel_ws = torch.empty(max(1, dsa.workspace_size(dsa.OP_SELECT, B, T, N, wl.H_I, wl.H, wl.d_v, wl.k)),
                         dtype=torch.uint8, device=dev)
    topk_ws = torch.empty(max(1, dsa.workspace_size(dsa.OP_TOPK, B, T, N, wl.H_I, wl.H, wl.d_v, wl.k)),
                          dtype=torch.uint8, device=dev)
    step_parts = {
        "select": lambda: dsa.indexer_select(g["q_idx"], g["k_idx"], g["w"], wl.k, wl.q_offset,
                                             q_idx_scale=g["q_idx_scale"],
                                             k_idx_scale=g["k_idx_scale"], out=idx, workspace=sel_ws),
        "attention": lambda: dsa.sparse_mla_attn(g["q"], g["kv"], idx, wl.d_v, wl.sm_scale,
                                                 out=out, lse=False, workspace=attn_ws),
    }
    components = {
        "indexer": lambda: dsa.indexer_scores(g["q_idx"], g["k_idx"], g["w"], wl.q_offset,
                                              q_idx_scale=g["q_idx_scale"],
                                              k_idx_scale=g["k_idx_scale"], out=scores),
        "topk": lambda: dsa.topk_select(scores, wl.k, wl.q_offset, out=idx, workspace=topk_ws),
    }
    phase_ms = timed_sequence(step_parts, args.steps, args.warmup, stream)
    comp_ms = timed_sequence(components, args.steps, args.warmup, stream)
    w = work(wl)
    dom = max(phase_ms, key=phase_ms.get)
    roof = roofline(dom, w[dom], phase_ms[dom] / 1e3)
    roof["traffic"] = measured_traffic(dom, wl)
    t_roof = sum(phase_floor(w[p]) for p in ("indexer", "topk", "attention"))
    per_kernel = {}
    for name, t_ms in {**phase_ms, **comp_ms}.items():
        r = roofline(name, w[name], t_ms / 1e3)
        per_kernel[name] = {"ms": round(t_ms, 4), "bound": r["bound"], "achieved": r["achieved"],
                            "unit": r["unit"], "frac": r["frac"]}

    line = {
        "metric": "DSA tokens/s (indexer+top-k+sparse attn) at 128K ctx; % of MFMA / HBM roofline",
        "value": round(B * T / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 indexer / bf16 attention" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded)",
        "config": {"workload": wl.name, "batch": B, "query_tokens": T, "context": N,
                   "q_offset": wl.q_offset, "indexer_heads": wl.H_I, "indexer_dim": wl.d_I,
                   "top_k": wl.k, "heads": wl.H, "d_qk": wl.d_qk, "d_v": wl.d_v,
                   "parallelism": "single GPU"},
        "phases_ms": {k: round(v, 4) for k, v in phase_ms.items()},
        "roofline": roof,
        "kernels": per_kernel,
        # the whole step against the sum of the phases' floors at published peaks
        "step_roofline": {"t_roof_ms": round(t_roof * 1e3, 4),
                          "frac": round(t_roof / (ms / 1e3), 4)},
    }
    # the step before the path (not part of the step): appending this step's
    # new tokens (one per query token) to the key and latent caches
    line["next"] = {"cache_append": time_cache_append(wl, g, args.steps, stream)}
    # the indexer's alignment objective on this step's score rows (dense
    # warm-up form) and on its selected slots (sparse form)
    line["next"].update(time_indexer_kl(wl, scores, idx, args.steps, stream))
    # the sparse attention backward on this step's selection
    if wl.dtype == "bf16":
        line["next"].update(time_attn_bwd(wl, g, idx, args.steps, stream))
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline")
        line["cpu_baseline"] = cpu_baseline(wl, g, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
