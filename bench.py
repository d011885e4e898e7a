"""Throughput of the DSA hot path (lightning indexer -> top-k -> sparse MQA
attention) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_128k]
    python bench.py --copy-calibration MIB   (a plain device copy, for counters)

A step is one dsa_forward call over one batch of seeded synthetic inputs that
are already resident in HBM.  The default workload is decode at 128K context:
64 sequences, each one new query token against a 131072-token cache (FP8
indexer keys [131072,128] and bf16 latent KV [131072,576] per sequence,
8 indexer heads, k = 2048, 128 query heads, value dim 512).  Prints one JSON
line; ``value`` is query tokens per second.

The line also carries:
  kernels     every kernel of the step: average HIP-event duration per launch
              (events recorded around each launch on its stream by the
              library's timing window), launches per step, and its position
              against the roofline that bounds it;
  roofline    the same for the step's dominant kernel (the one with the most
              time per step), with the fraction of the published peak and of
              the peak measured on this GPU (a streaming read, vendor GEMMs);
  phases_ms   selection and attention timed as the two entry points the
              step runs, called in sequence with HIP events between them;
  chunk_128k  with the default workload, the same measurements for chunked
              prefill at 128K (the indexer's FP8 target is judged there);
  the benchmark spec  the decode attention's HBM fraction and the chunked-prefill
              indexer's FP8 MFMA fraction;
  next        the neighbouring steps (cache append, the indexer's KL
              objective, the attention backward, MHA-mode attention);
  cpu_baseline the CPU oracle on a bounded sample of whole query rows of the
              same workload; those rows are also checked against the timed
              step's output (index-set rule and bf16 tolerances), and a
              mismatch makes the run exit non-zero before printing.
Before timing, the step's selection is checked bit for bit against the
separate score and top-k entry points.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import long_context_02_amd as dsa  # noqa: E402
from long_context_02_amd.synth import WORKLOADS, make_inputs, make_mha_inputs  # noqa: E402

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0     # dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0    # dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
BF16_MAX_ABS, BF16_MEAN_ABS, BAND_REL = 2e-2, 5e-3, 1e-3

# kernel -> the sources it is built from (a traffic summary is used only while
# they are unchanged)
_IDX = ("indexer.hip", "indexer_math.h", "topk_select.h")
_ATT = ("attention.hip", "attn_common.h")
KERNEL_SOURCES = {
    "indexer_fp8_stream": _IDX, "indexer_fp8_tiled": _IDX, "indexer_sample_threshold": _IDX,
    "topk_rows": ("topk.hip", "indexer_math.h", "topk_select.h"),
    "topk_cand_select": ("topk.hip", "indexer_math.h", "topk_select.h"),
    "topk_seg": ("topk.hip", "indexer_math.h", "topk_select.h"),
    "sparse_mla_attn_bf16": _ATT, "attn_combine": _ATT,
    "attn_bwd": ("attention_bwd.hip", "attn_common.h"),
    "mha": ("attention_mha.hip",), "sparse_mha_attn": ("attention_mha.hip",),
}


def _sources_of(kernel):
    for prefix, files in KERNEL_SOURCES.items():
        if kernel.startswith(prefix):
            return files
    raise KeyError(kernel)


def source_hash(kernel):
    """sha256 over the sources a kernel is built from (in a fixed order)."""
    h = hashlib.sha256()
    for name in _sources_of(kernel):
        with open(os.path.join(ROOT, "long_context_02_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def profile_name(kernel):
    """File-name form of a kernel name: indexer_fp8_stream<false, 1, true> ->
    indexer_fp8_stream_false_1_true."""
    return "".join(c if c.isalnum() or c == "_" else "_" for c in kernel).replace("__", "_").strip("_")


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


def kernel_work(kernel, w):
    """Algorithmic work a kernel of the step carries, or None for kernels that
    only handle the implementation's intermediates (sampling, partial
    merges, clearing)."""
    if kernel.startswith(("indexer_fp8_stream", "indexer_fp8_tiled", "indexer_f32")):
        return w["indexer"]
    if kernel.startswith(("topk_rows", "topk_seg_finalize")):
        return w["topk"]
    if kernel.startswith(("sparse_mla_attn_bf16", "sparse_attn_f32")):
        return w["attention"]
    return None


def phase_floor(w):
    """Seconds a phase needs at the published peaks: max(FLOP / MFMA peak, bytes / HBM)."""
    peak_f = {"fp8": PEAK_FP8_TFLOPS, "bf16": PEAK_BF16_TFLOPS, "f32": PEAK_F32_TFLOPS}.get(w["flop_unit"])
    t_mem = w["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_cmp = w["flops"] / (peak_f * 1e12) if peak_f else 0.0
    return max(t_mem, t_cmp)


def roofline(name, w, seconds, measured=None):
    """Roofline position of one kernel: which roof binds, the achieved rate,
    its fraction of the published peak and, when `measured` holds them, of
    the peaks measured on this GPU."""
    peak_f = {"fp8": PEAK_FP8_TFLOPS, "bf16": PEAK_BF16_TFLOPS, "f32": PEAK_F32_TFLOPS}.get(w["flop_unit"])
    t_mem = w["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_cmp = w["flops"] / (peak_f * 1e12) if peak_f else 0.0
    if t_cmp > t_mem:
        ach = w["flops"] / seconds / 1e12
        r = {"kernel": name, "bound": "mfma", "achieved": round(ach, 2), "peak": peak_f,
             "unit": "TFLOP/s", "frac": round(ach / peak_f, 4), "algorithmic": w["flops"]}
        mp = (measured or {}).get(f"{w['flop_unit']}_mfma_tflops")
    else:
        ach = w["bytes"] / seconds / 1e9
        r = {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
             "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "algorithmic": w["bytes"]}
        mp = (measured or {}).get("hbm_read_gbs")
    if mp:
        r["measured_peak"] = mp
        r["frac_of_measured"] = round(ach / mp, 4)
    return r


def measured_traffic(kernel, wl):
    """HBM bytes per launch of `kernel` on `wl` from its counter summary in
    profiles/ (FETCH_SIZE + WRITE_SIZE, scaled by the plain-copy
    calibration), or None when there is none or it was taken on other kernel
    sources."""
    path = os.path.join(ROOT, "profiles", f"{profile_name(kernel)}_{wl.name}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                key, val = ln.split("=", 1)
                fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != source_hash(kernel) or "hbm_bytes_per_launch" not in fields:
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


def kernel_table(step, steps, wl, measured):
    """Per-kernel HIP-event times of `steps` calls of step(): {kernel: {...}}."""
    times = dsa.kernel_times(lambda: [step() for _ in range(steps)], max_launches=64 * steps)
    torch.cuda.synchronize()
    w = work(wl)
    out = {}
    for name, (launches, total) in times.items():
        per_launch = total / launches
        e = {"ms": round(per_launch, 4), "launches_per_step": round(launches / steps, 3),
             "ms_per_step": round(total / steps, 4)}
        kw = kernel_work(name, w)
        if kw is not None and launches == steps:
            r = roofline(name, kw, per_launch / 1e3, measured)
            e.update({k: r[k] for k in ("bound", "achieved", "unit", "frac") if k in r})
            e["flop_unit"] = kw["flop_unit"]
        out[name] = e
    return out


def add_measured_fracs(entry, measured):
    """Add the fraction of the measured peak to a roofline entry (in place)."""
    if not isinstance(entry, dict) or entry.get("achieved") is None or not measured:
        return
    if entry.get("bound") == "hbm":
        mp = measured.get("hbm_read_gbs")
    elif entry.get("bound") == "mfma":
        mp = measured.get(f"{entry.get('flop_unit')}_mfma_tflops")
    else:
        mp = None
    if mp:
        entry["measured_peak"] = mp
        entry["frac_of_measured"] = round(entry["achieved"] / mp, 4)


def measure_peaks(dev):
    """What this GPU sustains, from the library's probes: a streaming read of
    2 GiB and back-to-back bf16 / FP8 MFMAs (the engine clock under MFMA load
    is in these); and, for reference, what vendor GEMMs reach (torch.matmul
    in bf16, torch._scaled_mm in FP8 e4m3, 8192^3)."""
    p = dsa.probe_peaks(dev)
    out = {"hbm_read_gbs": p["stream_read_gbs"], "bf16_mfma_tflops": p["mfma_bf16_tflops"],
           "fp8_mfma_tflops": p["mfma_fp8_tflops"]}
    stream = torch.cuda.current_stream(dev)
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    ms = min(timed(lambda: a @ b, 5, stream) for _ in range(3))
    out["bf16_vendor_gemm_tflops"] = round(2 * n ** 3 / (ms / 1e3) / 1e12, 1)
    try:
        a8 = a.to(torch.float8_e4m3fn)
        b8 = b.t().contiguous().to(torch.float8_e4m3fn).t()
        one = torch.ones((), device=dev)
        ms = min(timed(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one,
                                                out_dtype=torch.bfloat16), 5, stream) for _ in range(3))
        out["fp8_vendor_gemm_tflops"] = round(2 * n ** 3 / (ms / 1e3) / 1e12, 1)
    except Exception as e:  # FP8 GEMM not available in this torch build
        log(f"[bench] fp8 gemm peak not measured: {e}")
    out["how"] = ("library probes (best of 5): streaming read of 2 GiB, back-to-back MFMA loops; "
                  "vendor GEMMs (best of 3x5): torch.matmul 8192^3 bf16, torch._scaled_mm 8192^3 "
                  "e4m3 -> bf16")
    return out


# ---------------------------------------------------------------------------
class Step:
    """The inputs, outputs and workspace of one workload's dsa_forward step."""

    def __init__(self, wl, dev, seed=0):
        self.wl, self.dev = wl, dev
        log(f"[bench] generating {wl.name} inputs on {dev}")
        self.g = make_inputs(wl, seed=seed, device=dev)
        B, T, N = wl.B, wl.T, wl.N
        self.out = torch.empty(B, T, wl.H, wl.d_v, dtype=self.g["q"].dtype, device=dev)
        self.lse = torch.empty(B, T, wl.H, dtype=torch.float32, device=dev)
        self.idx = torch.empty(B, T, wl.k, dtype=torch.int32, device=dev)
        self.ws = torch.empty(dsa.workspace_size(dsa.OP_FORWARD, B, T, N, wl.H_I, wl.H, wl.d_v, wl.k),
                              dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)

    def __call__(self, keep=False):
        g, wl = self.g, self.wl
        dsa.forward(g["q_idx"], g["k_idx"], g["w"], g["q"], g["kv"], k=wl.k, q_offset=wl.q_offset,
                    d_v=wl.d_v, sm_scale=wl.sm_scale, q_idx_scale=g["q_idx_scale"],
                    k_idx_scale=g["k_idx_scale"], out=self.out,
                    lse=self.lse if keep else None, idx_out=self.idx if keep else None,
                    workspace=self.ws)


def check_selection_consistency(st):
    """dsa_forward's selection must equal, bit for bit, dsa_topk_select run on
    dsa_indexer_scores' output (same ranking rule, same scores)."""
    g, wl = st.g, st.wl
    st(keep=True)
    scores = dsa.indexer_scores(g["q_idx"], g["k_idx"], g["w"], wl.q_offset,
                                q_idx_scale=g["q_idx_scale"], k_idx_scale=g["k_idx_scale"])
    ref = dsa.topk_select(scores, wl.k, wl.q_offset)
    torch.cuda.synchronize()
    same = torch.equal(ref, st.idx)
    del scores
    if not same:
        bad = int((ref != st.idx).any(-1).sum().item())
        print(f"[bench] PARITY FAILURE: dsa_forward's selection differs from dsa_topk_select on "
              f"dsa_indexer_scores in {bad} rows of {wl.name}", file=sys.stderr, flush=True)
        sys.exit(3)
    return True


def time_step(st, steps, warmup, measured):
    """Headline timing of the step plus its per-kernel and per-phase tables."""
    wl, g = st.wl, st.g
    B, T, N = wl.B, wl.T, wl.N
    log(f"[bench] {wl.name}: warmup {warmup}, timing {steps} steps")
    for _ in range(warmup):
        st()
    torch.cuda.synchronize()
    ms = timed(st, steps, st.stream)
    kernels = kernel_table(st, steps, wl, measured)

    # the step's two parts, as dsa_forward runs them (scores + selection,
    # then attention), called in sequence through their entry points with
    # HIP events between them on the launch stream; then the standalone
    # score and top-k kernels the same way
    dev = st.dev
    scores = torch.empty(B, T, N, dtype=torch.float32, device=dev)
    idx = torch.empty(B, T, wl.k, dtype=torch.int32, device=dev)
    attn_ws = torch.empty(max(1, dsa.workspace_size(dsa.OP_ATTN, B, T, N, wl.H_I, wl.H, wl.d_v, wl.k)),
                          dtype=torch.uint8, device=dev)
    sel_ws = torch.empty(max(1, dsa.workspace_size(dsa.OP_SELECT, B, T, N, wl.H_I, wl.H, wl.d_v, wl.k)),
                         dtype=torch.uint8, device=dev)
    topk_ws = torch.empty(max(1, dsa.workspace_size(dsa.OP_TOPK, B, T, N, wl.H_I, wl.H, wl.d_v, wl.k)),
                          dtype=torch.uint8, device=dev)
    out = torch.empty_like(st.out)
    step_parts = {
        "select": lambda: dsa.indexer_select(g["q_idx"], g["k_idx"], g["w"], wl.k, wl.q_offset,
                                             q_idx_scale=g["q_idx_scale"],
                                             k_idx_scale=g["k_idx_scale"], out=idx, workspace=sel_ws),
        "attention": lambda: dsa.sparse_mla_attn(g["q"], g["kv"], idx, wl.d_v, wl.sm_scale,
                                                 out=out, lse=False, workspace=attn_ws),
    }
    standalone = {
        "indexer_scores": lambda: dsa.indexer_scores(g["q_idx"], g["k_idx"], g["w"], wl.q_offset,
                                                     q_idx_scale=g["q_idx_scale"],
                                                     k_idx_scale=g["k_idx_scale"], out=scores),
        "topk_select": lambda: dsa.topk_select(scores, wl.k, wl.q_offset, out=idx, workspace=topk_ws),
    }
    phase_ms = timed_sequence(step_parts, steps, warmup, st.stream)
    comp_ms = timed_sequence(standalone, steps, warmup, st.stream)
    w = work(wl)
    t_roof = sum(phase_floor(w[p]) for p in ("indexer", "topk", "attention"))
    phases = {}
    for name, t_ms in phase_ms.items():
        r = roofline(name, w[name], t_ms / 1e3, measured)
        phases[name] = {"ms": round(t_ms, 4), "bound": r["bound"], "achieved": r["achieved"],
                        "unit": r["unit"], "frac": r["frac"]}
    stand = {}
    for name, t_ms in comp_ms.items():
        r = roofline(name, w["indexer" if name == "indexer_scores" else "topk"], t_ms / 1e3, measured)
        stand[name] = {"ms": round(t_ms, 4), "bound": r["bound"], "achieved": r["achieved"],
                       "unit": r["unit"], "frac": r["frac"]}
    # the dominant kernel: the most time per step; its roofline position
    dom = max(kernels, key=lambda n: kernels[n]["ms_per_step"])
    kw = kernel_work(dom, w)
    roof = (dict(roofline(dom, kw, kernels[dom]["ms"] / 1e3, measured), flop_unit=kw["flop_unit"])
            if kw is not None
            else {"kernel": dom, "bound": None, "achieved": None, "peak": None, "unit": None,
                  "frac": None})
    roof["ms"] = kernels[dom]["ms"]
    roof["traffic"] = measured_traffic(dom, wl)
    return {
        "value": round(B * T / (ms / 1e3), 1),
        "ms_per_step": round(ms, 4),
        "kernels": kernels,
        "roofline": roof,
        "phases": phases,
        "standalone": stand,
        "step_roofline": {"t_roof_ms": round(t_roof * 1e3, 4), "frac": round(t_roof / (ms / 1e3), 4)},
        "_scores": scores,
        "_idx": idx,
    }


# ---------------------------------------------------------------------------
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
    kt = dsa.kernel_times(fn)
    return {"attn_bwd": {"ms": round(ms, 4), "rows": rows, "bound": "mfma", "achieved": round(ach, 1),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach / PEAK_BF16_TFLOPS, 4), "algorithmic_flop": flop,
                         "algorithmic_bytes": nbytes,
                         "hbm_floor_ms": round(nbytes / (PEAK_HBM_GBS * 1e9) * 1e3, 4),
                         "kernels_ms": {n: round(t, 4) for n, (_, t) in kt.items()},
                         "traffic": measured_traffic("attn_bwd", wl)}}


def time_attn_mha(wl, g, idx, steps, stream, seed=0):
    """dsa_sparse_mla_attn_mha (MLA's MHA mode) on the step's selection:
    the per-head keys and values of every latent row are up-projected, then
    each head attends over its own rows.  Algorithmic work: the up-projection
    (2 x 512 x 256 FLOP per latent row and head, the latent rows read, the
    per-head rows written) and, per (query, selected token, head), the
    head's 128-wide key part and 128-wide value gathered (512 bytes) for
    2 x 320 FLOP, plus per (query, selected token) the 64-wide rope key part
    that every head shares (128 bytes)."""
    dev = g["q"].device
    extra = make_mha_inputs(wl, seed=seed, device=dev)
    B, T, N, H = wl.B, wl.T, wl.N, wl.H
    out = torch.empty(B, T, H, 128, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(dsa.workspace_size(dsa.OP_ATTN_MHA, B, T, N, wl.H_I, H, 128, wl.k),
                     dtype=torch.uint8, device=dev)

    def fn():
        dsa.sparse_mla_attn_mha(extra["q_mha"], g["kv"], extra["w_uk"], extra["w_uv"], idx,
                                extra["sm_scale_mha"], out=out, lse=False, workspace=ws)

    fn()
    ms = timed(fn, steps, stream)
    kt = dsa.kernel_times(fn)
    n_valid = int(((idx >= 0) & (idx < N)).sum().item())
    up_flop = 2.0 * 512 * 256 * H * B * N
    up_bytes = B * N * (1152 + H * (128 + 128) * 2)
    gather_bytes = n_valid * (H * (128 + 128) * 2 + 64 * 2)
    res = {"ms": round(ms, 4), "rows": B * T, "kernels": {}}
    for name, (_, t) in kt.items():
        if name == "mha_up_project":
            ach = up_flop / (t / 1e3) / 1e12
            res["kernels"][name] = {"ms": round(t, 4), "bound": "mfma", "achieved": round(ach, 1),
                                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                                    "algorithmic_flop": up_flop, "algorithmic_bytes": up_bytes,
                                    "traffic": measured_traffic(name, wl)}
        else:
            ach = gather_bytes / (t / 1e3) / 1e9
            res["kernels"][name] = {"ms": round(t, 4), "bound": "hbm", "achieved": round(ach, 1),
                                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                                    "algorithmic_bytes": gather_bytes,
                                    "traffic": measured_traffic(name, wl),
                                    "note": "per-head rows gathered once per (query, token, head); "
                                            "rows shared by nearby queries may come from the caches"}
    return {"attn_mha": res}


# ---------------------------------------------------------------------------
def cpu_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    return model, cores, threads


def _check_row(gpu_idx, gpu_out, scores_row, sel_ref, attn_ref, wl, n_cand, where):
    """The parity rules for one row: index set (exact up to tokens within
    1e-3 relative of the oracle's k-th score) and bf16 attention tolerances
    (the oracle attends over the GPU's own selection)."""
    n = min(wl.k, n_cand)
    sel = np.asarray(gpu_idx, np.int64)
    if not (np.all(sel[n:] == -1) and np.all(np.diff(sel[:n]) > 0)
            and np.all((sel[:n] >= 0) & (sel[:n] < n_cand))):
        return f"{where}: malformed index row"
    diff = np.setxor1d(sel[:n], np.asarray(sel_ref)[:n])
    if diff.size:
        v = scores_row[:n_cand]
        thr = np.partition(v, n_cand - n)[n_cand - n] if n_cand > wl.k else -np.inf
        ok = (np.abs(scores_row[diff] - thr) <= BAND_REL * abs(thr)) if thr != 0 else scores_row[diff] == 0
        if not np.all(ok):
            return f"{where}: selection differs outside the 1e-3 band ({int((~ok).sum())} tokens)"
    d = np.abs(np.asarray(gpu_out, np.float64) - attn_ref)
    tol_max = BF16_MAX_ABS if wl.dtype == "bf16" else 1e-5
    if d.max() > tol_max or (wl.dtype == "bf16" and d.mean() > BF16_MEAN_ABS):
        return f"{where}: attention error max {d.max():.3e} mean {d.mean():.3e}"
    return None


def cpu_baseline(st, budget_s, max_rows=None):
    """The CPU oracle on a bounded sample of the same workload: whole rows
    (index scores -> selection -> attention), timed on this host's cores.
    Every row it computes is also checked against the timed step's output
    (st.idx, st.out, written by a step run with the index output kept)."""
    import oracle
    wl, g = st.wl, st.g
    model, cores, threads = cpu_info()
    fp8 = wl.dtype == "bf16"
    rng = np.random.default_rng(0)
    if wl.T == 1:
        order = [(int(b), 0) for b in rng.permutation(wl.B)]
    else:
        order = [(0, int(t)) for t in rng.permutation(wl.T)]
    gpu_idx = st.idx.cpu().numpy()
    done, spent, failures = 0, 0.0, []
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
        # parity of this row (not timed): the oracle's attention on the GPU's
        # own selection, and the selection rule
        o_ref, _ = oracle.sparse_mqa_attention_row(q, h["kv"], gpu_idx[b, t], wl.d_v, wl.sm_scale)
        err = _check_row(gpu_idx[b, t], st.out[b, t].double().cpu().numpy(), I, sel, o_ref, wl, n_cand,
                         f"{wl.name} row (b={b}, t={t})")
        if err:
            failures.append(err)
        if spent >= budget_s or (max_rows is not None and done >= max_rows):
            break
    return {"value": round(done / spent, 3), "unit": "tokens/s", "cores": int(cores),
            "blas_threads": int(threads), "cpu_model": model, "kind": "oracle",
            "sample": f"{done} query tokens of {wl.name} (whole rows: index scores, top-{wl.k}, "
                      f"attention; float64), {spent:.1f} s",
            "rows_checked_against_gpu": done, "parity_failures": failures}


def run_workload(wl, args, dev, measured, cpu_budget, with_next=True, cpu_rows=None):
    st = Step(wl, dev)
    check_selection_consistency(st)
    res = time_step(st, args.steps, args.warmup, measured)
    scores, idx = res.pop("_scores"), res.pop("_idx")
    if with_next:
        # the step before the path (not part of the step): appending this
        # step's new tokens to the key and latent caches; the indexer's
        # alignment objective on this step's rows; the attention backward;
        # MHA-mode attention on prefill-sized caches
        nxt = {"cache_append": time_cache_append(wl, st.g, args.steps, st.stream)}
        nxt.update(time_indexer_kl(wl, scores, idx, args.steps, st.stream))
        if wl.dtype == "bf16":
            nxt.update(time_attn_bwd(wl, st.g, idx, args.steps, st.stream))
            if wl.T > 1:
                nxt.update(time_attn_mha(wl, st.g, idx, 3, st.stream))
        res["next"] = nxt
    del scores
    if cpu_budget > 0:
        log(f"[bench] {wl.name}: cpu baseline and row parity")
        st(keep=True)
        torch.cuda.synchronize()
        cb = cpu_baseline(st, cpu_budget, cpu_rows)
        if cb["parity_failures"]:
            for f in cb["parity_failures"]:
                print(f"[bench] PARITY FAILURE: {f}", file=sys.stderr, flush=True)
            sys.exit(3)
        res["cpu_baseline"] = cb
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # untimed steps first: after a few the clocks have not settled yet (the
    # decode step times ~5 % slower after 3 warm-up steps than after 50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode_128k", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunk", action="store_true",
                    help="with the default workload, skip the chunked-prefill block")
    ap.add_argument("--no-next", action="store_true", help="skip the neighbouring steps")
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
    measured = None  # taken after the timed work, then added to the entries
    res = run_workload(wl, args, dev, measured, 0 if args.no_cpu_baseline else args.cpu_budget,
                       with_next=not args.no_next)
    torch.cuda.empty_cache()
    line = {
        "metric": "DSA tokens/s (indexer+top-k+sparse attn) at 128K ctx; % of MFMA / HBM roofline",
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 indexer / bf16 attention" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded)",
        "config": {"workload": wl.name, "batch": wl.B, "query_tokens": wl.T, "context": wl.N,
                   "q_offset": wl.q_offset, "indexer_heads": wl.H_I, "indexer_dim": wl.d_I,
                   "top_k": wl.k, "heads": wl.H, "d_qk": wl.d_qk, "d_v": wl.d_v,
                   "parallelism": "single GPU"},
        "roofline": res["roofline"],
        "kernels": res["kernels"],
        "phases_ms": {k: v["ms"] for k, v in res["phases"].items()},
        "phases": res["phases"],
        "standalone": res["standalone"],
        # the whole step against the sum of the phases' floors at published peaks
        "step_roofline": res["step_roofline"],
    }
    if "next" in res:
        line["next"] = res["next"]
    if "cpu_baseline" in res:
        line["cpu_baseline"] = res["cpu_baseline"]
    if args.workload == "decode_128k" and not args.no_chunk:
        # chunked prefill at 128K, where the indexer's FP8 target is judged
        del res
        torch.cuda.empty_cache()
        cw = WORKLOADS["chunk_128k"]
        cres = run_workload(cw, args, dev, measured, 0 if args.no_cpu_baseline else 4.0,
                            with_next=not args.no_next, cpu_rows=3)
        line["chunk_128k"] = {"value": cres["value"], "unit": "tokens/s",
                              "ms_per_step": cres["ms_per_step"], "roofline": cres["roofline"],
                              "kernels": cres["kernels"], "phases": cres["phases"],
                              "standalone": cres["standalone"],
                              "step_roofline": cres["step_roofline"]}
        if "next" in cres:
            line["chunk_128k"]["next"] = cres["next"]
        if "cpu_baseline" in cres:
            cb = cres["cpu_baseline"]
            line["chunk_128k"]["rows_checked_against_oracle"] = cb["rows_checked_against_gpu"]
        att = next((v for k, v in line["kernels"].items() if k.startswith("sparse_mla_attn_bf16")), None)
        ind = next((v for k, v in cres["kernels"].items() if k.startswith("indexer_fp8_tiled")), None)
        att_ms = sum(v["ms_per_step"] for k, v in line["kernels"].items()
                     if k.startswith(("sparse_mla_attn_bf16", "attn_combine")))
        att_bytes = work(wl)["attention"]["bytes"]
        line["north_star"] = {
            "decode_attention_hbm_frac": att["frac"] if att else None,
            "decode_attention_with_combine_ms": round(att_ms, 4),
            "decode_attention_with_combine_hbm_frac": round(att_bytes / (att_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)
            if att_ms > 0 else None,
            "chunk_indexer_fp8_frac": ind["frac"] if ind else None,
            "targets": {"decode_attention_hbm_frac": 0.60, "chunk_indexer_fp8_frac": 0.50},
        }
    torch.cuda.empty_cache()
    measured = measure_peaks(dev)
    log(f"[bench] measured peaks {measured}")
    line["measured_peaks"] = measured
    for blk in (line, line.get("chunk_128k", {})):
        for e in list(blk.get("kernels", {}).values()) + [blk.get("roofline")]:
            add_measured_fracs(e, measured)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
