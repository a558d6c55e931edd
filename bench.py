#!/usr/bin/env python3
"""Bench of the paged KV-cache hot path on one MI355X.

One step = one pass of the whole path over one batch of the workload:
  decode workloads:  the cache write of the step's new K/V rows through
                     slot_mapping (padding rows included), then paged decode
                     attention (split-K partitions + reduce, or one pass);
  prefill workloads: the cache write of the packed new rows, then causal
                     packed prefill over the paged cache.
Default workload: the 7B-like MHA decode layer (64 sequences, 32 heads,
head size 128, bf16, block size 16, context lengths U[200, 2048], 71 write
rows of which 7 are padding) over head-major (HND) pools.  Inputs are seeded synthetic data already
resident in device memory when the timed region starts.

--kv fp8 runs a workload over FP8 (E4M3) pools: the cache write quantises,
decode and prefill read one byte per element.

Prints ONE JSON line.  `value` = algorithmic KV bytes read per step / step
time (GB/s) for decode, algorithmic flops / step time (TFLOP/s) for prefill.
`roofline` covers the dominant kernel, timed with HIP events recorded on the
stream the kernels run on.  `cpu_baseline` is the fp64 oracle timed on a
bounded sample of the same workload on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode KV GB/s (fraction of HBM peak); prefill MFMA util; tokens/s"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, AMD published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16/fp16 MFMA, AMD published
# source file of each timed kernel (the hash of its code, comments excluded,
# ties a committed counter profile to the kernel it was taken on)
# (with the headers they include, so a change to shared device code also
# retires the profile)
KERNEL_SOURCES = {
    "decode_head": ["decode_head.hip", "decode_common.h", "kernel_common.h"],
    "decode_group": ["decode_group.hip", "decode_common.h", "kernel_common.h"],
    "decode_group_fp8": ["decode_group_fp8.hip", "decode_common.h", "kernel_common.h"],
    "prefill": ["prefill.hip", "kernel_common.h"],
}


def decode_kernel_kind(w, fp8: bool = False) -> str:
    """Which decode kernel the library dispatches for this workload: the
    grouped kernels for group sizes 4, 8, 16 (LDS-staged for 16-bit caches,
    matrix-core for FP8), the per-head kernel otherwise."""
    if w.dtype == "f32" or w.G not in (4, 8, 16):
        return "decode_head"
    return "decode_group_fp8" if fp8 else "decode_group"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed warm-up steps; -1 (default): as many as fill 0.3 s (at least 5), "
                         "so clocks have settled before the timed steps")
    ap.add_argument("--config", default="2", help="workload: 1, 2, 3, 4, 5a, 5b, 5c")
    ap.add_argument("--layout", choices=["nhd", "hnd"], default="hnd",
                    help="pool layout: hnd (head-major, default: a kv head's block is one "
                         "contiguous run) or nhd")
    ap.add_argument("--cascade", action="store_true",
                    help="shared-prefix decode workloads: attend the common blocks once "
                         "(pa_decode_cascade)")
    ap.add_argument("--kv", choices=["native", "fp8"], default="native",
                    help="keep the workload's cache type, or FP8 (E4M3) pools written by the "
                         "quantising cache write")
    ap.add_argument("--partition", type=int, default=-1,
                    help="decode partition size (-1 auto, 0 single pass)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU work budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def code_text(src: str) -> str:
    """The source with comments removed and whitespace collapsed: edits to
    comments leave the hash, and so a counter profile, valid."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_sha(kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "paged_kv_cache_134_amd", "csrc", name)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, kind: str):
    """HBM bytes per launch of the dominant kernel from a committed counter
    summary (profiles/<kind>_<workload>_traffic.txt), if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    sha = re.search(r"kernel_source_sha:\s*(\w+)", txt)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not sha or not val or sha.group(1) != source_sha(kind):
        return None
    return float(val.group(1))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); every step of this "
              "path runs on a single MI355X and no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    import paged_kv_cache_134_amd as P
    from paged_kv_cache_134_amd import metadata as M

    cfg = args.config if not args.config.isdigit() else int(args.config)
    w = workloads.make(cfg)
    layout = P.NHD if args.layout == "nhd" else P.HND
    fp8 = args.kv == "fp8"
    if fp8 and w.dtype == "f32":
        raise SystemExit("--kv fp8 needs a bf16 workload")
    ks, vs = workloads.FP8_K_SCALE, workloads.FP8_V_SCALE
    torch.cuda.set_device(0)
    t0 = time.time()
    dw = (M.setup(w, layout=layout, kv_dtype="e4m3", k_scale=ks, v_scale=vs) if fp8
          else M.setup(w, layout=layout))
    torch.cuda.synchronize()
    log(f"[bench] set-up of {w.name} took {time.time() - t0:.1f}s")
    stream = torch.cuda.current_stream()

    S, H, Hkv, D = w.S, w.H, w.Hkv, w.D
    eb = 1 if fp8 else w.elem_bytes  # bytes per cached element
    lens = w.context_lens.astype(np.int64)
    kv_bytes = int(lens.sum()) * Hkv * D * 2 * eb
    out = torch.empty(w.query_shape, dtype=torch.float32, device="cuda")
    kinds = []

    cascade = None
    if args.cascade:
        if w.kind != "decode" or w.prefix_len < w.bs:
            raise SystemExit("--cascade needs a decode workload with a shared prefix (5a)")
        common = (w.prefix_len // w.bs) * w.bs  # the fully shared blocks
        # unique bytes the method must read: the common blocks once, then each
        # sequence's own tokens
        unique = (common + int((lens - common).sum())) * Hkv * D * 2 * eb
        cascade = {"common_prefix_len": common, "unique_kv_bytes_per_step": unique}
        ps = args.partition if args.partition >= 0 else -1
        ws = torch.empty(P.pa_decode_cascade_workspace_size(S, H, D, dw.max_context_len, common, ps),
                         dtype=torch.uint8, device="cuda")

        def step(ev):
            ev[0].record(stream)
            M.write_step_rows(dw)
            ev[1].record(stream)
            if fp8:
                P.pa_decode_cascade_fp8(out, dw.query, dw.key_cache, dw.value_cache,
                                        dw.block_tables, dw.context_lens, dw.max_context_len,
                                        common, w.scale, ks, vs, ws, layout=layout,
                                        partition_size=ps)
            else:
                P.pa_decode_cascade(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                                    dw.context_lens, dw.max_context_len, common, w.scale, ws,
                                    layout=layout, partition_size=ps)
            ev[2].record(stream)
            ev[3].record(stream)
        kinds = ["reshape_and_cache", "decode_cascade", None]
        dominant = 1
        work_units = S
    elif w.kind == "decode":
        ps = args.partition if args.partition >= 0 else P.pa_decode_auto_partition(
            S, H, Hkv, P.PA_FP8_E4M3 if fp8 else P.KV_DTYPE[w.dtype],
            dw.max_context_len, int(lens.sum()))
        ws = None
        if ps > 0:
            ws = torch.empty(P.pa_decode_workspace_size(S, H, D, dw.max_context_len, ps),
                             dtype=torch.uint8, device="cuda")

        def step(ev):
            ev[0].record(stream)
            M.write_step_rows(dw)
            ev[1].record(stream)
            if ps > 0 and fp8:
                P.pa_decode_partitions_fp8(out, dw.query, dw.key_cache, dw.value_cache,
                                           dw.block_tables, dw.context_lens, dw.max_context_len,
                                           w.scale, ks, vs, ps, ws, layout=layout)
                ev[2].record(stream)
                P.pa_decode_reduce(out, dw.context_lens, dw.max_context_len, Hkv, ps, ws)
            elif ps > 0:
                P.pa_decode_partitions(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                                       dw.context_lens, dw.max_context_len, w.scale, ps, ws,
                                       layout=layout)
                ev[2].record(stream)
                P.pa_decode_reduce(out, dw.context_lens, dw.max_context_len, Hkv, ps, ws)
            elif fp8:
                P.pa_decode_fp8(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                                dw.context_lens, dw.max_context_len, w.scale, ks, vs,
                                layout=layout, partition_size=0)
                ev[2].record(stream)
            else:
                P.pa_decode(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                            dw.context_lens, dw.max_context_len, w.scale, layout=layout,
                            partition_size=0)
                ev[2].record(stream)
            ev[3].record(stream)
        kinds = ["reshape_and_cache", "decode_partitions" if ps > 0 else "decode_single_pass",
                 "decode_reduce"]
        dominant = 1
        work_units = S  # tokens decoded per step
    else:
        ps = None
        qlens = w.query_lens.astype(np.int64)
        ctx = w.context_lens.astype(np.int64)
        # causal-visible (query, key) pairs: row j of a sequence sees L - n + j + 1 keys
        pairs = int(sum(n * (L - n) + n * (n + 1) // 2 for n, L in zip(qlens, ctx)))
        flops = 4 * D * H * pairs
        max_q = int(qlens.max())

        def step(ev):
            ev[0].record(stream)
            M.write_step_rows(dw)
            ev[1].record(stream)
            if fp8:
                P.pa_prefill_fp8(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                                 dw.query_start_loc, dw.context_lens, max_q, dw.max_context_len,
                                 w.scale, ks, vs, layout=layout)
            else:
                P.pa_prefill(out, dw.query, dw.key_cache, dw.value_cache, dw.block_tables,
                             dw.query_start_loc, dw.context_lens, max_q, dw.max_context_len,
                             w.scale, layout=layout)
            ev[2].record(stream)
            ev[3].record(stream)
        kinds = ["reshape_and_cache", "prefill", None]
        dominant = 1
        work_units = int(qlens.sum())

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    if args.warmup >= 0:
        for _ in range(args.warmup):
            step(events())
        torch.cuda.synchronize()
    else:
        args.warmup, t_w = 0, time.perf_counter()
        while args.warmup < 5 or time.perf_counter() - t_w < 0.3:
            for _ in range(5):
                step(events())
            torch.cuda.synchronize()
            args.warmup += 5
    evs = [events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / max(args.steps, 1)
    kern_ms = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i in range(3)]
    kernels_us = {k: round(t * 1e3, 3) for k, t in zip(kinds, kern_ms) if k}

    # sampled parity of the last step's output against the oracle's plain definition
    # (FP8 pools: the oracle's codes of the same rows, read back times the scales)
    from oracle import attention as A
    from oracle import fp8 as F8
    got = out.cpu().numpy()
    errs = []
    sample_seqs = sorted({0, S // 2, S - 1}) if w.kind == "decode" else sorted({0, S - 1})
    for s in sample_seqs:
        K, V = w.kv(s)
        if fp8:
            Kf = F8.dequantize(F8.quantize(K, w.dtype, ks), ks)
            Vf = F8.dequantize(F8.quantize(V, w.dtype, vs), vs)
        else:
            Kf, Vf = A.bits_to_f64(K, w.dtype), A.bits_to_f64(V, w.dtype)
        qf = A.bits_to_f64(w.query, w.dtype)
        for h in sorted({0, H - 1}):
            if w.kind == "decode":
                ref, _ = A.attention_dense(qf[s, h], Kf[:, h // w.G], Vf[:, h // w.G], w.scale)
                errs.append(float(np.max(np.abs(got[s, h] - ref))))
            else:
                n = int(w.query_lens[s])
                L = int(w.context_lens[s])
                for j in sorted({0, n // 2, n - 1}):
                    a = L - n + j
                    r = int(w.query_start_loc[s]) + j
                    ref, _ = A.attention_dense(qf[r, h], Kf[:a + 1, h // w.G], Vf[:a + 1, h // w.G],
                                               w.scale)
                    errs.append(float(np.max(np.abs(got[r, h] - ref))))
    tol = 1e-5 if w.dtype == "f32" else 2e-3
    parity = {"max_abs": max(errs), "tolerance": tol, "ok": max(errs) <= tol,
              "sampled": f"sequences {sample_seqs}, heads {sorted({0, H - 1})}"}

    if w.kind == "decode":
        value = kv_bytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        dom_ms = kern_ms[dominant]
        # the cascade's roofline counts the bytes it must read (common blocks
        # once); the value keeps the logical KV bytes of the plain method
        achieved = (cascade["unique_kv_bytes_per_step"] if cascade else kv_bytes) / (dom_ms * 1e-3) / 1e9
        kind_src = decode_kernel_kind(w, fp8)
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
        alg = {"kv_bytes_per_step": kv_bytes}
    else:
        value = flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        dom_ms = kern_ms[dominant]
        achieved = flops / (dom_ms * 1e-3) / 1e12
        kind_src = "prefill"
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
        alg = {"flops_per_step": flops, "causal_pairs_per_head": pairs}
    roof["kernel"] = kinds[dominant]
    prof_name = w.name + ("-e4m3" if fp8 else "")
    roof["traffic"] = traffic_from_profile(prof_name, kind_src)
    roof["kernel_source_sha"] = source_sha(kind_src)

    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds, unit,
                                                         (ks, vs) if fp8 else None)
    pcache = prefix_cache_probe(w, P) if w.prefix_len >= w.bs else None

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 kv, bf16 q, fp32 accumulate" if fp8 else w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": S, "num_heads": H, "num_kv_heads": Hkv,
                   "head_size": D, "block_size": w.bs, "layout": args.layout.upper(),
                   "context_tokens": int(lens.sum()), "write_rows": w.T,
                   "partition_size": ps, "seed": w.seed,
                   **({"kv_cache_dtype": "e4m3", "k_scale": ks, "v_scale": vs} if fp8 else {}),
                   **({"path": "cascade", **cascade} if cascade else {})},
        "tokens_per_s": round(work_units / (ms_per_step * 1e-3), 1),
        "frac_hbm_peak_step": round(value / HBM_PEAK_GBS, 4) if unit == "GB/s" else None,
        "kernels_us": kernels_us,
        **alg,
        "parity": parity,
        **({"prefix_cache": pcache} if pcache else {}),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def prefix_cache_probe(w, P):
    """Host prefix cache on the workload's prompts: every sequence's prompt
    (shared prefix tokens, then its own) through pa_pool_add_seq_cached on a
    fresh pool.  Token ids are seeded draws; timed: the adds only."""
    import numpy as np
    rng = np.random.default_rng([w.seed, 99])
    prefix = rng.integers(0, 32000, w.prefix_len).astype(np.int32)
    prompts = [np.concatenate([prefix, rng.integers(0, 32000, int(L) - w.prefix_len).astype(np.int32)])
               for L in w.context_lens]
    nb = 2 * sum(-(-int(L) // w.bs) for L in w.context_lens)
    pool = P.BlockPool(nb, w.bs)
    t0 = time.perf_counter()
    hits = [pool.add_seq_cached(t)[1] for t in prompts]
    us = (time.perf_counter() - t0) * 1e6 / len(prompts)
    return {"sequences": len(prompts), "prompt_tokens": int(sum(len(t) for t in prompts)),
            "cached_tokens": int(sum(hits)), "cached_blocks": pool.num_cached(),
            "host_us_per_sequence": round(us, 2)}


def cpu_baseline(w, budget_s: float, unit: str, fp8_scales=None):
    """The fp64 oracle on a bounded sample of the workload, one host thread.

    The oracle's pool is built untimed.  Timed: the oracle cache write of the
    step's rows (charged pro rata to the sampled sequences) plus the oracle
    decode / prefill of whole sequences taken in order until the CPU budget
    is spent.  Reported in the metric's unit over the sample's own work.
    fp8_scales (k_scale, v_scale): FP8 pools, quantising write."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention as A
    from oracle.state import build_pool, build_state

    st = build_state(w)
    ks, vs = fp8_scales or (1.0, 1.0)
    kv = "e4m3" if fp8_scales else None
    kc, vc = build_pool(w, st, kv_dtype=kv, k_scale=ks, v_scale=vs)
    K, V = w.new_rows()
    lens = w.context_lens.astype(np.int64)
    eb = 1 if fp8_scales else w.elem_bytes
    done, secs, work = [], 0.0, 0.0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if fp8_scales:
            kc, vc = A.write_ref_fp8(kc, vc, K, V, st.step_slots, w.bs, w.dtype, ks, vs)
        else:
            kc, vc = A.write_ref(kc, vc, K, V, st.step_slots, w.bs)
        t_write = time.perf_counter() - t0
        # whole sequences in order, passing over the batch again while the
        # budget lasts (a short workload is timed over several passes)
        order = [s for _ in range(1000) for s in range(w.S)]
        for s in order:
            t0 = time.perf_counter()
            if w.kind == "decode":
                A.decode_ref(w.query[s:s + 1], kc, vc, st.block_tables[s:s + 1], lens[s:s + 1],
                             w.scale, w.bs, w.dtype, kv_dtype=kv, k_scale=ks, v_scale=vs)
                work += float(lens[s]) * w.Hkv * w.D * 2 * eb
            else:
                a, b = int(w.query_start_loc[s]), int(w.query_start_loc[s + 1])
                A.prefill_ref(w.query[a:b], kc, vc, st.block_tables[s:s + 1],
                              np.array([0, b - a]), lens[s:s + 1], w.scale, w.bs, w.dtype,
                              kv_dtype=kv, k_scale=ks, v_scale=vs)
                n, L = b - a, int(lens[s])
                work += 4.0 * w.D * w.H * (n * (L - n) + n * (n + 1) / 2)
            secs += time.perf_counter() - t0
            done.append(s)
            if secs >= budget_s:
                break
    secs += t_write * len(done) / w.S
    value = work / secs / (1e9 if unit == "GB/s" else 1e12)
    passes = len(done) / w.S
    what = (f"{len(done)} of {w.S} sequences" if len(done) < w.S
            else f"{passes:.2f} passes over the {w.S} sequences")
    return {"value": round(value, 6), "unit": unit, "cores": 1, "kind": "oracle",
            "seconds": round(secs, 2),
            "sample": f"{what} of {w.name} (all heads): oracle {w.kind} of those sequences + "
                      f"their share of the oracle write of the step rows; pool built untimed"}


if __name__ == "__main__":
    main()
