#!/usr/bin/env python3
"""Benchmark of the exact tiled attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. fa_fwd on causal multi-head prefill, bf16, B=2, H=32, N=8192, d=128 (K scaled by 2);
  2. fa_decode_splitk (split-K paged decode, partials merged in the same launch) on B=8
     sequences, 32 query heads over 8 KV heads, d=128, lengths uniform in [16384, 32768],
     16-token pages.
Inputs are generated once (seeded) and are resident in HBM before timing starts. The
default 30 untimed steps (about 35 ms of work) let the clock settle first: after an idle
period it ramps over the first 20 to 30 forward calls. After the
steps, each in a loop of its own: fa_fwd on the other two prefill workloads (causal B=4 H=16
N=2048 d=64, and causal GQA B=1 Hq=32 Hkv=8 N=32768 d=128), chunked prefill over the paged
cache, the block-sparse forward, the backward and the fp8 forward.

Prints ONE JSON line. `value` is the forward's algorithmic TFLOP/s (4*d per admissible
(query, key) pair, causal tiles skipped by the method are not counted) over the timed
steps; the decode's algorithmic HBM GB/s (K and V read once per KV head, plus q, o, the
block table and the lengths) is reported next to it. Kernel durations come from HIP
events recorded on the stream the kernels are launched on. `cpu_baseline` times the
float64 CPU oracle (one worker process per core of this process's affinity set, at most 16)
on bounded samples of the prefill and decode workloads and compares its results with the GPU
outputs of the timed runs element by element.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s & % MFMA peak; decode HBM GB/s & % peak (1×MI355X)"
PEAK_FP8_TFLOPS = 5000.0  # dense fp8 MFMA, MI355X public figure
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (no sparsity)
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--fwd-config", type=int, default=3, choices=[2, 3, 4])
    ap.add_argument("--decode-splits", type=int, default=0, help="0 = the library's plan")
    ap.add_argument("--kv-pools", type=int, default=2,
                    help="copies of the decode KV cache used in turn, so that no call finds the "
                         "previous call's pages in L2 or the Infinity Cache (1 = one cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads4", type=int, default=32,
                    help="heads of the N=32768 GQA workload the oracle runs on (of 32)")
    ap.add_argument("--only", choices=["fwd", "decode", "fwd2", "fwd4", "paged", "sparse", "bwd",
                                       "fp8", "fp8v"], default=None,
                    help="time one kernel only (profiling runs)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter scaling)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DB", "WRITE_DB"), default=None,
                    help="write profiles/traffic.json from FETCH_SIZE and WRITE_SIZE rocprofv3 "
                         "databases of runs made with --copy-mib, and exit (no GPU needed)")
    ap.add_argument("--summarize", nargs="+", metavar="DB", default=None,
                    help="print per-kernel averages (duration, counters) of rocprofv3 result "
                         "databases as markdown and exit (no GPU needed)")
    ap.add_argument("--kernel", default=None, help="with --summarize: only kernels whose name contains one of these "
                         "comma-separated fragments")
    return ap.parse_args()


def summarize(paths, kernel=None):
    """Per-kernel averages from rocprofv3 SQLite result databases, as markdown tables.

    `kernel`: comma-separated name fragments; keep only kernels whose name contains one.
    """
    import collections
    import sqlite3

    def short(name):
        name = name.replace("(anonymous namespace)::", "")
        return name.removeprefix("void ").split("(")[0]

    keep = [k for k in (kernel or "").split(",") if k]

    def wanted(name):
        return not keep or any(k in name for k in keep)

    for path in paths:
        con = sqlite3.connect(path)
        tables = {r[0] for r in con.execute("select name from sqlite_master")}
        print(f"\n#### {os.path.basename(path)}\n")
        if "counters_collection" in tables and con.execute(
                "select count(*) from counters_collection").fetchone()[0]:
            vals = collections.defaultdict(lambda: collections.defaultdict(list))
            disp = collections.defaultdict(dict)
            for name, counter, value, did, dur in con.execute(
                    "select kernel_name, counter_name, value, dispatch_id, duration "
                    "from counters_collection"):
                vals[short(name)][counter].append(value)
                disp[short(name)][did] = dur
            print("| kernel | dispatches | mean ns | counter | mean per dispatch |\n"
                  "|---|---|---|---|---|")
            for kname, cs in vals.items():
                if not wanted(kname):
                    continue
                d = disp[kname]
                for counter, v in sorted(cs.items()):
                    print(f"| `{kname}` | {len(d)} | {sum(d.values()) / len(d):.0f} | {counter} | "
                          f"{sum(v) / len(v):.6g} |")
        else:
            # One kernel can serve several bench legs (the dense d = 128 instance runs workload 3
            # in the step and workload 4 after it): a kernel's dispatches are split where their
            # sorted durations jump by more than 1.5x, one row per group.
            disp = collections.defaultdict(list)
            info = {}
            for r in con.execute(
                    "select name, duration, grid_x, grid_y, workgroup_x, vgpr_count, "
                    "accum_vgpr_count, sgpr_count, lds_size, scratch_size from kernels"):
                disp[r[0]].append(r[1])
                info[r[0]] = r[2:]
            rows = []
            for name, durs in disp.items():
                durs = sorted(durs)
                groups = [[durs[0]]]
                for x in durs[1:]:
                    if x > 1.5 * groups[-1][-1]:
                        groups.append([])
                    groups[-1].append(x)
                for gi, g in enumerate(groups):
                    tag = f" (group {gi + 1} of {len(groups)})" if len(groups) > 1 else ""
                    rows.append((short(name) + tag, len(g), sum(g) / len(g), g[0], g[-1], info[name]))
            print("| kernel | calls | mean ns | min ns | max ns | grid | wg | vgpr/agpr/sgpr | "
                  "lds B | scratch B |\n|---|---|---|---|---|---|---|---|---|---|")
            for name, n, mean, lo, hi, i in sorted(rows, key=lambda r: -r[1] * r[2]):
                if not wanted(name):
                    continue
                print(f"| `{name}` | {n} | {mean:.0f} | {lo} | {hi} | {i[0]}x{i[1]} | {i[2]} | "
                      f"{i[3]}/{i[4]}/{i[5]} | {i[6]} | {i[7]} |")


# Kernels whose HBM traffic is reported, with the source file each is compiled from.
TRAFFIC_KERNELS = {
    "fwd": ("fwd_bf16_sp_kernel<128, 0, false>", "exact_tiled_attention_24_amd/csrc/fwd_bf16_sp.hip"),
    "paged": ("fwd_bf16_sp_kernel<128, 1, false>", "exact_tiled_attention_24_amd/csrc/fwd_bf16_sp.hip"),
    "sparse": ("fwd_bf16_sp_kernel<128, 2, false>", "exact_tiled_attention_24_amd/csrc/fwd_bf16_sp.hip"),
    "fp8": ("fwd_bf16_sp_kernel<128, 3, false>", "exact_tiled_attention_24_amd/csrc/fwd_bf16_sp.hip"),
    "fp8v": ("fwd_bf16_sp_kernel<128, 4, false>", "exact_tiled_attention_24_amd/csrc/fwd_bf16_sp.hip"),
    "decode": ("decode_mx_kernel", "exact_tiled_attention_24_amd/csrc/decode_mx.hip"),
    "bwd_dkdv": ("bwd_dkdv_kernel<128>", "exact_tiled_attention_24_amd/csrc/bwd_bf16.hip"),
    "bwd_dq": ("bwd_dq_kernel<128>", "exact_tiled_attention_24_amd/csrc/bwd_bf16.hip"),
}
COPY_KERNEL = "copyBuffer"


def source_digest(rel):
    """Digest of a kernel source's code: comments and blank space do not count, so editing
    a comment does not invalidate counters taken on the same code."""
    import hashlib
    import re

    with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    code = " ".join(text.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def counter_values(path, counter):
    """Per-dispatch values of `counter`: a list of (kernel name, value)."""
    import sqlite3

    con = sqlite3.connect(path)
    return con.execute("select kernel_name, value from counters_collection "
                       "where counter_name = ?", (counter,)).fetchall()


def write_traffic(fetch_db, write_db, copy_mib):
    """HBM bytes per launch: raw counter KiB scaled by what the counter reads for a copy.

    The copy of `copy_mib` MiB reads and writes exactly copy_mib MiB; the ratio of that to
    what FETCH_SIZE / WRITE_SIZE report for it is the scale applied to the kernels.
    """
    fetch = counter_values(fetch_db, "FETCH_SIZE")
    write = counter_values(write_db, "WRITE_SIZE")

    def pick(table, key, largest=False):
        vals = [v for name, v in table if key in name]
        if not vals:
            raise SystemExit(f"no dispatch of a kernel named *{key}* in the counter database")
        if largest:  # the timed copy, not the small staging copies of the set-up
            vals = [v for v in vals if v >= 0.5 * max(vals)]
        return sum(vals) / len(vals), len(vals)

    exact_kib = copy_mib * 1024.0
    f_copy, _ = pick(fetch, COPY_KERNEL, largest=True)
    w_copy, _ = pick(write, COPY_KERNEL, largest=True)
    f_scale, w_scale = exact_kib / f_copy, exact_kib / w_copy
    doc = {"copy_mib": copy_mib, "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}
    for key, (kname, src) in TRAFFIC_KERNELS.items():
        f_kib, nf = pick(fetch, kname)
        w_kib, nw = pick(write, kname)
        doc[key] = {"kernel": kname, "source": src, "source_sha256_16": source_digest(src),
                    "dispatches": [nf, nw], "fetch_kib_raw": round(f_kib, 1),
                    "write_kib_raw": round(w_kib, 1),
                    "bytes": int(round((f_kib * f_scale + w_kib * w_scale) * 1024))}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(json.dumps(doc, indent=1))


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(*args.traffic_from, args.copy_mib or 1024)
        return
    if args.summarize:
        summarize(args.summarize, args.kernel)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the attention path here has no multi-GPU "
              "component (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_24_amd as fa
    from exact_tiled_attention_24_amd import inputs as gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    fa.load_library()  # fails loudly if the HIP library is missing
    props = torch.cuda.get_device_properties(dev)

    do_fwd = args.only in (None, "fwd")
    do_dec = args.only in (None, "decode")
    do_paged = args.only in (None, "paged")
    do_sparse = args.only in (None, "sparse")
    do_bwd = args.only in (None, "bwd")
    do_fp8 = args.only in (None, "fp8")
    do_fp8v = args.only in (None, "fp8v")
    do_fwd2 = args.only in (None, "fwd2") and args.fwd_config != 2
    # (the counter runs for traffic skip workload 4: it launches the same kernel instance as
    # the step's forward, and the counters are attributed by kernel name)
    do_fwd4 = args.only in (None, "fwd4") and args.fwd_config != 4 and not args.copy_mib

    # ---- inputs, resident in HBM ----
    fcfg = gen.CONFIGS[args.fwd_config]
    dcfg = gen.CONFIGS[5]
    fwd_flops = fcfg.flops()
    fx = None
    if do_fwd:
        fx = gen.config_fwd_inputs(fcfg)
    if do_fwd:
        q = gen.to_torch(fx.q, "bf16", dev)
        k = gen.to_torch(fx.k, "bf16", dev)
        v = gen.to_torch(fx.v, "bf16", dev)
        o = torch.empty_like(q)

    dec_bytes, splits, lens_sum = None, None, None
    if do_dec:
        dx = gen.config_decode_inputs(dcfg)
        dq = gen.to_torch(dx.q, "bf16", dev)
        kc = gen.to_torch(dx.k_cache, "bf16", dev)
        vc = gen.to_torch(dx.v_cache, "bf16", dev)
        pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(max(1, args.kv_pools) - 1)]
        table = torch.from_numpy(dx.block_table).to(dev)
        lens = torch.from_numpy(dx.lens.astype(np.int32)).to(dev)
        do = torch.empty_like(dq)
        ws_bytes = fa.fa_decode_workspace_bytes(dcfg.B, dcfg.Hq, dcfg.d, 16, dcfg.len_max,
                                                args.decode_splits)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        splits = args.decode_splits or fa.fa_decode_plan_splits(dcfg.B, dcfg.Hkv, 16,
                                                                dcfg.len_max)
        lens_sum = int(dx.lens.sum())
        dec_bytes = (dx.kv_bytes() + dq.numel() * 2 + do.numel() * 2
                     + 4 * int(sum(-(-int(L) // 16) for L in dx.lens)) + 4 * dcfg.B)
        dec_scale = dx.scale
        dec_inputs = dx

    paged_flops = None
    if do_paged:
        pcfg = gen.PREFILL_PAGED
        px = gen.config_prefill_paged_inputs(pcfg)
        p_q = gen.to_torch(px.q, "bf16", dev)
        p_kc = gen.to_torch(px.k_cache, "bf16", dev)
        p_vc = gen.to_torch(px.v_cache, "bf16", dev)
        p_tab = torch.from_numpy(px.block_table).to(dev)
        p_lens = torch.from_numpy(px.lens.astype(np.int32)).to(dev)
        p_o = torch.empty_like(p_q)
        paged_flops = px.flops()
        paged_scale = px.scale
        paged_lens = [int(L) for L in px.lens]
        del px

    sparse_flops = None
    if do_sparse:
        scfg = gen.BLOCK_SPARSE
        sx = gen.fwd_inputs(scfg.B, scfg.Hq, scfg.Hkv, scfg.N, scfg.d, scfg.seed, causal=scfg.causal)
        s_rows = gen.local_global_blocks(scfg.B, scfg.Hq, scfg.N, scfg.window, scfg.n_global,
                                         scfg.causal)
        s_offs, s_idx = gen.block_csr(s_rows)
        s_q, s_k, s_v = (gen.to_torch(t, "bf16", dev) for t in (sx.q, sx.k, sx.v))
        s_o = torch.empty_like(s_q)
        s_offs_t = torch.from_numpy(s_offs).to(dev)
        s_idx_t = torch.from_numpy(s_idx).to(dev)
        sparse_flops = 4.0 * scfg.d * gen.block_pairs(s_rows, scfg.B, scfg.Hq, scfg.N, scfg.causal)
        sparse_blocks = int(s_idx.size)
        del sx

    bwd_flops = None
    if do_bwd:
        # backward of the forward workload: 10 d FLOP per admissible pair (S, dP, dV, dK, dQ)
        bcfg = gen.CONFIGS[args.fwd_config]
        bx = gen.config_fwd_inputs(bcfg)
        b_q, b_k, b_v = (gen.to_torch(t, "bf16", dev) for t in (bx.q, bx.k, bx.v))
        b_do = gen.to_torch(gen.round_to_bf16(
            np.random.default_rng(bcfg.seed + 100).standard_normal(bx.q.shape, dtype=np.float32)),
            "bf16", dev)
        b_o, b_m, b_l = fa.fa_fwd(b_q, b_k, b_v, scale=bx.scale, causal=bcfg.causal,
                                  return_stats=True)
        b_ws = torch.empty(fa.fa_bwd_workspace_bytes(bcfg.B, bcfg.Hq, bcfg.N), dtype=torch.uint8,
                           device=dev)
        bwd_flops = 2.5 * bcfg.flops()
        bwd_scale = bx.scale
        del bx

    # the other prefill workloads, timed in loops of their own after the steps
    extra_fwd = {}
    for cid, on in ((2, do_fwd2), (4, do_fwd4)):
        if on:
            c = gen.CONFIGS[cid]
            x = gen.config_fwd_inputs(c)
            tq, tk, tv = (gen.to_torch(t, "bf16", dev) for t in (x.q, x.k, x.v))
            extra_fwd[cid] = dict(cfg=c, x=x, q=tq, k=tk, v=tv, o=torch.empty_like(tq))

    fp8_flops = None
    if do_fp8:
        # the forward workload with e4m3 Q and K (the same draws, a different rounding)
        f8cfg = gen.CONFIGS[args.fwd_config]
        f8x = gen.fp8_fwd_inputs(f8cfg.B, f8cfg.Hq, f8cfg.Hkv, f8cfg.N, f8cfg.d, f8cfg.seed,
                                 causal=f8cfg.causal, k_mult=f8cfg.k_mult)
        f8_q, f8_k = gen.to_torch(f8x.q, "e4m3", dev), gen.to_torch(f8x.k, "e4m3", dev)
        f8_v = gen.to_torch(f8x.v, "bf16", dev)
        f8_o = torch.empty(f8x.q.shape, dtype=torch.bfloat16, device=dev)
        fp8_flops = f8cfg.flops()
        fp8_scale = f8x.scale
        del f8x

    def run_fp8():
        fa.fa_fwd_fp8(f8_q, f8_k, f8_v, scale=fp8_scale, causal=f8cfg.causal, out=f8_o)

    if do_fp8v:
        # the forward workload with Q, K and V in e4m3 (P rounded to e4m3, P V on fp8 too)
        v8cfg = gen.CONFIGS[args.fwd_config]
        v8x = gen.fp8_fwd_inputs(v8cfg.B, v8cfg.Hq, v8cfg.Hkv, v8cfg.N, v8cfg.d, v8cfg.seed,
                                 causal=v8cfg.causal, k_mult=v8cfg.k_mult, v_fp8=True)
        v8_q, v8_k, v8_v = (gen.to_torch(t, "e4m3", dev) for t in (v8x.q, v8x.k, v8x.v))
        v8_o = torch.empty(v8x.q.shape, dtype=torch.bfloat16, device=dev)
        fp8v_flops = v8cfg.flops()
        fp8v_scale = v8x.scale
        del v8x

    def run_fp8v():
        fa.fa_fwd_fp8(v8_q, v8_k, v8_v, scale=fp8v_scale, causal=v8cfg.causal, out=v8_o)

    def run_bwd():
        fa.fa_bwd(b_q, b_k, b_v, b_o, b_do, b_m, b_l, scale=bwd_scale, causal=bcfg.causal,
                  workspace=b_ws)

    def run_sparse():
        fa.fa_fwd_block_sparse(s_q, s_k, s_v, s_offs_t, s_idx_t, scale=scfg.scale,
                               causal=scfg.causal, out=s_o)

    def run_paged():
        fa.fa_fwd_paged(p_q, p_kc, p_vc, p_tab, p_lens, scale=paged_scale, causal=pcfg.causal,
                        out=p_o)

    def run_fwd():
        fa.fa_fwd(q, k, v, scale=fx.scale, causal=fcfg.causal, out=o)

    calls = [0]

    def run_decode():
        kp, vp = pools[calls[0] % len(pools)]
        calls[0] += 1
        fa.fa_decode_splitk(dq, kp, vp, table, lens, dcfg.len_max, scale=dec_scale,
                            num_splits=args.decode_splits, out=do, workspace=ws)

    copy_src = copy_dst = None
    if args.copy_mib:
        copy_src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        copy_dst = torch.empty_like(copy_src)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        if do_fwd:
            run_fwd()
        if do_dec:
            run_decode()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        e = ev[s]
        e[0].record(stream)
        if do_fwd:
            run_fwd()
        e[1].record(stream)
        e[2].record(stream)
        if do_dec:
            run_decode()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if copy_src is not None:
        for _ in range(3):
            copy_dst.copy_(copy_src)
        torch.cuda.synchronize()

    def timed_loop(fn, reps, warmup):
        for _ in range(warmup):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    fwd_extra_ms = {}
    for cid, e in extra_fwd.items():
        def run(e=e):
            fa.fa_fwd(e["q"], e["k"], e["v"], scale=e["x"].scale, causal=e["cfg"].causal,
                      out=e["o"])
        fwd_extra_ms[cid] = timed_loop(run, max(10, args.steps), args.warmup)

    # chunked prefill over the paged cache: timed on its own, after the steps
    paged_ms = None
    if do_paged:
        for _ in range(args.warmup):
            run_paged()
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in pev:
            a.record(stream)
            run_paged()
            b.record(stream)
        torch.cuda.synchronize()
        paged_ms = np.array([a.elapsed_time(b) for a, b in pev])

    sparse_ms = None
    if do_sparse:
        for _ in range(args.warmup):
            run_sparse()
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in sev:
            a.record(stream)
            run_sparse()
            b.record(stream)
        torch.cuda.synchronize()
        sparse_ms = np.array([a.elapsed_time(b) for a, b in sev])

    fp8_ms = None
    if do_fp8:
        for _ in range(args.warmup):
            run_fp8()
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in fev:
            a.record(stream)
            run_fp8()
            b.record(stream)
        torch.cuda.synchronize()
        fp8_ms = np.array([a.elapsed_time(b) for a, b in fev])

    fp8v_ms = None
    if do_fp8v:
        for _ in range(args.warmup):
            run_fp8v()
        vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in vev:
            a.record(stream)
            run_fp8v()
            b.record(stream)
        torch.cuda.synchronize()
        fp8v_ms = np.array([a.elapsed_time(b) for a, b in vev])

    bwd_ms = None
    if do_bwd:
        for _ in range(min(args.warmup, 2)):
            run_bwd()
        bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(max(1, args.steps // 4))]
        for a, b in bev:
            a.record(stream)
            run_bwd()
            b.record(stream)
        torch.cuda.synchronize()
        bwd_ms = np.array([a.elapsed_time(b) for a, b in bev])

    fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    dec_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])

    fwd_tflops = fwd_flops / (fwd_ms.mean() * 1e-3) / 1e12 if do_fwd else None
    dec_gbps = dec_bytes / (dec_ms.mean() * 1e-3) / 1e9 if do_dec else None
    traffic = load_traffic()

    result = {
        "metric": METRIC,
        "value": round(fwd_tflops, 2) if fwd_tflops else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16-rounded; no dataset)",
        "config": {
            "workload": f"fwd: {fcfg.name}; decode: {dcfg.name}",
            "fwd": {"B": fcfg.B, "Hq": fcfg.Hq, "Hkv": fcfg.Hkv, "N": fcfg.N, "d": fcfg.d,
                    "causal": fcfg.causal, "algorithmic_flops": fwd_flops},
            "decode": {"B": dcfg.B, "Hq": dcfg.Hq, "Hkv": dcfg.Hkv, "d": dcfg.d, "page": 16,
                       "seq_lens_sum": lens_sum, "splits": splits,
                       "algorithmic_bytes": dec_bytes},
            "device": props.name, "cus": props.multi_processor_count,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(fwd_tflops, 2) if fwd_tflops else None,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4) if fwd_tflops else None,
            "traffic": traffic.get("fwd"),
            "kernel": "fwd_bf16_sp_kernel<128, 0, false>",
            "avg_launch_ms": round(float(fwd_ms.mean()), 5) if do_fwd else None,
        },
        "decode": {
            "value": round(dec_gbps, 1) if dec_gbps else None,
            "unit": "GB/s",
            "tokens_per_s": round(dcfg.B / (dec_ms.mean() * 1e-3), 1) if do_dec else None,
            "kv_tokens_per_s": round(lens_sum / (dec_ms.mean() * 1e-3), 1) if do_dec else None,
            "roofline": {
                "bound": "hbm",
                "achieved": round(dec_gbps, 1) if dec_gbps else None,
                "peak": PEAK_HBM_GBPS,
                "unit": "GB/s",
                "frac": round(dec_gbps / PEAK_HBM_GBPS, 4) if dec_gbps else None,
                "traffic": traffic.get("decode"),
                "avg_call_ms": round(float(dec_ms.mean()), 5) if do_dec else None,
            },
        },
        "fwd_tokens_per_s": round(fcfg.B * fcfg.N / (fwd_ms.mean() * 1e-3), 1) if do_fwd else None,
    }
    if fwd_extra_ms:
        result["fwd_configs"] = {}
    for cid, ms in fwd_extra_ms.items():
        c = extra_fwd[cid]["cfg"]
        tf = c.flops() / (ms.mean() * 1e-3) / 1e12
        result["fwd_configs"][str(cid)] = {
            "workload": c.name, "algorithmic_flops": c.flops(), "value": round(tf, 2),
            "unit": "TFLOP/s", "avg_call_ms": round(float(ms.mean()), 5), "calls": int(ms.size),
            "tokens_per_s": round(c.B * c.N / (ms.mean() * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "kernel": f"fwd_bf16_sp_kernel<{c.d}, 0, false>"},
        }
    if do_paged:
        p_tflops = paged_flops / (paged_ms.mean() * 1e-3) / 1e12
        result["paged_prefill"] = {
            "workload": pcfg.name, "seq_lens": paged_lens, "algorithmic_flops": paged_flops,
            "value": round(p_tflops, 2), "unit": "TFLOP/s",
            "avg_call_ms": round(float(paged_ms.mean()), 5),
            "tokens_per_s": round(pcfg.B * pcfg.Nq / (paged_ms.mean() * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(p_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(p_tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic.get("paged"), "kernel": "fwd_bf16_sp_kernel<128, 1, false>"},
        }
    if do_sparse:
        s_tflops = sparse_flops / (sparse_ms.mean() * 1e-3) / 1e12
        result["block_sparse"] = {
            "workload": scfg.name, "listed_blocks": sparse_blocks, "algorithmic_flops": sparse_flops,
            "value": round(s_tflops, 2), "unit": "TFLOP/s",
            "avg_call_ms": round(float(sparse_ms.mean()), 5),
            "tokens_per_s": round(scfg.B * scfg.N / (sparse_ms.mean() * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(s_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(s_tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic.get("sparse"), "kernel": "fwd_bf16_sp_kernel<128, 2, false>"},
        }
    if do_fp8:
        f_tflops = fp8_flops / (fp8_ms.mean() * 1e-3) / 1e12
        # half the work (S = Q K^T) on the fp8 matrix cores, half (P V) on the bf16 ones
        mixed_peak = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
        result["fp8_qk"] = {
            "workload": f"{f8cfg.name} with e4m3 Q and K", "algorithmic_flops": fp8_flops,
            "value": round(f_tflops, 2), "unit": "TFLOP/s",
            "avg_call_ms": round(float(fp8_ms.mean()), 5),
            "roofline": {"bound": "mfma", "achieved": round(f_tflops, 2),
                         "peak": round(mixed_peak, 1), "unit": "TFLOP/s",
                         "frac": round(f_tflops / mixed_peak, 4),
                         "peak_note": "S on fp8 (5.0 PFLOP/s), P V on bf16 (2.5 PFLOP/s)",
                         "traffic": traffic.get("fp8"), "kernel": "fwd_bf16_sp_kernel<128, 3, false>"},
        }
    if do_fp8v:
        v_tflops = fp8v_flops / (fp8v_ms.mean() * 1e-3) / 1e12
        result["fp8_qkv"] = {
            "workload": f"{v8cfg.name} with e4m3 Q, K and V (weights rounded to e4m3)",
            "algorithmic_flops": fp8v_flops, "value": round(v_tflops, 2), "unit": "TFLOP/s",
            "avg_call_ms": round(float(fp8v_ms.mean()), 5),
            "roofline": {"bound": "mfma", "achieved": round(v_tflops, 2), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(v_tflops / PEAK_FP8_TFLOPS, 4),
                         "traffic": traffic.get("fp8v"), "kernel": "fwd_bf16_sp_kernel<128, 4, false>"},
        }
    if do_bwd:
        b_tflops = bwd_flops / (bwd_ms.mean() * 1e-3) / 1e12
        result["backward"] = {
            "workload": f"backward of {bcfg.name}", "algorithmic_flops": bwd_flops,
            "value": round(b_tflops, 2), "unit": "TFLOP/s",
            "avg_call_ms": round(float(bwd_ms.mean()), 5), "calls": int(bwd_ms.size),
            "roofline": {"bound": "mfma", "achieved": round(b_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(b_tflops / PEAK_BF16_TFLOPS, 4),
                         "kernels": "bwd_dq_kernel, bwd_dkdv_kernel",
                         # HBM bytes of one call (both kernels), when both were counted
                         "traffic": (sum(traffic[k] for k in ("bwd_dq", "bwd_dkdv"))
                                     if all(traffic.get(k) for k in ("bwd_dq", "bwd_dkdv")) else None),
                         "traffic_by_kernel": {k: traffic.get(k) for k in ("bwd_dq", "bwd_dkdv")}},
        }
    try:  # the counter evidence behind the tile and split choices (from the sweeps)
        with open(os.path.join(ROOT, "profiles", "choices.json")) as f:
            result["choices"] = json.load(f)
    except (OSError, ValueError):
        result["choices"] = None
    if not args.no_cpu_baseline:
        legs = {}
        if do_fwd:
            legs[fcfg_id(fcfg)] = (fx, fcfg, o, fwd_ms, None)
        for cid, e in extra_fwd.items():
            heads = args.cpu_heads4 if cid == 4 else None
            legs[cid] = (e["x"], e["cfg"], e["o"], fwd_extra_ms[cid], heads)
        dec_leg = (dec_inputs, do, dec_ms) if do_dec else None
        result["cpu_baseline"] = cpu_baseline(legs, dec_leg, main_cfg=fcfg_id(fcfg))
    print(json.dumps(result), flush=True)


def fcfg_id(cfg):
    from exact_tiled_attention_24_amd import inputs as gen

    return next(k for k, c in gen.CONFIGS.items() if c is cfg)


def load_traffic():
    """Measured HBM bytes per launch, per kernel; None where the kernel's source has changed
    since the counters were taken (or no counters were taken)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return {}
    out = {}
    for key, (_, src) in TRAFFIC_KERNELS.items():
        ent = doc.get(key)
        if ent and ent.get("source_sha256_16") == source_digest(src):
            out[key] = ent["bytes"]
    return out


def cpu_baseline(legs, dec_leg, main_cfg):
    """The float64 oracle on bounded samples of the workloads, timed on this host's cores.

    `legs`: {config id: (inputs, config, GPU output tensor, GPU call times in ms, heads)}; the
    oracle runs `heads` evenly spaced heads (all when None) of each, one head per task in a
    pool of worker processes (one per core of the affinity set, at most 16, one BLAS thread
    each), and its results are compared with the GPU output of the timed calls. `dec_leg`:
    (decode inputs, GPU output, call times) for the decode workload (all sequences).
    """
    from oracle import pool
    import oracle

    workers = pool.worker_count()
    per = {}
    total_s = 0.0
    for cid, (x, c, o_gpu, ms, heads) in legs.items():
        G = c.Hq // c.Hkv
        all_heads = [(b, h) for b in range(c.B) for h in range(c.Hq)]
        n = len(all_heads) if heads is None else max(1, min(int(heads), len(all_heads)))
        pick = [all_heads[int(round(i * (len(all_heads) - 1) / max(1, n - 1)))] for i in range(n)]
        pick = sorted(set(pick))
        t0 = time.perf_counter()
        refs = list(pool.attention_heads(((x.q[b, h], x.k[b, h // G], x.v[b, h // G])
                                          for b, h in pick), x.scale, c.causal, workers=workers))
        dt = time.perf_counter() - t0
        total_s += dt
        err = 0.0
        for (b, h), (o_ref, _, _) in zip(pick, refs):
            got = o_gpu[b, h].float().cpu().numpy().astype(np.float64)
            err = max(err, float(np.abs(got - o_ref).max()))
        flops = c.flops() / len(all_heads) * len(pick)
        oracle_tflops = flops / dt / 1e12
        gpu_tflops = c.flops() / (ms.mean() * 1e-3) / 1e12
        per[str(cid)] = {
            "workload": c.name, "heads": f"{len(pick)} of {len(all_heads)}",
            "seconds": round(dt, 3), "value": round(oracle_tflops, 6), "unit": "TFLOP/s",
            "max_abs_err_vs_gpu": err, "gpu_over_oracle": round(gpu_tflops / oracle_tflops, 1),
            "extrapolated": len(pick) < len(all_heads),
        }
    if dec_leg is not None:
        dx, o_gpu, ms = dec_leg
        t0 = time.perf_counter()
        o_ref, _, _ = oracle.decode(dx.q, dx.k_seqs, dx.v_seqs, dx.scale)
        dt = time.perf_counter() - t0
        total_s += dt
        err = float(np.abs(o_gpu.float().cpu().numpy().astype(np.float64) - o_ref).max())
        kv = dx.kv_bytes()
        per["5"] = {"workload": "paged split-K decode (all sequences)", "seconds": round(dt, 3),
                    "value": round(kv / dt / 1e9, 3), "unit": "GB/s of K and V",
                    "max_abs_err_vs_gpu": err,
                    "gpu_over_oracle": round((kv / (ms.mean() * 1e-3)) / (kv / dt), 1),
                    "extrapolated": False, "cores": 1}
    main = per.get(str(main_cfg), next(iter(per.values())) if per else {})
    return {"value": main.get("value"), "unit": main.get("unit", "TFLOP/s"), "cores": workers,
            "kind": "oracle",
            "sample": f"float64 numpy oracle, one head per task on {workers} worker processes: "
                      + "; ".join(f"workload {k}: {v.get('heads', 'all sequences')}"
                                  for k, v in per.items()),
            "seconds": round(total_s, 3), "gpu_over_oracle": main.get("gpu_over_oracle"),
            "per_config": per}


if __name__ == "__main__":
    main()
