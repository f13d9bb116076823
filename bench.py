"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass over every form of the path, each on its own seeded
synthetic input resident in HBM:
  prefill  causal GQA prefill, 2048 x 2048, 16/8 heads, d 256, f16 K/V, f32 Q/O
           (mask tile classification + MFMA attention kernel)
  decode   paged decode, 64 sequences of 512..16384 tokens, 16-token pages in a
           permuted 65536-page pool, 32/8 heads, d 128, f16 K/V
           (split-KV partial pass + log-sum-exp reduce)
  verify   DFlash2 block verify, 4 lanes x 16 drafted rows, ring window 4096,
           32/8 heads, d 128: pack -> mask -> attention over the packed
           buffers, the pack-free verify attention read from the ring in
           place, then commit
  multi    prepare (Q/K RMS norm, rotary embedding, K/V into the pages) and
           multi-token paged attention: 16 sequences x 16 new tokens over
           contexts of 1024..8192 tokens in 16-token pages, 32/8 heads, d 128
           (block verify straight from the page table)
W untimed steps, then K timed steps bracketed by torch.cuda.synchronize().
Each row is timed with HIP events on the stream its kernels run on; a GPU
sleep ahead of each timed step lets the host enqueue the whole step first,
so an event pair brackets the GPU time of its call only.  ms_per_step is the
GPU time from the step's first call to its last; wall_ms_per_step is the
host clock (sleep included).

Prints ONE JSON line.  `value` is the prefill row's algorithmic TFLOP/s
(4 * n_heads * head_dim per visible (query, key) pair); the paged-decode
row's algorithmic KV GB/s and the verify rows are reported beside it, with
roofline fractions against MI355X peaks (dense fp16 MFMA 2.5 PFLOP/s, HBM
8 TB/s).  `cpu_baseline` times the fp64 oracle on a bounded sample of the
prefill workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

PEAK_F16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
COPY_PROBE_BYTES = 1 << 30
HERE = os.path.dirname(os.path.abspath(__file__))


def measured_traffic():
    """HBM bytes per paged-decode call from the committed counter summary, or None
    when a source the kernels are built from has changed since the counters were
    taken."""
    import hashlib
    path = os.path.join(HERE, "profiles", "paged_decode_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec.get("sources", []):
        with open(os.path.join(HERE, src), "rb") as f:
            h.update(f.read())
    return rec["bytes_per_launch"] if rec.get("sources") and h.hexdigest() == rec.get("sources_sha256") else None


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--rows-only", choices=["prefill", "decode", "verify", "multi", "chunked"], default=None,
                    help="time one row alone (profiling runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (the reference for scaling HBM byte counters)")
    return ap.parse_args()


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the path has no multi-GPU form here "
              "(one process drives one MI355X); --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import attention_flash_attn_03_amd as fa
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.int16)
            if bf16:
                t = t.view(torch.bfloat16)
        elif a.dtype == np.uint32:
            t = t.view(torch.int32)
        return t.to(dev)

    print("bench: building inputs", file=sys.stderr, flush=True)
    want = {"prefill", "decode", "verify", "multi"} if args.rows_only is None else {args.rows_only}
    # ---------------- prefill (causal, 2048 x 2048)
    pc = workloads.prefill_case("causal2k")
    m = pc.meta
    prefill_flops = 4.0 * m["n_heads"] * m["head_dim"] * pc.visible_pairs
    if "prefill" in want:
        pq, pk, pv, pm = to_dev(pc.q), to_dev(pc.k), to_dev(pc.v), to_dev(pc.mask)
        po = torch.empty(pc.q.shape, dtype=torch.float32, device=dev)
        pp = fa.prefill_params(pq, pk, pv, pm, po, scale=pc.scale)
        pws = torch.empty(max(1, fa.prefill_workspace_bytes(pp)), dtype=torch.uint8, device=dev)

    # ---------------- paged decode
    dm = dict(batch=64, page_size=16, num_pages=65536, n_heads=32, n_kv_heads=8, head_dim=128)
    if "decode" in want:
        dc = workloads.paged_case()
        dq = to_dev(dc.q)
        dkp, dvp = to_dev(dc.k_pool), to_dev(dc.v_pool)
        dpt, dctx = to_dev(dc.page_table), to_dev(dc.context_lens)
        do = torch.empty(dc.q.shape, dtype=torch.float32, device=dev)
        dp = fa.decode_params(dq, dkp, dvp, dpt, do, scale=dc.scale, max_context=dc.max_context)
        dws = torch.empty(fa.decode_workspace_bytes(dp), dtype=torch.uint8, device=dev)
        dm = dc.meta
        ctx = dc.context_lens.astype(np.int64)
        decode_bytes = (float(ctx.sum()) * dm["n_kv_heads"] * dm["head_dim"] * 2 * 2      # K and V rows, f16
                        + dc.q.nbytes + dc.q.nbytes                                       # Q in, O out (f32)
                        + 4.0 * float(np.sum(-(-ctx // dm["page_size"])))                 # page-table entries
                        + 4.0 * dm["batch"])                                              # context lengths
        decode_flops = 4.0 * dm["n_heads"] * dm["head_dim"] * float(ctx.sum())

    # ---------------- block verify
    vc = workloads.dflash_case() if "verify" in want else None
    b, h, hk, d, r, w = (4, 32, 8, 128, 16, 4096) if vc is None else vc.geom
    klen = w - 1 + r
    if vc is not None:
        vp = fa.DFlashParams(b, h, hk, d, r, w, klen, vc.max_commit)
        ring_k, ring_v = to_dev(vc.ring_k, True), to_dev(vc.ring_v, True)
        cq, ck, cv = to_dev(vc.cur_q), to_dev(vc.cur_k), to_dev(vc.cur_v)
        vL, vwp, vcnt = to_dev(vc.cache_lengths), to_dev(vc.write_positions), to_dev(vc.commit_counts)
        packed_q = torch.empty((b, h, r, d), dtype=torch.bfloat16, device=dev)
        packed_k = torch.empty((b, hk, klen, d), dtype=torch.bfloat16, device=dev)
        packed_v = torch.empty_like(packed_k)
        vmask = torch.empty((b, h, r, klen), dtype=torch.bfloat16, device=dev)
        vout = torch.empty((b, h, r, d), dtype=torch.float32, device=dev)
        # packed Q [b, h, r, d] seen as [batch, rows, heads, d]; packed K/V [b, hk, k, d] as [batch, k, hk, d]
        vq_view, vk_view, vv_view = (packed_q.permute(0, 2, 1, 3), packed_k.permute(0, 2, 1, 3),
                                     packed_v.permute(0, 2, 1, 3))
        vo_view = vout.permute(0, 2, 1, 3)
        vap = fa.prefill_params(vq_view, vk_view, vv_view, vmask, vo_view, scale=vc.scale)
        vws = torch.empty(max(1, fa.prefill_workspace_bytes(vap)), dtype=torch.uint8, device=dev)
        L = vc.cache_lengths.astype(np.int64)
        vis_cache = np.minimum(L, w - 1)
        pack_bytes = (vc.cur_q.nbytes + vc.cur_k.nbytes + vc.cur_v.nbytes + 8.0 * b
                      + float(vis_cache.sum()) * hk * d * 2 * 2
                      + b * h * r * d * 2 + 2.0 * b * hk * klen * d * 2)
        mask_bytes = 4.0 * b + b * h * r * klen * 2
        # rows visible per query row: r drafted + min(L, w - 1 - i) cached
        vis_rows = np.array([[r + min(int(Lb), w - 1 - i) for i in range(r)] for Lb in L])
        verify_attn_bytes = (b * h * r * d * 2 + b * h * r * d * 4 + b * h * r * klen * 2
                             + float(np.max(vis_rows, axis=1).sum()) * hk * d * 2 * 2)
        verify_attn_flops = 4.0 * d * h * float(vis_rows.sum())
        vfo = torch.empty((b, h, r, d), dtype=torch.float32, device=dev)
        vfws = torch.empty(fa.verify_workspace_bytes(vp), dtype=torch.uint8, device=dev)
        # pack-free verify: current Q/K/V (f32), lengths and positions, the visible ring rows, O (f32)
        fused_bytes = (vc.cur_q.nbytes + vc.cur_k.nbytes + vc.cur_v.nbytes + 8.0 * b
                       + float(vis_cache.sum()) * hk * d * 2 * 2 + b * h * r * d * 4)
        cnt = np.minimum(vc.commit_counts.astype(np.int64), vc.max_commit)
        commit_bytes = float(cnt.sum()) * hk * d * (4 + 2) * 2 + 8.0 * b

    # ---------------- multi-token paged attention: block verify straight from the page table
    if "multi" in want:
        mc = workloads.paged_multi_case(max_tokens=16, batch=16, ctx_lo=1024, ctx_hi=8192, num_pages=8192,
                                        n_heads=32, n_kv_heads=8, head_dim=128, seed=6, query_lens=np.full(16, 16))
        mpc = mc.paged
        mq = to_dev(mc.q)
        mkp, mvp = to_dev(mpc.k_pool), to_dev(mpc.v_pool)
        mpt, mql, mst = to_dev(mpc.page_table), to_dev(mc.query_lens), to_dev(mc.position_starts)
        mo = torch.empty(mc.q.shape, dtype=torch.float32, device=dev)
        mpp = fa.paged_prefill_params(mq, mkp, mvp, mpt, mo, scale=mpc.scale, max_context=mpc.max_context)
        mws = torch.empty(fa.paged_prefill_workspace_bytes(mpp), dtype=torch.uint8, device=dev)
        mctx = mpc.context_lens.astype(np.int64)
        # K and V rows of every context token, Q and O (f32), the page-table entries, lengths and starts
        multi_bytes = (float(mctx.sum()) * 8 * 128 * 2 * 2 + 2.0 * mc.q.nbytes
                       + 4.0 * float(np.sum(-(-mctx // 16))) + 8.0 * len(mctx))
        # prepare: raw Q/K/V projections of the new tokens, Q/K norm weights
        mqr = to_dev(workloads.normal_f32(16 * 16 * 32 * 128, [6, 20]).reshape(16, 16, 32, 128))
        mkr = to_dev(workloads.normal_f32(16 * 16 * 8 * 128, [6, 21]).reshape(16, 16, 8, 128))
        mvr = to_dev(workloads.normal_f32(16 * 16 * 8 * 128, [6, 22]).reshape(16, 16, 8, 128))
        mqn = torch.ones((1, 128), dtype=torch.float32, device=dev)
        mkn = torch.ones((1, 128), dtype=torch.float32, device=dev)
        # raw Q/K/V read (f32), prepared Q written (f32), K/V rows written (f16), lengths and starts
        prep_bytes = (mqr.numel() + mkr.numel() + mvr.numel() + mqr.numel()) * 4.0 + mkr.numel() * 2 * 2.0 + 8.0 * 16
        # 4 * heads * d per (query token, visible key): token i of a sequence sees start + i + 1 keys
        multi_flops = 4.0 * 32 * 128 * float(sum(int(st) * int(n) + int(n) * (int(n) + 1) // 2
                                                 for st, n in zip(mc.position_starts, mc.query_lens)))

    stream = torch.cuda.current_stream()

    def run_prefill():
        fa.attn_prefill(pq, pk, pv, pm, po, scale=pc.scale, workspace=pws)

    def run_decode():
        fa.attn_paged_decode(dq, dkp, dvp, dpt, dctx, do, scale=dc.scale, max_context=dc.max_context, workspace=dws)

    def run_pack():
        fa.dflash_pack(vp, ring_k, ring_v, cq, ck, cv, vL, vwp, packed_q, packed_k, packed_v)

    def run_mask():
        fa.dflash_mask(vp, vL, vmask)

    def run_verify_attn():
        fa.attn_prefill(vq_view, vk_view, vv_view, vmask, vo_view, scale=vc.scale, workspace=vws)

    def run_verify_fused():
        fa.dflash_verify_attention(vp, ring_k, ring_v, cq, ck, cv, vL, vwp, vfo, scale=vc.scale, workspace=vfws)

    def run_prepare():
        fa.attn_paged_prepare(mqr, mkr, mvr, mqn, mkn, mpt, mql, mst, mq, mkp, mvp, rope_dim=128, rope_theta=1e4,
                              rope_interleaved=False, epsilon=1e-6, max_context=mpc.max_context)

    def run_multi():
        fa.attn_paged_prefill(mq, mkp, mvp, mpt, mql, mst, mo, scale=mpc.scale, max_context=mpc.max_context,
                              workspace=mws)

    def run_commit():
        fa.dflash_commit(vp, ck, cv, vcnt, vwp, ring_k, ring_v)

    rows = []
    if "prefill" in want:
        rows.append(("prefill", run_prefill))
    if "decode" in want:
        rows.append(("decode", run_decode))
    if "verify" in want:
        rows += [("pack", run_pack), ("mask", run_mask), ("verify_attn", run_verify_attn),
                 ("verify_fused", run_verify_fused), ("commit", run_commit)]
    if "multi" in want:
        rows += [("prepare", run_prepare), ("paged_prefill", run_multi)]

    events = {name: [] for name, _ in rows}
    head_start = [0]  # GPU sleep (cycles) ahead of each timed step

    def step(record):
        if record and head_start[0]:
            # keeps the GPU busy while the host enqueues the step, so each call's
            # event pair brackets its own GPU time and not the host's launch work
            torch.cuda._sleep(head_start[0])
        for name, fn in rows:
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                events[name].append((e0, e1))
            else:
                fn()

    if args.copy_probe:
        # elementwise copy of known size: reads and writes COPY_PROBE_BYTES once per launch
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    avg_ms, ms_per_step, wall_ms_per_step = {}, None, None
    if rows:  # every row but the chunked prefill, which is timed on its own below
        print("bench: warmup", file=sys.stderr, flush=True)
        for _ in range(args.warmup):
            step(False)
        torch.cuda.synchronize()
        # size the head start: twice the host's enqueue time of one step, in sleep cycles
        t_host = time.perf_counter()
        step(False)
        t_host = time.perf_counter() - t_host
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        torch.cuda._sleep(1 << 20)
        c1.record(stream)
        torch.cuda.synchronize()
        cycles_per_ms = (1 << 20) / max(c0.elapsed_time(c1), 1e-3)
        head_start[0] = int(min(2.0 * t_host * 1e3 + 0.2, 20.0) * cycles_per_ms)
        print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        avg_ms = {name: float(np.mean([a.elapsed_time(b_) for a, b_ in ev])) for name, ev in events.items() if ev}
        # GPU time of a step: first call's start event to the last call's end event
        first, last = events[rows[0][0]], events[rows[-1][0]]
        ms_per_step = float(np.mean([a[0].elapsed_time(z[1]) for a, z in zip(first, last)]))
        wall_ms_per_step = 1e3 * wall / max(1, args.steps)

    # ---------------- chunked prefill at head_dim 512, timed on its own (outside the step)
    chunk = None
    if args.rows_only in (None, "chunked"):
        print("bench: chunked prefill (d 512)", file=sys.stderr, flush=True)
        if "decode" in want:
            del dkp, dvp
            torch.cuda.empty_cache()
        cc = workloads.prefill_case("chunked8k")
        cq3, ck3, cv3, cm3 = to_dev(cc.q), to_dev(cc.k), to_dev(cc.v), to_dev(cc.mask)
        co3 = torch.empty(cc.q.shape, dtype=torch.float32, device=dev)
        cp3 = fa.prefill_params(cq3, ck3, cv3, cm3, co3, scale=cc.scale)
        cws3 = torch.empty(max(1, fa.prefill_workspace_bytes(cp3)), dtype=torch.uint8, device=dev)
        for _ in range(2):
            fa.attn_prefill(cq3, ck3, cv3, cm3, co3, scale=cc.scale, workspace=cws3)
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(3, args.steps // 2)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fa.attn_prefill(cq3, ck3, cv3, cm3, co3, scale=cc.scale, workspace=cws3)
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        c_ms = float(np.mean([a.elapsed_time(b_) for a, b_ in ts]))
        c_flops = 4.0 * cc.meta["n_heads"] * cc.meta["head_dim"] * cc.visible_pairs
        chunk = {"workload": "chunked prefill 4096 rows x 8192 keys (10% holes), 16/2 heads, d 512",
                 "ms": c_ms, "tflops": c_flops / (c_ms * 1e-3) / 1e12,
                 "frac": c_flops / (c_ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, "gflop": c_flops / 1e9}

    # ---------------- CPU baseline: the oracle on a bounded sample of the prefill rows
    cpu = None
    if not args.no_cpu_baseline and args.rows_only is None:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        import oracle
        oracle.build()
        rows_all = pc.q.shape[1]
        cached = m["cached"]

        def run_rows(sel):
            t = time.perf_counter()
            oracle.attention(pc.q[:, sel], pc.k, pc.v, pc.mask[:, :, sel], scale=pc.scale)
            return time.perf_counter() - t

        def flops_of(sel):
            return 4.0 * m["n_heads"] * m["head_dim"] * float(np.minimum(cached + sel + 1, m["kv_len"]).sum())

        probe = np.linspace(0, rows_all - 1, 32).astype(np.int64)
        t_probe = run_rows(probe)
        rate = flops_of(probe) / max(t_probe, 1e-6)
        n = int(min(rows_all, max(32, rows_all * (args.cpu_seconds * rate / prefill_flops))))
        sel = np.linspace(0, rows_all - 1, n).astype(np.int64)
        t_cpu = run_rows(sel)
        cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
        cpu = {"value": flops_of(sel) / t_cpu / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": "%d of %d query rows (evenly spaced), all 16 heads, of the causal 2048x2048 prefill; "
                         "%.1f s of fp64 compute" % (n, rows_all, t_cpu)}

    def roofline_hbm(bytes_, ms):
        gbps = bytes_ / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
                "traffic": None}

    out = {"metric": "prefill attn TFLOP/s + paged decode KV GB/s, % of MI355X peak"}
    if "prefill" in avg_ms:
        pt = prefill_flops / (avg_ms["prefill"] * 1e-3) / 1e12
        out.update({"value": pt, "unit": "TFLOP/s"})
    else:
        out.update({"value": None, "unit": "TFLOP/s"})
    out.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
                "wall_ms_per_step": wall_ms_per_step,
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
                "data": "synthetic (seeded; shapes and distributions of the five workloads)"})
    out["config"] = {
        "workload": "attention hot path: causal GQA prefill 2048x2048 h16/8 d256 f16 K/V (value) + paged decode "
                    "64 seqs ctx 512..16384 h32/8 d128 + DFlash2 block verify 4x16 rows window 4096 h32/8 d128",
        "prefill": {"rows": 2048, "kv_len": 2048, "n_heads": 16, "n_kv_heads": 8, "head_dim": 256,
                    "gflop": prefill_flops / 1e9},
        "decode": {"batch": 64, "page_size": 16, "pool_pages": 65536, "n_heads": 32, "n_kv_heads": 8,
                   "head_dim": 128, "context_tokens": int(ctx.sum()) if "decode" in want else None,
                   "gbytes": decode_bytes / 1e9 if "decode" in want else None},
        "verify": {"lanes": b, "rows": r, "window": w, "packed_len": klen, "q_heads": h, "kv_heads": hk,
                   "head_dim": d},
        "parallelism": "single GPU",
    }
    comps = {}
    if "prefill" in avg_ms:
        comps["prefill"] = {"ms": avg_ms["prefill"], "tflops": out["value"], "frac": out["value"] / PEAK_F16_TFLOPS}
        out["roofline_prefill"] = {"bound": "mfma", "achieved": out["value"], "peak": PEAK_F16_TFLOPS,
                                   "unit": "TFLOP/s", "frac": out["value"] / PEAK_F16_TFLOPS, "traffic": None}
    if "decode" in avg_ms:
        comps["decode"] = {"ms": avg_ms["decode"], "gbps": decode_bytes / (avg_ms["decode"] * 1e-3) / 1e9,
                           "tflops": decode_flops / (avg_ms["decode"] * 1e-3) / 1e12}
        comps["decode"]["frac"] = comps["decode"]["gbps"] / PEAK_HBM_GBPS
        out["decode_kv_gbps"] = comps["decode"]["gbps"]
        out["roofline_decode"] = roofline_hbm(decode_bytes, avg_ms["decode"])
        out["roofline_decode"]["traffic"] = measured_traffic()
    verify_rows = ((("pack", pack_bytes), ("mask", mask_bytes), ("verify_attn", verify_attn_bytes),
                    ("verify_fused", fused_bytes), ("commit", commit_bytes)) if "verify" in want else ())
    for name, nbytes in verify_rows:
        if name in avg_ms:
            comps[name] = {"ms": avg_ms[name], "gbps": nbytes / (avg_ms[name] * 1e-3) / 1e9,
                           "frac": nbytes / (avg_ms[name] * 1e-3) / 1e9 / PEAK_HBM_GBPS, "mbytes": nbytes / 1e6}
    for name in ("verify_attn", "verify_fused"):
        if name in comps:
            comps[name]["tflops"] = verify_attn_flops / (avg_ms[name] * 1e-3) / 1e12
    if "prepare" in avg_ms:
        ms = avg_ms["prepare"]
        comps["prepare"] = {"workload": "16 sequences x 16 new tokens, 32/8 heads, d 128: Q/K RMS norm, rotary "
                                        "embedding on all 128 features, K/V into 16-token f16 pages",
                            "ms": ms, "gbps": prep_bytes / (ms * 1e-3) / 1e9, "mbytes": prep_bytes / 1e6}
    if "paged_prefill" in avg_ms:
        ms = avg_ms["paged_prefill"]
        comps["paged_prefill"] = {"workload": "16 sequences x 16 new tokens, contexts 1024..8192, 16-token pages, "
                                              "32/8 heads, d 128, f16 K/V",
                                  "ms": ms, "gbps": multi_bytes / (ms * 1e-3) / 1e9,
                                  "frac": multi_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                                  "mbytes": multi_bytes / 1e6, "tflops": multi_flops / (ms * 1e-3) / 1e12}
    if chunk:
        comps["chunked_prefill_d512"] = chunk
    # `roofline` describes the row that takes the most time in a step
    timed = {k: v for k, v in avg_ms.items() if k in ("prefill", "decode", "verify_attn")}
    if timed:
        dom = max(timed, key=timed.get)
        if dom == "prefill":
            out["roofline"] = dict(out["roofline_prefill"], kernel="causal2k prefill (classify + MFMA attention)")
        elif dom == "decode":
            out["roofline"] = dict(out["roofline_decode"], kernel="paged decode (split-KV partial + reduce)")
        else:
            out["roofline"] = dict(roofline_hbm(verify_attn_bytes, avg_ms["verify_attn"]),
                                   kernel="block-verify attention")
    out["components"] = comps
    out["cpu_baseline"] = cpu
    print(json.dumps(out))


if __name__ == "__main__":
    main()
