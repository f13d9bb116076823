"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass over every form of the path, each on its own seeded
synthetic input resident in HBM:
  prefill   chunked prefill at head_dim 512: 4096 new rows over 4096 cached +
            4096 new keys, 10% random holes below the causal frontier, 16/2
            heads, f16 K/V, f32 Q/O (mask tile classification + MFMA
            attention) -- the headline `value`
  causal2k  causal GQA prefill, 2048 x 2048, 16/8 heads, d 256
  decode    paged decode, 64 sequences of 512..16384 tokens, 16-token pages in a
            permuted 65536-page pool, 32/8 heads, d 128, f16 K/V
            (split-KV partial pass + log-sum-exp reduce)
  verify    DFlash2 block verify, 4 lanes x 16 drafted rows, ring window 4096,
            32/8 heads, d 128: pack -> mask -> attention over the packed
            buffers, the pack-free verify attention read from the ring in
            place, then commit
  multi     prepare (Q/K RMS norm, rotary embedding, K/V into the pages) and
            multi-token paged attention: 16 sequences x 16 new tokens over
            contexts of 1024..8192 tokens in 16-token pages, 32/8 heads, d 128

W untimed steps, then K timed steps bracketed by torch.cuda.synchronize().
Ahead of every call a 1 GiB scratch buffer is rewritten and then another
1 GiB buffer is read (both untimed), so no call finds its inputs in the 256 MB
last-level cache or the L2; the read leaves clean lines behind, so the
write-back of the rewrite's dirty lines does not fall inside the timed call
(it cost paged decode about 4 % when the rewrite came alone).  Each call
is timed with HIP events on the stream its kernels run on; a GPU sleep ahead
of each timed step lets the host enqueue the whole step first, so an event
pair brackets the GPU time of its call only.  Every per-call figure is the
median over the K steps; ms_per_step is the sum of the rows' medians (GPU
time of the hot path, flushes excluded) and step_span_ms the median GPU time
from a step's first call to its last (flushes included).

Prints ONE JSON line.  `value` is the chunked d 512 prefill's algorithmic
TFLOP/s (4 * n_heads * head_dim per (query, key) pair at or below the row's
causal frontier); the other rows are reported beside it with roofline
fractions against MI355X peaks (dense fp16 MFMA 2.5 PFLOP/s, HBM 8 TB/s).
`cpu_baseline` times the fp64 oracle on a bounded sample of the chunked
prefill's query rows on the host cores.

    python bench.py --summarize-traffic ROW FETCH_DIR WRITE_DIR

turns two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, each over
`bench.py --rows-only ROW --copy-probe`) into profiles/<row>_traffic.json:
HBM bytes per call, each counter scaled by what it reads for the copy probe,
tied to a digest of the sources the row's kernels are built from.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

PEAK_F16_TFLOPS = 2500.0
PEAK_HBM_GBPS = 8000.0
COPY_PROBE_BYTES = 1 << 30
FLUSH_BYTES = 1 << 30
HERE = os.path.dirname(os.path.abspath(__file__))

# Per row: the kernels of one call (name fragments in the trace) and the sources they are compiled from.
TRAFFIC_ROWS = {
    "decode": {"file": "paged_decode_traffic.json",
               "kernels": {"partial": "decode_partial_kernel", "reduce": "decode_reduce_kernel"},
               "sources": ["attention_flash_attn_03_amd/csrc/decode.hip",
                           "attention_flash_attn_03_amd/csrc/device_common.h"]},
    "prefill": {"file": "prefill_chunked8k_traffic.json",
                "kernels": {"classify": "classify_kernel", "attention": "wide_kernel"},
                "sources": ["attention_flash_attn_03_amd/csrc/prefill.hip",
                            "attention_flash_attn_03_amd/csrc/prefill_common.h",
                            "attention_flash_attn_03_amd/csrc/device_common.h",
                            "attention_flash_attn_03_amd/csrc/internal.h"]},
    "causal2k": {"file": "prefill_causal2k_traffic.json",
                 "kernels": {"classify": "classify_kernel", "attention": "narrow_kernel"},
                 "sources": ["attention_flash_attn_03_amd/csrc/prefill.hip",
                             "attention_flash_attn_03_amd/csrc/narrow.hip",
                             "attention_flash_attn_03_amd/csrc/prefill_common.h",
                             "attention_flash_attn_03_amd/csrc/device_common.h",
                             "attention_flash_attn_03_amd/csrc/internal.h"]},
}


def _sources_sha256(sources):
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(HERE, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(row="decode"):
    """HBM bytes per call of `row` from the committed counter summary, or None when
    a source its kernels are built from has changed since the counters were taken."""
    path = os.path.join(HERE, "profiles", TRAFFIC_ROWS[row]["file"])
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    srcs = rec.get("sources")
    return rec["bytes_per_launch"] if srcs and _sources_sha256(srcs) == rec.get("sources_sha256") else None


def summarize_traffic(row, fetch_dir, write_dir, algorithmic_bytes=None):
    """profiles/<row>_traffic.json from the counter CSVs of two rocprofv3 --pmc runs."""
    spec = TRAFFIC_ROWS[row]

    def per_kernel(d):
        out = {}
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    def pick(d, frag, last=None):
        ks = [k for k in d if frag in k]
        assert len(ks) >= 1, (frag, list(d))
        vals = [v for k in ks for v in d[k]]
        return statistics.median(vals if last is None else vals[-last:])

    f, w = per_kernel(fetch_dir), per_kernel(write_dir)
    cf, cw = pick(f, "neg_kernel"), pick(w, "neg_kernel")
    fs, ws = COPY_PROBE_BYTES / (cf * 1024), COPY_PROBE_BYTES / (cw * 1024)
    fk = {name: pick(f, frag) for name, frag in spec["kernels"].items()}
    wk = {name: pick(w, frag) for name, frag in spec["kernels"].items()}
    total = sum(fk.values()) * 1024 * fs + sum(wk.values()) * 1024 * ws
    path = os.path.join(HERE, "profiles", spec["file"])
    rec = {}
    if os.path.exists(path):
        with open(path) as fh:
            rec = json.load(fh)
    rec.update({
        "copy_probe": {"kernel": "torch.neg of a 1 GiB f32 tensor (reads 1 GiB, writes 1 GiB)",
                       "fetch_kib": cf, "write_kib": cw, "fetch_scale": fs, "write_scale": ws},
        "fetch_kib": fk, "write_kib": wk, "bytes_per_launch": total,
        "sources": spec["sources"], "sources_sha256": _sources_sha256(spec["sources"]),
    })
    if algorithmic_bytes is not None:
        rec["algorithmic_bytes"] = algorithmic_bytes
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--rows-only", choices=["prefill", "causal2k", "decode", "verify", "multi"], default=None,
                    help="time one row alone (profiling runs)")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache flush between calls")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (the reference for scaling HBM byte counters)")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("ROW", "FETCH_DIR", "WRITE_DIR"), default=None,
                    help="write profiles/<row>_traffic.json from two rocprofv3 --pmc output directories")
    ap.add_argument("--algorithmic-bytes", type=float, default=None)
    return ap.parse_args()


def prefill_row(fa, workloads, to_dev, dev, name):
    """Device inputs of a prefill configuration and its call."""
    import torch
    c = workloads.prefill_case(name)
    q, k, v, m = to_dev(c.q), to_dev(c.k), to_dev(c.v), to_dev(c.mask)
    o = torch.empty(c.q.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(fa.prefill_workspace_bytes(fa.prefill_params(q, k, v, m, o, scale=c.scale)),
                     dtype=torch.uint8, device=dev)
    flops = 4.0 * c.meta["n_heads"] * c.meta["head_dim"] * c.visible_pairs
    # algorithmic bytes: Q and O (f32), K and V rows (kv type), the mask (2 bytes per entry)
    nbytes = 2.0 * c.q.nbytes + c.k.nbytes + c.v.nbytes + c.mask.nbytes

    def run():
        fa.attn_prefill(q, k, v, m, o, scale=c.scale, workspace=ws)

    return c, run, flops, nbytes


def main():
    args = _parse()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, algorithmic_bytes=args.algorithmic_bytes)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the path has no multi-GPU form here "
              "(one process drives one MI355X); --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    sys.path.insert(0, HERE)
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
    want = {"prefill", "causal2k", "decode", "verify", "multi"} if args.rows_only is None else {args.rows_only}
    rows = []     # (name, callable) in step order
    info = {}     # name -> dict of algorithmic work

    # ---------------- prefill: chunked 4096 x 8192 keys, d 512 (the headline) and causal 2k, d 256
    if "prefill" in want:
        pc, run, flops, nbytes = prefill_row(fa, workloads, to_dev, dev, "chunked8k")
        rows.append(("prefill", run))
        info["prefill"] = {"flops": flops, "bytes": nbytes}
    if "causal2k" in want:
        c2, run, flops, nbytes = prefill_row(fa, workloads, to_dev, dev, "causal2k")
        rows.append(("causal2k", run))
        info["causal2k"] = {"flops": flops, "bytes": nbytes}

    # ---------------- paged decode
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
        info["decode"] = {
            "bytes": (float(ctx.sum()) * dm["n_kv_heads"] * dm["head_dim"] * 2 * 2     # K and V rows, f16
                      + dc.q.nbytes + dc.q.nbytes                                      # Q in, O out (f32)
                      + 4.0 * float(np.sum(-(-ctx // dm["page_size"])))                # page-table entries
                      + 4.0 * dm["batch"]),                                            # context lengths
            "flops": 4.0 * dm["n_heads"] * dm["head_dim"] * float(ctx.sum()),
            "context_tokens": int(ctx.sum())}

        def run_decode():
            fa.attn_paged_decode(dq, dkp, dvp, dpt, dctx, do, scale=dc.scale, max_context=dc.max_context,
                                 workspace=dws)
        rows.append(("decode", run_decode))

    # ---------------- block verify
    b, h, hk, d, r, w = 4, 32, 8, 128, 16, 4096
    klen = w - 1 + r
    if "verify" in want:
        vc = workloads.dflash_case()
        b, h, hk, d, r, w = vc.geom
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
        vws = torch.empty(fa.prefill_workspace_bytes(vap), dtype=torch.uint8, device=dev)
        L = vc.cache_lengths.astype(np.int64)
        vis_cache = np.minimum(L, w - 1)
        # rows visible per query row: r drafted + min(L, w - 1 - i) cached
        vis_rows = np.array([[r + min(int(Lb), w - 1 - i) for i in range(r)] for Lb in L])
        verify_attn_flops = 4.0 * d * h * float(vis_rows.sum())
        cnt = np.minimum(vc.commit_counts.astype(np.int64), vc.max_commit)
        info["pack"] = {"bytes": (vc.cur_q.nbytes + vc.cur_k.nbytes + vc.cur_v.nbytes + 8.0 * b
                                  + float(vis_cache.sum()) * hk * d * 2 * 2
                                  + b * h * r * d * 2 + 2.0 * b * hk * klen * d * 2)}
        info["mask"] = {"bytes": 4.0 * b + b * h * r * klen * 2}
        info["verify_attn"] = {"bytes": (b * h * r * d * 2 + b * h * r * d * 4 + b * h * r * klen * 2
                                         + float(np.max(vis_rows, axis=1).sum()) * hk * d * 2 * 2),
                               "flops": verify_attn_flops}
        # pack-free verify: current Q/K/V (f32), lengths and positions, the visible ring rows, O (f32)
        info["verify_fused"] = {"bytes": (vc.cur_q.nbytes + vc.cur_k.nbytes + vc.cur_v.nbytes + 8.0 * b
                                          + float(vis_cache.sum()) * hk * d * 2 * 2 + b * h * r * d * 4),
                                "flops": verify_attn_flops}
        info["commit"] = {"bytes": float(cnt.sum()) * hk * d * (4 + 2) * 2 + 8.0 * b}
        vfo = torch.empty((b, h, r, d), dtype=torch.float32, device=dev)
        vfws = torch.empty(fa.verify_workspace_bytes(vp), dtype=torch.uint8, device=dev)
        rows += [
            ("pack", lambda: fa.dflash_pack(vp, ring_k, ring_v, cq, ck, cv, vL, vwp, packed_q, packed_k, packed_v)),
            ("mask", lambda: fa.dflash_mask(vp, vL, vmask)),
            ("verify_attn", lambda: fa.attn_prefill(vq_view, vk_view, vv_view, vmask, vo_view, scale=vc.scale,
                                                    workspace=vws)),
            ("verify_fused", lambda: fa.dflash_verify_attention(vp, ring_k, ring_v, cq, ck, cv, vL, vwp, vfo,
                                                                scale=vc.scale, workspace=vfws)),
            ("commit", lambda: fa.dflash_commit(vp, ck, cv, vcnt, vwp, ring_k, ring_v)),
        ]

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
        # prepare: raw Q/K/V projections of the new tokens, Q/K norm weights
        mqr = to_dev(workloads.normal_f32(16 * 16 * 32 * 128, [6, 20]).reshape(16, 16, 32, 128))
        mkr = to_dev(workloads.normal_f32(16 * 16 * 8 * 128, [6, 21]).reshape(16, 16, 8, 128))
        mvr = to_dev(workloads.normal_f32(16 * 16 * 8 * 128, [6, 22]).reshape(16, 16, 8, 128))
        mqn = torch.ones((1, 128), dtype=torch.float32, device=dev)
        mkn = torch.ones((1, 128), dtype=torch.float32, device=dev)
        # raw Q/K/V read (f32), prepared Q written (f32), K/V rows written (f16), lengths and starts
        info["prepare"] = {"bytes": (mqr.numel() + mkr.numel() + mvr.numel() + mqr.numel()) * 4.0
                           + mkr.numel() * 2 * 2.0 + 8.0 * 16}
        # K and V rows of every context token, Q and O (f32), the page-table entries, lengths and starts;
        # 4 * heads * d per (query token, visible key): token i of a sequence sees start + i + 1 keys
        info["paged_prefill"] = {
            "bytes": (float(mctx.sum()) * 8 * 128 * 2 * 2 + 2.0 * mc.q.nbytes
                      + 4.0 * float(np.sum(-(-mctx // 16))) + 8.0 * len(mctx)),
            "flops": 4.0 * 32 * 128 * float(sum(int(st) * int(n) + int(n) * (int(n) + 1) // 2
                                                for st, n in zip(mc.position_starts, mc.query_lens)))}
        rows += [
            ("prepare", lambda: fa.attn_paged_prepare(mqr, mkr, mvr, mqn, mkn, mpt, mql, mst, mq, mkp, mvp,
                                                      rope_dim=128, rope_theta=1e4, rope_interleaved=False,
                                                      epsilon=1e-6, max_context=mpc.max_context)),
            ("paged_prefill", lambda: fa.attn_paged_prefill(mq, mkp, mvp, mpt, mql, mst, mo, scale=mpc.scale,
                                                            max_context=mpc.max_context, workspace=mws)),
        ]

    stream = torch.cuda.current_stream()
    flush_buf = None if args.no_flush else torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_read = None if args.no_flush else torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    events = {name: [] for name, _ in rows}
    spans = []
    head_start = [0]  # GPU sleep (cycles) ahead of each timed step

    def step(record):
        if record and head_start[0]:
            # keeps the GPU busy while the host enqueues the step, so each call's
            # event pair brackets its own GPU time and not the host's launch work
            torch.cuda._sleep(head_start[0])
        first = last = None
        for i, (name, fn) in enumerate(rows):
            if flush_buf is not None:
                flush_buf.fill_(float(i))  # evicts the previous calls' data from L2 and the last-level cache
                flush_read.sum()           # and replaces the rewrite's dirty lines with clean ones
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                events[name].append((e0, e1))
                first = first or e0
                last = e1
            else:
                fn()
        if record:
            spans.append((first, last))

    if args.copy_probe:
        # elementwise copy of known size: reads and writes COPY_PROBE_BYTES once per launch
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

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
    med_ms = {name: float(np.median([a.elapsed_time(z) for a, z in ev])) for name, ev in events.items() if ev}
    ms_per_step = float(sum(med_ms.values()))
    step_span_ms = float(np.median([a.elapsed_time(z) for a, z in spans]))
    wall_ms_per_step = 1e3 * wall / max(1, args.steps)

    # ---------------- CPU baseline: the oracle on a bounded sample of the headline prefill's rows
    cpu = None
    if not args.no_cpu_baseline and args.rows_only is None:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        import oracle
        oracle.build()
        m = pc.meta
        rows_all = pc.q.shape[1]

        def run_rows(sel):
            t = time.perf_counter()
            oracle.attention(pc.q[:, sel], pc.k, pc.v, pc.mask[:, :, sel], scale=pc.scale)
            return time.perf_counter() - t

        def flops_of(sel):
            return 4.0 * m["n_heads"] * m["head_dim"] * float(np.minimum(m["cached"] + sel + 1, m["kv_len"]).sum())

        probe = np.linspace(0, rows_all - 1, 16).astype(np.int64)
        rate = flops_of(probe) / max(run_rows(probe), 1e-6)
        n = int(min(rows_all, max(16, rows_all * (args.cpu_seconds * rate / info["prefill"]["flops"]))))
        sel = np.linspace(0, rows_all - 1, n).astype(np.int64)
        t_cpu = run_rows(sel)
        cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
        cpu_tflops = flops_of(sel) / t_cpu / 1e12
        gpu_tflops = info["prefill"]["flops"] / (med_ms["prefill"] * 1e-3) / 1e12
        cpu = {"value": cpu_tflops, "unit": "TFLOP/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
               "gpu_over_oracle": gpu_tflops / cpu_tflops,
               "sample": "%d of %d query rows (evenly spaced), all 16 heads, of the chunked prefill (4096 x 8192 "
                         "keys, d 512); %.1f s of fp64 compute on %d threads" % (n, rows_all, t_cpu, cores)}

    def rate(name):
        ms = med_ms[name]
        out = {"ms": ms}
        if "flops" in info[name]:
            out["tflops"] = info[name]["flops"] / (ms * 1e-3) / 1e12
        if "bytes" in info[name]:
            out["gbps"] = info[name]["bytes"] / (ms * 1e-3) / 1e9
            out["mbytes"] = info[name]["bytes"] / 1e6
        return out

    def roofline(name, bound, kernel):
        r_ = rate(name)
        if bound == "mfma":
            ach, peak, unit = r_["tflops"], PEAK_F16_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = r_["gbps"], PEAK_HBM_GBPS, "GB/s"
        traffic = measured_traffic(name) if name in TRAFFIC_ROWS else None
        return {"bound": bound, "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
                "traffic": traffic, "kernel": kernel, "ms": r_["ms"]}

    out = {"metric": "prefill attn TFLOP/s + paged decode KV GB/s, % of MI355X peak"}
    out["value"] = rate("prefill")["tflops"] if "prefill" in med_ms else None
    out["unit"] = "TFLOP/s"
    out.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
                "step_span_ms": step_span_ms, "wall_ms_per_step": wall_ms_per_step,
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
                "data": "synthetic (seeded; shapes and distributions of the five workloads)",
                "timing": "per-call medians over the timed steps; before every call 1 GiB rewritten, then 1 GiB read"
                          + (" (disabled)" if args.no_flush else "")})
    out["config"] = {
        "workload": "chunked prefill 4096 new rows x 8192 keys (4096 cached), 10% holes below the causal frontier, "
                    "16/2 heads, d 512, f16 K/V, f32 Q/O (value); beside it causal GQA prefill 2048x2048 h16/8 "
                    "d256, paged decode 64 seqs ctx 512..16384 h32/8 d128, DFlash2 block verify 4x16 rows window "
                    "4096 h32/8 d128, multi-token paged attention 16x16 tokens",
        "prefill": {"rows": 4096, "kv_len": 8192, "cached": 4096, "n_heads": 16, "n_kv_heads": 2, "head_dim": 512,
                    "holes": 0.1, "gflop": info["prefill"]["flops"] / 1e9 if "prefill" in info else None},
        "causal2k": {"rows": 2048, "kv_len": 2048, "n_heads": 16, "n_kv_heads": 8, "head_dim": 256,
                     "gflop": info["causal2k"]["flops"] / 1e9 if "causal2k" in info else None},
        "decode": {"batch": 64, "page_size": 16, "pool_pages": 65536, "n_heads": 32, "n_kv_heads": 8,
                   "head_dim": 128, "context_tokens": info.get("decode", {}).get("context_tokens"),
                   "gbytes": info["decode"]["bytes"] / 1e9 if "decode" in info else None},
        "verify": {"lanes": b, "rows": r, "window": w, "packed_len": klen, "q_heads": h, "kv_heads": hk,
                   "head_dim": d},
        "parallelism": "single GPU",
    }
    comps = {name: rate(name) for name in med_ms}
    for name in ("prefill", "causal2k", "verify_attn", "verify_fused", "paged_prefill"):
        if name in comps and "tflops" in comps[name]:
            comps[name]["frac_mfma"] = comps[name]["tflops"] / PEAK_F16_TFLOPS
    for name in ("decode", "pack", "mask", "verify_attn", "verify_fused", "commit", "prepare", "paged_prefill"):
        if name in comps:
            comps[name]["frac_hbm"] = comps[name]["gbps"] / PEAK_HBM_GBPS
    out["components"] = comps
    if "prefill" in med_ms:
        out["roofline_prefill"] = roofline("prefill", "mfma", "chunked prefill d 512 (classify + MFMA attention)")
    if "causal2k" in med_ms:
        out["roofline_causal2k"] = roofline("causal2k", "mfma", "causal2k prefill d 256 (classify + MFMA attention)")
    if "decode" in med_ms:
        out["decode_kv_gbps"] = comps["decode"]["gbps"]
        out["roofline_decode"] = roofline("decode", "hbm", "paged decode (split-KV partial + reduce)")
    # `roofline` describes the call that takes the most time in a step
    dom = {"prefill": "roofline_prefill", "causal2k": "roofline_causal2k", "decode": "roofline_decode"}
    timed = {k: v for k, v in med_ms.items() if k in dom}
    if timed:
        out["roofline"] = out[dom[max(timed, key=timed.get)]]
    out["cpu_baseline"] = cpu
    print(json.dumps(out))


if __name__ == "__main__":
    main()
