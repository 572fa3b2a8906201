"""Benchmark of the Hybrid HiSparse sparse-MLA decode step on one MI355X.

A step is one pass of the whole hot path over one batch: the indexer sweep + top-K select
(hisparse_index_topk), the fused resolver with its host-to-device miss copies
(hisparse_resolve), and sparse MLA decode attention for every layer sharing the top-K
(sparse_mla_decode).  Inputs are synthetic and seeded; every per-step input (queries, context
lengths) is staged in HBM before the timed region; the KV pool, indexer keys, block tables
and the pinned host pool are filled up front.

Default workload: 64 requests at 131,072-token context, MTP3 verification (4 query tokens per
request resolved together), FP8 rows and keys, newest 10 % of pages resident, the rest in the
pinned host pool, hot buffer (3 + 2) x 2,048 rows per request.

Prints one JSON line.  `value` is layer-steps/s (one layer-step = one sparse-MLA layer's decode
for the whole batch, including its share of index + resolve).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode layer-steps/s + achieved HBM GB/s (indexer+gather) at 128K ctx"
HBM_PEAK_GBPS = 8000.0
BF16_DENSE_TFLOPS = 2500.0
PCIE_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction, nominal (the host link of the misses)
MAT_PAGES_PER_REQ = 16  # pages per request whose materialisation (device -> host) is timed


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload index (3 = the 128K metric config)")
    ap.add_argument("--scale", type=int, default=1, help="divide context lengths (development only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-requests", type=int, default=64)
    ap.add_argument("--prefill-tokens", type=int, default=32768,
                    help="prompt length of the prefill measurement (0: skip it)")
    return ap.parse_args()


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(see DESIGN.md, 'More than one GPU'); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from sparse_mla_attention_score_amd import accounting as acc
    from sparse_mla_attention_score_amd import hisparse as hsb
    from sparse_mla_attention_score_amd import rocprof_summary as rprof

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # warm-up, the timed steps, then as many steps again with per-kernel timing on (kept out of
    # the timed region: its event pairs between launches would lengthen the step)
    total_steps = args.warmup + 2 * args.steps
    wl = synth.config(args.config, scale=args.scale, steps=total_steps)
    lay = synth.make_layout(wl)
    B, S, K, NL = wl.batch, wl.queries, wl.topk, wl.n_layers
    # the write side of the host pool is measured after the steps: complete resident pages
    # (not the tail) of every request get a spare host block each, to be materialised into
    mat_pages = []
    for b in range(B):
        tail = (int(wl.ctx[b]) - 1) // synth.BLOCK
        res = [int(p) for p in np.nonzero(lay.block_table[b] >= 0)[0] if p < tail]
        mat_pages += [(b, p) for p in res[:MAT_PAGES_PER_REQ]]
    for k, (b, p) in enumerate(mat_pages):
        lay.host_block_table[b, p] = lay.num_host_blocks + k
    lay.num_host_blocks += len(mat_pages)
    log(f"workload {wl.name}: B={B} S={S} ctx={wl.ctx[0]} layers={NL} gpu_blocks={lay.num_gpu_blocks} "
        f"host_blocks={lay.num_host_blocks} idx_blocks={lay.num_idx_blocks}")

    t0 = time.time()
    cfg = hsb.make_config(topk=K, kv_dtype=wl.kv_dtype, idx_dtype=wl.idx_dtype, n_layers=NL,
                          max_batch=B, max_queries=S, max_pages_per_req=wl.max_pages,
                          hot_rows_per_req=wl.hot_rows, num_gpu_blocks=lay.num_gpu_blocks,
                          num_idx_blocks=lay.num_idx_blocks, num_host_blocks=lay.num_host_blocks)
    ctx = hsb.Context(cfg, dev)
    stage = np.zeros(lay.num_idx_blocks * wl.idx_block_bytes, np.uint8)
    synth.fill_idx_pool(wl, lay, stage)
    ctx.idx_pool.copy_(torch.from_numpy(stage))
    del stage
    stage = np.zeros(NL * lay.num_gpu_blocks * 64 * wl.row_bytes, np.uint8)
    synth.fill_kv(wl, lay, stage, ctx.host_pool)
    ctx.kv_pool.copy_(torch.from_numpy(stage))
    del stage
    for name in ("idx_block_table", "block_table", "host_block_table", "hot_blocks"):
        getattr(ctx, name).copy_(torch.from_numpy(np.ascontiguousarray(getattr(lay, name))))
    chains = [synth.qidx(wl, b, total_steps * S) for b in range(B)]
    w = torch.from_numpy(synth.head_weights(wl)).to(dev)
    qidx_d, q_d, lens_d = [], [], []
    for step in range(total_steps):
        qidx_d.append(torch.from_numpy(synth.qidx_step(wl, step, chains).view(np.int16)).to(dev))
        q_d.append(torch.from_numpy(synth.mla_q(wl, step).view(np.int16)).to(dev))
        lens_d.append(torch.from_numpy(wl.ctx_at(step).astype(np.int32)).to(dev))
    topk = torch.empty((B, S, K), dtype=torch.int32, device=dev)
    rows = torch.empty_like(topk)
    stats = torch.empty((B, 4), dtype=torch.int32, device=dev)
    out = torch.empty((B, S, 64, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, S, 64), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(576.0)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f} s")

    stream = torch.cuda.current_stream()

    def run_step(step, ev=None):
        if ev is not None:
            ev[0].record(stream)
        ctx.index_topk(qidx_d[step].view(torch.bfloat16), w, lens_d[step], topk)
        if ev is not None:
            ev[1].record(stream)
        ctx.resolve(topk, lens_d[step], rows, stats)
        if ev is not None:
            ev[2].record(stream)
        for layer in range(NL):
            ctx.decode(layer, q_d[step].view(torch.bfloat16), rows, lens_d[step], scale, out, lse)
        if ev is not None:
            ev[3].record(stream)

    # warm-up steps, each timed on its own (step 0 starts from a cold hot buffer)
    misses_warm, warm_ms = [], []
    for step in range(args.warmup):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_step(step)
        e1.record(stream)
        torch.cuda.synchronize()
        warm_ms.append(e0.elapsed_time(e1))
        misses_warm.append(int(stats[:, 2].sum()))
    err = ctx.device_error()
    if err:
        log(f"device error word after warmup: {err:#x}")
        return 1

    # the timed region: K whole steps, nothing recorded between launches
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_host = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        run_step(args.warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    elapsed_ms = start.elapsed_time(end)
    timed_miss = int(stats[:, 2].sum())
    err = ctx.device_error()
    if err:
        log(f"device error word after timed steps: {err:#x}")
        return 1
    # the next K steps with per-call events and per-kernel HIP events (recorded by the library
    # on the stream each kernel is launched on): stage and kernel durations, the roofline
    first_inst = args.warmup + args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    ctx.kernel_timing(True)
    miss_acc = torch.zeros((), dtype=torch.int64, device=dev)  # misses of the instrumented steps
    torch.cuda.synchronize()
    for i in range(args.steps):
        run_step(first_inst + i, events[i])
        miss_acc += stats[:, 2].sum()  # after the step's last event: not inside any timing
    torch.cuda.synchronize()
    ktimes = ctx.kernel_times()
    ctx.kernel_timing(False)
    kernels_us = {k: round(ms * 1e3 / n, 1) for k, (ms, n) in ktimes.items() if n}
    kernel_launches = {k: n for k, (ms, n) in ktimes.items() if n}
    sel_list, sel_scores = ctx.select_paths()  # over every step since the context was reset
    # write side of the host pool: materialise the chosen pages (every layer, one launch);
    # one untimed launch, then MAT_REPS timed ones
    mat = None
    if mat_pages:
        pages_d = torch.tensor(mat_pages, dtype=torch.int32, device=dev)
        ctx.materialize_pages(pages_d)
        torch.cuda.synchronize()
        MAT_REPS = 5
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(MAT_REPS):
            ctx.materialize_pages(pages_d)
        e1.record(stream)
        torch.cuda.synchronize()
        mat_us = e0.elapsed_time(e1) * 1e3 / MAT_REPS
        mat_bytes = len(mat_pages) * synth.BLOCK * wl.row_bytes * NL
        mat_gbps = mat_bytes / (mat_us * 1e-6) / 1e9
        mat = {"pages": len(mat_pages), "bytes": mat_bytes, "us": round(mat_us, 1),
               "gbps": round(mat_gbps, 2), "peak": PCIE_PEAK_GBPS, "frac": round(mat_gbps / PCIE_PEAK_GBPS, 4)}
    err = ctx.device_error()
    if err:
        log(f"device error word after instrumented steps: {err:#x}")
        return 1
    # per-call durations (ms), averaged over the instrumented steps
    t_idx = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    t_res = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    t_dec = sum(e[2].elapsed_time(e[3]) for e in events) / args.steps
    last_miss = int(stats[:, 2].sum())  # misses of the last instrumented step

    ms_per_step = elapsed_ms / args.steps
    layer_steps_per_s = args.steps * NL / (elapsed_ms / 1e3)
    # algorithmic work of the instrumented steps (the roofline's kernel times are theirs)
    idx_b = gat_b = att_f = sweep_b = sweep_f = 0
    for i in range(args.steps):
        lens_i = wl.ctx_at(first_inst + i)
        wk = acc.step_work(lens_i, S, K, NL, wl.kv_dtype, wl.idx_dtype)
        idx_b += wk["indexer_bytes"]
        gat_b += wk["gather_bytes"]
        att_f += wk["attention_flops"]
        sweep_b += sum(acc.sweep_bytes(int(L), S, wl.idx_dtype) for L in lens_i)
        sweep_f += wk["indexer_flops"]
    idx_b /= args.steps
    gat_b /= args.steps
    att_f /= args.steps
    sweep_b /= args.steps
    sweep_f /= args.steps
    # roofline of the dominant kernel: the indexer score sweep (one launch per step)
    t_sweep_ms = ktimes["index_score"][0] / ktimes["index_score"][1]
    sweep_gbps = sweep_b / (t_sweep_ms * 1e-3) / 1e9
    traffic = rprof.read_traffic(os.path.join(ROOT, "profiles", f"index_score_kernel_{wl.name}_traffic.txt"))
    idx_gbps = idx_b / (t_idx * 1e-3) / 1e9
    gat_gbps = gat_b / (t_dec * 1e-3) / 1e9
    both_gbps = (idx_b + gat_b) / ((t_idx + t_dec) * 1e-3) / 1e9
    # the decode kernels' own time (plus the split-K merge where it runs), not the stage time
    # between events, which also holds launch gaps
    t_dec_kernels_ms = (ktimes["decode"][0] + ktimes["decode_merge"][0]) / args.steps
    mfma_util = att_f / (t_dec_kernels_ms * 1e-3) / (BF16_DENSE_TFLOPS * 1e12)
    stream_read = measure_stream_read(torch, dev)
    # host link: the copy kernel's rate over the instrumented steps' misses, and the rate over
    # the whole resolve stage (resolver + copy)
    inst_misses = int(miss_acc.item()) / args.steps
    copy_bytes = inst_misses * NL * wl.row_bytes
    copy_gbps = copy_bytes / (ktimes["miss_copy"][0] / ktimes["miss_copy"][1] * 1e-3) / 1e9 if ktimes["miss_copy"][1] else 0.0
    host_gbps = copy_bytes / (t_res * 1e-3) / 1e9

    pre = bench_prefill(torch, dev, args.prefill_tokens) if args.prefill_tokens > 0 else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, chains, args.cpu_sample_requests)
    all_ms = sum(warm_ms) + elapsed_ms
    n_all = args.warmup + args.steps

    splits = hsb.hs_decode_splits(ctx.ctx, B, S)
    line = {
        "metric": METRIC,
        "value": round(layer_steps_per_s, 3),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16",
        "dtype_detail": {
            "indexer": "bf16 MFMA over FP8 E4M3 keys converted to bf16 exactly; fp32 accumulate and weighted ReLU sum",
            "attention_qk_nope": "FP8 E4M3 MFMA; the bf16 query as two exact E4M3 parts under a per-head power-of-two scale; fp32 accumulate",
            "attention_qk_rope_and_pv": "bf16 MFMA, fp32 accumulate",
            "softmax": "fp32", "outputs": "bf16 (lse fp32)"},
        "data": "synthetic (seeded; FP8 E4M3 rows and keys, bf16 queries)",
        "rates": {"steady_layer_steps_per_s": round(layer_steps_per_s, 3),
                  "all_steps_layer_steps_per_s": round(n_all * NL / (all_ms / 1e3), 3),
                  "all_steps_note": f"{args.warmup} warm-up steps (the first from a cold hot buffer) "
                                    f"and the {args.steps} timed steps",
                  "cold_step0_ms": round(warm_ms[0], 4) if warm_ms else None,
                  "warmup_steps_ms": [round(x, 4) for x in warm_ms],
                  "request_layer_steps_per_s": round(layer_steps_per_s * B, 1),
                  "query_tokens_per_s": round(layer_steps_per_s / NL * B * S, 1)},
        "config": {"workload": wl.name, "batch": B, "queries_per_request": S,
                   "ctx": int(wl.ctx[0]), "topk": K, "layers": NL, "hot_rows": wl.hot_rows,
                   "resident_fraction": wl.residency[0][1], "scale": args.scale,
                   "decode_splits": splits},
        "hbm_gbps_indexer_gather": round(both_gbps, 1),
        "stages_ms": {"index_topk": round(t_idx, 4), "resolve": round(t_res, 4),
                      "sparse_mla_decode": round(t_dec, 4)},
        "indexer": {"algorithmic_bytes": int(idx_b), "gbps": round(idx_gbps, 1),
                    "frac_hbm_peak": round(idx_gbps / HBM_PEAK_GBPS, 4),
                    "selections_from_candidate_list": sel_list, "selections_from_scores": sel_scores},
        "gather": {"algorithmic_bytes": int(gat_b), "gbps": round(gat_gbps, 1),
                   "frac_hbm_peak": round(gat_gbps / HBM_PEAK_GBPS, 4)},
        "attention": {"algorithmic_flops": int(att_f),
                      "kernel_us_per_step": round(t_dec_kernels_ms * 1e3, 1),
                      "tflops": round(att_f / (t_dec_kernels_ms * 1e-3) / 1e12, 2),
                      "mfma_util_bf16_dense": round(mfma_util, 4),
                      "stage_tflops": round(att_f / (t_dec * 1e-3) / 1e12, 2)},
        "materialize": mat,
        "host_link": {"misses_last_step": last_miss, "misses_last_timed_step": timed_miss,
                      "misses_warmup_steps": misses_warm,
                      "misses_per_instrumented_step": round(inst_misses, 1),
                      "copy_kernel_gbps": round(copy_gbps, 2), "resolve_stage_gbps": round(host_gbps, 2),
                      "peak": PCIE_PEAK_GBPS, "frac": round(copy_gbps / PCIE_PEAK_GBPS, 4)},
        "kernels_us": kernels_us,
        "kernel_launches": kernel_launches,
        "roofline": {"kernel": "index_score_kernel (indexer sweep, steady state: every key scored, candidates listed)",
                     "bound": "hbm", "achieved": round(sweep_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(sweep_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(sweep_b),
                     "avg_launch_us": round(t_sweep_ms * 1e3, 1),
                     "measured_stream_read_gbps": round(stream_read, 1),
                     "frac_of_measured_stream_read": round(sweep_gbps / stream_read, 4),
                     "mfma_frac_bf16_dense": round(sweep_f / (t_sweep_ms * 1e-3) / (BF16_DENSE_TFLOPS * 1e12), 4)},
        "prefill": pre,
        "cpu_baseline": cpu,
        "host_wall_s": round(t_host, 4),
    }
    print(json.dumps(line), flush=True)
    ctx.close()
    return 0


def bench_prefill(torch, dev, P: int) -> dict:
    """One request's prompt of P tokens (all pages resident, FP8 rows and keys, K = 2,048): the
    prefill indexer (every new token scores every earlier token, then its top-K) and sparse MLA
    attention of one layer on the decode kernel over those selections.  Compute-bound: the
    roofline is bf16 dense MFMA.  Queries are seeded N(0,1) drawn on the device (timing only;
    the prefill parity tests use the host generator)."""
    import numpy as np

    import synth
    from sparse_mla_attention_score_amd import accounting as acc
    from sparse_mla_attention_score_amd import hisparse as hsb

    K = 2048
    wl = synth.toy(seed=synth.SEED_BASE + 6, batch=1, queries=4, ctx=(P,), topk=K, steps=1,
                   residency=[(synth.RES_FULL, 1.0)])
    lay = synth.make_layout(wl)
    max_batch = 256                              # chunks of 256 x 4 prompt tokens
    pad = ((0, max_batch - 1), (0, 0))
    cfg = hsb.make_config(topk=K, n_layers=1, max_batch=max_batch, max_queries=4,
                          max_pages_per_req=wl.max_pages, num_gpu_blocks=lay.num_gpu_blocks,
                          num_idx_blocks=lay.num_idx_blocks, num_host_blocks=0)
    ctx = hsb.Context(cfg, dev)
    stage = np.zeros(lay.num_idx_blocks * wl.idx_block_bytes, np.uint8)
    synth.fill_idx_pool(wl, lay, stage)
    ctx.idx_pool.copy_(torch.from_numpy(stage))
    stage = np.zeros(lay.num_gpu_blocks * 64 * wl.row_bytes, np.uint8)
    synth.fill_kv(wl, lay, stage, None)
    ctx.kv_pool.copy_(torch.from_numpy(stage))
    del stage
    ctx.idx_block_table.copy_(torch.from_numpy(np.pad(lay.idx_block_table, pad, constant_values=-1)))
    ctx.block_table.copy_(torch.from_numpy(np.pad(lay.block_table, pad, constant_values=-1)))
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    qidx = torch.randn((P, 32, 128), generator=g, device=dev).to(torch.bfloat16)
    w = torch.rand((P, 32), generator=g, device=dev)
    q = torch.randn((P, 64, 576), generator=g, device=dev).to(torch.bfloat16)
    topk = torch.empty((P, K), dtype=torch.int32, device=dev)
    out = torch.empty((P, 64, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((P, 64), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(576.0)
    t_idx, t_att = [], []
    for rep in range(4):                         # the first pass warms up
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        ctx.prefill_index_topk(0, qidx, w, P, topk)
        e[1].record()
        ctx.prefill(0, 0, q, topk, P, scale, out, lse)
        e[2].record()
        torch.cuda.synchronize()
        if rep:
            t_idx.append(e[0].elapsed_time(e[1]))
            t_att.append(e[1].elapsed_time(e[2]))
    # one more pass with the library's per-kernel timing: where the prefill's time goes
    ctx.kernel_timing(True)
    torch.cuda.synchronize()
    ctx.prefill_index_topk(0, qidx, w, P, topk)
    ctx.prefill(0, 0, q, topk, P, scale, out, lse)
    torch.cuda.synchronize()
    kt = {k: (round(ms * 1e3, 1), n) for k, (ms, n) in ctx.kernel_times().items() if n}
    ctx.kernel_timing(False)
    err = ctx.device_error()
    ctx.close()
    if err:
        log(f"device error word after the prefill: {err:#x}")
        return {"error": err}
    ms_idx, ms_att = min(t_idx), min(t_att)
    visible = np.arange(1, P + 1, dtype=np.int64)
    idx_flops = float(acc.IDX_FLOPS_PER_KEY) * float(visible.sum())
    att_flops = float(np.minimum(visible, K).sum()) * 64 * acc.FLOPS_PER_HEAD_ROW
    return {"workload": f"prefill_{P}_fp8", "tokens": P, "topk": K, "layers": 1,
            "indexer_ms": round(ms_idx, 3), "attention_ms": round(ms_att, 3),
            "tokens_per_s": round(P / ((ms_idx + ms_att) * 1e-3), 1),
            "indexer": {"algorithmic_flops": idx_flops, "tflops": round(idx_flops / (ms_idx * 1e-3) / 1e12, 2),
                        "bound": "mfma", "peak_tflops": BF16_DENSE_TFLOPS,
                        "frac": round(idx_flops / (ms_idx * 1e-3) / (BF16_DENSE_TFLOPS * 1e12), 4)},
            "attention": {"algorithmic_flops": att_flops, "tflops": round(att_flops / (ms_att * 1e-3) / 1e12, 2),
                          "bound": "mfma", "peak_tflops": BF16_DENSE_TFLOPS,
                          "frac": round(att_flops / (ms_att * 1e-3) / (BF16_DENSE_TFLOPS * 1e12), 4)},
            "kernels_us_total_launches": kt,
            "note": "indexer + top-K of every prompt token, then one layer of sparse MLA on the "
                    "decode kernel; run as groups of 4 tokens, 1,024 tokens per chunk"}


def measure_stream_read(torch, dev) -> float:
    """The box's streaming-read rate (GB/s): a plain read of a 4 GiB buffer by the library's
    measurement kernel, best of 5."""
    from sparse_mla_attention_score_amd import hisparse as hsb
    x = torch.ones(1 << 30, dtype=torch.float32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    g = hsb.hs_measure_read_gbps(x.data_ptr(), x.numel() * 4, sink.data_ptr(), 5)
    del x
    return g


def cpu_info() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "model": model}


def oracle_one_thread_8k():
    """The oracle on the 8K single-request workload (bf16 rows and keys), all stages, with the
    BLAS pool held to one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    wl = synth.config(1)
    chains = [synth.qidx(wl, 0, 1)]
    w = synth.head_weights(wl)
    q = synth.mla_q(wl, 0)
    lay = synth.make_layout(wl)
    L = int(wl.ctx_at(0)[0])
    codes, sc = synth.idx_tokens(wl, 0, 0, L)
    rows_all = synth.latent_tokens(wl, 0, 0, np.arange(L))
    reps, t = 3, 0.0
    with threadpool_limits(limits=1):
        for _ in range(reps):
            t0 = time.perf_counter()
            keys = oracle.dequant_idx_keys(codes, sc)
            scores = oracle.indexer_scores(np.stack(chains[0][:1]), w[0], keys)
            tk = oracle.topk_select(scores[0], wl.topk)
            st = oracle.HotState.cold(wl.hot_rows, wl.max_pages * 64)
            oracle.resolve(tk[None], lay.block_table[0], lay.host_block_table[0], lay.hot_blocks[0], st)
            toks = tk[tk >= 0]
            lat = oracle.decode_latent_rows(rows_all[toks], wl.kv_dtype)
            oracle.attention(q[0, 0], lat, 1.0 / math.sqrt(576.0))
            t += time.perf_counter() - t0
    return {"workload": wl.name, "value": round(reps / t, 3), "unit": "layer-steps/s", "threads": 1}


def cpu_baseline(wl, chains, n_req: int):
    """The oracle, as it stands, on a bounded sample of the same workload: the first
    `n_req` requests of the first decode step (cold hot buffer), all stages.  Scaled to
    layer-steps/s of the full batch."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import synth

    S, K = wl.queries, wl.topk
    w = synth.head_weights(wl)
    q = synth.mla_q(wl, 0, batches=range(n_req))
    lay = synth.make_layout(wl)
    lens = wl.ctx_at(0)
    scale = 1.0 / math.sqrt(576.0)
    t_total = 0.0
    for b in range(n_req):
        L = int(lens[b])
        codes, sc = synth.idx_tokens(wl, b, 0, L)
        qidx = np.stack(chains[b][:S])
        t = time.perf_counter()
        keys = oracle.dequant_idx_keys(codes, sc)
        scores = oracle.indexer_scores(qidx, w[b], keys)
        tk = np.stack([oracle.topk_select(s, K) for s in scores])
        st = oracle.HotState.cold(wl.hot_rows, wl.max_pages * 64)
        oracle.resolve(tk, lay.block_table[b], lay.host_block_table[b], lay.hot_blocks[b], st)
        t_total += time.perf_counter() - t
        for layer in range(wl.n_layers):
            for j in range(S):
                toks = tk[j][tk[j] >= 0]
                rows = synth.latent_tokens(wl, b, layer, toks)      # input fetch, not timed
                t = time.perf_counter()
                lat = oracle.decode_latent_rows(rows, wl.kv_dtype)
                oracle.attention(q[b, j], lat, scale)
                t_total += time.perf_counter() - t
    per_step_s = t_total / n_req * wl.batch
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": round(wl.n_layers / per_step_s, 6), "unit": "layer-steps/s", "cores": threads,
            "kind": "oracle", "host": cpu_info(), "one_thread_8k": oracle_one_thread_8k(),
            "sample": f"{n_req} of {wl.batch} requests, decode step 0 (cold hot buffer), all stages; "
                      f"{t_total:.1f} s of oracle time scaled by {wl.batch}/{n_req}"}


if __name__ == "__main__":
    sys.exit(main())
