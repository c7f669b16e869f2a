"""Throughput of the sparse path (indexer + Top-K + sparse MLA attention) on one
MI355X.

Default workload: speculative decode, 64 sequences x 131072 positions, two draft
tokens per sequence (128 query tokens), fp8 index-K (64 heads x 128) with
per-token scales, Top-2048, bf16 latent KV (576/512) with 128 attention heads,
page size 64, shuffled page tables. One step = one fused indexer + Top-K pass
and one sparse attention pass over every query token, with all inputs resident
in HBM. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="spec_decode_128k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true",
                   help="leave out the 16K causal prefill figures")
    p.add_argument("--graph", action="store_true",
                   help="replay every call from a HIP graph instead of launching it from the host "
                        "(measured the same as host launches on this path)")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="instead of the path, run a plain device copy of this many bytes "
                        "(calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


# Sources of the kernels the roofline line reports on: a traffic figure taken
# from hardware counters is only valid for the code it was measured on.
KERNEL_SOURCES = ["indexer.hip", "sia_device.h", "sia_select.h", "sia_kernels.h", "sia_sched.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_traffic_spec_decode_128k.md")


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank space removed, so that
    only a change of the code itself invalidates a counter figure."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "indexer_top_sparse_02_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(ln.strip() for ln in text.splitlines() if ln.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per indexer call from the committed counter summary, or None
    when there is none for this workload or the kernels changed since."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("workload") != workload or fields.get("kernel source hash") != kernel_source_hash():
        return None
    try:
        return float(fields["hbm bytes per call"])
    except (KeyError, ValueError):
        return None


def copy_calibration(nbytes: int):
    """A plain device-to-device copy of nbytes, five times: the bytes a perfect
    counter would report per dispatch are nbytes read and nbytes written."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "dispatches": 5}))


def algorithmic_bytes(wl, idx):
    """Bytes the method must move per step: every visible index-K row (+ scale)
    of each sequence once, each selected latent row once per sequence (rows
    shared by a sequence's draft tokens count once), queries, weights, outputs
    and the page-table entries used."""
    import torch
    s = wl.spec
    lens = wl.seq_lens.long()
    es = 1 if s.idx_fp8 else 2
    row_idx = s.dim_idx * es + (4 if s.idx_fp8 else 0)
    idx_bytes = int(lens.sum()) * row_idx
    # latent rows: union of the selected positions of each sequence's queries
    B = int(lens.numel())
    q_seq = wl.q_seq.long()
    key = (q_seq[:, None] * (1 << 32) + idx.long())[idx >= 0]
    uniq = int(torch.unique(key).numel())
    kv_bytes = uniq * 576 * 2
    Q = wl.num_q
    q_bytes = Q * (s.heads_idx * s.dim_idx * 2 + s.heads_idx * 4 + s.heads_attn * 576 * 2)
    out_bytes = Q * (s.heads_attn * 512 * 2 + s.topk * 4)
    pt_bytes = int(((lens + 63) // 64).sum()) * 4
    return dict(index_k=idx_bytes, latent=kv_bytes, queries=q_bytes, outputs=out_bytes,
                page_table=pt_bytes, total=idx_bytes + kv_bytes + q_bytes + out_bytes + pt_bytes,
                indexer=idx_bytes + Q * (s.heads_idx * s.dim_idx * 2 + s.heads_idx * 4) + pt_bytes
                + Q * s.topk * 4)


def cpu_baseline(wl_gpu, s, budget_s: float = 12.0):
    """The oracle on a bounded sample of the same workload: whole sequences,
    taken in order until about budget_s seconds of CPU work are done."""
    import oracle
    import workloads as W
    oracle.build(force=False)
    nq, dt, seqs = 0, 0.0, 0
    for seq in range(int(wl_gpu.seq_lens.numel())):
        sub = W.subset(wl_gpu, [seq], device="cpu")
        t0 = time.perf_counter()
        oracle.run(sub, attention=True)
        dt += time.perf_counter() - t0
        nq += sub.num_q
        seqs += 1
        if dt >= budget_s:
            break
    return {"value": nq / dt, "unit": "query tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{nq} query tokens of {seqs} sequences ({s.ctx_hi} positions each) of "
                      f"{s.name}: indexer, Top-K and attention, {dt:.1f} s"}


METRIC = "decode queries/s and HBM GB/s at 128K ctx; prefill tokens/s (indexer+TopK+sparse attn)"


GRAPH = False   # replay each call from a HIP graph (set from --graph)


def time_path(sia, wl, s, group, steps, warmup, sched=-1, attention_too=True):
    """Times `steps` passes of the whole path (indexer + Top-K, then sparse
    attention) with HIP events on the stream the library runs on. Returns the
    indices of the last pass, ms per step and ms per phase. `sched` picks the
    causal prefill tile schedule (-1: the library's default). With GRAPH, each
    call is captured once into a HIP graph after the eager warmup and the timed
    steps replay the graphs (the same kernels and arguments, without the host
    launch path); the events sit between the replays."""
    import torch
    dev = wl.q_idx.device
    maxv = int(torch.minimum(wl.q_pos.long() + 1, wl.seq_lens.long()[wl.q_seq.long()]).max())
    ws_i = sia.new_workspace(sia.indexer_workspace_size(wl.page_table, wl.seq_lens, wl.idx_k,
                                                        wl.idx_scale, wl.q_seq, wl.q_pos,
                                                        s.heads_idx, s.topk, group=group,
                                                        max_visible=maxv), dev)
    ws_a = sia.new_workspace(sia.mla_workspace_size(wl.num_q, s.heads_attn, s.topk), dev)
    idx = torch.empty((wl.num_q, s.topk), dtype=torch.int32, device=dev)
    out = torch.empty((wl.num_q, s.heads_attn, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((wl.num_q, s.heads_attn), dtype=torch.float32, device=dev)

    def indexer():
        sia.sparse_indexer_topk(wl.page_table, wl.seq_lens, wl.idx_k, wl.idx_scale, wl.q_seq,
                                wl.q_pos, wl.q_idx, wl.w, s.topk, group=group, max_visible=maxv,
                                out_idx=idx, workspace=ws_i, sched=sched)

    def attention():
        if attention_too:
            sia.sparse_mla_attention(wl.page_table, wl.seq_lens, wl.kv, wl.q_seq, wl.q_attn, idx,
                                     s.sm_scale, out=out, lse=lse, workspace=ws_a)

    for _ in range(max(1, warmup)):
        indexer()
        attention()
    torch.cuda.synchronize()
    if GRAPH:
        g_idx = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_idx):
            indexer()
        indexer = g_idx.replay
        if attention_too:
            g_att = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_att):
                attention()
            attention = g_att.replay
        torch.cuda.synchronize()
        for _ in range(max(1, warmup)):
            indexer()
            attention()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for e0, e1, e2 in ev:
        e0.record()
        indexer()
        e1.record()
        attention()
        e2.record()
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / steps
    idx_ms = sum(e0.elapsed_time(e1) for e0, e1, _ in ev) / steps
    att_ms = sum(e1.elapsed_time(e2) for _, e1, e2 in ev) / steps
    return idx, ms, idx_ms, att_ms


def prefill_flops(s, wl):
    """Algorithmic flops of one causal prefill pass: 2*H_I*d_I per visible
    (query, position) for the indexer, 2*H_A*(576 + 512) per selected
    (query, row) for attention."""
    t = wl.q_pos.long().cpu() + 1
    vis = float(t.sum())
    sel = float(torch_min(t, s.topk).sum())
    return 2.0 * s.heads_idx * s.dim_idx * vis, 2.0 * s.heads_attn * (576 + 512) * sel


def torch_min(t, k):
    import torch
    return torch.clamp(t, max=k)


def prefill_line(wl, s, steps, warmup):
    """Causal prefill: every position of the sequence is a query that sees
    positions 0..t. Reports tokens/s and MFMA throughput of each phase."""
    import indexer_top_sparse_02_amd as sia
    idx, ms, idx_ms, att_ms = time_path(sia, wl, s, wl.num_q, steps, warmup)
    f_idx, f_att = prefill_flops(s, wl)
    # the causal tile schedules of the fused indexer, timed alone (same results)
    sched_ms = {}
    for name, code in (("naive", 0), ("heavy_first", 1), ("zigzag", 2)):
        sched_ms[name] = time_path(sia, wl, s, wl.num_q, max(2, steps // 2), 1, sched=code,
                                   attention_too=False)[2]
    ti, ta = f_idx / (idx_ms * 1e-3) / 1e12, f_att / (att_ms * 1e-3) / 1e12
    dominant = ("sparse_mla_attention call (sparse_mla_kernel)", ta, f_att, att_ms) \
        if att_ms >= idx_ms else ("sparse_indexer_topk call (indexer_stream_kernel)", ti, f_idx, idx_ms)
    return {
        "metric": METRIC, "value": wl.num_q / (ms * 1e-3), "unit": "prefill tokens/s",
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) caches and queries, shuffled page table)",
        "config": {"workload": s.name, "tokens": wl.num_q, "indexer_heads": s.heads_idx,
                   "index_dim": s.dim_idx, "topk": s.topk, "attention_heads": s.heads_attn,
                   "page_size": 64, "launch": "hip graph per call" if GRAPH else "eager"},
        "phases_ms": {"indexer_topk": idx_ms, "attention": att_ms},
        "indexer_schedule_ms": sched_ms,
        "algorithmic_tflop": {"indexer": f_idx / 1e12, "attention": f_att / 1e12},
        "phase_tflops": {"indexer": ti, "attention": ta},
        "mfma_frac_step": (f_idx + f_att) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "kernel": dominant[0], "achieved": dominant[1],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": dominant[1] / PEAK_BF16_TFLOPS,
                     "traffic": None, "algorithmic_tflop_per_call": dominant[2] / 1e12,
                     "call_ms": dominant[3]},
    }


def chunked_line(wl, s, steps, warmup):
    """Chunked causal prefill: the sequence's queries in chunks of s.chunk, each
    chunk one indexer call and one attention call against the paged caches
    (a chunk's queries see positions 0..t, so later rows already in the cache
    stay invisible, as in a cache that grows chunk by chunk). Reports the time
    of every chunk: the causal work grows linearly with the chunk index."""
    import indexer_top_sparse_02_amd as sia
    n_chunks = wl.num_q // s.chunk
    chunks = []
    tot_ms = tot_i = tot_a = f_i_all = f_a_all = 0.0
    for c in range(n_chunks):
        sub = wl.queries(c * s.chunk, (c + 1) * s.chunk)
        _, ms, i_ms, a_ms = time_path(sia, sub, s, s.chunk, steps, warmup)
        f_i, f_a = prefill_flops(s, sub)
        chunks.append({"chunk": c, "ms": ms, "indexer_ms": i_ms, "attention_ms": a_ms,
                       "indexer_tflops": f_i / (i_ms * 1e-3) / 1e12,
                       "attention_tflops": f_a / (a_ms * 1e-3) / 1e12})
        print(f"chunk {c}: {ms:.3f} ms (indexer {i_ms:.3f}, attention {a_ms:.3f})", file=sys.stderr,
              flush=True)
        tot_ms += ms
        tot_i += i_ms
        tot_a += a_ms
        f_i_all += f_i
        f_a_all += f_a
    dominant = ("sparse_indexer_topk calls (indexer_stream_kernel)", f_i_all / (tot_i * 1e-3) / 1e12,
                f_i_all, tot_i) if tot_i >= tot_a else \
        ("sparse_mla_attention calls (sparse_mla_kernel)", f_a_all / (tot_a * 1e-3) / 1e12, f_a_all, tot_a)
    return {
        "metric": METRIC, "value": wl.num_q / (tot_ms * 1e-3), "unit": "prefill tokens/s",
        "ms_per_step": tot_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded fp8 index-K with per-token scales, N(0,1) "
                                 "latent KV and queries, shuffled page table)",
        "config": {"workload": s.name, "tokens": wl.num_q, "chunk": s.chunk, "indexer_heads": s.heads_idx,
                   "index_dim": s.dim_idx, "topk": s.topk, "attention_heads": s.heads_attn,
                   "page_size": 64, "launch": "hip graph per call" if GRAPH else "eager"},
        "phases_ms": {"indexer_topk": tot_i, "attention": tot_a},
        "algorithmic_tflop": {"indexer": f_i_all / 1e12, "attention": f_a_all / 1e12},
        "mfma_frac_step": (f_i_all + f_a_all) / (tot_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "chunks": chunks,
        "roofline": {"bound": "mfma", "kernel": dominant[0], "achieved": dominant[1],
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": dominant[1] / PEAK_BF16_TFLOPS,
                     "traffic": None, "algorithmic_tflop_per_call": dominant[2] / 1e12 / n_chunks,
                     "call_ms": dominant[3] / n_chunks},
    }


def main():
    a = _args()
    if a.copy_bytes:
        copy_calibration(a.copy_bytes)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this implementation runs on one GPU (no sharding or "
                                   "collectives); --gpus must be 1", "n_gpus": a.gpus}))
        sys.exit(2)
    import torch

    import indexer_top_sparse_02_amd as sia
    import workloads as W

    global GRAPH
    GRAPH = a.graph
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = W.spec(a.config)
    if s.prefill:
        if s.chunk:
            line = chunked_line(W.make(s, device=dev), s, max(1, a.steps // 4), max(1, a.warmup))
        else:
            line = prefill_line(W.make(s, device=dev), s, a.steps, a.warmup)
        line.update({"n_gpus": 1, "steps": a.steps, "warmup": a.warmup})
        print(json.dumps(line))
        return
    wl = W.make(s, device=dev)
    group = s.q_per_seq
    idx, ms, idx_ms, att_ms = time_path(sia, wl, s, group, a.steps, a.warmup)
    by = algorithmic_bytes(wl, idx)
    step_gbs = by["total"] / (ms * 1e-3) / 1e9
    idx_gbs = by["indexer"] / (idx_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": wl.num_q / (ms * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "dtype_detail": "fp8 e4m3fn index keys fed raw to fp8 MFMA against a two-term e4m3 split "
                        "of the bf16 query (equal to the bf16 product up to rounding order), fp32 "
                        "accumulate; bf16 latent KV with bf16 MFMA; fp32 softmax",
        "data": "synthetic (seeded N(0,1) caches and queries, shuffled page tables)",
        "config": {"workload": s.name, "batch": s.batch, "context": s.ctx_hi,
                   "query_tokens": wl.num_q, "indexer_heads": s.heads_idx, "index_dim": s.dim_idx,
                   "topk": s.topk, "attention_heads": s.heads_attn, "page_size": 64,
                   "launch": "hip graph per call" if GRAPH else "eager"},
        "hbm_gbs_step": step_gbs,
        "phases_ms": {"indexer_topk": idx_ms, "attention": att_ms},
        "algorithmic_bytes": by,
        "roofline": {"bound": "hbm",
                     "kernel": "sparse_indexer_topk call (indexer_pair_kernel score pass + "
                               "topk_rows_kernel selection pass)",
                     "achieved": idx_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": idx_gbs / PEAK_HBM_GBS, "traffic": measured_traffic(s.name),
                     "algorithmic_bytes_per_call": by["indexer"],
                     "call_ms": idx_ms},
    }
    del wl, idx
    torch.cuda.empty_cache()
    if not a.no_prefill:
        ps = W.spec("prefill_16k")
        line["prefill"] = prefill_line(W.make(ps, device=dev), ps, max(2, a.steps // 4),
                                       max(1, a.warmup))
        torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(W.make(s, device=dev), s)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
