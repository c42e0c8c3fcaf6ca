"""Benchmark of the attention forward hot path on one MI355X.

One step is one pass over the whole path on seeded synthetic inputs already
resident in HBM:

  1. causal GQA prefill of a Llama-8B-like layer (B=1, 32 query heads, 8 K/V
     heads, D=128, bf16) over 16384 tokens processed as 32 microbatches of 512
     queries, microbatch u attending to keys [0, 512(u+1)) -- 32 calls of
     fa_prefill_ex (key splits and their combine as the planner chooses);
  2. paged MLA decode, batch 128 x 64 heads, 2048 cached tokens each,
     D_qk = 576 (512 latent + 64 rope), D_v = 512, page_size 1 with a random
     page permutation, scale 1/sqrt(192) -- one fa_decode_paged call (+ combine).

Between the two parts a 512 MiB buffer is read, so the decode finds the
last-level cache (256 MB) full of clean, unrelated lines.

Printed JSON: ``value`` is the prefill throughput in TFLOP/s (algorithmic
FLOP: 4*D per visible (query, key) pair and head) over the prefill part's
device time; ``decode`` holds the decode throughput in GB/s (algorithmic bytes:
the K/V rows of every cached token once, Q, O, page table and lengths). Each has
a ``roofline`` entry against MI355X's published peaks (2.5 PFLOP/s dense bf16,
8 TB/s HBM). ``cpu_baseline`` is the CPU oracle timed on a bounded sample of the
prefill rows on this host. Device times come from HIP events recorded on the
stream the library launches on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (%MFMA peak); paged decode GB/s (%HBM peak)"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
UB = 512


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(Sq_total, ub, Hq, D):
    total = 0
    for u in range(Sq_total // ub):
        off = ub * u
        total += ub * off + ub * (ub + 1) // 2
    return total * Hq * 4 * D


def decode_bytes(inp):
    kv = int(inp.seq_lens.astype("int64").sum()) * inp.D_qk * 2
    q = inp.B * inp.Hq * inp.D_qk * 2
    o = inp.B * inp.Hq * inp.D_v * 2
    pt = int(sum((int(n) + inp.page_size - 1) // inp.page_size for n in inp.seq_lens)) * 4
    return kv + q + o + pt + inp.B * 4


def split_decode_bytes(inp):
    """Algorithmic bytes of paged GQA decode: K and V rows of every cached token once
    per K/V head, q and o of the Sq new tokens, the page-table entries used and the lengths."""
    kv = int(inp.seq_lens.astype("int64").sum()) * inp.Hkv * 2 * inp.D_qk * 2
    q = inp.B * inp.Sq * inp.Hq * inp.D_qk * 2
    o = inp.B * inp.Sq * inp.Hq * inp.D_v * 2
    pt = int(sum((int(n) + inp.page_size - 1) // inp.page_size for n in inp.seq_lens)) * 4
    return kv + q + o + pt + inp.B * 4


def source_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "flashattention_forward_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, sha):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic.json),
    used only while the kernel source still hashes to what was measured."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not t or t.get("source_sha") != sha:
        return None
    return t.get("bytes_per_launch"), t.get("launch")


def cpu_baseline(inp3, budget_s):
    """Oracle rows of the prefill workload, sized to about ``budget_s`` seconds."""
    import numpy as np

    import oracle
    threads = oracle.default_threads()
    k = oracle.widen(inp3.k, "bf16")
    v = oracle.widen(inp3.v, "bf16")
    r = np.random.default_rng(7)

    def sample(n):
        rows = np.stack([np.zeros(n, np.int64), r.integers(0, inp3.Hq, n),
                         r.integers(0, inp3.Sq, n)], axis=1)
        q = oracle.widen(inp3.q[0, rows[:, 2], rows[:, 1]], "bf16")
        t = time.perf_counter()
        oracle.attention_rows(q, rows[:, 0], rows[:, 1], rows[:, 2], k, v, inp3.Hq, inp3.Sq,
                              True, inp3.scale, threads)
        dt = time.perf_counter() - t
        flops = float(((rows[:, 2] + 1) * 4 * inp3.D).sum())  # Sq == Skv: row i sees i+1 keys
        return flops, dt

    f0, t0 = sample(256)
    n = int(min(inp3.Sq * inp3.Hq, max(256, 256 * budget_s / max(t0, 1e-3))))
    f1, t1 = sample(n)
    return {"value": f1 / t1 / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} random query rows of the causal GQA prefill (B=1, 32 heads, "
                      f"16384 tokens, D=128), fp64, {t1:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of CPU oracle work for the baseline (0 = skip)")
    ap.add_argument("--mla-page-sizes", action="store_true",
                    help="also time the MLA decode workload with page sizes 16 and 64 "
                         "(fresh pools and page tables of the same seeded recipe)")
    ap.add_argument("--no-mask", action="store_true",
                    help="skip the masked-prefill measurement (fa_prefill_mask)")
    ap.add_argument("--traffic", action="store_true",
                    help="run only the launches that the HBM-traffic counter runs measure: a "
                         "256 MiB device copy (calibration), the last prefill microbatch "
                         "(keys [0, 16384)), the MLA decode and the small-batch GQA decode, "
                         "3 times each")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU sharding "
              "of this path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fa_inputs as fi
    import flashattention_forward_amd as fa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    eprint(f"device: {props.name}, {props.multi_processor_count} CUs, "
           f"{props.total_memory / 2**30:.0f} GiB")

    def to_dev(bits, dtype="bf16"):
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(dev)

    # ---- inputs, resident in HBM before timing ----
    inp3 = fi.workload(3)
    q3, k3, v3 = to_dev(inp3.q), to_dev(inp3.k), to_dev(inp3.v)
    o3 = torch.empty_like(q3)
    Hq, Hkv, D, S = inp3.Hq, inp3.Hkv, inp3.D, inp3.Sq
    n_ub = S // UB
    ws3_bytes = max(fa.fa_prefill_workspace_size(1, Hq, Hkv, UB, UB * (u + 1), D, 1, fa.FA_BF16)
                    for u in range(n_ub))
    ws3 = torch.empty(max(ws3_bytes, 16) // 4 + 4, dtype=torch.float32, device=dev)
    ub_args = [(q3[:, UB * u:UB * (u + 1)], k3[:, :UB * (u + 1)], v3[:, :UB * (u + 1)],
                o3[:, UB * u:UB * (u + 1)], UB * (u + 1)) for u in range(n_ub)]

    inp4 = fi.workload(4)
    q4, pool4 = to_dev(inp4.q), to_dev(inp4.pool)
    pt4 = torch.from_numpy(inp4.page_table).to(dev)
    sl4 = torch.from_numpy(inp4.seq_lens).to(dev)
    o4 = torch.empty((inp4.B, inp4.Hq, inp4.D_v), dtype=torch.bfloat16, device=dev)
    ws4_bytes = fa.fa_decode_workspace_size(inp4.B, inp4.Hq, 1, 576, 512, 1, inp4.max_seq_len,
                                            fa.FA_KV_MLA_SHARED)
    ws4 = torch.empty(max(ws4_bytes, 16) // 4 + 4, dtype=torch.float32, device=dev)
    n_split4 = fa.fa_decode_num_splits(inp4.B, inp4.Hq, 1, 576, 512, 1, inp4.max_seq_len,
                                       fa.FA_KV_MLA_SHARED)
    flush = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sid = stream.cuda_stream

    def prefill_pass():
        for q, k, v, o, skv in ub_args:
            fa.fa_prefill_ex(q, k, v, o, None, 1, Hq, Hkv, UB, skv, D, 1, inp3.scale,
                             fa.FA_BF16, fa.FA_BF16, ws3, ws3_bytes, stream=sid)

    # The same 32 microbatches with an explicit additive mask (a distance bias,
    # slope 1/8, with -inf above the causal diagonal; the causal rule is on too).
    masks3 = None
    if not args.no_mask and not args.traffic:
        masks3 = [to_dev(fi.bias_mask(UB, UB * (u + 1), 3)) for u in range(n_ub)]

    def prefill_mask_pass():
        for (q, k, v, o, skv), m in zip(ub_args, masks3):
            fa.fa_prefill_mask(q, k, v, m, skv, 0, o, None, 1, Hq, Hkv, UB, skv, D, 1,
                               inp3.scale, fa.FA_BF16, fa.FA_BF16, ws3, ws3_bytes, stream=sid)

    # Workload 5's small batch (4 sequences of 1024..32768 tokens, 32 query / 8 K/V
    # heads, page 16) decoding 4 new tokens per sequence at once.
    inp5 = fi.split_decode_inputs(5, 4, 32, 8, 128, fi.random_lens(5, 4, 1024, 32768), 16, Sq=4)
    q5, pool5 = to_dev(inp5.q), to_dev(inp5.pool)
    pt5 = torch.from_numpy(inp5.page_table).to(dev)
    sl5 = torch.from_numpy(inp5.seq_lens).to(dev)
    o5 = torch.empty((inp5.B, inp5.Sq, inp5.Hq, 128), dtype=torch.bfloat16, device=dev)
    ws5_bytes = fa.fa_decode_multi_workspace_size(inp5.B, inp5.Sq, inp5.Hq, inp5.Hkv, 128, 128,
                                                  16, inp5.max_seq_len, fa.FA_KV_SPLIT)
    ws5 = torch.empty(max(ws5_bytes, 16) // 4 + 4, dtype=torch.float32, device=dev)

    # Workload 2: non-causal MHA prefill, B=4, 16 heads, 2048 tokens, D=64, bf16
    # (one fa_prefill_ex call, planner-chosen workgroups and splits).
    inp2 = fi.workload(2)
    q2, k2, v2 = to_dev(inp2.q), to_dev(inp2.k), to_dev(inp2.v)
    o2 = torch.empty_like(q2)
    ws2_bytes = fa.fa_prefill_workspace_size(inp2.B, inp2.Hq, inp2.Hkv, inp2.Sq, inp2.Skv,
                                             inp2.D, 0, fa.FA_BF16)
    ws2 = torch.empty(max(ws2_bytes, 16) // 4 + 4, dtype=torch.float32, device=dev)

    def mha_pass():
        fa.fa_prefill_ex(q2, k2, v2, o2, None, inp2.B, inp2.Hq, inp2.Hkv, inp2.Sq, inp2.Skv,
                         inp2.D, 0, inp2.scale, fa.FA_BF16, fa.FA_BF16, ws2, ws2_bytes,
                         stream=sid)

    # Workload 5: small-batch GQA decode, one new token per sequence (4 sequences of
    # U[1024, 32768] tokens, 32 query / 8 K/V heads, D=128, page 16).
    inp5s = fi.workload(5)
    q5s, pool5s = to_dev(inp5s.q), to_dev(inp5s.pool)
    pt5s = torch.from_numpy(inp5s.page_table).to(dev)
    sl5s = torch.from_numpy(inp5s.seq_lens).to(dev)
    o5s = torch.empty((inp5s.B, inp5s.Hq, 128), dtype=torch.bfloat16, device=dev)
    ws5s_bytes = fa.fa_decode_workspace_size(inp5s.B, inp5s.Hq, inp5s.Hkv, 128, 128, 16,
                                             inp5s.max_seq_len, fa.FA_KV_SPLIT)
    ws5s = torch.empty(max(ws5s_bytes, 16) // 4 + 4, dtype=torch.float32, device=dev)
    n_split5s = fa.fa_decode_num_splits(inp5s.B, inp5s.Hq, inp5s.Hkv, 128, 128, 16,
                                        inp5s.max_seq_len, fa.FA_KV_SPLIT)

    def decode_gqa_pass():
        fa.fa_decode_paged(q5s, pool5s, pt5s, sl5s, pool5s.shape[0], o5s, None, inp5s.B,
                           inp5s.Hq, inp5s.Hkv, 128, 128, 16, inp5s.max_pages,
                           inp5s.max_seq_len, fa.FA_KV_SPLIT, inp5s.scale, 0, fa.FA_BF16, ws5s,
                           ws5s_bytes, stream=sid)

    # Workload 4 decoding 2 new tokens per sequence at once (the same pool and table).
    q4m = to_dev(fi.normal_bits((inp4.B, 2, inp4.Hq, 576), "bf16", fi.rng_for(4, fi.T_Q)))
    o4m = torch.empty((inp4.B, 2, inp4.Hq, 512), dtype=torch.bfloat16, device=dev)
    ws4m_bytes = fa.fa_decode_multi_workspace_size(inp4.B, 2, inp4.Hq, 1, 576, 512, 1,
                                                   inp4.max_seq_len, fa.FA_KV_MLA_SHARED)
    ws4m = torch.empty(max(ws4m_bytes, 16) // 4 + 4, dtype=torch.float32, device=dev)

    def decode_mla_multi_pass():
        fa.fa_decode_paged_multi(q4m, pool4, pt4, sl4, pool4.shape[0], o4m, None, inp4.B, 2,
                                 inp4.Hq, 1, 576, 512, 1, inp4.max_pages, inp4.max_seq_len,
                                 fa.FA_KV_MLA_SHARED, inp4.scale, 0, fa.FA_BF16, ws4m,
                                 ws4m_bytes, stream=sid)

    def decode_multi_pass():
        fa.fa_decode_paged_multi(q5, pool5, pt5, sl5, pool5.shape[0], o5, None, inp5.B, inp5.Sq,
                                 inp5.Hq, inp5.Hkv, 128, 128, 16, inp5.max_pages,
                                 inp5.max_seq_len, fa.FA_KV_SPLIT, inp5.scale, 0, fa.FA_BF16,
                                 ws5, ws5_bytes, stream=sid)

    def decode_pass():
        fa.fa_decode_paged(q4, pool4, pt4, sl4, pool4.shape[0], o4, None, inp4.B, inp4.Hq, 1, 576,
                           512, 1, inp4.max_pages, inp4.max_seq_len, fa.FA_KV_MLA_SHARED,
                           inp4.scale, 0, fa.FA_BF16, ws4, ws4_bytes, stream=sid)

    if args.traffic:
        src = torch.ones(64 * 2**20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        q, k, v, o, skv = ub_args[-1]
        for _ in range(3):
            dst.copy_(src)
            flush_sum = flush.sum()
            fa.fa_prefill_ex(q, k, v, o, None, 1, Hq, Hkv, UB, skv, D, 1, inp3.scale,
                             fa.FA_BF16, fa.FA_BF16, ws3, ws3_bytes, stream=sid)
            flush_sum = flush.sum()
            decode_pass()
            flush_sum = flush.sum()
            decode_gqa_pass()
        torch.cuda.synchronize()
        eprint("traffic launches done (copy 268435456 B read + written per launch)")
        return

    def step(evs):
        evs[0].record(stream)
        prefill_pass()
        evs[1].record(stream)
        flush_sum = flush.sum()
        evs[2].record(stream)
        decode_pass()
        evs[3].record(stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(4)]  # noqa: E731
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    events = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in events:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_pfm = None
    if masks3 is not None:
        for _ in range(2):
            prefill_mask_pass()
        ev_m = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
        for e0, e1 in ev_m:
            e0.record(stream)
            prefill_mask_pass()
            e1.record(stream)
        torch.cuda.synchronize()
        t_pfm = sum(e0.elapsed_time(e1) for e0, e1 in ev_m) / 1e3

    def timed_cold(fn):
        for _ in range(2):
            fn()
        evs = []
        for _ in range(args.steps):
            flush_sum = flush.sum()  # noqa: F841
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in evs) / 1e3

    def timed_warm(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3

    t_mha = timed_warm(mha_pass)
    t_d5s = timed_cold(decode_gqa_pass)
    t_d5 = timed_cold(decode_multi_pass)
    t_d4m = timed_cold(decode_mla_multi_pass)

    t_pf = sum(e[0].elapsed_time(e[1]) for e in events) / 1e3  # s
    t_dec = sum(e[2].elapsed_time(e[3]) for e in events) / 1e3
    K = args.steps
    flops3 = prefill_flops(S, UB, Hq, D)
    bytes4 = decode_bytes(inp4)
    pf_tflops = flops3 * K / t_pf / 1e12
    dec_gbs = bytes4 * K / t_dec / 1e9

    sha_pf = source_sha("prefill_kernel.h", "prefill.hip", "combine.hip", "fa_device.h")
    sha_dec = source_sha("decode_mla.hip", "combine.hip", "fa_device.h")
    sha_gqa = source_sha("decode.hip", "combine.hip", "fa_device.h")
    tr_pf, tr_pf_launch = traffic_for("prefill", sha_pf) or (None, None)
    tr_dec, tr_dec_launch = traffic_for("decode_mla", sha_dec) or (None, None)
    tr_gqa, tr_gqa_launch = traffic_for("decode_gqa", sha_gqa) or (None, None)

    result = {
        "metric": METRIC,
        "value": round(pf_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal GQA prefill B=1 Hq=32 Hkv=8 D=128 bf16, 16384 tokens as 32 "
                        "microbatches of 512 queries; then paged MLA decode batch=128 heads=64 "
                        "seq_len=2048 D_qk=576 D_v=512 page_size=1",
            "prefill_calls_per_step": n_ub,
            "prefill_flop_per_step": flops3,
            "prefill_ms_per_step": round(t_pf / K * 1e3, 4),
            "decode_bytes_per_step": bytes4,
            "decode_us_per_step": round(t_dec / K * 1e6, 2),
            "decode_splits": n_split4,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(pf_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pf_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": tr_pf,
            "traffic_launch": tr_pf_launch,
            "kernel": "fa_prefill_ex call (prefill kernel + split combine), averaged over the "
                      "32 microbatch launches",
        },
        "decode": {
            "metric": "paged MLA decode GB/s (%HBM peak)",
            "value": round(dec_gbs, 1),
            "unit": "GB/s",
            "roofline": {
                "bound": "hbm",
                "achieved": round(dec_gbs, 1),
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                "traffic": tr_dec,
                "traffic_launch": tr_dec_launch,
                "kernel": "fa_decode_paged call (MLA decode kernel + split combine)",
            },
            "tflops": round(36507222016 * K / t_dec / 1e12, 1),
        },
        "cpu_baseline": None,
    }
    flops2 = 4 * inp2.B * inp2.Hq * inp2.Sq * inp2.Skv * inp2.D
    mha_tflops = flops2 * K / t_mha / 1e12
    result["prefill_mha"] = {
        "metric": "non-causal MHA prefill attn TFLOP/s (%MFMA peak)",
        "value": round(mha_tflops, 2),
        "unit": "TFLOP/s",
        "us_per_call": round(t_mha / K * 1e6, 2),
        "flop_per_call": flops2,
        "workload": "non-causal MHA B=4 Hq=Hkv=16 Sq=Skv=2048 D=64 bf16, scale 1/8; warm "
                    "(inputs resident, back-to-back calls)",
        "splits": max(1, ws2_bytes // (inp2.B * inp2.Sq * inp2.Hq * (inp2.D * 2 + 4))),
        "roofline": {
            "bound": "mfma",
            "achieved": round(mha_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(mha_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "kernel": "fa_prefill_ex call (prefill kernel, plus the split combine if the "
                      "planner splits)",
        },
    }
    bytes5s = split_decode_bytes(inp5s)
    d5s_gbs = bytes5s * K / t_d5s / 1e9
    result["decode_gqa"] = {
        "metric": "small-batch paged GQA decode GB/s (%HBM peak)",
        "value": round(d5s_gbs, 1),
        "unit": "GB/s",
        "us_per_call": round(t_d5s / K * 1e6, 2),
        "bytes_per_call": bytes5s,
        "workload": "4 sequences of U[1024, 32768] tokens (seeded: "
                    + "/".join(str(int(n)) for n in inp5s.seq_lens)
                    + "), 32 query / 8 K/V heads, D=128, page 16, one new token each, bf16; "
                      "cold (after a cache-evicting read)",
        "splits": n_split5s,
        "roofline": {
            "bound": "hbm",
            "achieved": round(d5s_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(d5s_gbs / PEAK_HBM_GBS, 4),
            "traffic": tr_gqa,
            "traffic_launch": tr_gqa_launch,
            "kernel": "fa_decode_paged call (GQA decode kernel + split combine)",
        },
    }
    bytes5 = split_decode_bytes(inp5)
    d5_gbs = bytes5 * K / t_d5 / 1e9
    result["decode_multi"] = {
        "metric": "paged GQA decode of 4 new tokens per sequence GB/s (%HBM peak)",
        "value": round(d5_gbs, 1),
        "unit": "GB/s",
        "us_per_call": round(t_d5 / K * 1e6, 2),
        "bytes_per_call": bytes5,
        "workload": "4 sequences of U[1024, 32768] tokens (seeded), 32 query / 8 K/V heads, "
                    "D=128, page 16, 4 new tokens each (causal among themselves), bf16; "
                    "cold (after a cache-evicting read)",
        "splits": max(1, ws5_bytes // (inp5.B * inp5.Sq * inp5.Hq * (128 * 2 + 4))),
        "roofline": {
            "bound": "hbm",
            "achieved": round(d5_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(d5_gbs / PEAK_HBM_GBS, 4),
            "traffic": None,
            "kernel": "fa_decode_paged_multi call (GQA decode kernel + split combine)",
        },
    }
    bytes4m = decode_bytes(inp4) + inp4.B * inp4.Hq * (576 + 512) * 2  # a second q and o row
    d4m_gbs = bytes4m * K / t_d4m / 1e9
    result["decode_mla_multi"] = {
        "metric": "paged MLA decode of 2 new tokens per sequence GB/s (%HBM peak)",
        "value": round(d4m_gbs, 1),
        "unit": "GB/s",
        "us_per_call": round(t_d4m / K * 1e6, 2),
        "bytes_per_call": bytes4m,
        "workload": "MLA batch 128 x 64 heads x 2048 tokens, page 1, 2 new tokens each "
                    "(causal among themselves), bf16; cold",
        "roofline": {
            "bound": "hbm",
            "achieved": round(d4m_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(d4m_gbs / PEAK_HBM_GBS, 4),
            "traffic": None,
            "kernel": "fa_decode_paged_multi call (MLA decode kernel, 64-row workgroups)",
        },
    }
    if args.mla_page_sizes:
        per_ps = {}
        for ps in (1, 16, 64):
            inp_ps = fi.mla_decode_inputs(4, 128, 64, 2048, page_size=ps)
            q_ps, pool_ps = to_dev(inp_ps.q), to_dev(inp_ps.pool)
            pt_ps = torch.from_numpy(inp_ps.page_table).to(dev)
            sl_ps = torch.from_numpy(inp_ps.seq_lens).to(dev)
            wsb_ps = fa.fa_decode_workspace_size(128, 64, 1, 576, 512, ps, 2048,
                                                 fa.FA_KV_MLA_SHARED)
            ws_ps = torch.empty(max(wsb_ps, 16) // 4 + 4, dtype=torch.float32, device=dev)

            def ps_pass():
                fa.fa_decode_paged(q_ps, pool_ps, pt_ps, sl_ps, pool_ps.shape[0], o4, None, 128,
                                   64, 1, 576, 512, ps, inp_ps.max_pages, 2048,
                                   fa.FA_KV_MLA_SHARED, inp_ps.scale, 0, fa.FA_BF16, ws_ps,
                                   wsb_ps, stream=sid)
            t_ps = timed_cold(ps_pass)
            per_ps[str(ps)] = {"us_per_call": round(t_ps / K * 1e6, 2),
                               "GB/s": round(decode_bytes(inp_ps) * K / t_ps / 1e9, 1)}
            del q_ps, pool_ps, pt_ps, sl_ps, ws_ps
        result["decode_mla_page_sizes"] = per_ps
    if t_pfm is not None:
        pfm_tflops = flops3 * K / t_pfm / 1e12
        result["prefill_mask"] = {
            "metric": "masked prefill attn TFLOP/s (%MFMA peak)",
            "value": round(pfm_tflops, 2),
            "unit": "TFLOP/s",
            "ms_per_pass": round(t_pfm / K * 1e3, 4),
            "mask": "explicit additive [512, keys] bf16 mask per microbatch: distance bias "
                    "-(p_i - j)/8, -inf above the causal diagonal; causal rule also on",
            "roofline": {
                "bound": "mfma",
                "achieved": round(pfm_tflops, 2),
                "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(pfm_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": None,
                "kernel": "fa_prefill_mask call (masked prefill kernel + split combine), "
                          "averaged over the 32 microbatch launches",
            },
        }
    if args.cpu_budget > 0:
        eprint("timing the CPU oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(inp3, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
