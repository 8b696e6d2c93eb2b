#!/usr/bin/env python3
"""Benchmark of the DSA hot path on one MI355X.

One step = one pass of the whole path over each workload the headline metric names:
  * prefill, 1 sequence of 32768 tokens (all tokens are queries), indexer H_I=64 x d_I=128 in fp8,
    top-2048 selection, sparse MLA (128 heads, 576/512) in bf16;
  * decode, 64 sequences x one query against 131072 cached tokens, same shapes.
Each workload is one call of the exported entry point (dsa_forward_prefill, dsa_forward_decode) on one
stream, timed with HIP events around the call; inputs are generated on the GPU before the timed region.
The same work is then run as separate stage calls (indexer -> top-k -> sparse attention) with events
between them, for the per-kernel durations behind the roofline figures.

Prints ONE JSON line: value = prefill tokens/s at 32K (whole job, one GPU); decode queries/s, per-stage
times and roofline fractions, the prefill 8K and chunked 128K configurations, and a parity summary against
the oracle are in the same line.  The oracle (plain C on the host cores) is timed on a bounded sample of
rows and extrapolated with the per-row work model.
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

# MI355X published peaks (dense)
PEAK_FP8_TFLOPS = 5000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0

IDX_FLOP_PER_PAIR = 2 * 64 * 128          # one causal (query, key) pair: 64 heads x 128-dim dot
ATT_FLOP_PER_ENTRY = 2 * 128 * (576 + 512)  # one selected entry: QK (576) and PV (512) for 128 heads
MHA_FLOP_PER_PAIR = 2 * 128 * (192 + 128)   # masked MHA mode: QK (192) and PV (128) per (query, key), 128 heads


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefill-len", type=int, default=32768)
    ap.add_argument("--decode-batch", type=int, default=64)
    ap.add_argument("--decode-len", type=int, default=131072)
    ap.add_argument("--k", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None)
    ap.add_argument("--no-proj", action="store_true", help="skip the MQA-mode projection measurement")
    ap.add_argument("--no-extra-prefill", action="store_true",
                    help="skip the prefill 8K and chunked 128K measurements")
    ap.add_argument("--no-warmup-loss", action="store_true", help="skip the indexer warm-up loss measurement")
    ap.add_argument("--no-sparse-bwd", action="store_true", help="skip the sparse training backward measurement")
    ap.add_argument("--mha-lens", default="4096,8192,12288,16384",
                    help="prefill lengths of the masked-MHA vs sparse-MQA attention sweep ('' to skip)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference kernel for the HBM byte "
                         "counters), then exit")
    return ap.parse_args()


# HBM traffic of the dominant kernel, from two rocprofv3 counter passes (FETCH_SIZE, WRITE_SIZE) over
# `bench.py --only prefill --steps 1 --warmup 0 --no-cpu-baseline`, each scaled by the reading of the same
# counter for a plain copy of known size (`bench.py --calib-copy`).  Valid only for the kernel source it
# was measured on: the sha256 of that source is stored with it and checked at run time.
MEASURED_TRAFFIC = {
    "prefill.sparse_mla": {"bytes_per_launch": 14851565568,  # 10.540 GB read + 4.312 GB written
                           "src_sha256": "fa47cf722a806e7512a0d254ef106b91900de98267c36519d725397c3e087733",
                           "profile": "profiles/dsa_kernels_prefill32k_hbm_traffic.md"},
}
KERNEL_SOURCES = {
    "prefill.sparse_mla": "sparse_attention_13_amd/csrc/sparse_mla.hip",
    "prefill.indexer": "sparse_attention_13_amd/csrc/indexer.hip",
    "prefill.topk": "sparse_attention_13_amd/csrc/topk.hip",
    "decode.indexer": "sparse_attention_13_amd/csrc/indexer.hip",
}


def source_sha(stage):
    import hashlib
    path = os.path.join(ROOT, KERNEL_SOURCES[stage])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(stage):
    """HBM bytes per launch of `stage`'s kernel from the stored counter passes, or None when there is no
    measurement or the kernel's source has changed since it was taken."""
    m = MEASURED_TRAFFIC.get(stage)
    if not m or m["src_sha256"] != source_sha(stage):
        return None
    return m["bytes_per_launch"]


def calib_copy():
    """A plain device copy of 2^30 bytes (read 1 GiB, write 1 GiB), five times: the reference reading for
    the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    dev = torch.device("cuda:0")
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(5):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / 5
    print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4, "ms": round(ms, 4),
                      "GB/s": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}), flush=True)


def causal_work(L: int, n_q: int, k: int):
    """(indexer causal pairs, selected entries, score reads) for the last n_q queries of L tokens."""
    pairs, entries = 0, 0
    for t in range(L - n_q, L):
        pairs += t + 1
        entries += min(k, t + 1)
    return pairs, entries


def prefill_roofline_ms(L: int, n_q: int, k: int) -> float:
    """Roofline time of one prefill call (the last n_q of L tokens are queries): indexer flops at the FP8 peak,
    the score matrix written and read plus the selection written at the HBM peak, attention flops at the bf16
    peak."""
    pairs, entries = causal_work(L, n_q, k)
    return (pairs * IDX_FLOP_PER_PAIR / (PEAK_FP8_TFLOPS * 1e12) + (2 * pairs * 4 + n_q * k * 4) / (PEAK_HBM_GBS * 1e9)
            + entries * ATT_FLOP_PER_ENTRY / (PEAK_BF16_TFLOPS * 1e12)) * 1e3


def decode_bytes(B: int, S: int, k: int):
    """HBM bytes of one decode step per stage: indexer (keys, key scales, scores written, q and w), top-k
    (scores read, selection written), attention (selected rows, selection read, q, out)."""
    i_bytes = B * S * (128 + 4 + 4) + B * 64 * (128 + 8)
    k_bytes = B * S * 4 + B * k * 4
    a_bytes = B * k * 1152 + B * 128 * 576 * 2 + B * 128 * 512 * 2 + B * k * 4
    return i_bytes, k_bytes, a_bytes


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path has no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return
    import torch

    from sparse_attention_13_amd import dsa, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    k = args.k
    sm = 1.0 / math.sqrt(576)

    def timed(calls, steps):
        """Run `calls` (list of (name, fn)) `steps` times with events between them; per-call mean ms."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
        acc = [0.0] * len(calls)
        for _ in range(steps):
            ev[0].record(stream)
            for i, (_, fn) in enumerate(calls):
                fn()
                ev[i + 1].record(stream)
            torch.cuda.synchronize()
            for i in range(len(calls)):
                acc[i] += ev[i].elapsed_time(ev[i + 1])
        return {name: acc[i] / max(steps, 1) for i, (name, _) in enumerate(calls)}

    # ------------------------------------------------------------------ prefill workload (32K, all tokens queries)
    pre = None
    if args.only in (None, "prefill"):
        L = args.prefill_len
        print(f"[bench] generating prefill inputs L={L}", file=sys.stderr, flush=True)
        x = synth.prefill(L, seed=0, device=dev, n_needles=256, needle_layout="random")
        q8, qs, k8, ks, w = (x["q8"][None], x["q_scale"][None], x["k8"][None], x["k_scale"][None], x["w"][None])
        q, kv = x["q"][None], x["kv"][None]
        out = torch.empty((1, L, 128, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((1, L, 128), dtype=torch.float32, device=dev)
        idx_f = torch.empty((1, L, k), dtype=torch.int32, device=dev)
        fws = torch.empty(dsa.forward_workspace_size(1, L, L, 128, 576, 512, k, dsa.DSA_BF16), dtype=torch.uint8,
                          device=dev)
        # stage-by-stage buffers (the per-kernel breakdown and the parity sample)
        ld = ((L + 63) // 64) * 64
        scores = torch.empty((1, L, ld), dtype=torch.float32, device=dev)
        idx = torch.empty((1, L, k), dtype=torch.int32, device=dev)
        s_out = torch.empty_like(out)
        s_lse = torch.empty_like(lse)
        tk_ws = torch.empty(max(dsa.topk_workspace_size(1, L, L, k), 256), dtype=torch.uint8, device=dev)
        ws_n = dsa.lib().dsa_sparse_mla_attn_workspace_size(1, L, L, 128, 576, 512, k, dsa.DSA_BF16)
        ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device=dev)
        pre = dict(L=L, x=x, idx=idx, out=s_out, lse=s_lse, scores=scores,
                   forward=("prefill", lambda: dsa.forward(q8, qs, k8, ks, w, q, kv, k, 512, sm, out=out, lse=lse,
                                                           idx_out=idx_f, workspace=fws)),
                   stages=[("prefill.indexer", lambda: dsa.indexer_scores(q8, qs, k8, ks, w, scores)),
                           ("prefill.topk", lambda: dsa.topk(scores, L, k, idx=idx, workspace=tk_ws)),
                           ("prefill.sparse_mla", lambda: dsa.sparse_mla_attn(q, kv, idx, 512, sm, out=s_out, lse=s_lse,
                                                                              workspace=ws))])

    # ------------------------------------------------------------------ decode workload (64 x 1 query over 128K)
    dec = None
    if args.only in (None, "decode"):
        B, S = args.decode_batch, args.decode_len
        print(f"[bench] generating decode inputs B={B} S={S}", file=sys.stderr, flush=True)
        y = synth.decode(B, S, seed=0, device=dev)
        d_out = torch.empty((B, 128, 512), dtype=torch.bfloat16, device=dev)
        d_lse = torch.empty((B, 128), dtype=torch.float32, device=dev)
        d_idx_f = torch.empty((B, k), dtype=torch.int32, device=dev)
        d_fws = torch.empty(dsa.forward_workspace_size(B, 1, S, 128, 576, 512, k, dsa.DSA_BF16), dtype=torch.uint8,
                            device=dev)
        ld = ((S + 63) // 64) * 64
        d_scores = torch.empty((B, ld), dtype=torch.float32, device=dev)
        d_idx = torch.empty((B, k), dtype=torch.int32, device=dev)
        s_dout = torch.empty_like(d_out)
        s_dlse = torch.empty_like(d_lse)
        d_tk_ws = torch.empty(max(int(dsa.lib().dsa_topk_decode_workspace_size(B, S, k)), 256), dtype=torch.uint8,
                              device=dev)
        ws_n = int(dsa.lib().dsa_sparse_mla_attn_decode_workspace_size(B, S, 128, 576, 512, k, dsa.DSA_BF16))
        d_ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device=dev)
        yq8, yqs, yk8, yks, yw, yq, ykv = y["q8"], y["q_scale"], y["k8"], y["k_scale"], y["w"], y["q"], y["kv"]
        dec = dict(B=B, S=S, y=y, idx=d_idx, out=s_dout, lse=s_dlse, scores=d_scores,
                   forward=("decode", lambda: dsa.forward(yq8, yqs, yk8, yks, yw, yq, ykv, k, 512, sm, decode=True,
                                                          out=d_out, lse=d_lse, idx_out=d_idx_f, workspace=d_fws)),
                   stages=[("decode.indexer", lambda: dsa.indexer_scores_decode(yq8, yqs, yk8, yks, yw, d_scores)),
                           ("decode.topk", lambda: dsa.topk_decode(d_scores, S, k, idx=d_idx, workspace=d_tk_ws)),
                           ("decode.sparse_mla", lambda: dsa.sparse_mla_attn_decode(yq, ykv, d_idx, 512, sm,
                                                                                    out=s_dout, lse=s_dlse,
                                                                                    workspace=d_ws))])

    # ------------------------------------------------------------------ the timed steps: the forward entry points
    step_calls = [w_["forward"] for w_ in (pre, dec) if w_]
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    if args.warmup > 0:
        timed(step_calls, args.warmup)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    st = timed(step_calls, args.steps)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / max(args.steps, 1) * 1e3
    # per-stage breakdown: the same work as separate stage calls (one kernel launch per stage at these shapes,
    # except the split attention and top-k at decode), events between them
    stage_calls = (pre["stages"] if pre else []) + (dec["stages"] if dec else [])
    print(f"[bench] stage breakdown, {args.steps} steps", file=sys.stderr, flush=True)
    timed(stage_calls, 1)
    sst = timed(stage_calls, args.steps)

    res = {"metric": "DSA prefill tokens/s at 32K ctx + decode queries/s at 128K ctx; % roofline",
           "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(sum(st.values()), 4), "wall_ms_per_step": round(wall, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8+bf16",
           "data": "synthetic (seeded; N(0,1) inputs, fp8 e4m3 indexer with amax scales, needles)",
           "config": {"workload": ("prefill 1x32768 tokens (all queries) + decode 64x1 query over 131072 "
                                   "cached tokens; H_I=64 d_I=128 fp8, k=2048, 128 heads d_qk=576 d_v=512 bf16"),
                      "timed": "dsa_forward_prefill + dsa_forward_decode per step"}}
    rooflines = {}
    if pre:
        L = pre["L"]
        pairs, entries = causal_work(L, L, k)
        t_fwd = st["prefill"]
        t_i, t_k, t_a = sst["prefill.indexer"], sst["prefill.topk"], sst["prefill.sparse_mla"]
        idx_tf = pairs * IDX_FLOP_PER_PAIR / (t_i * 1e-3) / 1e12
        tk_bytes = pairs * 4 + L * k * 4
        tk_gbs = tk_bytes / (t_k * 1e-3) / 1e9
        att_tf = entries * ATT_FLOP_PER_ENTRY / (t_a * 1e-3) / 1e12
        roof_ms = prefill_roofline_ms(L, L, k)
        res["value"] = round(L / (t_fwd * 1e-3), 1)
        res["prefill"] = {"tokens_per_s": res["value"], "ms": round(t_fwd, 4), "roofline_ms": round(roof_ms, 4),
                          "frac_of_roofline": round(roof_ms / t_fwd, 4),
                          "stages_ms": {"indexer": round(t_i, 4), "topk": round(t_k, 4), "sparse_mla": round(t_a, 4)},
                          "stages_sum_ms": round(t_i + t_k + t_a, 4),
                          "indexer": {"TFLOP/s": round(idx_tf, 1), "frac_fp8_peak": round(idx_tf / PEAK_FP8_TFLOPS, 4)},
                          "topk": {"GB/s": round(tk_gbs, 1), "frac_hbm": round(tk_gbs / PEAK_HBM_GBS, 4)},
                          "sparse_mla": {"TFLOP/s": round(att_tf, 1),
                                         "frac_bf16_peak": round(att_tf / PEAK_BF16_TFLOPS, 4)}}
        rooflines["prefill.indexer"] = (t_i, {"bound": "mfma", "achieved": round(idx_tf, 2), "peak": PEAK_FP8_TFLOPS,
                                              "unit": "TFLOP/s", "frac": round(idx_tf / PEAK_FP8_TFLOPS, 4),
                                              "traffic": None})
        rooflines["prefill.topk"] = (t_k, {"bound": "hbm", "achieved": round(tk_gbs, 1), "peak": PEAK_HBM_GBS,
                                           "unit": "GB/s", "frac": round(tk_gbs / PEAK_HBM_GBS, 4), "traffic": None})
        rooflines["prefill.sparse_mla"] = (t_a, {"bound": "mfma", "achieved": round(att_tf, 2),
                                                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                                 "frac": round(att_tf / PEAK_BF16_TFLOPS, 4), "traffic": None})
    if dec:
        B, S = dec["B"], dec["S"]
        t_fwd = st["decode"]
        t_i, t_k, t_a = sst["decode.indexer"], sst["decode.topk"], sst["decode.sparse_mla"]
        i_bytes, k_bytes, a_bytes = decode_bytes(B, S, k)
        roof_ms = (i_bytes + k_bytes + a_bytes) / (PEAK_HBM_GBS * 1e9) * 1e3
        i_gbs = i_bytes / (t_i * 1e-3) / 1e9
        a_gbs = a_bytes / (t_a * 1e-3) / 1e9
        res["decode"] = {"queries_per_s": round(B / (t_fwd * 1e-3), 1), "unit": "queries/s", "ms": round(t_fwd, 4),
                         "roofline_ms": round(roof_ms, 4), "frac_of_hbm_roofline": round(roof_ms / t_fwd, 4),
                         "stages_ms": {"indexer": round(t_i, 4), "topk": round(t_k, 4), "sparse_mla": round(t_a, 4)},
                         "stages_sum_ms": round(t_i + t_k + t_a, 4),
                         "indexer": {"GB/s": round(i_gbs, 1), "frac_hbm": round(i_gbs / PEAK_HBM_GBS, 4)},
                         "topk": {"GB/s": round(k_bytes / (t_k * 1e-3) / 1e9, 1),
                                  "frac_hbm": round(k_bytes / (t_k * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
                         "sparse_mla": {"GB/s": round(a_gbs, 1), "frac_hbm": round(a_gbs / PEAK_HBM_GBS, 4)}}
        rooflines["decode.indexer"] = (t_i, {"bound": "hbm", "achieved": round(i_gbs, 1), "peak": PEAK_HBM_GBS,
                                             "unit": "GB/s", "frac": round(i_gbs / PEAK_HBM_GBS, 4), "traffic": None})
        if res["value"] is None:
            res["value"] = res["decode"]["queries_per_s"]
            res["unit"] = "queries/s"
    # dominant kernel = the stage with the largest time in the step
    dom = max(rooflines.items(), key=lambda kv_: kv_[1][0]) if rooflines else None
    if dom:
        roof = dict(dom[1][1], kernel=dom[0])
        roof["traffic"] = measured_traffic(dom[0]) if dom[0] in KERNEL_SOURCES else None
        res["roofline"] = roof

    # ------------------------------------------------------------------ CPU oracle baseline and parity sample
    if not args.no_cpu_baseline and pre:
        base, par = cpu_baseline_prefill(pre, k, sm)
        res["cpu_baseline"] = base
        res["parity"] = {"prefill_32k": par}
        if dec:
            dbase, dpar = cpu_baseline_decode(dec, k, sm)
            res["decode"]["cpu_baseline"] = dbase
            res["parity"]["decode_128k"] = dpar
    del pre, dec
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------ further prefill configurations
    if args.only in (None, "prefill") and not args.no_extra_prefill:
        res["prefill_8k"] = prefill_leg(8192, 1, k, dev, stream, max(args.steps, 3), n_needles=64, layout="random")
        res["chunked_128k"] = prefill_leg(131072, 16, k, dev, stream, max(2, args.steps // 4), n_needles=1024,
                                          layout="even")
    # ------------------------------------------------------------------ masked MHA mode (short prefill)
    if args.only in (None, "prefill") and args.mha_lens:
        res["masked_mha"] = masked_mha_sweep([int(v) for v in args.mha_lens.split(",")], k, dev, stream)
    if args.only in (None, "prefill") and not args.no_proj:
        res["mla_projections"] = projections_bench(args.prefill_len, dev, stream)
    if args.only in (None, "prefill") and not args.no_warmup_loss:
        res["warmup_loss"] = warmup_bench(args.prefill_len, dev, stream)
    if args.only in (None, "prefill") and not args.no_sparse_bwd:
        res["sparse_backward"] = sparse_backward_bench(args.prefill_len, k, dev, stream)
    print(json.dumps(res), flush=True)


def prefill_leg(L, n_chunks, k, dev, stream, steps, n_needles, layout):
    """One prefill of L tokens as n_chunks calls of dsa_forward_prefill (chunk c: queries c*L/n_chunks ..
    (c+1)*L/n_chunks - 1 over the keys 0 .. (c+1)*L/n_chunks - 1), timed per whole prefill with events around
    the calls; reported with the roofline of the same calls."""
    import torch

    from sparse_attention_13_amd import dsa, synth

    C = L // n_chunks
    print(f"[bench] prefill leg L={L} in {n_chunks} call(s) of {C} queries", file=sys.stderr, flush=True)
    x = synth.prefill(L, seed=0, device=dev, n_needles=n_needles, needle_layout=layout)
    sm = 1.0 / math.sqrt(576)
    out = torch.empty((1, C, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, C, 128), dtype=torch.float32, device=dev)
    fws = torch.empty(dsa.forward_workspace_size(1, C, L, 128, 576, 512, k, dsa.DSA_BF16), dtype=torch.uint8,
                      device=dev)
    views = []
    for c in range(n_chunks):
        lo, hi = c * C, (c + 1) * C
        views.append((x["q8"][None, lo:hi], x["q_scale"][None, lo:hi], x["k8"][None, :hi], x["k_scale"][None, :hi],
                      x["w"][None, lo:hi], x["q"][None, lo:hi], x["kv"][None, :hi]))

    def run():
        for v in views:
            dsa.forward(*v, k, 512, sm, out=out, lse=lse, workspace=fws)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        ev[0].record(stream)
        run()
        ev[1].record(stream)
        torch.cuda.synchronize()
        ts.append(ev[0].elapsed_time(ev[1]))
    t = sorted(ts)[len(ts) // 2]
    roof = sum(prefill_roofline_ms((c + 1) * C, C, k) for c in range(n_chunks))
    res = {"workload": (f"prefill 1x{L} tokens as {n_chunks} dsa_forward_prefill call(s) of {C} queries; "
                        f"{n_needles} needles ({layout}); indexer 64x128 fp8, k={k}, 128 heads 576/512 bf16"),
           "ms": round(t, 4), "tokens_per_s": round(L / (t * 1e-3), 1), "roofline_ms": round(roof, 4),
           "frac_of_roofline": round(roof / t, 4), "steps": steps}
    del x, views, out, lse, fws
    torch.cuda.empty_cache()
    return res


SBWD_FLOP_PER_ENTRY = 2 * 128 * (576 + 512 + 576 + 576 + 512)  # S, dP, dq, dK, dV per selected entry


def sparse_backward_bench(L, k, dev, stream):
    """The sparse training stage's backward through the attention on a prefill of L tokens with k selected
    entries per query (a host-drawn top-k-shaped selection): dq and dkv (and the head-mean target) from
    dout, given the forward's out and lse.  Matrix-core work per selected entry: S, dP, dq, dK and dV over
    128 heads (SBWD_FLOP_PER_ENTRY); HBM traffic beyond it: P and dS (512 B per entry) and the entry's
    dkv terms (1152 B per entry), each written once and read once."""
    import torch

    from sparse_attention_13_amd import dsa, synth

    print(f"[bench] sparse backward at {L} tokens, k={k}", file=sys.stderr, flush=True)
    x = synth.prefill(L, seed=0, device=dev)
    idx = torch.from_numpy(synth.selection(L, L, k, seed=1)).to(dev)
    mq_ws = dsa.lib().dsa_sparse_mla_attn_workspace_size(1, L, L, 128, 576, 512, k, dsa.DSA_BF16)
    ws_f = torch.empty(max(mq_ws, 256), dtype=torch.uint8, device=dev)
    out, lse = dsa.sparse_mla_attn(x["q"][None], x["kv"][None], idx, 512, x["sm_scale"], workspace=ws_f)
    dout = synth.sparse_grad((1, L, 128, 512), seed=0, device=dev)
    ws = torch.empty(dsa.sparse_mla_backward_workspace_size(1, L, L, k), dtype=torch.uint8, device=dev)
    dq = torch.empty((1, L, 128, 576), dtype=torch.float32, device=dev)
    dkv = torch.empty((1, L, 576), dtype=torch.float32, device=dev)
    pbar = torch.empty((1, L, k), dtype=torch.float32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tf, tb = [], []
    for rep in range(5):
        ev[0].record(stream)
        dsa.sparse_mla_attn(x["q"][None], x["kv"][None], idx, 512, x["sm_scale"], out=out, lse=lse, workspace=ws_f)
        ev[1].record(stream)
        dsa.sparse_mla_backward(x["q"][None], x["kv"][None], idx, out, lse, dout, x["sm_scale"], dq=dq, dkv=dkv,
                                pbar=pbar, workspace=ws)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if rep:
            tf.append(ev[0].elapsed_time(ev[1]))
            tb.append(ev[1].elapsed_time(ev[2]))
    t_f, t_b = sorted(tf)[len(tf) // 2], sorted(tb)[len(tb) // 2]
    entries = sum(min(k, t + 1) for t in range(L))
    tflops = entries * SBWD_FLOP_PER_ENTRY / (t_b * 1e-3) / 1e12
    res = {"workload": f"1x{L} tokens, k={k}, 128 heads, d_qk=576, d_v=512, bf16 (host-drawn selection)",
           "forward_ms": round(t_f, 4), "backward_ms": round(t_b, 4), "backward_over_forward": round(t_b / t_f, 2),
           "tokens_per_s": round(L / (t_b * 1e-3), 1), "TFLOP/s": round(tflops, 1),
           "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / PEAK_BF16_TFLOPS, 4)},
           "workspace_bytes": int(ws.numel())}
    del x, idx, out, lse, dout, ws, ws_f, dq, dkv, pbar
    torch.cuda.empty_cache()
    return res


def warmup_bench(L, dev, stream):
    """One indexer warm-up step on a prefill of L tokens: index scores (fp8), the loss (target from the main
    attention: 128 heads x 576 over every causal pair, bf16; KL; gradient) and the gradients through the
    indexer (dq, dw: 2 x 64 x 128 x 2 flop per pair; dk the same).  The main attention's log-sum-exp is an
    input (the frozen main model's dense forward pass produces it), made beforehand with the attention kernel
    over the full causal selection."""
    import torch

    from sparse_attention_13_amd import dsa, synth

    print(f"[bench] indexer warm-up step at {L} tokens", file=sys.stderr, flush=True)
    x = synth.prefill(L, seed=0, device=dev, n_needles=max(1, L // 128), needle_layout="random")
    pos = torch.arange(L, device=dev)[:, None]
    s_ = torch.arange(L, device=dev)[None, :]
    idx = torch.where(s_ <= pos, s_, torch.full_like(s_, -1)).to(torch.int32)[None]
    del pos, s_
    _, lse = dsa.sparse_mla_attn(x["q"][None], x["kv"][None], idx, 512, x["sm_scale"])
    del idx
    torch.cuda.empty_cache()
    scores = torch.empty((1, L, L), dtype=torch.float32, device=dev)
    target = torch.empty_like(scores)
    loss = torch.empty((1, L), dtype=torch.float32, device=dev)
    dq = torch.empty((1, L, 64, 128), dtype=torch.float32, device=dev)
    dw = torch.empty((1, L, 64), dtype=torch.float32, device=dev)
    dk = torch.empty((1, L, 128), dtype=torch.float32, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ts = [[], [], []]
    for rep in range(6):
        ev[0].record(stream)
        dsa.indexer_scores(x["q8"][None], x["q_scale"][None], x["k8"][None], x["k_scale"][None], x["w"][None], scores)
        ev[1].record(stream)
        dsa.warmup_loss(x["q"][None], x["kv"][None], lse, scores, x["sm_scale"], target=target, loss=loss)
        ev[2].record(stream)
        dsa.warmup_indexer_backward(x["q8"][None], x["q_scale"][None], x["k8"][None], x["k_scale"][None],
                                    x["w"][None], scores, dq=dq, dw=dw, dk=dk)
        ev[3].record(stream)
        torch.cuda.synchronize()
        if rep:
            for i in range(3):
                ts[i].append(ev[i].elapsed_time(ev[i + 1]))
    t_i, t_l, t_b = (sorted(v)[len(v) // 2] for v in ts)
    pairs = L * (L + 1) // 2
    tgt_flop = pairs * 2 * 128 * 576
    bwd_flop = pairs * 2 * (2 * 64 * 128 * 2)
    res = {"workload": f"1x{L} tokens, dense causal; indexer 64x128 fp8, main attention 128 heads x 576 bf16",
           "ms": round(t_i + t_l + t_b, 4),
           "stages_ms": {"indexer": round(t_i, 4), "loss": round(t_l, 4), "backward": round(t_b, 4)},
           "tokens_per_s": round(L / ((t_i + t_l + t_b) * 1e-3), 1),
           "indexer_TFLOP/s": round(pairs * IDX_FLOP_PER_PAIR / (t_i * 1e-3) / 1e12, 1),
           "loss_target_TFLOP/s": round(tgt_flop / (t_l * 1e-3) / 1e12, 1),
           "backward_TFLOP/s": round(bwd_flop / (t_b * 1e-3) / 1e12, 1)}
    res["roofline"] = {"bound": "mfma", "kernel": "loss (target product)", "achieved": res["loss_target_TFLOP/s"],
                       "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(res["loss_target_TFLOP/s"] / PEAK_BF16_TFLOPS, 4)}
    res["backward_roofline"] = {"bound": "mfma", "achieved": res["backward_TFLOP/s"], "peak": PEAK_BF16_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(res["backward_TFLOP/s"] / PEAK_BF16_TFLOPS, 4)}
    del x, lse, scores, target, loss, dq, dw, dk
    torch.cuda.empty_cache()
    return res


def projections_bench(L, dev, stream):
    """The MQA-mode projections at the prefill size (L tokens x 128 heads): query absorption of W_UK
    (reads the 192-wide per-head query, writes the 576-wide latent query) and the output up-projection
    W_UV (reads the 512-wide latent output, writes 128).  HBM-bound: bytes per (token, head) are
    384 + 1152 and 1024 + 256 (weights, 16 MiB each, stay in cache)."""
    import torch

    from sparse_attention_13_amd import dsa, synth

    H = 128
    print(f"[bench] MQA-mode projections at {L} tokens", file=sys.stderr, flush=True)
    g = torch.Generator(device=dev).manual_seed(0)
    q = torch.randn((L, H, 192), generator=g, device=dev).to(torch.bfloat16)
    o_lat = torch.randn((L, H, 512), generator=g, device=dev).to(torch.bfloat16)
    w = synth.mla_weights(H, seed=0, device=dev)
    q_mqa = torch.empty((L, H, 576), dtype=torch.bfloat16, device=dev)
    o = torch.empty((L, H, 128), dtype=torch.bfloat16, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ta, tb = [], []
    for rep in range(6):
        ev[0].record(stream)
        dsa.mla_absorb_q(q, w["w_ukt"], q_mqa)
        ev[1].record(stream)
        dsa.mla_out_proj(o_lat, w["w_uv"], o)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if rep:
            ta.append(ev[0].elapsed_time(ev[1]))
            tb.append(ev[1].elapsed_time(ev[2]))
    res = {"workload": f"{L} tokens x {H} heads, bf16; absorb 128->512 (+64 rope), out 512->128"}
    for name, ts, per, flop in (("absorb_q", ta, 384 + 1152, 2 * 128 * 512), ("out_proj", tb, 1024 + 256, 2 * 512 * 128)):
        t = sorted(ts)[len(ts) // 2]
        gbs = L * H * per / (t * 1e-3) / 1e9
        res[name] = {"ms": round(t, 4), "GB/s": round(gbs, 1), "TFLOP/s": round(L * H * flop / (t * 1e-3) / 1e12, 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(gbs / PEAK_HBM_GBS, 4)}}
    return res


def masked_mha_sweep(lens, k, dev, stream):
    """Attention of one prefill of L tokens in both modes, on the same selection (indexer + top-k of the
    sequence): masked MHA mode (MHA form: 128 heads, d_qk 192, d_v 128; the mask build included) and
    sparse MQA mode (latent rows, d_qk 576, d_v 512).  Reported: both times per L, the masked-MHA rate at
    8K against the bf16 peak (dense-equivalent: every causal pair is computed, masked or not), and the
    length where the two modes cross (linear interpolation between the measured lengths)."""
    import torch

    from sparse_attention_13_amd import dsa, synth

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def t_ms(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]))
        return sorted(ts)[len(ts) // 2]

    sweep = []
    for L in lens:
        print(f"[bench] masked MHA vs sparse MQA at L={L}", file=sys.stderr, flush=True)
        x = synth.prefill(L, seed=0, device=dev, n_needles=max(1, L // 128), needle_layout="random")
        scores = torch.empty((1, L, L), dtype=torch.float32, device=dev)
        dsa.indexer_scores(x["q8"][None], x["q_scale"][None], x["k8"][None], x["k_scale"][None], x["w"][None], scores)
        idx = dsa.topk(scores, L, k)
        del scores
        m = synth.mha_heads(L, seed=0, device=dev)
        ws = torch.empty(max(dsa.masked_mha_workspace_size(1, L, L), 256), dtype=torch.uint8, device=dev)
        o1 = torch.empty((1, L, 128, 128), dtype=torch.bfloat16, device=dev)
        l1 = torch.empty((1, L, 128), dtype=torch.float32, device=dev)
        t_mha = t_ms(lambda: dsa.masked_mha_attn(m["q"][None], m["k"][None], m["v"][None], idx, m["sm_scale"], out=o1,
                                                 lse=l1, workspace=ws))
        del m, ws, o1, l1
        mq_ws = dsa.lib().dsa_sparse_mla_attn_workspace_size(1, L, L, 128, 576, 512, k, dsa.DSA_BF16)
        ws2 = torch.empty(max(mq_ws, 256), dtype=torch.uint8, device=dev)
        o2 = torch.empty((1, L, 128, 512), dtype=torch.bfloat16, device=dev)
        l2 = torch.empty((1, L, 128), dtype=torch.float32, device=dev)
        t_mqa = t_ms(lambda: dsa.sparse_mla_attn(x["q"][None], x["kv"][None], idx, 512, x["sm_scale"], out=o2, lse=l2,
                                                 workspace=ws2))
        del x, idx, ws2, o2, l2
        torch.cuda.empty_cache()
        pairs, entries = causal_work(L, L, k)
        sweep.append({"L": L, "masked_mha_ms": round(t_mha, 4), "sparse_mqa_ms": round(t_mqa, 4),
                      "masked_mha_dense_TFLOP/s": round(pairs * MHA_FLOP_PER_PAIR / (t_mha * 1e-3) / 1e12, 1),
                      "masked_mha_useful_TFLOP/s": round(entries * MHA_FLOP_PER_PAIR / (t_mha * 1e-3) / 1e12, 1),
                      "sparse_mqa_TFLOP/s": round(entries * ATT_FLOP_PER_ENTRY / (t_mqa * 1e-3) / 1e12, 1)})
    res = {"workload": ("prefill 1xL, attention only, both modes on the same top-k (k=%d) selection; masked MHA: "
                        "128 heads d_qk=192 d_v=128 bf16; sparse MQA: 128 heads d_qk=576 d_v=512 bf16" % k),
           "sweep": sweep}
    ref = next((e for e in sweep if e["L"] == 8192), sweep[0] if sweep else None)
    if ref:
        tf = ref["masked_mha_dense_TFLOP/s"]
        res["roofline"] = {"bound": "mfma", "L": ref["L"], "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    cut = None
    for a, b in zip(sweep, sweep[1:]):
        da, db = a["masked_mha_ms"] - a["sparse_mqa_ms"], b["masked_mha_ms"] - b["sparse_mqa_ms"]
        if da <= 0.0 < db:
            cut = round(a["L"] + (b["L"] - a["L"]) * (-da) / (db - da))
            break
    res["cutover_L"] = cut
    res["cutover_rule"] = "masked MHA mode below cutover_L, sparse MQA mode above (attention time only)"
    return res


def _parity_summary(oracle, parity, g_scores, o_scores, mag, absmag, gi, res, g_out, g_lse, pos):
    """Parity of the GPU's stage outputs on the sampled rows against the oracle's own run on the same rows:
    indexer score errors (the asserted magnitude-relative bound and the plain relative figure), the selection
    under the band rule, and the attention on the rows whose selection is identical."""
    rep = parity.indexer_report(g_scores, o_scores, mag, absmag, pos)
    ok, exact = parity.topk_band_match(gi, res["idx"], res["scores"], res["kth"], pos)
    same = [r for r in range(len(pos)) if (gi[r] == res["idx"][r]).all()]
    ratio, mx, lse_err = parity.attention_errors(g_out[same], res["out"][same], g_lse[same], res["lse"][same])
    return {"rows": int(len(pos)), "indexer_entries": rep["n"],
            "indexer_worst_over_bound": round(rep["worst_bound_ratio"], 4),
            "indexer_rel_err_wellcond": float(f"{rep['rel_wellcond']:.3g}"),
            "indexer_frac_wellcond": round(rep["frac_wellcond"], 4),
            "indexer_rel_err_q999_all": float(f"{rep['rel_q999']:.3g}"),
            "selection_band_ok_rows": int(ok), "selection_identical_rows": int(exact),
            "selection_band_exchange_rows": int(ok - exact), "attention_rows_compared": len(same),
            "attention_worst_over_bound": round(ratio, 4), "attention_max_abs_err": float(f"{mx:.3g}"),
            "lse_max_abs_err": float(f"{lse_err:.3g}"),
            "pass": bool(rep["worst_bound_ratio"] <= 1.0 and rep["rel_wellcond"] <= parity.IDX_REL and ok == len(pos)
                         and ratio <= 1.0 and lse_err <= parity.LSE_ABS)}


def cpu_baseline_prefill(pre, k, sm):
    """The oracle timed on a bounded sample of the 32K prefill's query rows (full path per row), extrapolated
    to every row with the per-row work model; the same rows then give the parity summary of the GPU's stage
    outputs (scores, selection, attention)."""
    import numpy as np
    import torch

    import oracle
    from sparse_attention_13_amd import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity
    L, x = pre["L"], pre["x"]
    gen = np.random.default_rng(0)
    fixed = np.concatenate([np.arange(0, 64), np.arange(k - 32, k + 32), np.arange(L - 64, L)])
    rest = np.setdiff1d(np.arange(L), fixed)
    rows = np.unique(np.concatenate([fixed, gen.choice(rest, 512 - len(np.unique(fixed)), replace=False)]))
    rows = rows.astype(np.int64)
    rsel = torch.from_numpy(rows).to(x["q8"].device)
    q_i = oracle.dequant_e4m3(synth.u8(x["q8"][rsel]), x["q_scale"][rsel].cpu().numpy())
    w = x["w"][rsel].cpu().numpy()
    k_i = oracle.dequant_e4m3(synth.u8(x["k8"]), x["k_scale"].cpu().numpy())
    qb = oracle.bf16_to_f32(synth.bf16_bits(x["q"][rsel]))
    kvb = oracle.bf16_to_f32(synth.bf16_bits(x["kv"]))
    t0 = time.perf_counter()
    res = oracle.forward(q_i, w, k_i, qb, kvb, rows, k, 512, sm)
    t = time.perf_counter() - t0
    work = lambda p: IDX_FLOP_PER_PAIR * (p + 1) + ATT_FLOP_PER_ENTRY * min(k, p + 1)
    w_sample = sum(work(int(p)) for p in rows)
    w_total = sum(work(p) for p in range(L))
    full_s = t * w_total / w_sample
    base = {"value": round(L / full_s, 3), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": (f"{len(rows)} of {L} query rows (first 64, 64 around position k-1, last 64, the rest "
                       f"uniform), {t:.1f} s, extrapolated to all rows by the per-row work model"),
            "sample_seconds": round(t, 2)}
    _, mag, absmag = oracle.indexer(q_i, w, k_i, rows, ld=L, with_mag=True)
    g_scores = pre["scores"][0, rsel, :L].cpu().numpy()
    par = _parity_summary(oracle, parity, g_scores, res["scores"][:, :L], mag, absmag, pre["idx"][0, rsel].cpu().numpy(),
                          res, pre["out"][0, rsel].float().cpu().numpy(), pre["lse"][0, rsel].cpu().numpy(), rows)
    par["workload"] = "prefill 32K, the stage calls' outputs on the cpu_baseline rows"
    return base, par


def cpu_baseline_decode(dec, k, sm):
    """The oracle's full decode path for a bounded number of sequences, and the parity summary of the GPU's
    decode stage outputs on them."""
    import numpy as np

    import oracle
    from sparse_attention_13_amd import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity
    y, S = dec["y"], dec["S"]
    nb = min(12, dec["B"])
    t_total = 0.0
    pos = np.array([S - 1], np.int64)
    acc = []
    for b in range(nb):
        q_i = oracle.dequant_e4m3(synth.u8(y["q8"][b:b + 1]), y["q_scale"][b:b + 1].cpu().numpy())
        k_i = oracle.dequant_e4m3(synth.u8(y["k8"][b]), y["k_scale"][b].cpu().numpy())
        qb = oracle.bf16_to_f32(synth.bf16_bits(y["q"][b:b + 1]))
        kvb = oracle.bf16_to_f32(synth.bf16_bits(y["kv"][b]))
        w = y["w"][b:b + 1].cpu().numpy()
        t0 = time.perf_counter()
        res = oracle.forward(q_i, w, k_i, qb, kvb, pos, k, 512, sm)
        t_total += time.perf_counter() - t0
        _, mag, absmag = oracle.indexer(q_i, w, k_i, pos, ld=S, with_mag=True)
        acc.append((dec["scores"][b:b + 1, :S].cpu().numpy(), res, mag, absmag, dec["idx"][b:b + 1].cpu().numpy(),
                    dec["out"][b:b + 1].float().cpu().numpy(), dec["lse"][b:b + 1].cpu().numpy()))
    base = {"value": round(nb / t_total, 4), "unit": "queries/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{nb} of {dec['B']} sequences, full path, {t_total:.1f} s"}
    cat = lambda i: np.concatenate([a[i] for a in acc])
    res = {key: np.concatenate([a[1][key] for a in acc]) for key in ("scores", "kth", "idx", "out", "lse")}
    par = _parity_summary(oracle, parity, cat(0), res["scores"], cat(2), cat(3), cat(4), res, cat(5), cat(6),
                          np.full(nb, S - 1, np.int64))
    par["workload"] = f"decode 64x131072, the decode stage calls' outputs for {nb} sequences"
    return base, par


if __name__ == "__main__":
    main()
