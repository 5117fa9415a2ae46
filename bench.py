#!/usr/bin/env python3
"""Benchmark of the Sparse-to-Dense (StD) decoding hot path on one MI355X.

Workload: the 140k-token long-video case -- 28 layers of Qwen2-VL-7B-shaped
attention (28 query heads, 4 KV heads, head_dim 128), bf16 KV cache of
140,000 visual + 2,048 text positions (~8.2 GB resident in HBM), top-K
K = 4,096 per (layer, KV head), draft length gamma = 6.  Inputs are seeded
synthetic tensors (no weights or video datasets are available), generated on
the GPU before timing.

One step = one request through the whole hot path:
  (a) prefill-time selection for all 28 layers (std_select_topk), then
  draft-verify cycles until 256 new tokens exist, each cycle being
  (b) gamma sparse draft steps x 28 layers (std_sparse_decode_attn),
  (c) one dense verify pass x 28 layers with gamma+1 queries
      (std_dense_verify_attn),
  (d) greedy acceptance (std_accept), which advances the device-resident
      cache length by n + 1; n_out is copied to pinned host memory without
      a wait and read one cycle later, so the host only counts tokens while
      the GPU runs the next cycle (no per-cycle host round trip).
The acceptance step sees synthetic draft tokens and logits (vocab 152,064)
in which each draft agrees with the dense argmax with probability
alpha = 0.95 (the pages report that top-K KV keeps the original prediction
for about 95% of tokens); the cycles' accepted counts come from the GPU.
Non-attention model work (projections, MLP, LM head) is outside the path.

value = new tokens per second of the whole request (selection included).
Also reported: dense-only decoding tokens/s (the same dense kernel with one
query per token, no selection), per-kernel HBM GB/s and % of 8 TB/s, and the
attention bytes per emitted token (measured, and projected per acceptance
rate against a dense decode step).

  python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_BF16 = 2.5e15         # MI355X dense bf16 MFMA, flop/s
COPY_BYTES = 1 << 30        # the counter calibration copy (bytes read = bytes written)
CPU_LAYERS = 4             # layers of the workload the CPU baseline samples
CPU_ROWS = 384             # text rows per sampled layer for the CPU selection
METRIC = "sparse/dense attn HBM GB/s (% of peak) + draft-verify tokens/sec @140k ctx"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--new-tokens", type=int, default=256)
    ap.add_argument("--alpha", type=float, default=0.95)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dense-tokens", type=int, default=8)
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the calls one by one instead of replaying captured phases")
    ap.add_argument("--sel-streams", type=int, default=2,
                    help="streams the per-layer selections are dealt over")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill text attention + selection measurement")
    ap.add_argument("--batch-seqs", type=int, default=4,
                    help="sequences in the batched decode-cycle measurement")
    ap.add_argument("--no-batch", action="store_true",
                    help="skip the batched sparse draft measurement")
    ap.add_argument("--no-prefill-lse", action="store_true",
                    help="skip the selection timing with a caller-supplied row LSE")
    ap.add_argument("--no-toy", action="store_true",
                    help="skip the end-to-end toy decoder measurement")
    ap.add_argument("--no-gamma-sweep", action="store_true",
                    help="skip the draft-length sweep (verify timed at gamma + 1 queries)")
    ap.add_argument("--sync-each-cycle", action="store_true",
                    help="read each cycle's n_out before launching the next (the blocking "
                         "loop, for comparison)")
    return ap.parse_args()


def say(msg):
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print(msg, file=sys.stderr, flush=True)


def attn_bytes_dense(cfg, length, n_q):
    e = 2
    return 2 * cfg.n_kv_heads * length * cfg.head_dim * e + 2 * n_q * cfg.n_q_heads * cfg.head_dim * e


def attn_bytes_sparse(cfg, length):
    e = 2
    keys = cfg.topk + length - cfg.vis_len
    return (2 * cfg.n_kv_heads * keys * cfg.head_dim * e + 4 * cfg.n_kv_heads * cfg.topk
            + 2 * cfg.n_q_heads * cfg.head_dim * e)


def prefill_flops(cfg):
    """Matrix-unit flops of the text rows' prefill attention per layer: QK^T
    and PV, 2 d flops per (row, visible key) each."""
    nt = cfg.n_text
    pairs = nt * cfg.text_start + nt * (nt + 1) // 2
    return 4 * cfg.head_dim * cfg.n_q_heads * pairs


def select_flops(cfg):
    d, hq, nt = cfg.head_dim, cfg.n_q_heads, cfg.n_text
    lse = nt * cfg.text_start + nt * (nt + 1) // 2
    return 2 * d * hq * (lse + nt * cfg.vis_len)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_draft_speculative_amd as sd
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    sd.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = synth.config("c4", extra=args.new_tokens + 8)
    L = args.layers
    G = cfg.gamma
    print(f"# generating {L} layers of c4 inputs (capacity {cfg.capacity})", file=sys.stderr,
          flush=True)
    layers = [synth.attention_layer(cfg, l, device="cuda") for l in range(L)]
    for lay in layers:
        lay.pop("planted")
    torch.cuda.synchronize()
    cpu_layers = [] if args.no_cpu_baseline else [
        {k_: t_.cpu() for k_, t_ in layers[l].items()} for l in range(min(CPU_LAYERS, L))]

    # ---------------------------------------------------------------- setup
    shape = sd.attn_shape(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim)
    k0 = layers[0]["k"]
    max_len = cfg.capacity
    ws_dense = torch.zeros(max(sd.std_dense_verify_workspace(shape, G + 1, k0, max_len), 256),
                           dtype=torch.uint8, device=dev)
    ws_sparse = torch.zeros(max(sd.std_sparse_decode_workspace(shape, k0, max_len, cfg.vis_start,
                                                              cfg.vis_len, cfg.topk), 256),
                            dtype=torch.uint8, device=dev)
    ws_sel = torch.zeros(max(sd.std_select_topk_workspace(shape, cfg.n_text, cfg.vis_start,
                                                         cfg.vis_len, cfg.topk, k0, cfg.ctx), 256),
                         dtype=torch.uint8, device=dev)
    idx = [torch.zeros(cfg.n_kv_heads, cfg.topk, dtype=torch.int32, device=dev) for _ in range(L)]
    out_sp = torch.empty(cfg.n_q_heads, cfg.head_dim, dtype=torch.bfloat16, device=dev)
    out_dv = torch.empty(G + 1, cfg.n_q_heads, cfg.head_dim, dtype=torch.bfloat16, device=dev)

    # Every call runs on one stream and reads the valid cache length from
    # the device scalar `seq` (the position of the pending token x_t), which
    # the acceptance step advances; so each phase is captured once as a HIP
    # graph and replayed every cycle (--no-graph launches the same calls
    # one by one instead).
    st = torch.cuda.Stream()
    seq = torch.zeros(1, dtype=torch.int32, device=dev)
    # Selection deals layers round-robin over --sel-streams streams (each
    # with its own workspace), so one layer's tail kernels (top-K runs one
    # workgroup per KV head) and the big kernels' last partial rounds
    # overlap the next layer's passes.
    nss = max(1, args.sel_streams)
    st_sel = [st] + [torch.cuda.Stream() for _ in range(nss - 1)]
    ws_sels = [ws_sel] + [torch.zeros_like(ws_sel) for _ in range(nss - 1)]
    sel_calls = [sd.prepare_select_topk(lay["q_text"], lay["k"], cfg.ctx, cfg.text_start,
                                        cfg.vis_start, cfg.vis_len, cfg.topk, idx[l],
                                        ws_sels[l % nss], stream=st_sel[l % nss])
                 for l, lay in enumerate(layers)]

    def select_all(calls=sel_calls):
        """The 28 selections, enqueued on st; the other streams join st
        before and after (their calls overwrite index lists that the previous
        request's draft steps read, and the draft steps read their output)."""
        fork = torch.cuda.Event()
        fork.record(st)
        for x in st_sel[1:]:
            x.wait_event(fork)
        for c in calls:
            c()
        for x in st_sel[1:]:
            join = torch.cuda.Event()
            join.record(x)
            st.wait_event(join)
    q_draft = [[lay["q_draft"][j].contiguous() for j in range(G)] for lay in layers]
    sp_calls = [[sd.prepare_sparse_decode_dlen(q_draft[l][j], lay["k"], lay["v"], cfg.vis_start,
                                               cfg.vis_len, idx[l], out_sp, ws_sparse, seq, 1 + j,
                                               max_len=max_len, stream=st)
                 for l, lay in enumerate(layers)] for j in range(G)]
    dv_calls = [sd.prepare_dense_verify_dlen(lay["q_verify"], lay["k"], lay["v"], out_dv,
                                             ws_dense, seq, G + 1, max_len=max_len, stream=st)
                for lay in layers]
    q_one = [lay["q_verify"][:1].contiguous() for lay in layers]
    out_one = torch.empty(1, cfg.n_q_heads, cfg.head_dim, dtype=torch.bfloat16, device=dev)
    dn_calls = [sd.prepare_dense_verify_dlen(q_one[l], lay["k"], lay["v"], out_one, ws_dense,
                                             seq, 1, max_len=max_len, stream=st)
                for l, lay in enumerate(layers)]

    vocab = 152064
    pool = []
    for s_ in range(16):
        draft, logits = synth.accept_case(G, vocab, args.alpha, seed=1000 + s_,
                                          dtype=torch.bfloat16)
        pool.append((draft.to(dev), logits.to(dev)))
    toks = torch.empty(G + 1, dtype=torch.int32, device=dev)
    n_out = torch.zeros(1, dtype=torch.int32, device=dev)
    acc_calls = [sd.prepare_accept(d_, lg, toks, n_out, seq_len=seq, stream=st)
                 for d_, lg in pool]

    def draft_phase():
        for j in range(G):
            for l in range(L):
                sp_calls[j][l]()

    def verify_phase():
        for c in dv_calls:
            c()

    def dense_token():
        for c in dn_calls:
            c()
        seq.add_(1)

    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        seq.fill_(cfg.ctx)
        draft_phase()                      # warm-up launches outside any capture
        verify_phase()
        dense_token()
        for c in acc_calls:
            c()
    torch.cuda.synchronize()
    # one plain device copy of COPY_BYTES: the calibration point for the
    # HBM byte counters (FETCH_SIZE / WRITE_SIZE) in a counter run
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    if args.no_graph:
        run_draft, run_verify, run_dense = draft_phase, verify_phase, dense_token
        run_accept = acc_calls
    else:
        def capture(fn):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                fn()
            return g
        g_draft, g_verify, g_dense = capture(draft_phase), capture(verify_phase), capture(dense_token)
        g_acc = [capture(c) for c in acc_calls]
        run_draft, run_verify, run_dense = g_draft.replay, g_verify.replay, g_dense.replay
        run_accept = [g.replay for g in g_acc]
        torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    nvtx = torch.cuda.nvtx

    # n_out of each cycle lands in pinned host memory by an asynchronous copy
    # on the bench stream; the host reads it one cycle late (after launching
    # the next cycle), so the GPU never waits for the host between cycles.
    # A cycle is launched only while the tokens it could add are certainly
    # still needed: known tokens + (cycles in flight) x (gamma + 1) < target,
    # so no cycle is ever wasted; the host waits only for the oldest cycle
    # in flight, and only once no further cycle is certainly needed.
    RING = 64
    n_host = torch.zeros(RING, dtype=torch.int32, pin_memory=True)

    def run_request(timing):
        """One request; returns (new tokens, cycles, phase times ms or None)."""
        e_sel = (ev(), ev())
        cyc_ev = []
        inflight = []                      # (ring slot, copy-done event)
        with torch.cuda.stream(st):
            # host-side ranges (roctx through torch.cuda.nvtx) for a marker trace
            nvtx.range_push("selection")
            e_sel[0].record()
            select_all()
            e_sel[1].record()
            nvtx.range_pop()
            seq.fill_(cfg.ctx)
            t = cfg.ctx
            produced = 1                   # the pending token x_t comes from prefill
            cycles = 0
            emitted = 0
            sp_bytes = dv_bytes = 0
            while produced < args.new_tokens or inflight:
                if (produced + len(inflight) * (G + 1) < args.new_tokens
                        and len(inflight) < RING):
                    es = (ev(), ev(), ev(), ev())
                    es[0].record()
                    nvtx.range_push("draft")
                    run_draft()
                    es[1].record()
                    nvtx.range_pop()
                    nvtx.range_push("verify")
                    run_verify()
                    es[2].record()
                    nvtx.range_pop()
                    nvtx.range_push("accept")
                    run_accept[cycles % len(run_accept)]()
                    es[3].record()
                    nvtx.range_pop()
                    cyc_ev.append(es)
                    slot = cycles % RING
                    n_host[slot:slot + 1].copy_(n_out, non_blocking=True)
                    done = torch.cuda.Event()
                    done.record(st)
                    inflight.append((slot, done))
                    cycles += 1
                    if not args.sync_each_cycle:
                        continue
                slot, done = inflight.pop(0)
                done.synchronize()
                n = int(n_host[slot])      # token count only; the device length is advanced
                sp_bytes += sum(L * attn_bytes_sparse(cfg, t + 1 + j) for j in range(G))
                dv_bytes += L * attn_bytes_dense(cfg, t + G + 1, G + 1)
                emitted += n
                produced += n
                t += n
        torch.cuda.synchronize()
        ph = None
        if timing:
            ph = {"select_ms": e_sel[0].elapsed_time(e_sel[1]),
                  "cycle_ms": [a.elapsed_time(d) for a, _, _, d in cyc_ev],
                  "gap_ms": [cyc_ev[i][3].elapsed_time(cyc_ev[i + 1][0])
                             for i in range(len(cyc_ev) - 1)],
                  "draft_ms": sum(a.elapsed_time(b) for a, b, _, _ in cyc_ev),
                  "verify_ms": sum(b.elapsed_time(c) for _, b, c, _ in cyc_ev),
                  "accept_ms": sum(c.elapsed_time(d) for _, _, c, d in cyc_ev),
                  "sparse_bytes": sp_bytes, "dense_bytes": dv_bytes, "emitted": emitted}
        return min(produced, args.new_tokens), cycles, ph

    say("# timing the requests")
    for _ in range(args.warmup):
        run_request(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    results = [run_request(True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    new_tok = sum(r[0] for r in results)
    cycles = sum(r[1] for r in results)
    cycle_ms = sorted(x for r in results for x in r[2]["cycle_ms"])
    gap_ms = sorted(x for r in results for x in r[2]["gap_ms"])
    ph = {k: sum(r[2][k] for r in results) for k in results[0][2]
          if k not in ("cycle_ms", "gap_ms")}

    # selection with the row normaliser (step 1) supplied by the caller, as
    # a prefill attention kernel returns it; the LSE itself is computed here
    # in fp32 torch, outside the timed region
    say(f"# requests done: {new_tok / wall:.1f} tokens/s; selection with a caller LSE")
    sel_prefill = None
    if not args.no_prefill_lse:
        lses = [prefill_lse(lay, cfg) for lay in layers]
        idx2 = [torch.zeros_like(t) for t in idx]
        sel2 = [sd.prepare_select_topk(lay["q_text"], lay["k"], cfg.ctx, cfg.text_start,
                                       cfg.vis_start, cfg.vis_len, cfg.topk, idx2[l],
                                       ws_sels[l % nss], lse=lses[l], stream=st_sel[l % nss])
                for l, lay in enumerate(layers)]
        torch.cuda.synchronize()               # the LSEs come from the current stream
        select_all(sel2)                       # warm-up
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        with torch.cuda.stream(st):
            e0.record()
            select_all(sel2)
            e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        same = sum(len(set(a.tolist()) & set(b.tolist()))
                   for x, y in zip(idx, idx2) for a, b in zip(x.cpu(), y.cpu()))
        sel_prefill = {"ms_per_layer": round(ms / L, 3), "ms_per_request": round(ms, 3),
                       "idx_overlap_with_full_selection": round(same / (L * cfg.n_kv_heads * cfg.topk), 6),
                       "note": "step 1 (row LSE) supplied by the caller, as the prefill's "
                               "attention returns it; steps 2-3 timed"}

    # Selection beside the prefill: the text rows' prefill attention returns
    # their normalisers (std_prefill_text_attn) and the selection takes
    # those instead of computing its first pass
    say("# prefill text attention, then selection on its normalisers")
    pf = None
    if not args.no_prefill:
        pf_ws = torch.zeros(max(sd.std_prefill_text_attn_workspace(shape, cfg.text_start,
                                                                   cfg.n_text), 256),
                            dtype=torch.uint8, device=dev)
        pf_out = torch.empty_like(layers[0]["q_text"])
        pf_lse = [torch.empty(cfg.n_q_heads, cfg.n_text, dtype=torch.float32, device=dev)
                  for _ in range(L)]
        pf_calls = [sd.prepare_prefill_text_attn(lay["q_text"], lay["k"], lay["v"], cfg.ctx,
                                                 cfg.text_start, pf_out, pf_lse[l], pf_ws,
                                                 stream=st)
                    for l, lay in enumerate(layers)]
        idx3 = [torch.zeros_like(t) for t in idx]
        sel3 = [sd.prepare_select_topk(lay["q_text"], lay["k"], cfg.ctx, cfg.text_start,
                                       cfg.vis_start, cfg.vis_len, cfg.topk, idx3[l],
                                       ws_sels[l % nss], lse=pf_lse[l], stream=st_sel[l % nss])
                for l, lay in enumerate(layers)]
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            for c in pf_calls:                 # warm-up
                c()
            select_all(sel3)
        torch.cuda.synchronize()
        e0, e1, e2 = ev(), ev(), ev()
        with torch.cuda.stream(st):
            e0.record()
            for c in pf_calls:
                c()
            e1.record()
            select_all(sel3)
            e2.record()
        torch.cuda.synchronize()
        pf_ms, sel3_ms = e0.elapsed_time(e1) / L, e1.elapsed_time(e2) / L
        same = sum(len(set(a.tolist()) & set(b.tolist()))
                   for x, y in zip(idx, idx3) for a, b in zip(x.cpu(), y.cpu()))
        pf_flops = prefill_flops(cfg)
        pf = {"prefill_ms_per_layer": round(pf_ms, 3),
              "prefill_tflops": round(pf_flops / (pf_ms * 1e-3) / 1e12, 1),
              "prefill_frac_of_bf16_peak": round(pf_flops / (pf_ms * 1e-3) / PEAK_BF16, 4),
              "selection_ms_per_layer": round(sel3_ms, 3),
              "idx_overlap_with_full_selection": round(same / (L * cfg.n_kv_heads * cfg.topk),
                                                       6),
              "note": "std_prefill_text_attn (output + normalisers of the 2,048 text rows over "
                      "their causal keys, 28 layers), then the 28 selections fed those "
                      "normalisers"}

    say("# batched launches")
    batch_sparse = None if args.no_batch else batched_sparse(sd, cfg, layers[0], idx[0], st)
    batch_cycles = None if args.no_batch else batched_cycles(sd, cfg, layers, idx, st, pool,
                                                             args.batch_seqs)
    # the same batch with a draft length of its own per sequence
    mixed = [G - 2 * (b % 3) for b in range(args.batch_seqs)]
    batch_mixed = None if args.no_batch else batched_cycles(sd, cfg, layers, idx, st, pool,
                                                            args.batch_seqs, gammas=mixed)

    say("# dense-only decoding and the read probe")
    # dense-only decoding baseline: 28 dense n_q=1 calls per token
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    with torch.cuda.stream(st):
        seq.fill_(cfg.ctx)
        e0.record()
        for i in range(args.dense_tokens):
            run_dense()
        e1.record()
    torch.cuda.synchronize()
    dense_ms_per_tok = e0.elapsed_time(e1) / args.dense_tokens
    dense_gbps = L * attn_bytes_dense(cfg, cfg.ctx + 1, 1) / (dense_ms_per_tok * 1e-3) / 1e9

    n_sp_calls = cycles * G * L
    n_dv_calls = cycles * L
    sp_call_us = ph["draft_ms"] * 1e3 / n_sp_calls
    dv_call_us = ph["verify_ms"] * 1e3 / n_dv_calls
    sp_gbps = ph["sparse_bytes"] / (ph["draft_ms"] * 1e-3) / 1e9
    dv_gbps = ph["dense_bytes"] / (ph["verify_ms"] * 1e-3) / 1e9
    sel_ms_layer = ph["select_ms"] / (args.steps * L)
    sel_tflops = select_flops(cfg) / (sel_ms_layer * 1e-3) / 1e12

    probe = read_probe(sd, attn_bytes_dense(cfg, cfg.verify_len, G + 1))
    acc_us = ph["accept_ms"] * 1e3 / max(cycles, 1)
    gsweep = None
    if not args.no_gamma_sweep:
        say("# draft-length sweep")
        gsweep = gamma_sweep(sd, cfg, layers, st, sp_call_us, acc_us, dense_ms_per_tok)

    def hbm_roof(gbps, bytes_per_launch):
        return {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(gbps * 1e9 / PEAK_HBM, 4),
                "traffic": None, "bytes_per_launch": int(bytes_per_launch),
                "frac_of_attainable": round(gbps / probe["gbps"], 4)}

    dense_roof = hbm_roof(dv_gbps, attn_bytes_dense(cfg, cfg.verify_len, G + 1))
    dense_roof.update(kernel="dense verify (std_dense_verify_attn)",
                      us_per_launch=round(dv_call_us, 2))
    sparse_roof = hbm_roof(sp_gbps, attn_bytes_sparse(cfg, cfg.ctx + 1))
    sparse_roof.update(kernel="sparse draft (std_sparse_decode_attn)",
                       us_per_launch=round(sp_call_us, 2))
    sel_roof = {"bound": "mfma", "achieved": round(sel_tflops, 1), "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s", "frac": round(sel_tflops * 1e12 / PEAK_BF16, 4),
                "traffic": None, "kernel": "selection (std_select_topk)",
                "ms_per_layer": round(sel_ms_layer, 3)}
    # acceptance: (gamma + 1) bf16 logit rows of the vocabulary read per call,
    # one call per cycle (argmax per row + commit); latency-bound at this size
    acc_bytes = (G + 1) * vocab * 2
    acc_roof = {"bound": "hbm", "achieved": round(acc_bytes / (acc_us * 1e-6) / 1e9, 1),
                "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": round(acc_bytes / (acc_us * 1e-6) / PEAK_HBM, 4), "traffic": None,
                "kernel": "acceptance (std_accept)", "bytes_per_launch": acc_bytes,
                "us_per_launch": round(acc_us, 2)}
    phases = {"select": ph["select_ms"], "draft": ph["draft_ms"], "verify": ph["verify_ms"]}
    # The roofline object is the dense verify kernel: the single kernel with
    # the largest share of GPU time in the request (the kernel trace under
    # profiles/ ranks them) and the metric's own HBM-bound kernel.  Its
    # measured HBM traffic comes from the committed counter summary while
    # the kernel source it was taken on is unchanged.
    dense_roof["traffic"] = recorded_traffic()
    sparse_roof["traffic"] = recorded_traffic("sparse_traffic_bytes_per_launch")
    dense_roof["kernel_only"] = recorded_kernel_times("dense")
    sparse_roof["kernel_only"] = recorded_kernel_times("sparse")
    roofline = dense_roof

    line = {
        "metric": METRIC,
        "value": round(new_tok / wall, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "c4 long-video decode: 28 layers, 28/4/128 GQA, 140,000 visual + "
                        "2,048 text positions, K=4096, gamma=6, 256 new tokens per request, "
                        f"synthetic acceptance alpha={args.alpha}",
            "layers": L, "ctx": cfg.ctx, "topk": cfg.topk, "gamma": G,
            "new_tokens": args.new_tokens, "parallelism": "single GPU",
        },
        "roofline": roofline,
        "dense_attn": dense_roof,
        "sparse_attn": sparse_roof,
        "selection": sel_roof,
        "accept": acc_roof,
        "phases_ms_per_step": {k: round(v / args.steps, 3) for k, v in
                               {**phases, "accept": ph["accept_ms"]}.items()},
        "accepted_tokens_per_cycle": round(ph["emitted"] / max(cycles, 1), 3),
        "attn_mb_per_emitted_token": round((ph["sparse_bytes"] + ph["dense_bytes"])
                                           / max(ph["emitted"], 1) / 1e6, 1),
        "dense_only_tokens_per_s": round(1e3 / dense_ms_per_tok, 2),
        # emitted tokens over the event-timed decode cycles alone: the selection
        # (once per request, at prefill) and the host gaps between cycles are out
        "decode_tokens_per_s": round(ph["emitted"] / (sum(cycle_ms) * 1e-3), 2),
        "decode_speedup_vs_dense_only": round(ph["emitted"] / (sum(cycle_ms) * 1e-3)
                                              * dense_ms_per_tok / 1e3, 3),
        "dense_only_attn_gbps": round(dense_gbps, 1),
        "cycle_ms": cycle_stats(cycle_ms),
        "inter_cycle_gap_ms": cycle_stats(gap_ms),
        "host_read_per_cycle": "blocking" if args.sync_each_cycle else
                               "asynchronous, one cycle late",
        "selection_prefill_lse": sel_prefill,
        "prefill_then_selection": pf,
        "batched_sparse": batch_sparse,
        "batched_decode": batch_cycles,
        "batched_decode_per_sequence_gamma": batch_mixed,
        "hbm_read_probe": probe,
        "gamma_sweep": gsweep,
        "projection": projection(cycle_ms, G, dense_ms_per_tok,
                                 L * attn_bytes_sparse(cfg, cfg.ctx + 1),
                                 L * attn_bytes_dense(cfg, cfg.verify_len, G + 1),
                                 L * attn_bytes_dense(cfg, cfg.ctx + 1, 1)),
    }
    if not args.no_toy:
        say("# toy decoder end to end")
        line["toy_e2e"] = toy_e2e()
    if not args.no_cpu_baseline:
        say("# oracle on the host (bounded sample)")
        line["cpu_baseline"] = cpu_baseline(cfg, cpu_layers, args, cycles / args.steps)
    print(json.dumps(line), flush=True)


def read_probe(sd, nbytes, regions=4, reps=40):
    """Attainable HBM read bandwidth: std_hbm_read_probe (a plain streaming
    read, one workgroup per CU) over `regions` distinct buffers of the dense
    verify call's size, launched round-robin so that together they exceed
    the 256 MB last-level cache and no launch is served from it."""
    import torch
    nbytes = int(nbytes) // 16384 * 16384
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(regions)]
    sink = torch.empty(65536, dtype=torch.int32, device="cuda")
    for b in bufs:
        sd.std_hbm_read_probe(b, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        sd.std_hbm_read_probe(bufs[r % regions], sink)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    gbps = nbytes / (us * 1e-6) / 1e9
    del bufs
    torch.cuda.empty_cache()
    return {"gbps": round(gbps, 1), "us_per_launch": round(us, 2), "bytes_per_launch": nbytes,
            "frac_of_peak": round(gbps * 1e9 / PEAK_HBM, 4),
            "note": "plain streaming read, 256 workgroups x 256 lanes, 16 KB tiles, "
                    f"{regions} buffers round-robin"}


def batched_sparse(sd, cfg, lay, idx, st, batches=(1, 4, 16, 24), reps=20, llc_bytes=256e6):
    """Sparse draft attention and dense verify attention of one c4 layer for
    B independent sequences, one launch each (std_sparse_decode_attn_batch,
    std_dense_verify_attn_batch; B copies of the layer's cache and index
    list at distinct addresses), each sequence at ctx + 1 keys for the draft
    step and ctx + gamma + 1 for the verify pass: HBM GB/s against B x the
    single-sequence algorithmic bytes.

    A draft launch reads B x 12.66 MB, less than the 256 MB last-level cache
    for small B, while the decode loop's draft step (28 layers) reads more
    than it; so consecutive launches rotate over enough distinct copies of
    the B sequences that together they hold at least twice that cache, and
    no launch finds its rows there."""
    import math
    import torch
    G = cfg.gamma
    sp_bytes = int(attn_bytes_sparse(cfg, cfg.ctx + 1))
    dv_bytes = int(attn_bytes_dense(cfg, cfg.verify_len, G + 1))
    out = {"layer_bytes_per_sequence": sp_bytes, "verify_bytes_per_sequence": dv_bytes}

    def timed(calls):
        for c in calls[:3]:
            c()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(st):
            e0.record()
            for r in range(reps):
                calls[(r + 3) % len(calls)]()
            e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    shape = sd.attn_shape(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim)
    for B in batches:
        sets = max(2, math.ceil(2 * llc_bytes / (B * sp_bytes)))
        rep = lambda t: t[None].expand(sets * B, *t.shape).contiguous()   # noqa: E731
        k, v = rep(lay["k"]), rep(lay["v"])
        q, qv, ib = rep(lay["q_draft"][0]), rep(lay["q_verify"]), rep(idx)
        o = torch.empty_like(q[:B])
        ov = torch.empty_like(qv[:B])
        ws = torch.zeros(max(sd.std_sparse_decode_batch_workspace(shape, B, k[:B], cfg.ctx + 1,
                                                                  cfg.vis_start, cfg.vis_len,
                                                                  cfg.topk), 256),
                         dtype=torch.uint8, device=q.device)
        wsv = torch.zeros(max(sd.std_dense_verify_batch_workspace(shape, G + 1, B, k[:B],
                                                                  cfg.verify_len), 256),
                          dtype=torch.uint8, device=q.device)
        part = [slice(i * B, (i + 1) * B) for i in range(sets)]
        # the copies above ran on the current stream, the calls run on st
        torch.cuda.synchronize()
        us = timed([lambda p=p: sd.std_sparse_decode_attn_batch(
            q[p], k[p], v[p], cfg.ctx + 1, cfg.vis_start, cfg.vis_len, ib[p], out=o,
            workspace=ws, stream=st) for p in part])
        usv = timed([lambda p=p: sd.std_dense_verify_attn_batch(
            qv[p], k[p], v[p], cfg.verify_len, out=ov, workspace=wsv, stream=st) for p in part])
        gbps = B * sp_bytes / (us * 1e-6) / 1e9
        gbpsv = B * dv_bytes / (usv * 1e-6) / 1e9
        out[f"batch{B}"] = {"us_per_launch": round(us, 2), "achieved_gbps": round(gbps, 1),
                            "frac": round(gbps * 1e9 / PEAK_HBM, 4),
                            "verify_us_per_launch": round(usv, 2),
                            "verify_gbps": round(gbpsv, 1),
                            "verify_frac": round(gbpsv * 1e9 / PEAK_HBM, 4),
                            "copies_rotated": sets}
        del k, v, q, qv, ib, o, ov, ws, wsv
        torch.cuda.empty_cache()
    return out


def batched_cycles(sd, cfg, layers, idx, st, pool, B, cycles=24, gammas=None):
    """Decode cycles for B sequences through the batched calls: per cycle
    gamma x 28 batched draft launches, 28 batched verify launches and one
    batched acceptance, captured as three graphs and replayed; every
    sequence keeps its own device length, advanced by its own n + 1.  The
    sequences are copies of the 28 c4 layers (distinct addresses), so the
    bytes moved are B times a single sequence's.  ``gammas`` (one per
    sequence, each <= gamma) gives every sequence its own draft length:
    draft step j runs only the sequences with j < gamma_b, the verify pass
    takes 1 + gamma queries and each acceptance reads its own rows."""
    import torch
    G, L = cfg.gamma, len(layers)
    dev = layers[0]["k"].device
    rep = lambda t: t[None].expand(B, *t.shape).contiguous()   # noqa: E731
    kb = [rep(lay["k"]) for lay in layers]
    vb = [rep(lay["v"]) for lay in layers]
    qd = [[rep(lay["q_draft"][j]) for j in range(G)] for lay in layers]
    qv = [rep(lay["q_verify"]) for lay in layers]
    ib = [rep(t) for t in idx]
    cap = cfg.capacity
    shape = sd.attn_shape(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim)
    ws_s = torch.zeros(max(sd.std_sparse_decode_batch_workspace(shape, B, kb[0], cap,
                                                                cfg.vis_start, cfg.vis_len,
                                                                cfg.topk), 256),
                       dtype=torch.uint8, device=dev)
    ws_d = torch.zeros(max(sd.std_dense_verify_batch_workspace(shape, G + 1, B, kb[0], cap), 256),
                       dtype=torch.uint8, device=dev)
    o_s = torch.empty_like(qd[0][0])
    o_d = torch.empty_like(qv[0])
    seq = torch.full((B,), cfg.ctx, dtype=torch.int32, device=dev)
    draft = torch.stack([pool[b % len(pool)][0] for b in range(B)]).contiguous()
    logits = torch.stack([pool[b % len(pool)][1] for b in range(B)]).contiguous()
    toks = torch.empty(B, G + 1, dtype=torch.int32, device=dev)
    n_out = torch.zeros(B, dtype=torch.int32, device=dev)
    total = torch.zeros(B, dtype=torch.int32, device=dev)
    gdev = None if gammas is None else torch.tensor(gammas, dtype=torch.int32, device=dev)
    G_run = G if gammas is None else max(gammas)
    torch.cuda.synchronize()

    def draft_phase():
        for j in range(G_run):
            for l in range(L):
                sd.std_sparse_decode_attn_batch(qd[l][j], kb[l], vb[l], cap, cfg.vis_start,
                                                cfg.vis_len, ib[l], len_dev=seq, len_offset=1 + j,
                                                gamma_dev=gdev, step=j, out=o_s, workspace=ws_s,
                                                stream=st)

    def verify_phase():
        for l in range(L):
            sd.std_dense_verify_attn_batch(qv[l], kb[l], vb[l], cap, len_dev=seq,
                                           len_offset=G + 1, out=o_d, workspace=ws_d, stream=st)

    def accept():
        sd.std_accept_batch(draft, logits, out_tokens=toks, n_out=n_out, seq_len=seq,
                            gamma_dev=gdev, stream=st)
        total.add_(n_out)

    with torch.cuda.stream(st):
        draft_phase()
        verify_phase()
        accept()
    torch.cuda.synchronize()
    graphs = []
    for fn in (draft_phase, verify_phase, accept):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            fn()
        graphs.append(g)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(st):
        seq.fill_(cfg.ctx)
        total.zero_()
        e0.record()
        for _ in range(cycles):
            for g in graphs:
                g.replay()
        e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    emitted = int(total.sum().item())
    out = {"sequences": B, "cycles": cycles, "ms_per_cycle": round(ms / cycles, 4),
           "gammas": list(gammas) if gammas is not None else [G] * B,
           "tokens_emitted": emitted,
           "decode_tokens_per_s": round(emitted / (ms * 1e-3), 1),
           "note": "28 c4 layers per sequence, gamma draft steps + verify + acceptance per "
                   "cycle for all B sequences, selection not included"}
    del kb, vb, qd, qv, ib, ws_s, ws_d, graphs
    torch.cuda.empty_cache()
    return out


def prefill_lse(lay, cfg):
    """Natural-log LSE of every text row over the keys it sees (the prompt
    up to its own position), in fp32 torch: the value a prefill attention
    kernel returns with its output."""
    import torch
    q, k = lay["q_text"].float(), lay["k"].float()
    hq, n_text, d = q.shape
    G = hq // k.shape[0]
    n_keys = cfg.text_start + n_text
    keypos = torch.arange(n_keys, device=q.device)[:, None]
    rowpos = cfg.text_start + torch.arange(n_text, device=q.device)[None, :]
    out = torch.empty(hq, n_text, dtype=torch.float32, device=q.device)
    for h in range(hq):
        s = (k[h // G, :n_keys] @ q[h].T) * (1.0 / math.sqrt(d))
        s.masked_fill_(keypos > rowpos, float("-inf"))
        out[h] = torch.logsumexp(s, dim=0)
        del s
    return out


def cycle_stats(ms):
    """Median, p10 and p90 of the per-cycle times (draft + verify + accept)."""
    if not ms:
        return None
    q = lambda f: ms[min(len(ms) - 1, int(f * (len(ms) - 1) + 0.5))]  # noqa: E731
    return {"cycles": len(ms), "median": round(q(0.5), 4), "p10": round(q(0.1), 4),
            "p90": round(q(0.9), 4)}


def projection(cycle_ms, gamma, dense_ms_per_tok, step_bytes, verify_bytes, dense_tok_bytes):
    """Attention-only decode rate projected from the measured median cycle
    time: E(alpha) = (1 - alpha^(gamma+1)) / (1 - alpha) tokens per cycle
    under independent per-token acceptance, for alpha in {0.8, 0.9, 0.95},
    against dense-only decoding (selection not included).

    Beside it, the attention I/O per emitted token (the pages' I/O argument:
    drafting reads only the kept KV, so once acceptance is high a token
    costs fewer bytes than a dense decode step; technical summary, Main
    contributions).  The pages print no formula; the reading used here is a
    cycle's algorithmic bytes, gamma draft steps (step_bytes each, all
    layers) plus one verify pass (verify_bytes), over E(alpha), against
    dense_tok_bytes for one dense decode step."""
    t = cycle_ms[len(cycle_ms) // 2]
    cycle_bytes = gamma * step_bytes + verify_bytes
    out = {"label": "attention-only, projected", "t_cycle_ms": round(t, 4),
           "dense_only_tokens_per_s": round(1e3 / dense_ms_per_tok, 2),
           "dense_mb_per_token": round(dense_tok_bytes / 1e6, 1),
           "cycle_mb": round(cycle_bytes / 1e6, 1)}
    for a in (0.8, 0.9, 0.95):
        e = (1 - a ** (gamma + 1)) / (1 - a)
        out[f"alpha_{a}"] = {"tokens_per_cycle": round(e, 3),
                             "tokens_per_s": round(e * 1e3 / t, 1),
                             "speedup_vs_dense": round(e * dense_ms_per_tok / t, 3),
                             "mb_per_token": round(cycle_bytes / e / 1e6, 1),
                             "io_reduction_vs_dense": round(dense_tok_bytes * e / cycle_bytes, 3)}
    return out


def gamma_sweep(sd, cfg, layers, st, sp_call_us, acc_us, dense_ms_per_tok,
                gammas=(2, 4, 6, 8, 9, 10, 12, 14, 16), reps=5):
    """Draft length against the projected attention-only decode rate (the
    pages' ablation finds the speed-up rising with gamma up to about 9,
    technical summary, Experimental results).  For each gamma the verify
    pass is timed: 28 dense calls with gamma + 1 queries at ctx + gamma + 1
    keys (graph-replayed on the bench stream).  A cycle is then gamma draft
    steps at the measured per-call draft time (its list grows by one entry
    per step, which the call time does not see), that verify pass and one
    acceptance at the measured call time (latency-bound: its (gamma + 1)
    logit rows change it little).  Tokens per cycle under independent
    acceptance, E = (1 - alpha^(gamma+1)) / (1 - alpha), over the cycle time
    gives the rate for alpha in {0.8, 0.9, 0.95}; selection is not included."""
    import torch
    L = len(layers)
    dev = layers[0]["k"].device
    shape = sd.attn_shape(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim)
    cap = cfg.capacity
    nq_max = max(gammas) + 1
    if cfg.ctx + nq_max > cap:
        raise ValueError("cache capacity too small for the sweep")
    ws = torch.zeros(max(sd.std_dense_verify_workspace(shape, nq_max, layers[0]["k"], cap), 256),
                     dtype=torch.uint8, device=dev)
    seq = torch.full((1,), cfg.ctx, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    draft_step_ms = sp_call_us * L / 1e3
    rows, best = [], {}
    for g in gammas:
        nq = g + 1
        qs = [torch.randn(nq, cfg.n_q_heads, cfg.head_dim, device=dev, generator=gen)
              .to(torch.bfloat16) for _ in range(L)]
        out = torch.empty(nq, cfg.n_q_heads, cfg.head_dim, dtype=torch.bfloat16, device=dev)
        calls = [sd.prepare_dense_verify_dlen(qs[l], lay["k"], lay["v"], out, ws, seq, nq,
                                              max_len=cap, stream=st)
                 for l, lay in enumerate(layers)]
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            for c in calls:                    # warm-up outside the capture
                c()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=st):
            for c in calls:
                c()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(st):
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
        torch.cuda.synchronize()
        verify_ms = e0.elapsed_time(e1) / reps
        call_us = verify_ms * 1e3 / L
        vbytes = attn_bytes_dense(cfg, cfg.ctx + nq, nq)
        t = g * draft_step_ms + verify_ms + acc_us / 1e3
        row = {"gamma": g, "verify_us_per_call": round(call_us, 2),
               "verify_frac": round(vbytes / (call_us * 1e-6) / PEAK_HBM, 4),
               "cycle_ms": round(t, 4)}
        for a in (0.8, 0.9, 0.95):
            e = (1 - a ** (g + 1)) / (1 - a)
            row[f"alpha_{a}"] = {"tokens_per_s": round(e * 1e3 / t, 1),
                                 "speedup_vs_dense": round(e * dense_ms_per_tok / t, 3)}
            if a not in best or e / t > best[a][1]:
                best[a] = (g, e / t)
        rows.append(row)
        del graph, calls, qs, out
    del ws
    torch.cuda.empty_cache()
    return {"label": "attention-only, projected from measured calls",
            "draft_step_ms": round(draft_step_ms, 4), "accept_ms": round(acc_us / 1e3, 4),
            "rows": rows,
            "best_gamma": {f"alpha_{a}": best[a][0] for a in (0.8, 0.9, 0.95)}}


def toy_e2e(n_new=256, gammas=(2, 4, 6), seed=0):
    """Draft-verify decoding of a random-init toy decoder, measured end to end.

    Decoder: 4 layers, hidden 512, 8 query / 2 KV heads of 64, SwiGLU MLP
    1,536, vocab 8,192, bf16 weights N(0, 0.02^2) and cache; prompt = 8,192
    synthetic visual embeddings (5% carry a planted direction) + 128 random
    text ids; K = 512.  Every attention runs on the library; the rest of the
    model is torch.  Tokens/s counts tokens 2..n_new (token 1 comes from the
    prefill); selection is part of the prefill and timed separately.
    """
    import torch
    import synth
    from sparse_draft_speculative_amd.toy_decoder import ToyDecoder

    cfg = dict(synth.TOY_C5)
    params = synth.toy_params(cfg, seed=seed, std=0.02)
    vis, text = synth.toy_prompt(cfg, seed=seed)
    n_vis = cfg["n_vis"]
    prompt_len = n_vis + cfg["n_text"]
    dec = ToyDecoder(params, prompt_len + n_new + max(gammas) + 2, dtype=torch.bfloat16)
    first, q_text = dec.prefill(vis, text)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    idx = dec.select(q_text, prompt_len, 0, n_vis, cfg["topk"])
    torch.cuda.synchronize()
    sel_ms = (time.perf_counter() - t0) * 1e3
    snap = dec.snapshot()

    def timed(fn):
        dec.restore(snap)
        fn()                                   # warm-up pass
        dec.restore(snap)
        torch.cuda.synchronize()
        t = time.perf_counter()
        res = fn()
        torch.cuda.synchronize()
        return res, time.perf_counter() - t

    dense, t_dense = timed(lambda: dec.decode_dense(first, prompt_len, n_new))
    out = {"workload": "toy decoder 4x512, 8/2/64 GQA, MLP 1536, vocab 8192, bf16, "
                       f"prompt {n_vis} visual + {cfg['n_text']} text, K={cfg['topk']}, "
                       f"{n_new} new tokens, weights N(0, 0.02^2)",
           "selection_ms": round(sel_ms, 3),
           "dense_only_tokens_per_s": round((n_new - 1) / t_dense, 2), "std": {}}
    def run(sel, g):
        (toks, acc), t_std = timed(lambda: dec.decode_std(first, prompt_len, n_new, sel, 0,
                                                           n_vis, g))
        return {
            "tokens_per_s": round((n_new - 1) / t_std, 2),
            "speedup_vs_dense": round(t_dense / t_std, 3),
            "accepted_tokens_per_dense_step": round(float(np.mean([a + 1 for a in acc])), 3),
            "alpha_hat": round(float(np.mean(acc)) / g, 4),
            "cycles": len(acc),
            "stream_equals_dense": toks == dense,
        }

    for g in gammas:
        out["std"][f"gamma{g}"] = run(idx, g)
    # Comparator: the same draft kernel over the streaming lists
    # (std_static_window_idx: the first STREAM_SINK visual positions and the
    # last topk - STREAM_SINK) in place of the attention-ranked top-K (sizes
    # are this harness's choice; the pages give none).
    topk = cfg["topk"]
    static = dec.select_static(0, n_vis, STREAM_SINK, topk)
    out["static_window"] = {"sink": STREAM_SINK, "window": topk - STREAM_SINK,
                            "std": {f"gamma{g}": run(static, g) for g in gammas}}
    return out


STREAM_SINK = 64          # visual positions kept from the start in the static-set comparator

TRAFFIC_SUMMARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "traffic_attention_c4.md")
TRACE_SUMMARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                             "kernel_trace_c4_request.md")
KERNEL_SOURCES = ["attention.hip", "tile.hpp", "common.hpp", "internal.hpp"]


def kernel_source_digest():
    """sha256 over the dense verify kernel's sources with comments and
    whitespace removed (counter values taken on other code do not describe
    this kernel; an edited comment does not change it)."""
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "sparse_draft_speculative_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(base, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def recorded_kernel_times(prefix):
    """Kernel-only times of one attention call (main kernel, combine) in us
    from the committed kernel-trace summary, or None when it is missing or
    was taken on different kernel sources."""
    try:
        text = open(TRACE_SUMMARY).read()
    except OSError:
        return None
    vals = dict(re.findall(r"^- (\w+): (\S+)$", text, flags=re.M))
    if vals.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return {"main_kernel_us": float(vals[f"{prefix}_main_kernel_us"]),
                "combine_us": float(vals[f"{prefix}_combine_us"]),
                "source": "rocprofv3 kernel trace (profiles/kernel_trace_c4_request.md)"}
    except (KeyError, ValueError):
        return None


def recorded_traffic(key="traffic_bytes_per_launch"):
    """HBM bytes per launch of a kernel from the committed FETCH_SIZE /
    WRITE_SIZE summary (copy-calibrated): ``traffic_bytes_per_launch`` for
    the dense verify call, ``sparse_traffic_bytes_per_launch`` for the
    sparse draft call (main kernel + combine).  None when that summary is
    missing or was taken on different kernel sources."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    vals = dict(re.findall(r"^- (\w+): (\S+)$", text, flags=re.M))
    if vals.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return int(vals[key])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, cpu_layers, args, cycles_per_request):
    """The float64 oracle on the host, on a bounded sample of the workload.

    Sample: for each of the first CPU_LAYERS layers, one dense verify pass
    (7 queries x 28 heads over 142k keys), gamma sparse draft steps and the
    selection scores of one KV head over CPU_ROWS text rows; plus one
    acceptance.  Per-request CPU time is extrapolated to 28 layers x
    (selection scaled to 4 heads x 2,048 rows + cycles x (draft + verify)) +
    cycles x accept.
    """
    import oracle
    import synth

    G = cfg.gamma
    gpg = cfg.n_q_heads // cfg.n_kv_heads
    rows = CPU_ROWS
    # a valid index set for the sparse steps: every (vis_len // K)-th visual
    # position (the planted runs are not needed for timing)
    idx = np.tile(np.arange(cfg.topk) * (cfg.vis_len // cfg.topk), (cfg.n_kv_heads, 1))
    t_verify = t_draft = t_sel = 0.0
    for lay in cpu_layers:
        k = lay["k"].double().numpy()
        v = lay["v"].double().numpy()
        qv = lay["q_verify"].double().numpy()
        qd = lay["q_draft"].double().numpy()
        qt = lay["q_text"].double().numpy()
        t0 = time.perf_counter()
        oracle.dense_verify(qv, k, v, cfg.verify_len)
        t_verify += time.perf_counter() - t0
        t0 = time.perf_counter()
        for j in range(G):
            oracle.sparse_decode(qd[j], k, v, cfg.draft_len(j), cfg.vis_start, cfg.vis_len, idx)
        t_draft += time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.selection_scores(qt[:gpg, :rows], k[:1], cfg.text_start, cfg.vis_start,
                                cfg.vis_len)
        t_sel += time.perf_counter() - t0
    n = len(cpu_layers)
    draft, logits = synth.accept_case(G, 152064, args.alpha, seed=1000)
    t0 = time.perf_counter()
    oracle.accept(draft.numpy(), logits.double().numpy())
    t_accept = time.perf_counter() - t0
    sel_layer = (t_sel / n) * cfg.n_kv_heads * (cfg.n_text / rows)
    per_req = (cfg.n_layers * (sel_layer + cycles_per_request * (t_draft + t_verify) / n)
               + cycles_per_request * t_accept)
    try:
        from threadpoolctl import threadpool_info
        threads = max(p["num_threads"] for p in threadpool_info()) or 1
    except Exception:
        threads = os.cpu_count()
    return {
        "value": round(args.new_tokens / per_req, 4), "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"layers 0-{n - 1} of the workload: dense verify (7x28 rows, 142k keys) "
                   f"{t_verify:.2f}s, {G} sparse steps per layer {t_draft:.2f}s, selection of "
                   f"1 KV head x {rows} text rows per layer {t_sel:.2f}s, one acceptance "
                   f"{t_accept:.3f}s; extrapolated to 28 layers x {cycles_per_request:.1f} "
                   f"cycles/request + full selection (4 KV heads x {cfg.n_text} rows)"),
        "sample_seconds": round(t_verify + t_draft + t_accept + t_sel, 2),
    }


if __name__ == "__main__":
    main()
