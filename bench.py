#!/usr/bin/env python3
"""Benchmark of the W12 tree-verification pass on one MI355X.

Workload: the 27B-like dense target (64 layers, hidden 5120, GQA 40/8 x 128,
SwiGLU 17408, vocab 151936, random-init W12 weights), committed context 4096,
32-node best-first draft trees whose tokens come from the target's own top-4
(p = 0.7), one ``verify_step`` per step (forward over all nodes, LM-head
argmax, acceptance walk, KV commit) plus the readback of the accepted length.

Prints one JSON line: verify steps/s (``value``), tokens/s, the achieved HBM
GB/s of the whole step (also as a fraction of a streaming-read probe run on
the same GPU), the roofline entry of the dominant kernel (the fused
gate/up W12 GEMM and the launch that finishes its K-sliced remaining
groups, timed together with HIP events on their stream) and the CPU
oracle's rate on a bounded sample.
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

METRIC = "W12 tree-verify steps/s + achieved HBM GB/s (27B-like, 32-node tree), 1 GPU"
HBM_PEAK_GBS = 8000.0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# HBM traffic of the gate/up launch measured with rocprofv3 --pmc (FETCH_SIZE,
# WRITE_SIZE), recorded with a hash of the kernel's sources: the figure is
# reported only while the sources are unchanged.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "w12_skinny_gateup_27b_pmc.md")
KERNEL_SOURCES = ["tree_verification_pass_amd/csrc/w12_gemm.hip", "tree_verification_pass_amd/csrc/common.h",
                  "tree_verification_pass_amd/csrc/internal.h", "include/tvp.h"]


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(alg_bytes: int):
    """Bytes per launch from the committed counter summary, if it was taken on
    the current sources and on this launch (the same algorithmic bytes, i.e.
    the same weight shape and rows); else None."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    if fields.get("algorithmic_bytes_per_launch") != str(int(alg_bytes)):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def w12_algorithmic_bytes(n_out: int, k_in: int, n_esc: int) -> int:
    """Bytes of the canonical W12 format: planes, base, escape pointers, 4 per escape."""
    return n_out * k_in + n_out * ((k_in + 1) // 2) + n_out + 4 * (n_out + 1) + 4 * n_esc


def build_model(cfg, seed: int, s_max: int, max_nodes: int, kv_fn=None, with_hi8: bool = False):
    import torch

    from synth.configs import gen_embed, gen_final_norm, gen_kv_context, gen_layer, gen_lm_head
    from tree_verification_pass_amd.model import DeviceModel, Dims

    dev = torch.device("cuda:0")

    def layer_fn(layer):
        if layer % 8 == 0:
            log(f"bench: converting layer {layer}/{cfg.n_layers} to W12")
        return gen_layer(cfg, seed, layer, device=dev, gains="ones")

    if kv_fn is None:
        def kv_fn(layer):
            return gen_kv_context(cfg, seed, layer, cfg.ctx_len, s_max, device=dev)

    t0 = time.perf_counter()
    dm = DeviceModel(Dims.of(cfg), gen_embed(cfg, seed, dev), gen_final_norm(cfg, seed, dev),
                     gen_lm_head(cfg, seed, dev), layer_fn, kv_fn, s_max=s_max, max_nodes=max_nodes,
                     with_hi8=with_hi8)
    torch.cuda.synchronize()
    log(f"bench: model ready in {time.perf_counter() - t0:.1f} s")
    return dm


def make_trees(dm, cfg, n_trees: int, seed: int):
    import torch

    import tree_verification_pass_amd as tvp
    from synth import best_first_topology
    from synth.trees import assign_tokens_by_depth

    rng = np.random.default_rng(seed)
    dev = torch.device("cuda:0")
    trees = []
    for _ in range(n_trees):
        parents, rank, _ = best_first_topology(rng, cfg.n_nodes)
        root = int(rng.integers(cfg.vocab))

        def topk_fn(tokens, par):
            r = tvp.verify_step(dm.plan, cfg.ctx_len, torch.as_tensor(tokens, device=dev),
                                torch.as_tensor(par, device=dev), commit=False, want_logits=True)
            return torch.topk(r.logits, 4, dim=1).indices.cpu().numpy()

        tokens = assign_tokens_by_depth(rng, parents, rank, root, cfg.vocab, topk_fn, p_top=0.7)
        trees.append((torch.as_tensor(tokens.astype(np.int32), device=dev),
                      torch.as_tensor(parents.astype(np.int32), device=dev)))
    return trees


def step_bytes(dm, cfg, mean_accepted: float, n: int = 0) -> float:
    """Algorithmic HBM bytes of one step over n nodes (default: the config's
    tree size): W12 stream + KV + embedding rows + commit."""
    n = n or cfg.n_nodes
    L, hkv, d = cfg.ctx_len, cfg.n_kv_heads, cfg.head_dim
    w = 0
    for p in [dm.lm_head] + [x for Lr in dm.layers for x in (Lr.wqkv, Lr.wo, Lr.wgu, Lr.wdown)]:
        w += w12_algorithmic_bytes(p.n_out, p.k_in, int(p.desc.n_esc))
    per_layer_kv = 2 * (L + n) * hkv * d * 2 + 2 * n * hkv * d * 2
    commit = cfg.n_layers * 2 * 2 * mean_accepted * hkv * d * 2
    return float(w + cfg.n_layers * per_layer_kv + n * cfg.hidden * 2 + commit)


def time_gateup(dm, cfg, iters: int):
    """Dominant kernel: the fused gate/up W12 GEMM, rotated over the 64 layers'
    distinct weights (no cache reuse), timed with HIP events on its stream."""
    import torch

    import tree_verification_pass_amd as tvp

    dev = torch.device("cuda:0")
    n, H, F = cfg.n_nodes, cfg.hidden, cfg.ffn
    x = torch.randn(n, H, device=dev).to(torch.bfloat16)
    # the launch configuration of the verification pass: packed activations in and out
    xp = tvp.w12_pack_x(x)
    u = torch.empty(tvp.w12_packed_x_elems(F), dtype=torch.bfloat16, device=dev)
    # arrival counters of the remaining groups' K slices, zero and left at
    # zero by every call, as the pass holds them (no clearing launch)
    cnt = torch.zeros(tvp.TVP_GEMM_COUNTERS, dtype=torch.int32, device=dev)
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=u.data_ptr(), y_packed=1, counters=cnt.data_ptr())
    layers = dm.layers
    for i in range(len(layers)):
        tvp.w12_gemm_px(xp, n, layers[i].wgu, epi)
    torch.cuda.synchronize()
    # the library launches on torch's current stream, where these events are
    # recorded: one pair around each launch, so the figure is the kernel's own
    # duration (the launch gaps between back-to-back calls are not counted)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record()
        tvp.w12_gemm_px(xp, n, layers[i % len(layers)].wgu, epi)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = sum(s.elapsed_time(e) for s, e in ev) / iters
    p = layers[0].wgu
    nbytes = (sum(w12_algorithmic_bytes(L.wgu.n_out, L.wgu.k_in, int(L.wgu.desc.n_esc)) for L in layers)
              / len(layers) + n * H * 2 + n * F * 2)
    return ms, nbytes, p


def time_gateup_rows(dm, cfg, m: int, iters: int):
    """The fused gate/up W12 GEMM at m rows in row-major layout (the batched
    pass's wide kernel and its fix-up), rotated over the layers' distinct
    weights, timed with HIP events around each launch on its stream."""
    import torch

    import tree_verification_pass_amd as tvp

    dev = torch.device("cuda:0")
    H, F = cfg.hidden, cfg.ffn
    x = torch.randn(m, H, device=dev).to(torch.bfloat16)
    u = torch.empty(m, F, dtype=torch.bfloat16, device=dev)
    epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_SWIGLU, y=u.data_ptr(), ldy=F)
    layers = dm.layers
    for i in range(len(layers)):
        tvp.w12_gemm_ex(x, layers[i].wgu, epi)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record()
        tvp.w12_gemm_ex(x, layers[i % len(layers)].wgu, epi)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / iters
    nbytes = (sum(w12_algorithmic_bytes(L.wgu.n_out, L.wgu.k_in, int(L.wgu.desc.n_esc)) for L in layers)
              / len(layers) + m * H * 2 + m * F * 2)
    return ms, nbytes


def read_probe_gbs(gib: int = 4, iters: int = 5) -> float:
    """Sustained HBM read rate of a plain sequential stream on this GPU
    (``tvp_read_probe`` over ``gib`` GiB, past the memory-side cache)."""
    import torch

    import tree_verification_pass_amd as tvp

    dev = torch.device("cuda:0")
    src = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    tvp.tvp_read_probe(src, sink)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        tvp.tvp_read_probe(src, sink)
    e.record()
    torch.cuda.synchronize()
    rate = iters * src.numel() / (s.elapsed_time(e) * 1e-3) / 1e9
    del src
    torch.cuda.empty_cache()
    return rate


def cpu_baseline(dm, cfg, seed: int, tree, n_sample: int = 4):
    """The oracle (untuned) on ``n_sample`` of the decoder layers of one step:
    W12 decode of each layer's four weights plus the layer's forward over the
    nodes; the step estimate scales that by total / sampled streamed weights.
    The first sampled layer is also timed on one thread."""
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import model as om
    from oracle import w12 as ow12
    from oracle.bf16 import from_bits
    from synth.configs import gen_layer
    from synth.weights import bf16_bits_numpy

    dev = torch.device("cuda:0")
    tokens, parents = (t.cpu().numpy() for t in tree)
    h_bits = bf16_bits_numpy(dm.embed[torch.as_tensor(tokens.astype(np.int64), device=dev)])
    dims = om.Dims.of(cfg)
    n_sample = max(1, min(n_sample, cfg.n_layers))

    def layer_inputs(li):  # weight generation and W12 encoding are not timed
        layer = gen_layer(cfg, seed, li, device=dev, gains="ones")
        bits = {k: bf16_bits_numpy(v) for k, v in layer.items()}
        del layer
        enc = {k: (ow12.encode(v) if k in ("wqkv", "wo", "wgu", "wdown") else v) for k, v in bits.items()}
        kc = bf16_bits_numpy(dm.layers[li].k_cache[:, : cfg.ctx_len])
        vc = bf16_bits_numpy(dm.layers[li].v_cache[:, : cfg.ctx_len])
        return enc, bits["attn_norm"][:1], kc, vc

    def one_layer(enc, norm, kc, vc) -> float:
        t0 = time.perf_counter()
        model = om.OracleModel.from_w12(dims, np.zeros((1, cfg.hidden), np.uint16), [enc], norm, None)
        h = from_bits(h_bits)
        pos = cfg.ctx_len + om._accept.depths(parents)
        om.layer_forward(model, 0, h, pos, from_bits(kc), from_bits(vc), om.ancestor_mask(parents))
        return time.perf_counter() - t0

    t_sample, t_one = 0.0, 0.0
    for li in range(n_sample):
        inp = layer_inputs(li)
        t_sample += one_layer(*inp)
        if li == 0:
            with threadpool_limits(limits=1):
                t_one = one_layer(*inp)
        del inp
    w_layer = sum(a * b for a, b in cfg.linear_shapes().values())
    scale = cfg.streamed_params() / (w_layer * n_sample)
    est, est_1 = t_sample * scale, t_one * scale * n_sample
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": 1.0 / est, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{n_sample} of {cfg.n_layers} decoder layers of one {len(tokens)}-node verify step (W12 "
                       f"decode of their weights + fp64 forward, ctx {cfg.ctx_len}): {t_sample:.2f} s, scaled by "
                       f"streamed weights ({scale:.2f}x) to a whole step of {est:.1f} s"),
            "one_thread": {"value": 1.0 / est_1, "unit": "steps/s", "cores": 1,
                           "sample": (f"the first sampled layer on 1 thread: {t_one:.2f} s, a whole step of "
                                      f"{est_1:.1f} s")}}


# once-per-pass kernels, by the name they carry in a trace
SMALL_ROLES = (("argmax_finalize_kernel", "LM-head argmax finalize"), ("tree_prep_kernel", "tree preparation"),
               ("rope_table_kernel", "RoPE table"), ("embed_kernel", "embedding"),
               ("accept_kernel", "acceptance walk"), ("kv_commit_kernel", "KV commit"))


def pass_roles(trace_csv: str) -> dict:
    """Durations (us) of the pass's launches by role, from a rocprofv3 kernel
    trace: the library's dispatches in start order, each named by its kernel
    and, where one kernel serves two roles, by the launch before it (the O
    projection follows tree attention, the down projection the gate/up
    GEMM; each residual + RMSNorm is named for the projection it follows).
    Gate/up launches outside the pass (bench.py's own timing leg) follow
    another gate/up launch and are left out."""
    import csv
    import re

    rows = []
    for r in csv.DictReader(open(trace_csv)):
        if "tvp::" in r["Kernel_Name"]:
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()

    def kind(name):
        m = re.search(r"w12_skinny_kernel<\d+, \d+, \d+, (\d+)(?:, \d+)?>", name)
        if m:
            return {"3": "gateup", "4": "qkv", "5": "lmhead", "16": "partial"}.get(m.group(1), "gemm")
        for key, lab in (("wide_fixup", "wfix"), ("w12_wide_kernel", "wide"),
                         ("tree_attn_kernel", "attn"), ("resid_norm", "norm")):
            if key in name:
                return lab
        for key, lab in SMALL_ROLES:
            if key in name:
                return lab
        return "other"

    kinds = [kind(r[2]) for r in rows]
    out = {}
    role_of = []
    for i, k in enumerate(kinds):
        prev = role_of[i - 1] if i else None
        role = None
        if k == "qkv":
            role = "QKV GEMM + RoPE + KV write"
        elif k == "attn":
            role = "tree attention"
        elif k == "partial":
            role = {"tree attention": "O GEMM (K slices)", "gate/up GEMM": "down GEMM (K slices)"}.get(prev)
        elif k == "norm":
            role = {"O GEMM (K slices)": "residual + norm after O", "wide O GEMM (split sums)": "residual + norm after O",
                    "down GEMM (K slices)": "residual + norm after down",
                    "wide down GEMM (split sums)": "residual + norm after down"}.get(prev, "norm (first or final)")
        elif k == "gateup":
            role = "gate/up GEMM" if prev == "residual + norm after O" else None
        elif k == "lmhead":
            role = "LM head + argmax"
        elif k == "wide":  # more than 32 rows: named by the launch before it
            role = {"norm (first or final)": "wide QKV GEMM", "residual + norm after down": "wide QKV GEMM",
                    "tree attention": "wide O GEMM (split sums)",
                    "residual + norm after O": "wide gate/up GEMM",
                    "wide gate/up fix-up (SwiGLU)": "wide down GEMM (split sums)"}.get(prev)
            if role == "wide QKV GEMM" and i + 2 < len(kinds) and kinds[i + 2] == "LM-head argmax finalize":
                role = "wide LM head"
        elif k == "wfix":
            role = {"wide QKV GEMM": "wide QKV fix-up (RoPE, KV write)", "wide gate/up GEMM": "wide gate/up fix-up (SwiGLU)",
                    "wide LM head": "wide LM-head fix-up (argmax keys)"}.get(prev)
        elif k != "other":
            role = k
        role_of.append(role)
        if role:
            out.setdefault(role, []).append((rows[i][1] - rows[i][0]) / 1e3)
    order = ["QKV GEMM + RoPE + KV write", "wide QKV GEMM", "wide QKV fix-up (RoPE, KV write)", "tree attention",
             "O GEMM (K slices)", "wide O GEMM (split sums)", "residual + norm after O",
             "gate/up GEMM", "wide gate/up GEMM", "wide gate/up fix-up (SwiGLU)",
             "down GEMM (K slices)", "wide down GEMM (split sums)", "residual + norm after down",
             "norm (first or final)", "LM head + argmax", "wide LM head", "wide LM-head fix-up (argmax keys)"] + \
        [r for _, r in SMALL_ROLES]
    return {r: out[r] for r in order if r in out}


def rocprof_summary(out_dir: str, top: int = 24) -> None:
    """Prints the short text summary of a rocprofv3 csv output folder: the
    per-kernel duration table of ``--kernel-trace --stats`` runs and, for
    ``--pmc`` runs, each kernel's counters summed over their instances and
    averaged over its dispatches."""
    import csv
    import glob
    from collections import defaultdict

    for path in sorted(glob.glob(os.path.join(out_dir, "**", "*_kernel_stats.csv"), recursive=True)):
        rows = list(csv.DictReader(open(path)))
        print(f"kernel stats ({os.path.basename(path)}): calls, total us, avg us, min us, max us, %, name")
        for r in rows[:top]:
            print(f"{int(r['Calls']):7d} {float(r['TotalDurationNs']) / 1e3:12.1f} {float(r['AverageNs']) / 1e3:9.2f} "
                  f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}  "
                  f"{r['Name'][:110]}")
    for path in sorted(glob.glob(os.path.join(out_dir, "**", "*_kernel_trace.csv"), recursive=True)):
        roles = pass_roles(path)
        if roles:
            print(f"per-role durations inside the pass ({os.path.basename(path)}): role, dispatches, mean us, "
                  f"median us")
            for role, vals in roles.items():
                vals.sort()
                print(f"  {role:28s} {len(vals):7d} {sum(vals) / len(vals):9.2f} {vals[len(vals) // 2]:9.2f}")
    for path in sorted(glob.glob(os.path.join(out_dir, "**", "*_counter_collection.csv"), recursive=True)):
        per = defaultdict(float)
        names = {}
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"], r["Counter_Name"], r["Dispatch_Id"])
            per[key] += float(r["Counter_Value"])
            names[key[:2]] = r["Grid_Size"]
        agg = defaultdict(list)
        for (kn, cn, _), v in per.items():
            agg[(kn, cn)].append(v)
        print(f"counters ({os.path.basename(path)}): dispatches, mean per dispatch, min, max, counter, kernel")
        for (kn, cn), vals in sorted(agg.items(), key=lambda kv: -sum(kv[1]))[:top]:
            print(f"{len(vals):7d} {sum(vals) / len(vals):14.1f} {min(vals):14.1f} {max(vals):14.1f}  {cn}  {kn[:100]}")


def bench_ar(args, cfg, dm) -> int:
    """Greedy autoregressive decoding with the same pass on a one-node tree:
    each step feeds the previous bonus token back as the root (the step's one
    readback), at a fixed committed length, and emits one token."""
    import torch

    import tree_verification_pass_amd as tvp

    dev = torch.device("cuda:0")
    out = tvp._alloc_out(dm.plan, 1, 1, False)
    parents = torch.full((1,), -1, dtype=torch.int32, device=dev)
    tok = torch.full((1,), 11, dtype=torch.int32, device=dev)

    enq = []  # host time to enqueue a step's launches

    def step():
        ta = time.perf_counter()
        tvp.verify_step(dm.plan, cfg.ctx_len, tok, parents, commit=True, out=out)
        enq.append(time.perf_counter() - ta)
        tok.fill_(int(out.bonus.item()))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} greedy decode steps")
    enq.clear()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    gbs = step_bytes(dm, cfg, 0.0, n=1) / (ms * 1e-3) / 1e9
    enq_ms = float(np.mean(enq)) * 1000.0
    log(f"bench: {ms:.3f} ms/token, {1000.0 / ms:.1f} tokens/s, {gbs:.0f} GB/s, host enqueue {enq_ms:.2f} ms/step")
    line = {
        "metric": "W12 greedy AR decode tokens/s (27B-like, one node per pass), 1 GPU",
        "value": round(1000.0 / ms, 3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "achieved_hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "host_enqueue_ms_per_step": round(enq_ms, 4),
        "config": {"workload": f"{cfg.name}-like greedy decode, ctx {cfg.ctx_len}", "n_layers": cfg.n_layers,
                   "hidden": cfg.hidden, "nodes": 1, "ctx_len": cfg.ctx_len},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_tlv(args, cfg) -> int:
    """Two-level verification on the 27B-like target: the Q pass (the 32-node
    draft tree through the 8-bit leading views of the weights), the exact
    pass alone, and whole TLV steps (Q pass, readback of its path and bonus,
    a re-drafted subtree attached, one exact 32-node pass with commit) at a
    fixed committed length.  Reports the Q pass's cost as a fraction of an
    exact step, the bytes each pass streams, and the Q pass's top-1 agreement
    with the exact pass on the same trees.  The synthetic drafter for the
    subtree draws best-first trees with uniform tokens (random weights admit
    no meaningful drafter)."""
    import torch

    import tree_verification_pass_amd as tvp
    from synth import best_first_topology
    from tree_verification_pass_amd.tlv import tlv_step

    s_max = cfg.ctx_len + 64
    dm = build_model(cfg, args.seed, s_max, cfg.n_nodes, with_hi8=True)
    trees = make_trees(dm, cfg, args.trees, args.seed + 1)
    dev = torch.device("cuda:0")
    out_q = tvp._alloc_out(dm.q_plan, cfg.n_nodes, 1, False)
    out_e = tvp._alloc_out(dm.plan, cfg.n_nodes, 1, False)

    def timed(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1000.0 / n

    def q_pass(i):
        tokens, parents = trees[i % len(trees)]
        tvp.verify_step(dm.q_plan, cfg.ctx_len, tokens, parents, commit=False, out=out_q)
        int(out_q.n_accepted.item())

    def exact_pass(i):
        tokens, parents = trees[i % len(trees)]
        tvp.verify_step(dm.plan, cfg.ctx_len, tokens, parents, commit=False, out=out_e)
        int(out_e.n_accepted.item())

    rng = np.random.default_rng(args.seed + 7)

    def redraft(q_path, q_bonus):
        sp = best_first_topology(rng, cfg.n_nodes - len(q_path))[0]
        st = rng.integers(0, cfg.vocab, len(sp))
        st[0] = q_bonus
        return sp, st

    accepted = []

    def tlv(i):
        tokens, parents = trees[i % len(trees)]
        r = tlv_step(dm, cfg.ctx_len, tokens, parents, redraft, commit=True)
        accepted.append(int(r.exact.n_accepted.item()))

    agree = []
    for i in range(len(trees)):
        q_pass(i)
        exact_pass(i)
        agree.append((out_q.argmax == out_e.argmax).float().mean().item())
    for fn in (q_pass, exact_pass, tlv):
        timed(fn, args.warmup)
    accepted.clear()
    log(f"bench: timing {args.steps} Q passes, exact passes and TLV steps")
    ms_q = timed(q_pass, args.steps)
    ms_e = timed(exact_pass, args.steps)
    ms_t = timed(tlv, args.steps)
    q_bytes = dm.stream_bytes(hi8=True)
    e_bytes = dm.stream_bytes()
    log(f"bench: Q pass {ms_q:.3f} ms, exact pass {ms_e:.3f} ms (Q / exact = {ms_q / ms_e:.3f}), TLV step "
        f"{ms_t:.3f} ms; packed weights streamed: {q_bytes / 1e9:.2f} GB (8-bit views) vs {e_bytes / 1e9:.2f} GB")
    line = {
        "metric": "W12 two-level verification: Q-pass cost / exact step, TLV steps/s (27B-like, 32-node tree), 1 GPU",
        "value": round(ms_q / ms_e, 4), "unit": "Q-pass ms / exact-pass ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "ms_q_pass": round(ms_q, 4), "ms_exact_pass": round(ms_e, 4), "ms_tlv_step": round(ms_t, 4),
        "tlv_steps_per_s": round(1000.0 / ms_t, 3), "mean_accepted_tlv": round(float(np.mean(accepted)), 3),
        "q_exact_top1_agreement": round(float(np.mean(agree)), 4),
        "packed_bytes_hi8": int(q_bytes), "packed_bytes_w12": int(e_bytes),
        "config": {"workload": f"{cfg.name}-like TLV step, {cfg.n_nodes}-node trees, ctx {cfg.ctx_len}",
                   "drafter": "draft trees from the target's top-4 (p = 0.7); re-drafted subtrees uniform"},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_batched(args, cfg) -> int:
    """Batched verification: 24 requests share a 192-node budget (per-request
    trees of 4-16 nodes, best-first topology, drafts from the target's own
    top-4 at p = 0.7), each over its own committed context (uniform in
    [512, 8192]) in its own KV region; one ``verify_step_batched`` per step
    (every GEMM over all 192 rows, attention, acceptance and commit per
    request) plus the readback of the accepted lengths."""
    import torch

    import tree_verification_pass_amd as tvp
    from synth import best_first_topology
    from synth.configs import gen_kv_context
    from synth.trees import assign_tokens_by_depth, batch_sizes

    dev = torch.device("cuda:0")
    n_req, total, cap, ctx_lo, ctx_hi = 24, 192, 16, 512, 8192
    rng = np.random.default_rng(args.seed + 2)
    sizes = batch_sizes(rng, n_req=n_req, total=total, start=4, cap=cap)
    ctxs = rng.integers(ctx_lo, ctx_hi + 1, n_req)
    s_req = ctx_hi + cap
    s_max = n_req * s_req
    hkv, d = cfg.n_kv_heads, cfg.head_dim

    def kv_fn(layer):  # request r's committed context in slots [r * s_req, r * s_req + ctx_r)
        kc = torch.zeros(hkv, s_max, d, dtype=torch.bfloat16, device=dev)
        vc = torch.zeros_like(kc)
        for r in range(n_req):
            k_r, v_r = gen_kv_context(cfg, args.seed * 1000 + r, layer, int(ctxs[r]), int(ctxs[r]), device=dev)
            kc[:, r * s_req: r * s_req + ctxs[r]] = k_r
            vc[:, r * s_req: r * s_req + ctxs[r]] = v_r
        return kc, vc

    dm = build_model(cfg, args.seed, s_max, total, kv_fn=kv_fn)
    node_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    log("bench: drafting the batch's trees from the target's top-4")
    batches = []
    for _ in range(2):
        trees = [best_first_topology(rng, int(sizes[r])) for r in range(n_req)]
        toks = np.zeros(total, np.int32)
        par = np.concatenate([t[0] for t in trees]).astype(np.int32)
        P = torch.as_tensor(par, device=dev)
        for r in range(n_req):
            sl = slice(node_ptr[r], node_ptr[r + 1])

            def topk_fn(tokens, parents, sl=sl):  # the other requests do not affect request r
                toks[sl] = tokens
                res = tvp.verify_step_batched(dm.plan, ctxs.tolist(), node_ptr.tolist(), s_req,
                                              torch.as_tensor(toks, device=dev), P, commit=False,
                                              want_logits=True)
                return torch.topk(res.logits[sl], 4, dim=1).indices.cpu().numpy()

            toks[sl] = assign_tokens_by_depth(rng, trees[r][0], trees[r][1], int(rng.integers(cfg.vocab)),
                                              cfg.vocab, topk_fn, p_top=0.7)
        batches.append((torch.as_tensor(toks.copy(), device=dev), P))
    out = tvp._alloc_out(dm.plan, total, n_req, False)

    def step(i):
        T, P = batches[i % len(batches)]
        tvp.verify_step_batched(dm.plan, ctxs.tolist(), node_ptr.tolist(), s_req, T, P, commit=True, out=out)
        return out.n_accepted.cpu().numpy()  # the step's one device-to-host readback

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} batched steps")
    acc = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        acc.append(step(i))
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    acc = np.asarray(acc, dtype=np.float64)
    emitted = float(np.mean(acc.sum(axis=1) + n_req))  # accepted + one bonus per request
    w = sum(w12_algorithmic_bytes(p.n_out, p.k_in, int(p.desc.n_esc))
            for p in [dm.lm_head] + [x for Lr in dm.layers for x in (Lr.wqkv, Lr.wo, Lr.wgu, Lr.wdown)])
    kv_read = sum(2 * (int(ctxs[r]) + int(sizes[r])) * hkv * d * 2 for r in range(n_req))
    kv_write = 2 * total * hkv * d * 2
    commit = 2 * 2 * float(np.mean(acc.sum(axis=1))) * hkv * d * 2
    nbytes = w + cfg.n_layers * (kv_read + kv_write + commit) + total * cfg.hidden * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"bench: {ms:.3f} ms/step, {1000.0 / ms:.2f} steps/s, {emitted * 1000.0 / ms:.0f} tokens/s, {gbs:.0f} GB/s")
    g_ms, g_bytes = time_gateup_rows(dm, cfg, total, max(args.gemm_iters, 2 * cfg.n_layers))
    g_gbs = g_bytes / (g_ms * 1e-3) / 1e9
    log(f"bench: gate/up W12 GEMM at {total} rows {g_ms * 1000.0:.1f} us/launch, {g_gbs:.0f} GB/s")
    line = {
        "metric": "W12 batched tree-verify steps/s (27B-like, 24 requests sharing a 192-node budget), 1 GPU",
        "value": round(1000.0 / ms, 3), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "tokens_per_s": round(emitted * 1000.0 / ms, 2), "mean_emitted_per_step": round(emitted, 2),
        "achieved_hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": int(nbytes),
        "roofline": {"kernel": (f"w12_wide_kernel + w12_wide_fixup_kernel (fused gate/up SwiGLU, "
                                f"{2 * cfg.ffn}x{cfg.hidden}, {total} rows)"),
                     "bound": "hbm", "achieved": round(g_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(g_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "us_per_launch": round(g_ms * 1000.0, 2), "bytes_per_launch": int(g_bytes),
                     "note": (f"{2 * total * 2 * cfg.ffn * cfg.hidden / g_bytes:.0f} flop per byte: the bf16 MFMA "
                              f"bound ({2 * total * 2 * cfg.ffn * cfg.hidden / 2.5e15 * 1e6:.1f} us) is below the "
                              f"HBM bound ({g_bytes / 8e12 * 1e6:.1f} us)")},
        "config": {"workload": (f"{cfg.name}-like batched verify step, {n_req} requests, {total} nodes "
                                f"(trees of {int(sizes.min())}-{int(sizes.max())}), ctx {int(ctxs.min())}-"
                                f"{int(ctxs.max())} (mean {float(ctxs.mean()):.0f})"),
                   "n_layers": cfg.n_layers, "hidden": cfg.hidden, "nodes": total, "requests": n_req},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_cost_curve(args, cfg, dm) -> int:
    """Verify cost against tree size: T(N) for best-first trees of N = 1, 8,
    16, 32 nodes over the same context (random draft tokens; the pass does
    the same work whatever is accepted), and c(N) = T(N) / T(1), where the
    one-node pass is one step of greedy decoding."""
    import torch

    import tree_verification_pass_amd as tvp
    from synth import best_first_topology

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(args.seed + 3)
    times = {}
    for n in (1, 8, 16, 32):
        parents = best_first_topology(rng, n)[0] if n > 1 else np.asarray([-1])
        tokens = rng.integers(0, cfg.vocab, n)
        T = torch.as_tensor(np.asarray(tokens, np.int32), device=dev)
        P = torch.as_tensor(np.asarray(parents, np.int32), device=dev)
        out = tvp._alloc_out(dm.plan, n, 1, False)
        for _ in range(args.warmup):
            tvp.verify_step(dm.plan, cfg.ctx_len, T, P, commit=True, out=out)
            int(out.n_accepted.item())
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            tvp.verify_step(dm.plan, cfg.ctx_len, T, P, commit=True, out=out)
            int(out.n_accepted.item())  # each step's one readback
        torch.cuda.synchronize()
        times[n] = (time.perf_counter() - t0) * 1000.0 / args.steps
        log(f"bench: N = {n:2d}: {times[n]:.3f} ms/step, c(N) = {times[n] / times[1]:.3f}")
    line = {
        "metric": "W12 verify cost curve c(N) = T(N)/T(1) (27B-like), 1 GPU",
        "value": round(times[32] / times[1], 4), "unit": "c(32)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
        "ms_per_step": {str(n): round(t, 4) for n, t in times.items()},
        "c": {str(n): round(t / times[1], 4) for n, t in times.items()},
        "config": {"workload": f"{cfg.name}-like verify step, best-first trees of 1-32 nodes, ctx {cfg.ctx_len}"},
    }
    print(json.dumps(line), flush=True)
    return 0


# Standalone W12 GEMM shapes of the 27B-like target, (n_out, k_in): the
# weights [5120 x 17408], [17408 x 5120] and [5120 x 6144] read as K_in x N_out.
GEMM_SHAPES = ((17408, 5120), (5120, 17408), (6144, 5120))
GEMM_ROWS = (1, 16, 32)


def bench_gemm(args) -> int:
    """The standalone skinny W12 GEMM at the 27B-like shapes, M in {1, 16, 32}:
    Y = X W^T, X bf16 N(0,1) in the GEMM's packed activation layout, Y bf16.
    Per shape, distinct encoded copies totalling at least 512 MB (twice the
    256 MB memory-side cache) are cycled, so every launch streams its weights
    from HBM; each launch is timed with HIP events on the stream it runs on
    (the median over the timed launches is reported)."""
    import torch

    import tree_verification_pass_amd as tvp
    from synth import gen_linear_bf16, make_generator
    from synth.configs import LARGE_RECIPE
    from synth.weights import bf16_bits_numpy, sub_seed

    dev = torch.device("cuda:0")
    probe = read_probe_gbs()
    cases = []
    cpu = None
    for si, (n_out, k_in) in enumerate(GEMM_SHAPES):
        per_copy = n_out * k_in * 1.55
        n_copies = max(4, int(np.ceil(512e6 / per_copy)))
        log(f"bench: gemm {n_out}x{k_in}: encoding {n_copies} copies")
        copies, alg = [], []
        for c in range(n_copies):
            w = gen_linear_bf16(make_generator(sub_seed(args.seed, 90, si, c), dev), n_out, k_in, LARGE_RECIPE,
                                device=dev)
            t = tvp.w12_encode(w)
            alg.append(w12_algorithmic_bytes(n_out, k_in, t.n_esc))
            copies.append(tvp.w12_pack(t))
            if c == 0 and si == 0 and not args.no_cpu_baseline:
                cpu = gemm_cpu_baseline(bf16_bits_numpy(w))
            del t, w
        torch.cuda.synchronize()
        for m in GEMM_ROWS:
            x = torch.randn(m, k_in, generator=make_generator(sub_seed(args.seed, 91, m))).to(torch.bfloat16).to(dev)
            xp = tvp.w12_pack_x(x)
            y = torch.empty(m, n_out, dtype=torch.bfloat16, device=dev)
            cnt = torch.zeros(tvp.TVP_GEMM_COUNTERS, dtype=torch.int32, device=dev)  # held zero, as in the pass
            epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_BF16, y=y.data_ptr(), ldy=n_out, counters=cnt.data_ptr())
            for c in range(n_copies):
                tvp.w12_gemm_px(xp, m, copies[c], epi)
            torch.cuda.synchronize()
            iters = max(args.gemm_iters, 4 * n_copies)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
            for i in range(iters):
                ev[i][0].record()
                tvp.w12_gemm_px(xp, m, copies[i % n_copies], epi)
                ev[i][1].record()
            torch.cuda.synchronize()
            us = float(np.median([s.elapsed_time(e) for s, e in ev])) * 1000.0
            nbytes = float(np.mean(alg)) + m * k_in * 2 + m * n_out * 2
            gbs = nbytes / (us * 1e-6) / 1e9
            cases.append({"n_out": n_out, "k_in": k_in, "m": m, "us_per_launch": round(us, 2),
                          "bytes_per_launch": int(nbytes), "achieved_gbs": round(gbs, 1),
                          "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "probe_frac": round(gbs / probe, 4),
                          "copies": n_copies})
            log(f"bench: gemm {n_out}x{k_in} m={m}: {us:.2f} us, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.3f} of 8 TB/s)")
        del copies
        torch.cuda.empty_cache()
    gm = float(np.exp(np.mean([np.log(c["achieved_gbs"]) for c in cases])))
    line = {
        "metric": "W12 skinny GEMM achieved HBM GB/s (27B-like shapes, M = 1/16/32), 1 GPU",
        "value": round(gm, 1), "unit": "GB/s (geometric mean over shapes and M)", "n_gpus": 1,
        "steps": max(args.gemm_iters, 1), "warmup": 1, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "read_probe_gbs": round(probe, 1),
        "config": {"workload": "standalone W12 GEMM, weights [5120x17408], [17408x5120], [5120x6144] (K_in x N_out), "
                               "M in {1,16,32}, X bf16 N(0,1), fp32 accumulation, bf16 out",
                   "weights": "per-channel sigma log-uniform [0.005,0.05], 1% zeros, 0.05% outliers x1000",
                   "rotation": ">= 512 MB of distinct encoded copies per shape"},
        "cases": cases,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_lmhead(args) -> int:
    """The 27B-like LM head (151936 x 5120) at 32 and 1 rows: the W12 head
    (skinny GEMM with the argmax epilogue, plus its finalize) against the
    INT8 head with the Cauchy-Schwarz certified candidate filter (norms,
    GEMM on the int8 tiles with the approximate-logit epilogue, threshold,
    candidate scan with exact rescoring from the canonical W12 rows, result).
    Each call is timed with HIP events on its stream (median of the timed
    calls); both return the exact greedy token of every row."""
    import torch

    import tree_verification_pass_amd as tvp
    from synth import gen_linear_bf16, make_generator
    from synth.configs import CONFIGS, LARGE_RECIPE
    from synth.weights import sub_seed

    cfg = CONFIGS["27b"]
    V, H = cfg.vocab, cfg.hidden
    dev = torch.device("cuda:0")
    w = gen_linear_bf16(make_generator(sub_seed(args.seed, 95), dev), V, H, LARGE_RECIPE, device=dev)
    exact = tvp.w12_encode(w)
    pw = tvp.w12_pack(exact)
    head = tvp.lmhead_i8_encode(w)
    del w
    torch.cuda.synchronize()
    rows = {}
    for m in (32, 1):
        x = torch.randn(m, H, generator=make_generator(sub_seed(args.seed, 96, m))).to(torch.bfloat16).to(dev)
        xp = tvp.w12_pack_x(x)
        am = torch.zeros(m, dtype=torch.int32, device=dev)
        epi = tvp.TvpGemmEpilogue(mode=tvp.TVP_EPI_ARGMAX, argmax=am.data_ptr())

        def w12_call():
            tvp.w12_gemm_px(xp, m, pw, epi)

        def i8_call():
            return tvp.lmhead_i8_argmax(xp, m, head, exact)

        res = {}
        for name, fn in (("w12", w12_call), ("i8", i8_call)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
            for s, e in ev:
                s.record()
                fn()
                e.record()
            torch.cuda.synchronize()
            res[name] = float(np.median([s.elapsed_time(e) for s, e in ev])) * 1000.0
        a8, nc, _ = i8_call()
        w12_call()
        torch.cuda.synchronize()
        rows[m] = {"us_w12_head": round(res["w12"], 1), "us_i8_head": round(res["i8"], 1),
                   "i8_over_w12": round(res["i8"] / res["w12"], 3),
                   "same_argmax_rows": int((a8 == am).sum().item()),
                   "candidates_mean": round(float(nc.float().mean().item()), 2), "candidates_max": int(nc.max().item())}
        log(f"bench: LM head m={m}: W12 {res['w12']:.1f} us, INT8 certified {res['i8']:.1f} us, "
            f"candidates mean {rows[m]['candidates_mean']}, same argmax on {rows[m]['same_argmax_rows']}/{m} rows")
    line = {
        "metric": "LM head (151936x5120) greedy token: W12 head vs INT8 head with certified candidate filter, 1 GPU",
        "value": rows[32]["us_i8_head"], "unit": "us per call (INT8 certified head, 32 rows)", "n_gpus": 1,
        "steps": 20, "warmup": 3, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "bytes_w12_head": int(pw.stream_bytes()), "bytes_i8_head": int(head.stream_bytes()),
        "rows": {str(k): v for k, v in rows.items()},
        "config": {"workload": "27B-like LM head, 151936 x 5120, large-recipe weights, X bf16 N(0,1)"},
    }
    print(json.dumps(line), flush=True)
    return 0


def gdn_bytes(n: int, hk: int, hv: int, dk: int, dv: int) -> int:
    """Algorithmic bytes of one Gated DeltaNet tree verify: the fp32 state
    once, q, k, v, g, beta of the n nodes once, the bf16 outputs once."""
    return hv * dv * dk * 4 + 2 * n * hk * dk * 2 + n * hv * dv * 2 + 2 * n * hv * 4 + n * hv * dv * 2


def bench_gdn(args) -> int:
    """The Gated DeltaNet layers of the 27B-hybrid-like stand-in (48
    recurrent layers of 8 key heads and 40 value heads x 128) over a 32-node
    best-first tree: per layer the WY-form verify and the path verify (one
    launch each per layer, every layer's own state and inputs, the 48
    launches captured in a HIP graph and replayed between two events), then
    one commit launch for all 48 layers along an accepted path of up to 4
    nodes (events around each launch, median).  The WY verify's achieved
    bytes (fp32 state, inputs and outputs once) are set against 8 TB/s."""
    import torch

    import tree_verification_pass_amd as tvp
    from synth import best_first_topology
    from synth.gdn import GDN_LAYERS_27B_HYBRID, GDN_SHAPES, gen_gdn_inputs

    shape = GDN_SHAPES["27b_hybrid"]
    L, n = GDN_LAYERS_27B_HYBRID, 32
    dev = torch.device("cuda:0")
    parents_np = np.asarray(best_first_topology(np.random.default_rng(args.seed + 5), n)[0], dtype=np.int32)
    parents = torch.as_tensor(parents_np, device=dev)
    inps = [gen_gdn_inputs(args.seed, l, n, shape) for l in range(L)]
    state = torch.stack([i.state for i in inps]).to(dev).contiguous()
    q = torch.stack([i.q for i in inps]).to(dev).contiguous()
    k = torch.stack([i.k for i in inps]).to(dev).contiguous()
    v = torch.stack([i.v for i in inps]).to(dev).contiguous()
    g = torch.stack([i.g for i in inps]).to(dev).contiguous()
    beta = torch.stack([i.beta for i in inps]).to(dev).contiguous()
    out = torch.empty(L, n, shape.hv, shape.dv, dtype=torch.bfloat16, device=dev)
    status = torch.zeros(L, dtype=torch.int32, device=dev)
    res = {}
    steps = max(args.steps // 10, 5)
    for name, fn in (("wy", tvp.gdn_tree_verify), ("path", tvp.gdn_path_verify)):
        def all_layers(fn=fn):
            for l in range(L):
                fn(q[l], k[l], v[l], g[l], beta[l], state[l], parents, out=out[l], status=status[l:l + 1])
        all_layers()
        torch.cuda.synchronize()
        eager = out.clone()
        # the 48 launches of a pass, captured once and replayed: the host's
        # per-call cost stays out of the timed region
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            all_layers()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(out.view(torch.int16), eager.view(torch.int16)) or int(status.abs().sum()) != 0:
            raise RuntimeError(f"GDN {name} verify: graph replay differs from the eager launches")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per_layer = e0.elapsed_time(e1) * 1000.0 / (steps * L)
        res[name] = (per_layer, per_layer * L)
        log(f"bench: GDN {name} verify: {per_layer:.2f} us per layer ({L} launches replayed from a graph)")
        del graph
    # commit of a 4-node accepted path into all layers (in place on a copy)
    path_np = [0]
    for i in range(1, n):
        if parents_np[i] == path_np[-1] and len(path_np) < 4:
            path_np.append(i)
    pbuf = torch.full((n,), -1, dtype=torch.int32, device=dev)
    pbuf[:len(path_np)] = torch.as_tensor(path_np, dtype=torch.int32)
    na = torch.tensor([len(path_np) - 1], dtype=torch.int32, device=dev)
    ok = torch.zeros(1, dtype=torch.int32, device=dev)
    work = state.clone()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        work.copy_(state)
        a.record()
        tvp.gdn_commit(work, k, v, g, beta, pbuf, na, ok)
        b.record()
    torch.cuda.synchronize()
    commit_us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1000.0
    commit_bytes = 2 * L * shape.hv * shape.dv * shape.dk * 4
    log(f"bench: GDN commit ({len(path_np)} nodes, {L} layers): {commit_us:.1f} us, "
        f"{commit_bytes / commit_us / 1e3:.0f} GB/s")
    nbytes = gdn_bytes(n, shape.hk, shape.hv, shape.dk, shape.dv)
    gbs = nbytes / (res["wy"][0] * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import gdn as ogdn
        from threadpoolctl import threadpool_info
        heads = 4  # a bounded sample: 4 of the 40 value heads of one layer
        i0 = inps[0]
        S = i0.state.double().numpy()[:heads]
        args_np = [S] + [t.double().numpy() for t in (i0.q, i0.k)] + \
                  [i0.v.double().numpy()[:, :heads], i0.g.double().numpy()[:, :heads],
                   i0.beta.double().numpy()[:, :heads]]
        hk_s = 1
        args_np[1], args_np[2] = args_np[1][:, :hk_s], args_np[2][:, :hk_s]
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0 or reps == 0:
            ogdn.tree_outputs(*args_np, parents_np)
            reps += 1
        per_layer_s = (time.perf_counter() - t0) / reps * (shape.hv / heads)
        threads = max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
        cpu = {"value": round(per_layer_s * 1e6, 1), "unit": "us per GDN layer verify (32 nodes, 40 value heads)",
               "cores": threads, "kind": "oracle",
               "sample": f"{reps} oracle runs over 4 of 40 value heads of one layer, scaled x10"}
    line = {
        "metric": "Gated DeltaNet tree verify (27B-hybrid-like, 48 recurrent layers, 32-node tree), 1 GPU",
        "value": round(res["wy"][0], 2), "unit": "us per layer (WY-form verify, 48 launches replayed)", "n_gpus": 1,
        "steps": steps, "warmup": 1, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32 state, bf16 io", "data": "synthetic",
        "us_per_layer": {"wy_verify": round(res["wy"][0], 2), "path_verify": round(res["path"][0], 2)},
        "us_all_layers": {"wy_verify": round(res["wy"][1], 1), "path_verify": round(res["path"][1], 1)},
        "commit_us_48_layers": round(commit_us, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gdn_wy_kernel", "bytes_per_launch": int(nbytes)},
        "config": {"workload": "27B-hybrid-like Gated DeltaNet layers: 48 layers, 8 key / 40 value heads x 128, "
                               "fp32 state, 32-node best-first tree (branching <= 4, depth <= 8)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def gemm_cpu_baseline(w_bits):
    """The oracle (untuned) on the 17408 x 5120 shape at 32 rows: exact W12
    decode of the canonical tensor plus the fp64 product (the encode is the
    offline conversion and is not timed)."""
    from threadpoolctl import threadpool_info

    from oracle import w12 as ow12
    from oracle.bf16 import from_bits

    t = ow12.encode(w_bits)
    x = np.random.default_rng(0).standard_normal((32, w_bits.shape[1]))
    t0 = time.perf_counter()
    y = from_bits(ow12.decode(t)) @ x.T
    dt = time.perf_counter() - t0
    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    return {"value": round(1e6 * dt, 1), "unit": "us per GEMM (17408x5120, M=32)", "cores": threads,
            "kind": "oracle", "sample": "one W12 decode + fp64 matmul of the 17408x5120 weight at M=32",
            "checksum": float(np.abs(y).sum())}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="27b")
    ap.add_argument("--trees", type=int, default=8)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--gemm-iters", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ar", action="store_true",
                    help="time W12 greedy autoregressive decoding instead (one node per pass, M = 1)")
    ap.add_argument("--cost-curve", action="store_true",
                    help="time the pass at 1, 8, 16 and 32 nodes instead and report c(N) = T(N)/T(1)")
    ap.add_argument("--batched", action="store_true",
                    help="time the batched pass instead (24 requests sharing a 192-node budget)")
    ap.add_argument("--lmhead", action="store_true",
                    help="time the W12 LM head against the INT8 head with the certified candidate filter instead")
    ap.add_argument("--tlv", action="store_true",
                    help="time two-level verification (Q pass on the 8-bit weight views + exact pass) instead")
    ap.add_argument("--gdn", action="store_true",
                    help="time the Gated DeltaNet tree verify (WY form, path form) and commit of a hybrid target")
    ap.add_argument("--gemm", action="store_true",
                    help="time the standalone W12 GEMM at the 27B-like shapes and M = 1, 16, 32 instead")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run three plain device copies of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--rocprof-summary", metavar="DIR", default="",
                    help="only print the summary of a rocprofv3 csv output folder (no GPU use)")
    ap.add_argument("--source-hash", action="store_true",
                    help="only print the hash of the GEMM kernel's sources (recorded with counter summaries)")
    args = ap.parse_args()
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary)
        return 0
    if args.source_hash:
        print(kernel_source_hash())
        return 0
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the verification pass runs on one GPU "
              f"(one GPU's weights and KV cache, no collectives); run with --gpus 1", flush=True)
        return 2

    import torch

    if args.copy_calibration:
        # an elementwise kernel that reads nb bytes and writes nb bytes
        nb = args.copy_calibration << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"bench: negated-copied {nb} bytes 3 times")
        return 0

    import tree_verification_pass_amd as tvp
    from synth.configs import CONFIGS

    cfg = CONFIGS[args.config]
    if args.gemm:
        return bench_gemm(args)
    if args.gdn:
        return bench_gdn(args)
    if args.tlv:
        return bench_tlv(args, cfg)
    if args.lmhead:
        return bench_lmhead(args)
    if args.batched:
        return bench_batched(args, cfg)
    s_max = cfg.ctx_len + 64
    dm = build_model(cfg, args.seed, s_max, cfg.n_nodes)
    if args.ar:
        return bench_ar(args, cfg, dm)
    if args.cost_curve:
        return bench_cost_curve(args, cfg, dm)
    log("bench: drafting trees from the target's top-4")
    trees = make_trees(dm, cfg, args.trees, args.seed + 1)
    out = tvp._alloc_out(dm.plan, cfg.n_nodes, 1, False)

    enq = []  # host time to enqueue a step's launches (the call returns before the GPU is done)

    def step(i):
        tokens, parents = trees[i % len(trees)]
        ta = time.perf_counter()
        tvp.verify_step(dm.plan, cfg.ctx_len, tokens, parents, commit=True, out=out)
        enq.append(time.perf_counter() - ta)
        return int(out.n_accepted.item())  # the step's one device-to-host readback

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    acc = []
    enq.clear()
    per_step = []  # wall time of each step (each ends in its readback)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        ts = time.perf_counter()
        acc.append(step(i))
        per_step.append((time.perf_counter() - ts) * 1000.0)
    ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1000.0 / args.steps
    dev_ms = ev0.elapsed_time(ev1) / args.steps
    enq_ms = float(np.mean(enq)) * 1000.0
    mean_acc = float(np.mean(acc))
    steps_s = 1000.0 / ms
    nbytes = step_bytes(dm, cfg, mean_acc)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"bench: {ms:.3f} ms/step, {steps_s:.1f} steps/s, {gbs:.0f} GB/s, mean accepted {mean_acc:.2f}, "
        f"host enqueue {enq_ms:.2f} ms/step")

    g_ms, g_bytes, _ = time_gateup(dm, cfg, args.gemm_iters)
    g_gbs = g_bytes / (g_ms * 1e-3) / 1e9
    log(f"bench: gate/up W12 GEMM {g_ms * 1000:.1f} us/launch, {g_gbs:.0f} GB/s")
    probe = read_probe_gbs()
    log(f"bench: streaming-read probe {probe:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a sample")
        cpu = cpu_baseline(dm, cfg, args.seed, trees[0])

    line = {
        "metric": METRIC,
        "value": round(steps_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_p10_median_p90": [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)],
        "device_ms_per_step": round(dev_ms, 4),
        "host_enqueue_ms_per_step": round(enq_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "tokens_per_s": round(steps_s * (mean_acc + 1.0), 2),
        "mean_accepted": round(mean_acc, 3),
        "achieved_hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "read_probe_gbs": round(probe, 1),
        "probe_frac": round(gbs / probe, 4),
        "bytes_per_step": int(nbytes),
        "config": {"workload": f"{cfg.name}-like verify step, {cfg.n_nodes}-node best-first tree, ctx {cfg.ctx_len}",
                   "n_layers": cfg.n_layers, "hidden": cfg.hidden, "heads": f"{cfg.n_heads}/{cfg.n_kv_heads}x{cfg.head_dim}",
                   "ffn": cfg.ffn, "vocab": cfg.vocab, "nodes": cfg.n_nodes, "ctx_len": cfg.ctx_len,
                   "weights": "W12 (random-init bf16, per-channel sigma log-uniform [0.005,0.05], 1% zeros, "
                              "0.05% outliers x1000)", "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": (f"w12_skinny_kernel, SWIGLU epilogue (fused gate/up, {2 * cfg.ffn}x{cfg.hidden}; "
                                "the remaining groups' K slices finished in the launch)"), "bound": "hbm",
                     "achieved": round(g_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(g_gbs / HBM_PEAK_GBS, 4), "probe_frac": round(g_gbs / probe, 4),
                     "traffic": recorded_traffic(g_bytes),
                     "us_per_launch": round(g_ms * 1000.0, 2), "bytes_per_launch": int(g_bytes)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
