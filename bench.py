"""Benchmark of the SALA hybrid attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * prefill of the hybrid 4-layer attention stack L, L, L, S at 262,144 tokens (batch 1;
    linear layers: 32 heads, d = 128; sparse layer: 32 query heads over 2 KV heads, top-64
    blocks of 64 with block 0 and 2 local blocks forced), and
  * one decode step of the same 4-layer stack at a 1,048,576-token context, batch 8
    (3 linear-state updates + KV append, block selection over 16,384 pooled key blocks and
    sparse attention).
Inputs are seeded N(0,1) bf16 tensors drawn on the GPU before timing (already resident in
HBM). `value` is prefill tokens per second of the whole step (262,144 tokens / step time,
decode time included). Per-layer prefill rates, decode microseconds per step and per token,
and roofline fractions come from HIP events recorded on the launch stream around each call.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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

METRIC = "attn-layer prefill tokens/s at 256K (linear, sparse); decode µs/token at 1M"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s


def sparse_prefill_flops(N, Hq, d, topk, block=64):
    """Algorithmic flops of block-sparse attention over a prompt of N tokens: 4*d per
    (query, head, attended key) — 2d for q.k and 2d for p.v — with every query block i
    attending min(topk, i+1) blocks and a causal diagonal block."""
    total_keys = 0
    nqb = -(-N // block)
    for i in range(nqb):
        rows = min(block, N - i * block)
        nsel = min(topk, i + 1)
        total_keys += rows * (nsel - 1) * block + rows * (rows + 1) // 2
    return 4.0 * d * Hq * total_keys


def cpu_baseline_sample(W, seconds_budget=20.0):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload and scale to
    the stack's prefill tokens/s. Sample: linear layer on 1 of 32 heads over 32,768 tokens;
    sparse layer on 1 of 2 KV groups (16 query heads) for query blocks 192..223 of a
    14,336-token prefix (each attending 64 blocks). Scaled linearly in heads and in attended
    key blocks to the 262,144-token stack."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle as O
    from hybrid_sparse_linear_causal_amd.inputs import host_normal

    N, H, d = W.seq_len, W.n_heads, W.head_dim
    # --- linear layer sample
    nl = 32768
    q, k, v, g = (host_normal(W.seed, t, (1, nl, 1, d)) for t in range(4))
    t0 = time.perf_counter()
    O.linear_prefill(q, k, v, g)
    t_lin = time.perf_counter() - t0
    t_lin_layer = t_lin * (N / nl) * H
    # --- sparse layer sample (one KV group = 16 query heads)
    G = W.n_heads // W.n_kv_heads
    blk_lo, nb = 192, 32
    P = (blk_lo + nb) * 64
    qs = host_normal(W.seed + 3, 0, (1, nb * 64, G, d))
    gs = host_normal(W.seed + 3, 3, (1, nb * 64, G, d))
    ks = host_normal(W.seed + 3, 1, (1, P, 1, d))
    vs = host_normal(W.seed + 3, 2, (1, P, 1, d))
    t0 = time.perf_counter()
    kh = O.qk_norm(ks)
    kb = O.pool_keys(kh, 64)
    qh = O.qk_norm(qs)
    sel = np.full((1, 1, blk_lo + nb, W.topk), -1, dtype=np.int64)
    qpos = np.arange(blk_lo * 64, P)
    for r in range(nb):
        i = blk_lo + r
        qt = qh[:, r * 64:(r + 1) * 64].mean(axis=1).sum(axis=1)[0]
        sc = np.full(i - W.n_local + 1, -np.inf)
        sc[:] = O.block_scores(qt, kb[0, 0, : i - W.n_local + 1])
        sel[0, 0, i] = O.select_row(sc, i, W.topk, W.n_local)
    o = O.sparse_attention(qh, kh, vs, sel, 64, 1.0 / math.sqrt(d), q_positions=qpos)
    _ = o * O.sigmoid(gs)
    t_sp = time.perf_counter() - t0
    sample_keys = nb * (64 * (W.topk - 1) * 64 + 64 * 65 // 2)  # attended keys per head
    full_keys = sparse_prefill_flops(N, 1, 1, W.topk) / 4.0
    t_sp_layer = t_sp * (full_keys / sample_keys) * W.n_kv_heads
    t_stack = 3 * t_lin_layer + t_sp_layer
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    return {
        "value": N / t_stack,
        "unit": "tokens/s",
        "cores": max(blas) if blas else 1,
        "kind": "oracle",
        "sample": (f"numpy float64 oracle: linear layer 1/{H} heads x {nl} tokens ({t_lin:.1f} s), "
                   f"sparse layer 1/{W.n_kv_heads} KV groups x {nb} query blocks with {W.topk} "
                   f"blocks each ({t_sp:.1f} s); scaled linearly to the {N}-token L,L,L,S stack "
                   f"(extrapolated {t_stack:.0f} s); host cores visible {len(os.sched_getaffinity(0))}"),
    }


def kernel_source_sha(files):
    """sha256 over the source files a kernel is built from (for matching stored counters)."""
    import hashlib

    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(kernel, launches_per_profile=1):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC summary
    (profiles/pmc_traffic.json), scaled by the copy-kernel calibration it records, or None if
    the summary is missing or the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get(kernel)
    if not rec or rec.get("source_sha256") != kernel_source_sha(rec["sources"]):
        return None
    return (rec["fetch_kb"] * rec["fetch_scale"] + rec["write_kb"] * rec["write_scale"]) * 1024.0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no "
              f"multi-GPU path; the sharding design is described in DESIGN.md.", file=sys.stderr)
        sys.exit(2)

    import torch

    from hybrid_sparse_linear_causal_amd import sala as S
    from hybrid_sparse_linear_causal_amd.inputs import WORKLOADS, device_normal

    torch.cuda.set_device(0)
    W, Dw = WORKLOADS["stack_256k"], WORKLOADS["decode_1m"]
    N, H, Hkv, d = W.seq_len, W.n_heads, W.n_kv_heads, W.head_dim
    bf = torch.bfloat16
    dev = "cuda"

    # ---------------- prefill inputs (independent seeds per layer), outputs, workspaces
    lin = []
    for li in range(3):
        sd = W.seed + li
        t = [device_normal(sd, tid, (1, N, H, d)) for tid in range(4)]
        lin.append(dict(qkvg=t, out=torch.empty_like(t[0]),
                        state=torch.empty((1, H, d, d), dtype=torch.float32, device=dev)))
    ldesc = S.linear_desc(lin[0]["qkvg"][0], 0, W.rope_base, W.norm_eps)
    ws_lin = torch.empty(max(1, S.workspace_bytes(S.OP_LINEAR_PREFILL, ldesc)), dtype=torch.uint8, device=dev)
    sd = W.seed + 3
    sq, sg = device_normal(sd, 0, (1, N, H, d)), device_normal(sd, 3, (1, N, H, d))
    sk, sv = device_normal(sd, 1, (1, N, Hkv, d)), device_normal(sd, 2, (1, N, Hkv, d))
    cap = N
    kc = torch.zeros((1, Hkv, cap, d), dtype=bf, device=dev)
    vc = torch.zeros_like(kc)
    kp = torch.zeros((1, Hkv, cap // 64, d), dtype=torch.float32, device=dev)
    nqb = N // 64
    sel = torch.empty((1, Hkv, nqb, W.topk), dtype=torch.int32, device=dev)
    sdesc = S.sparse_desc(batch=1, n_q=N, n_heads=H, n_kv_heads=Hkv, head_dim=d, dtype=bf, kv_len=N,
                          kv_capacity=cap, topk=W.topk, n_local=W.n_local)
    ws_sel = torch.empty(S.workspace_bytes(S.OP_BLOCK_SELECT, sdesc), dtype=torch.uint8, device=dev)
    sout = torch.empty_like(sq)

    # ---------------- decode inputs: 1M-token context, batch 8
    B, L = Dw.batch, Dw.seq_len
    dl = []
    for li in range(3):
        sd = Dw.seed + li
        t = [device_normal(sd, tid, (B, H, d)) for tid in range(4)]
        dl.append(dict(qkvg=t, out=torch.empty_like(t[0]),
                       state=device_normal(sd, 4, (B, H, d, d), dtype="f32", std=1024.0)))
    sd = Dw.seed + 3
    dq, dg = device_normal(sd, 0, (B, 1, H, d)), device_normal(sd, 3, (B, 1, H, d))
    dkn, dvn = device_normal(sd, 1, (B, 1, Hkv, d)), device_normal(sd, 2, (B, 1, Hkv, d))
    dkc = torch.empty((B, Hkv, L, d), dtype=bf, device=dev)
    dvc = torch.empty_like(dkc)
    for b in range(B):  # cache contents: N(0,1), taken as already-normalised keys
        dkc[b] = device_normal(sd * 100 + b, 5, (Hkv, L, d))
        dvc[b] = device_normal(sd * 100 + b, 6, (Hkv, L, d))
    dkp = torch.zeros((B, Hkv, L // 64, d), dtype=torch.float32, device=dev)
    S.kv_pool(dkc, dkp, L - 1, 0, (L - 1) // 64)
    dsel = torch.empty((B, Hkv, 1, Dw.topk), dtype=torch.int32, device=dev)
    ddesc = S.sparse_desc(batch=B, n_q=1, n_heads=H, n_kv_heads=Hkv, head_dim=d, dtype=bf, kv_len=L,
                          kv_capacity=L, topk=Dw.topk, n_local=Dw.n_local)
    ws_dsel = torch.empty(S.workspace_bytes(S.OP_BLOCK_SELECT, ddesc), dtype=torch.uint8, device=dev)
    ws_datt = torch.empty(S.workspace_bytes(S.OP_SPARSE_ATTN, ddesc), dtype=torch.uint8, device=dev)
    dsout = torch.empty_like(dq)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    marks = {}

    def step(record):
        e = {}
        if record:
            e["t0"] = ev(); e["t0"].record()
        for li, Lr in enumerate(lin):
            q, k, v, g = Lr["qkvg"]
            S.linear_prefill(q, k, v, g, rope_base=W.rope_base, eps=W.norm_eps, state_out=Lr["state"],
                             out=Lr["out"], workspace=ws_lin)
            if record:
                e[f"lin{li}"] = ev(); e[f"lin{li}"].record()
        S.kv_append(sk, sv, kc, vc, kp, N, eps=W.norm_eps, n_heads=H)
        if record:
            e["append"] = ev(); e["append"].record()
        S.block_select(sq, kp, N, cap, n_kv_heads=Hkv, topk=W.topk, n_local=W.n_local, eps=W.norm_eps,
                       sel=sel, workspace=ws_sel)
        if record:
            e["select"] = ev(); e["select"].record()
        S.sparse_attn(sq, kc, vc, sg, sel, N, n_local=W.n_local, eps=W.norm_eps, out=sout)
        if record:
            e["attn"] = ev(); e["attn"].record()
        for li, Dr in enumerate(dl):
            q, k, v, g = Dr["qkvg"]
            S.linear_decode_step(q, k, v, g, Dr["state"], L - 1, rope_base=W.rope_base, eps=W.norm_eps,
                                 out=Dr["out"])
        if record:
            e["dlin"] = ev(); e["dlin"].record()
        S.kv_append(dkn, dvn, dkc, dvc, dkp, L, eps=W.norm_eps, n_heads=H)
        S.block_select(dq, dkp, L, L, n_kv_heads=Hkv, topk=Dw.topk, n_local=Dw.n_local, eps=W.norm_eps,
                       sel=dsel, workspace=ws_dsel)
        if record:
            e["dsel"] = ev(); e["dsel"].record()
        S.sparse_attn(dq, dkc, dvc, dg, dsel, L, n_local=Dw.n_local, eps=W.norm_eps, out=dsout,
                      workspace=ws_datt)
        if record:
            e["end"] = ev(); e["end"].record()
        return e

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        recs.append(step(True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def avg(a, b):
        return sum(r[a].elapsed_time(r[b]) for r in recs) / len(recs)  # ms

    ms_step = wall * 1e3 / args.steps
    t_lin = [avg("t0", "lin0"), avg("lin0", "lin1"), avg("lin1", "lin2")]
    t_app, t_sel, t_att = avg("lin2", "append"), avg("append", "select"), avg("select", "attn")
    t_sparse = t_app + t_sel + t_att
    t_dlin, t_dsel, t_datt = avg("attn", "dlin"), avg("dlin", "dsel"), avg("dsel", "end")
    t_dec = t_dlin + t_dsel + t_datt
    t_prefill = sum(t_lin) + t_sparse

    flops_attn = sparse_prefill_flops(N, H, d, W.topk)
    att_tflops = flops_attn / (t_att * 1e-3) / 1e12
    lin_bytes = N * H * d * 2 * 5  # q, k, v, g in; out
    lin_gbs = lin_bytes / (sum(t_lin) / 3 * 1e-3) / 1e9
    dec_bytes_lin = B * H * d * d * 4 * 2 + B * H * d * 2 * 5
    n_cand = (L - 1) // 64 - Dw.n_local  # candidate blocks 1 .. i - n_local
    dec_bytes_sp = (B * Hkv * (n_cand + 1) * d * 4 + B * Hkv * Dw.topk * 64 * d * 2 * 2
                    + B * H * d * 2 * 3 + B * Hkv * 64 * d * 2)
    dec_gbs = (3 * dec_bytes_lin + dec_bytes_sp) / (t_dec * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 on the GPU; no trained weights)",
        "config": {"workload": "stack_256k prefill (L,L,L,S) + decode_1m step (4 layers, batch 8)",
                   "seq_len": N, "batch": 1, "heads": H, "kv_heads_sparse": Hkv, "head_dim": d,
                   "block": 64, "topk": W.topk, "n_local": W.n_local, "linear_chunk": 64,
                   "decode_batch": B, "decode_context": L},
        "roofline": {"kernel": "sparse_prefill_bf16_kernel", "bound": "mfma", "achieved": att_tflops,
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": att_tflops / BF16_PEAK_TFLOPS,
                     "traffic": stored_traffic("sparse_prefill_bf16_kernel"),
                     "flops_per_launch": flops_attn, "avg_launch_ms": t_att},
        "breakdown": {
            "prefill_ms": t_prefill,
            "linear_layer_ms": t_lin,
            "linear_layer_tokens_per_s": N / (sum(t_lin) / 3 * 1e-3),
            "linear_layer_hbm_frac": lin_gbs / HBM_PEAK_GBS,
            "sparse_layer_ms": t_sparse,
            "sparse_layer_tokens_per_s": N / (t_sparse * 1e-3),
            "sparse_parts_ms": {"kv_append": t_app, "block_select": t_sel, "attention": t_att},
            "decode_step_us": t_dec * 1e3,
            "decode_us_per_token": t_dec * 1e3 / B,
            "decode_parts_us": {"linear_x3": t_dlin * 1e3, "append_select": t_dsel * 1e3,
                                "attention": t_datt * 1e3},
            "decode_hbm_frac": dec_gbs / HBM_PEAK_GBS,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_sample(W)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
