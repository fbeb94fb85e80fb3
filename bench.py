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


def measured_peaks(torch):
    """Ceilings measured on this GPU by the committed peak kernels (libsala_peaks.so, built from
    hybrid_sparse_linear_causal_amd/csrc/peaks/peaks.hip): the best over a few grid sizes of a
    4 GiB streaming read (16-byte loads), a 2 GiB copy (bytes read plus written) and of loops of
    independent bf16 MFMA products, timed with HIP events."""
    import ctypes

    path = os.path.join(ROOT, "hybrid_sparse_linear_causal_amd", "libsala_peaks.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.sala_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.sala_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    lib.sala_peak_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.sala_peak_mfma32.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")  # >= the largest grid * 256

    def call(rc):
        if rc != 0:
            raise RuntimeError(f"peak kernel launch failed ({rc})")

    read = {}
    for wgs in (1024, 2048, 4096, 8192):
        ms = _time_events(torch, lambda: call(lib.sala_peak_read(buf.data_ptr(), nbytes, sink.data_ptr(), wgs, st)), 5)
        read[wgs] = nbytes / (ms * 1e-3) / 1e9
    # copy: 2 GiB read and 2 GiB written (bytes moved = both)
    half = nbytes // 2
    dst = buf[half // 4:]
    copy = {}
    for wgs in (1024, 2048, 4096, 8192):
        ms = _time_events(torch, lambda: call(lib.sala_peak_copy(buf.data_ptr(), dst.data_ptr(), half, wgs, st)), 5)
        copy[wgs] = 2 * half / (ms * 1e-3) / 1e9
    del buf, dst
    # cold ceilings at the decode step's sizes (a linear layer's state traffic as a 16.8 MB copy,
    # the selection's pooled keys as a 134 MB read, the attention's K/V as a 33.5 MB read): each
    # transfer after a 1 GiB read outside the timed region, HIP events, median of 5, best grid
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    fsink = torch.empty(1, dtype=torch.float32, device="cuda")
    buf = torch.ones(1 << 28, dtype=torch.int32, device="cuda")

    def cold_us(fn):
        ts = []
        for _ in range(5):
            torch.sum(flush, dim=0, keepdim=True, out=fsink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return sorted(ts)[2]

    half_gib = 512 << 20
    cold = {
        "copy_16.8MB": min(cold_us(lambda w=w: call(lib.sala_peak_copy(buf.data_ptr(), buf.data_ptr() + half_gib,
                                                                       16 << 20, w, st))) for w in (256, 512, 1024)),
        "read_134MB": min(cold_us(lambda w=w: call(lib.sala_peak_read(buf.data_ptr(), 128 << 20, sink.data_ptr(), w,
                                                                      st))) for w in (256, 512, 1024)),
        "read_33.5MB": min(cold_us(lambda w=w: call(lib.sala_peak_read(buf.data_ptr(), 32 << 20, sink.data_ptr(), w,
                                                                       st))) for w in (256, 512, 1024)),
        "empty_region": cold_us(lambda: None),
    }
    del flush, buf
    iters = 2048
    mfma, mfma32 = {}, {}
    for wgs in (256, 512, 1024, 2048, 4096):
        ms = _time_events(torch, lambda: call(lib.sala_peak_mfma(sink.data_ptr(), iters, wgs, st)), 3)
        mfma[wgs] = wgs * 4 * 8 * iters * 16384 / (ms * 1e-3) / 1e12
        ms = _time_events(torch, lambda: call(lib.sala_peak_mfma32(sink.data_ptr(), iters, wgs, st)), 3)
        mfma32[wgs] = wgs * 4 * 4 * iters * 32768 / (ms * 1e-3) / 1e12
    return {"hbm_read_gbs": max(read.values()), "hbm_copy_gbs": max(copy.values()),
            "bf16_mfma_tflops": max(mfma.values()), "bf16_mfma_32x32x16_tflops": max(mfma32.values()),
            "hbm_read_gbs_by_grid": read, "hbm_copy_gbs_by_grid": copy, "bf16_mfma_tflops_by_grid": mfma,
            "bf16_mfma_32x32x16_tflops_by_grid": mfma32, "cold_at_decode_sizes_us": cold,
            "method": "libsala_peaks.so: 4 GiB streaming read (uint4 loads, 4 in flight per lane); 2 GiB copy "
                      "(read + written bytes); the same kernels at the decode step's sizes after a 1 GiB read "
                      "(event-timed like the decode calls; empty_region is an event pair around nothing); "
                      "8 independent v_mfma_f32_16x16x32_bf16 (4 of v_mfma_f32_32x32x16_bf16) chains per "
                      "wave; best over grid sizes"}


def stored_mfma_busy(kernel):
    """MFMA busy fraction of `kernel` from the committed rocprofv3 counter summary
    (profiles/pmc_mfma.json: SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x CUs x 4 SIMDs, and
    the executed bf16 MFMA flops), or None if missing or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", "pmc_mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get(kernel)
    if not rec or rec.get("source_sha256") != kernel_source_sha(rec["sources"]):
        return None
    return {k: rec[k] for k in ("mfma_busy_frac", "executed_flops_per_launch", "counters", "command") if k in rec}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the per-configuration breakdown measurements that follow the timed steps "
                         "(for a kernel trace of the step alone)")
    ap.add_argument("--workload", default="stack_256k", choices=["stack_256k", "segmented_1m"],
                    help="stack_256k: the headline line; segmented_1m: 1M-token prefill in segments + decode")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library has no "
              f"multi-GPU path; each GPU would run its own heads or sequences independently.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "segmented_1m":
        segmented_1m(args)
        return

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
    ws_dstep = torch.empty(S.workspace_bytes(S.OP_SPARSE_DECODE_STEP, ddesc), dtype=torch.uint8, device=dev)
    dkvl = torch.full((B,), L, dtype=torch.int64, device=dev)  # every sequence at L tokens after the append
    dsout = torch.empty_like(dq)

    def sparse_decode_step():
        # append, select and attend in one call (three launches)
        S.sparse_decode_step(dq[:, 0], dkn[:, 0], dvn[:, 0], dg[:, 0], dkc, dvc, dkp, dkvl, L, topk=Dw.topk,
                             n_local=Dw.n_local, eps=W.norm_eps, sel=dsel[:, :, 0], out=dsout[:, 0],
                             workspace=ws_dstep)
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
        sparse_decode_step()
        if record:
            e["end"] = ev(); e["end"].record()
        return e

    # the decode step's calls with their algorithmic HBM bytes: a linear layer reads and writes
    # its fp32 state (plus q, k, v, g, out); the append writes the new k, v and, as the token
    # completes a block, reads its 64 keys and writes the pooled key; the selection reads the
    # pooled keys of every candidate block; the attention reads the selected blocks' K and V
    n_cand = (L - 1) // 64 - Dw.n_local  # candidate blocks 1 .. i - n_local
    bytes_lin = B * H * d * d * 4 * 2 + B * H * d * 2 * 5
    bytes_app = B * Hkv * (2 * d * 2 + 64 * d * 2 + d * 4)
    bytes_sel = B * Hkv * n_cand * d * 4 + B * H * d * 2
    bytes_att = B * Hkv * Dw.topk * 64 * d * 2 * 2 + B * H * d * 2 * 3

    def dlin_call(Dr):
        q, k, v, g = Dr["qkvg"]
        return lambda: S.linear_decode_step(q, k, v, g, Dr["state"], L - 1, rope_base=W.rope_base, eps=W.norm_eps,
                                            out=Dr["out"])

    decode_calls = [(f"linear_layer_{li}", dlin_call(Dr), bytes_lin) for li, Dr in enumerate(dl)] + [
        ("sparse_decode_step", sparse_decode_step, bytes_app + bytes_sel + bytes_att)]
    # the sparse layer's decode as three separate calls (same results), for comparison
    sparse_parts = [
        ("kv_append", lambda: S.kv_append(dkn, dvn, dkc, dvc, dkp, L, eps=W.norm_eps, n_heads=H), bytes_app),
        ("block_select", lambda: S.block_select(dq, dkp, L, L, n_kv_heads=Hkv, topk=Dw.topk, n_local=Dw.n_local,
                                                eps=W.norm_eps, sel=dsel, workspace=ws_dsel), bytes_sel),
        ("sparse_attn", lambda: S.sparse_attn(dq, dkc, dvc, dg, dsel, L, n_local=Dw.n_local, eps=W.norm_eps,
                                              out=dsout, workspace=ws_datt), bytes_att)]

    def decode_step():
        for _, fn, _ in decode_calls:
            fn()

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
    t_dlin, t_dsp = avg("attn", "dlin"), avg("dlin", "end")
    t_dec = t_dlin + t_dsp
    t_prefill = sum(t_lin) + t_sparse

    flops_attn = sparse_prefill_flops(N, H, d, W.topk)
    att_tflops = flops_attn / (t_att * 1e-3) / 1e12
    lin_bytes = N * H * d * 2 * 5  # q, k, v, g in; out
    lin_gbs = lin_bytes / (sum(t_lin) / 3 * 1e-3) / 1e9
    dec_bytes = sum(b for _, _, b in decode_calls)
    dec_gbs = dec_bytes / (t_dec * 1e-3) / 1e9

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
            "decode_step_in_stack_us": t_dec * 1e3,
            "decode_parts_in_stack_us": {"linear_x3": t_dlin * 1e3, "sparse_decode_step": t_dsp * 1e3},
            "decode_in_stack_hbm_frac": dec_gbs / HBM_PEAK_GBS,
            "decode_bytes_per_step": dec_bytes,
        },
    }
    peaks = measured_peaks(torch)
    result["measured_peaks"] = peaks
    r = result["roofline"]
    r["peak_measured"] = peaks["bf16_mfma_tflops"]
    r["frac_of_measured"] = att_tflops / peaks["bf16_mfma_tflops"]
    r["mfma_busy_counters"] = stored_mfma_busy("sparse_prefill_bf16_kernel")
    result["breakdown"]["linear_layer_hbm_frac_of_measured"] = lin_gbs / peaks["hbm_read_gbs"]
    result["linear_layer_tokens_per_s"] = result["breakdown"]["linear_layer_tokens_per_s"]
    result["sparse_layer_tokens_per_s"] = result["breakdown"]["sparse_layer_tokens_per_s"]
    if not args.no_extras:
        ex = extra_measurements(S, torch, W, decode_step, decode_calls, sparse_parts, dl, B, L, H, Hkv, d, peaks)
        result["breakdown"].update(ex)
        # the decode headline: the step with the last-level cache flushed before it
        result["decode_step_us"] = ex["decode_cold_step_us_median"]
        result["decode_us_per_token"] = ex["decode_cold_step_us_median"] / B
        result["decode_hbm_frac"] = dec_bytes / (ex["decode_cold_step_us_median"] * 1e-6) / 1e9 / HBM_PEAK_GBS
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_sample(W)
    print(json.dumps(result))


def _time_events(torch, fn, reps):
    """Average ms of fn() over reps calls, HIP events on the current stream."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def extra_measurements(S, torch, W, decode_step, decode_calls, sparse_parts, dl, B, L, H, Hkv, d, peaks):
    """Per-configuration layer times (32K linear, 128K sparse), the decode step as one graph
    replay, and the decode step with the 256 MB last-level cache flushed before each step (whole
    and call by call, with each call's HBM rate; flushed by reading, and for comparison by
    writing)."""
    from hybrid_sparse_linear_causal_amd.inputs import WORKLOADS, device_normal

    res = {}
    # linear prefill, 32,768 tokens x 32 heads
    Wl = WORKLOADS["linear_32k"]
    t = [device_normal(Wl.seed, tid, (1, Wl.seq_len, H, d)) for tid in range(4)]
    out = torch.empty_like(t[0])
    st = torch.empty((1, H, d, d), dtype=torch.float32, device="cuda")
    ld = S.linear_desc(t[0], 0, W.rope_base, W.norm_eps)
    ws = torch.empty(max(1, S.workspace_bytes(S.OP_LINEAR_PREFILL, ld)), dtype=torch.uint8, device="cuda")
    ms = _time_events(torch, lambda: S.linear_prefill(*t, state_out=st, out=out, workspace=ws), 10)
    res["linear_32k"] = {"ms": ms, "tokens_per_s": Wl.seq_len / (ms * 1e-3),
                         "hbm_frac": Wl.seq_len * H * d * 2 * 5 / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del t, out
    # sparse prefill, 131,072 tokens (append + select + attention)
    Ws = WORKLOADS["sparse_128k"]
    N = Ws.seq_len
    q, g = device_normal(Ws.seed, 0, (1, N, H, d)), device_normal(Ws.seed, 3, (1, N, H, d))
    k, v = device_normal(Ws.seed, 1, (1, N, Hkv, d)), device_normal(Ws.seed, 2, (1, N, Hkv, d))
    kc = torch.zeros((1, Hkv, N, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((1, Hkv, N // 64, d), dtype=torch.float32, device="cuda")
    sel = torch.empty((1, Hkv, N // 64, Ws.topk), dtype=torch.int32, device="cuda")
    sd = S.sparse_desc(batch=1, n_q=N, n_heads=H, n_kv_heads=Hkv, head_dim=d, dtype=torch.bfloat16,
                       kv_len=N, kv_capacity=N, topk=Ws.topk, n_local=Ws.n_local)
    wsel = torch.empty(S.workspace_bytes(S.OP_BLOCK_SELECT, sd), dtype=torch.uint8, device="cuda")
    so = torch.empty_like(q)

    def sparse_layer():
        S.kv_append(k, v, kc, vc, kp, N, n_heads=H)
        S.block_select(q, kp, N, N, n_kv_heads=Hkv, topk=Ws.topk, n_local=Ws.n_local, sel=sel, workspace=wsel)
        S.sparse_attn(q, kc, vc, g, sel, N, n_local=Ws.n_local, out=so)

    ms = _time_events(torch, sparse_layer, 5)
    ms_att = _time_events(torch, lambda: S.sparse_attn(q, kc, vc, g, sel, N, n_local=Ws.n_local, out=so), 5)
    fl = sparse_prefill_flops(N, H, d, Ws.topk)
    res["sparse_128k"] = {"ms": ms, "tokens_per_s": N / (ms * 1e-3), "attention_ms": ms_att,
                          "attention_mfma_frac": fl / (ms_att * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    # backward of the sparse layer's attention for the same selection and a synthetic upstream
    # gradient. Algorithmic flops: five products per attended (query, head, key) — S, dP, dV,
    # dK, dQ — 2.5x the forward's; the kernels execute nine (S is recomputed twice).
    dout = device_normal(Ws.seed, 10, (1, N, H, d))
    wsb = torch.empty(S.workspace_bytes(S.OP_SPARSE_ATTN_BACKWARD, sd), dtype=torch.uint8, device="cuda")
    ms_b = _time_events(torch, lambda: S.sparse_attn_backward(q, kc, vc, g, sel, N, dout, topk=Ws.topk,
                                                               n_local=Ws.n_local, workspace=wsb), 3)
    # the same with the forward's out and lse saved (no forward rerun inside the backward)
    lse = torch.empty((1, N, H), dtype=torch.float32, device="cuda")
    S.sparse_attn(q, kc, vc, g, sel, N, n_local=Ws.n_local, out=so, lse=lse)
    ms_s = _time_events(torch, lambda: S.sparse_attn_backward(q, kc, vc, g, sel, N, dout, topk=Ws.topk,
                                                               n_local=Ws.n_local, out=so, lse=lse, workspace=wsb), 3)
    res["sparse_backward_128k"] = {"ms": ms_b, "tokens_per_s": N / (ms_b * 1e-3),
                                   "mfma_frac": 2.5 * fl / (ms_b * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                   "ms_saved_forward": ms_s,
                                   "mfma_frac_saved_forward": 2.5 * fl / (ms_s * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    del q, g, k, v, kc, vc, so, dout, wsb, lse
    # backward of the linear layer (32 heads, d 128) at 32,768 and 262,144 tokens; HBM bytes
    # per (token, head): q, k, v, g, dout read in bf16 and dq, dk, dv, dg written in fp32
    for name, key in (("linear_backward_32k", "linear_32k"), ("linear_backward_256k", "stack_256k")):
        Wb = WORKLOADS[key]
        Nb = Wb.seq_len
        tb = [device_normal(Wb.seed, tid, (1, Nb, H, d)) for tid in (0, 1, 2, 3, 10)]
        lb = S.linear_desc(tb[0], 0, W.rope_base, W.norm_eps)
        wsl = torch.empty(S.workspace_bytes(S.OP_LINEAR_BACKWARD, lb), dtype=torch.uint8, device="cuda")
        ms_l = _time_events(torch, lambda: S.linear_backward(*tb, rope_base=W.rope_base, eps=W.norm_eps,
                                                             need_norm_w_grads=True, workspace=wsl), 3)
        byts = Nb * H * d * (5 * 2 + 4 * 4)
        res[name] = {"ms": ms_l, "tokens_per_s": Nb / (ms_l * 1e-3),
                     "hbm_frac": byts / (ms_l * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del tb, wsl
    res["varlen_256k"] = varlen_measurement(S, torch, W, H, Hkv, d)
    # decode step: individual launches (above) vs one graph replay; linear states restored after
    saved = [Dr["state"].clone() for Dr in dl]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        decode_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        decode_step()
    us_graph = _time_events(torch, graph.replay, 20) * 1e3
    # last-level-cache-cold decode: between steps (outside the timed region) a 1 GiB buffer, four
    # times the 256 MB last-level cache, is read through, which leaves the caches holding only
    # clean lines of other data. A second series writes 512 MB instead: then every cache line
    # the step brings in first evicts a dirty line of the flush, whose write-back the step pays.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    flush.fill_(0)
    fl32 = flush.view(torch.float32)
    sink = torch.empty(1, dtype=torch.float32, device="cuda")
    dirty = flush[: 512 << 20]

    def flush_read(r):
        torch.sum(fl32, dim=0, keepdim=True, out=sink)

    def flush_write(r):
        dirty.fill_(r)

    def cold_steps(flush_fn):
        ts = []
        for r in range(10):
            flush_fn(r)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            decode_step()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts.sort()
        return ts[len(ts) // 2]

    cold = cold_steps(flush_read)
    cold_dirty = cold_steps(flush_write)
    def cold_calls(call_list):
        # call by call: events between the calls of each flushed step
        per = {name: [] for name, _, _ in call_list}
        for r in range(10):
            flush_read(r)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(call_list) + 1)]
            evs[0].record()
            for x, (_, fn, _) in enumerate(call_list):
                fn()
                evs[x + 1].record()
            torch.cuda.synchronize()
            for x, (name, _, _) in enumerate(call_list):
                per[name].append(evs[x].elapsed_time(evs[x + 1]) * 1e3)
        calls = {}
        for name, _, byts in call_list:
            v = sorted(per[name])[len(per[name]) // 2]
            gbs = byts / (v * 1e-6) / 1e9
            calls[name] = {"us": v, "bytes": byts, "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                           "frac_of_measured_read": gbs / peaks["hbm_read_gbs"],
                           "frac_of_measured_copy": gbs / peaks["hbm_copy_gbs"]}
        return calls

    calls = cold_calls(decode_calls)
    parts = cold_calls(sparse_parts)
    for Dr, s0 in zip(dl, saved):
        Dr["state"].copy_(s0)
    res["decode_graph_step_us_warm"] = us_graph
    res["decode_graph_us_per_token_warm"] = us_graph / B
    res["decode_cold_step_us_median"] = cold
    res["decode_cold_flush"] = "1 GiB read between steps (clean caches)"
    res["decode_cold_step_us_dirty_flush"] = cold_dirty
    res["decode_cold_calls"] = calls
    res["decode_cold_sparse_as_three_calls"] = parts
    return res


def varlen_measurement(S, torch, W, H, Hkv, d):
    """Packed batch of 16 prompts of mixed lengths (262,144 tokens) through L, L, L, S with the
    varlen entry points (one launch per kernel for the linear layers and the attention), and
    the same prompts one call per sequence, both timed with HIP events (3 repetitions)."""
    from hybrid_sparse_linear_causal_amd.inputs import WORKLOADS, device_normal, varlen_lengths

    Wv = WORKLOADS["varlen_256k"]
    lens = varlen_lengths(Wv.seed, Wv.batch, Wv.seq_len)
    T, ns = sum(lens), len(lens)
    vl = S.Varlen(lens)
    cu = vl.cu
    cap = ((max(lens) + 63) // 64) * 64
    q, k, v, g = (device_normal(Wv.seed, t, (T, H, d)) for t in range(4))
    sk, sv = device_normal(Wv.seed, 11, (T, Hkv, d)), device_normal(Wv.seed, 12, (T, Hkv, d))
    out = torch.empty_like(q)
    st = torch.empty((ns, H, d, d), dtype=torch.float32, device="cuda")
    kc = torch.zeros((ns, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((ns, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    ld = S.LinearDesc(ns, T, H, H, d, S.SALA_BF16, 0, W.rope_base, W.norm_eps)
    wsl = torch.empty(max(1, S.varlen_workspace_bytes(S.OP_LINEAR_PREFILL, ld, vl)), dtype=torch.uint8,
                      device="cuda")
    sd = S._sparse_varlen_desc(vl, H, Hkv, d, cap, Wv.topk, Wv.n_local, W.norm_eps)
    wss = torch.empty(max(1, S.varlen_workspace_bytes(S.OP_BLOCK_SELECT, sd, vl)), dtype=torch.uint8, device="cuda")
    sel = torch.empty((vl.query_blocks() * Hkv, Wv.topk), dtype=torch.int32, device="cuda")
    sout = torch.empty_like(q)
    parts = {}

    def lin():
        for _ in range(3):
            S.linear_prefill_varlen(q, k, v, g, vl, rope_base=W.rope_base, eps=W.norm_eps, state_out=st, out=out,
                                    workspace=wsl)

    def sparse():
        S.kv_append_varlen(sk, sv, kc, vc, kp, vl, n_heads=H, eps=W.norm_eps)
        S.block_select_varlen(q, kp, vl, cap, n_kv_heads=Hkv, topk=Wv.topk, n_local=Wv.n_local, eps=W.norm_eps,
                              sel=sel, workspace=wss)
        S.sparse_attn_varlen(q, kc, vc, g, sel, vl, n_local=Wv.n_local, eps=W.norm_eps, out=sout)

    parts["linear_x3_ms"] = _time_events(torch, lin, 3)
    parts["sparse_ms"] = _time_events(torch, sparse, 3)
    parts["attention_ms"] = _time_events(torch, lambda: S.sparse_attn_varlen(
        q, kc, vc, g, sel, vl, n_local=Wv.n_local, eps=W.norm_eps, out=sout), 3)

    def per_sequence():
        for s in range(ns):
            a, b = cu[s], cu[s + 1]
            n = b - a
            qs, ks, vs, gs = (x[a:b].unsqueeze(0) for x in (q, k, v, g))
            for _ in range(3):
                S.linear_prefill(qs, ks, vs, gs, rope_base=W.rope_base, eps=W.norm_eps, state_out=st[s:s + 1],
                                 out=out[a:b].unsqueeze(0))
            S.kv_append(sk[a:b].unsqueeze(0), sv[a:b].unsqueeze(0), kc[s:s + 1], vc[s:s + 1], kp[s:s + 1], n,
                        eps=W.norm_eps, n_heads=H)
            ss = S.block_select(qs, kp[s:s + 1], n, cap, n_kv_heads=Hkv, topk=Wv.topk, n_local=Wv.n_local,
                                eps=W.norm_eps)
            S.sparse_attn(qs, kc[s:s + 1], vc[s:s + 1], gs, ss, n, n_local=Wv.n_local, eps=W.norm_eps,
                          out=sout[a:b].unsqueeze(0))

    ms = parts["linear_x3_ms"] + parts["sparse_ms"]
    ms_seq = _time_events(torch, per_sequence, 3)
    fl = sum(sparse_prefill_flops(n, H, d, Wv.topk) for n in lens)
    res = {"lengths": lens, "ms": ms, "tokens_per_s": T / (ms * 1e-3), "per_sequence_calls_ms": ms_seq,
           "linear_layer_hbm_frac": T * H * d * 2 * 5 * 3 / (parts["linear_x3_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "attention_mfma_frac": fl / (parts["attention_ms"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    res.update(parts)
    return res


def segmented_1m(args):
    """One 1,048,576-token sequence through the L,L,L,S stack, prefilled in segments of 131,072
    tokens (linear state carried through state_in/pos0, KV and pooled caches grown through
    kv_len), then decode steps at position 1,048,576. Inputs of each segment are drawn on the
    GPU before its calls (not timed); only the library calls are timed, with HIP events."""
    import torch

    from hybrid_sparse_linear_causal_amd import sala as S
    from hybrid_sparse_linear_causal_amd.inputs import device_normal

    torch.cuda.set_device(0)
    N, SEG, H, Hkv, d, topk, n_local = 1 << 20, 1 << 17, 32, 2, 128, 64, 2
    bf = torch.bfloat16
    cap = N + 64 * 64  # room for the decode tokens
    states = [torch.zeros((1, H, d, d), dtype=torch.float32, device="cuda") for _ in range(3)]
    kc = torch.zeros((1, Hkv, cap, d), dtype=bf, device="cuda")
    vc = torch.zeros_like(kc)
    kp = torch.zeros((1, Hkv, cap // 64, d), dtype=torch.float32, device="cuda")
    lout = torch.empty((1, SEG, H, d), dtype=bf, device="cuda")
    sout = torch.empty_like(lout)
    ld = S.linear_desc(lout, 0, 10000.0, 1e-6)
    ws_lin = torch.empty(max(1, S.workspace_bytes(S.OP_LINEAR_PREFILL, ld)), dtype=torch.uint8, device="cuda")
    sd_last = S.sparse_desc(batch=1, n_q=SEG, n_heads=H, n_kv_heads=Hkv, head_dim=d, dtype=bf, kv_len=N,
                            kv_capacity=cap, topk=topk, n_local=n_local)
    ws_sel = torch.empty(S.workspace_bytes(S.OP_BLOCK_SELECT, sd_last), dtype=torch.uint8, device="cuda")
    sel = torch.empty((1, Hkv, SEG // 64, topk), dtype=torch.int32, device="cuda")

    def prefill(record):
        for st in states:
            st.zero_()
        kp.zero_()
        ms = {"linear": 0.0, "sparse": 0.0}
        for s in range(N // SEG):
            s0, s1 = s * SEG, (s + 1) * SEG
            lin_in = [[device_normal(1000 * li + s, tid, (1, SEG, H, d)) for tid in range(4)] for li in range(3)]
            sq, sg = device_normal(3000 + s, 0, (1, SEG, H, d)), device_normal(3000 + s, 3, (1, SEG, H, d))
            sk, sv = device_normal(3000 + s, 1, (1, SEG, Hkv, d)), device_normal(3000 + s, 2, (1, SEG, Hkv, d))
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            for li in range(3):
                S.linear_prefill(*lin_in[li], pos0=s0, state_in=states[li], state_out=states[li], out=lout,
                                 workspace=ws_lin)
            e[1].record()
            S.kv_append(sk, sv, kc, vc, kp, s1, n_heads=H)
            S.block_select(sq, kp, s1, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local, sel=sel, workspace=ws_sel)
            S.sparse_attn(sq, kc, vc, sg, sel, s1, n_local=n_local, out=sout)
            e[2].record()
            torch.cuda.synchronize()
            ms["linear"] += e[0].elapsed_time(e[1])
            ms["sparse"] += e[1].elapsed_time(e[2])
            del lin_in, sq, sg, sk, sv
        return ms

    prefill(False)
    ms = prefill(True)
    # decode at position N, N+1, ... (batch 1): 3 linear layers + the sparse layer
    dl = [[device_normal(5000 + li, tid, (1, H, d)) for tid in range(4)] for li in range(3)]
    dq, dg = device_normal(5100, 0, (1, 1, H, d)), device_normal(5100, 3, (1, 1, H, d))
    dk, dv = device_normal(5100, 1, (1, 1, Hkv, d)), device_normal(5100, 2, (1, 1, Hkv, d))
    ddesc = S.sparse_desc(batch=1, n_q=1, n_heads=H, n_kv_heads=Hkv, head_dim=d, dtype=bf, kv_len=N + 1,
                          kv_capacity=cap, topk=topk, n_local=n_local)
    ws_ds = torch.empty(S.workspace_bytes(S.OP_BLOCK_SELECT, ddesc), dtype=torch.uint8, device="cuda")
    ws_da = torch.empty(S.workspace_bytes(S.OP_SPARSE_ATTN, ddesc), dtype=torch.uint8, device="cuda")
    dsel = torch.empty((1, Hkv, 1, topk), dtype=torch.int32, device="cuda")
    douts = [torch.empty((1, H, d), dtype=bf, device="cuda") for _ in range(3)]
    dso = torch.empty_like(dq)

    def dstep(p):
        for li in range(3):
            S.linear_decode_step(*dl[li], states[li], p, out=douts[li])
        S.kv_append(dk, dv, kc, vc, kp, p + 1, n_heads=H)
        S.block_select(dq, kp, p + 1, cap, n_kv_heads=Hkv, topk=topk, n_local=n_local, sel=dsel, workspace=ws_ds)
        S.sparse_attn(dq, kc, vc, dg, dsel, p + 1, n_local=n_local, out=dso, workspace=ws_da)

    dstep(N)
    torch.cuda.synchronize()
    steps = 32
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(steps):
        dstep(N + 1 + t)
    e1.record()
    torch.cuda.synchronize()
    dec_us = e0.elapsed_time(e1) * 1e3 / steps
    t_prefill = ms["linear"] + ms["sparse"]
    resident = {
        "linear_state_per_layer": H * d * d * 4,
        "sparse_kv_cache_per_layer": 2 * Hkv * cap * d * 2,
        "sparse_pooled_keys_per_layer": Hkv * (cap // 64) * d * 4,
        "segment_activations_per_layer": SEG * H * d * 2 * 5,
        "select_workspace": ws_sel.numel(),
        "linear_workspace": ws_lin.numel(),
    }
    result = {
        "metric": "prefill tokens/s at 1M (segmented, L,L,L,S, batch 1); decode us/step at 1M (batch 1)",
        "value": N / (t_prefill * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": 1,
        "warmup": 1,
        "ms_per_step": t_prefill,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 on the GPU, drawn per segment; no trained weights)",
        "config": {"workload": "segmented_1m: 1,048,576 tokens in 8 segments of 131,072 through L,L,L,S, "
                               "then decode at 1M", "seq_len": N, "segment": SEG, "batch": 1, "heads": H,
                   "kv_heads_sparse": Hkv, "head_dim": d, "topk": topk, "n_local": n_local},
        "breakdown": {"linear_ms_total_3_layers": ms["linear"], "sparse_ms_total": ms["sparse"],
                      "decode_step_us": dec_us, "resident_bytes": resident},
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
