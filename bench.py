#!/usr/bin/env python3
"""Benchmark of the IndexMem hot path on one MI355X.

Workload: 32 Llama-3.1-8B-shaped layers (32 query / 8 KV heads, head dim 128, hidden
4096), batch 8, 16384-token prefill evicted to B = 1638 (recent window 32 inside the
budget), indexer 32 heads x d_I 64 with a 64-query window, memory decay 0.995, then 512
decode steps.  One step = prefill index+evict of all 32 layers (indexer scores, top-k,
compaction + memory build) followed by the 512 decode steps x 32 layers (split-K
attention + memory read-out).  Inputs are seeded N(0,1) bf16 drawn on the device,
resident in HBM before timing.

Prints one JSON line: decode tokens/s (value), prefill index+evict ms, the decode
kernel's roofline against 8 TB/s HBM, and the fp64 oracle timed on a bounded sample on
the host (cpu_baseline).
"""
import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2516.6   # dense bf16 matrix cores: 256 CU x 2.4 GHz x 4096 flop/clk
METRIC = "decode tok/s & %HBM peak (evicted cache+memory); index+evict ms @16K prefill"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--graph-chunk", type=int, default=32, help="decode steps per captured HIP graph")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--n-split", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-decode-steps", type=int, default=32)
    ap.add_argument("--no-rows", action="store_true", help="skip the streaming and MomentKV row timings")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy a few times (HBM counter calibration)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_inputs(cfg, layers, T, torch, dev):
    """Seeded N(0,1) bf16 tensors of the workload's shapes, drawn on the device."""
    b, L, D, Hq, Hkv, d, HI, dI, W = cfg.b, cfg.L, cfg.D, cfg.H_q, cfg.H_kv, cfg.d, cfg.H_I, cfg.d_I, cfg.W
    bf = torch.bfloat16
    layers_in = []
    for l in range(layers):
        g = torch.Generator(device=dev)
        g.manual_seed(3_000_000 + l)
        rn = lambda *s, std=1.0: (torch.randn(*s, generator=g, device=dev, dtype=torch.float32) * std).to(bf)
        X = torch.empty((b, L, D), dtype=bf, device=dev)
        for i in range(b):
            X[i] = rn(L, D)
        li = dict(
            X=X, Q=rn(b, W, Hq, d), K=rn(b, L, Hkv, d), V=rn(b, L, Hkv, d),
            W_kI=rn(dI, D, std=D ** -0.5), W_qI=rn(HI, dI, d, std=d ** -0.5), W_g=rn(HI, D, std=D ** -0.5),
            w_g=rn(Hq, d, std=d ** -0.5),
            gk=torch.ones(dI, device=dev), gq=torch.ones(dI, device=dev),
            q=rn(T, b, Hq, d), kn=rn(T, b, Hkv, d), vn=rn(T, b, Hkv, d),
        )
        layers_in.append(li)
        if (l + 1) % 8 == 0:
            log(f"inputs: {l + 1}/{layers} layers drawn")
    return layers_in


def decode_bytes(cfg, n_attended, elem=2):
    """Algorithmic HBM bytes of one decode launch (one layer, whole batch): K and V of the
    attended slots, M and b of every (sequence, KV head), q, the new K/V row and o."""
    pairs = cfg.b * cfg.H_kv
    kv = pairs * n_attended * cfg.d * 2 * elem
    mem = pairs * (cfg.d * cfg.d + cfg.d) * 4
    qo = cfg.b * cfg.H_q * cfg.d * (elem + 4) + cfg.H_q * cfg.d * elem
    new = pairs * cfg.d * 2 * elem * 2          # read k_new/v_new, write them into the cache
    return kv + mem + qo + new


def prefill_bytes(cfg, keep, elem=2):
    """Algorithmic HBM bytes of index+evict for one layer: read X (key projection), read
    K and V once, write the kept rows, read/write the fp32 normalised keys between the
    projection and the score pass is implementation traffic and not counted."""
    tok = cfg.b * cfg.L
    return tok * cfg.D * elem + tok * cfg.H_kv * cfg.d * 2 * elem + cfg.b * keep * cfg.H_kv * cfg.d * 2 * elem


PMC_SUMMARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "decode_layer_step_cfg3_pmc.txt")
DECODE_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "learned_kv_cache_mqa_amd", "csrc", "decode.hip")


def measured_traffic():
    """HBM bytes per decode layer-step from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE scaled by a plain copy's counters), or None if the decode source changed
    since the counters were taken."""
    import hashlib
    try:
        kv = {}
        with open(PMC_SUMMARY) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        with open(DECODE_SRC, "rb") as fh:
            src = hashlib.sha256(fh.read()).hexdigest()
        if kv.get("source_sha256") != src:
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def calibrate_copy():
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 4}), flush=True)
    return 0


def time_rows(torch, api, KL, dev):
    """Timings of the rows outside the IndexMem decode path, at their workloads' shapes
    (device-drawn inputs): the streaming step (131072-token workload, pool 1024 + 64) and
    MomentKV's alpha, one score round and the read-out (Qwen3-4B shape, 32K tokens, batch 4)."""
    from synth import WORKLOADS
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(4_000_000)
    rn = lambda *sh, std=1.0: (torch.randn(*sh, generator=g, device=dev) * std).to(bf)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    rows = {}
    # A7: streaming eviction step + decode over the pool
    c4 = WORKLOADS["llama8b_layer_131k_stream"]
    P = c4.B + c4.R
    cap = api.cache_cap(P)
    Kc = rn(1, c4.H_kv, cap, c4.d)
    Vc = rn(1, c4.H_kv, c4.d, cap)
    M = torch.zeros((1, c4.H_kv, c4.d, c4.d), device=dev)
    bv = torch.ones((1, c4.H_kv, c4.d), device=dev)
    kh = torch.randn((1, P, c4.d_I), generator=g, device=dev)
    Ip = torch.rand((1, P), generator=g, device=dev)
    pos = torch.cat([torch.arange(0, c4.L - c4.R, (c4.L - c4.R) // c4.B, device=dev)[:c4.B],
                     torch.arange(c4.L - c4.R, c4.L, device=dev)]).to(torch.int32)[None].contiguous()
    npos = torch.full((1,), c4.L, dtype=torch.int32, device=dev)
    lens = torch.full((1,), P, dtype=torch.int32, device=dev)
    W = [rn(c4.d_I, c4.D, std=c4.D ** -0.5), torch.ones(c4.d_I, device=dev), rn(c4.H_I, c4.d_I, c4.d, std=c4.d ** -0.5),
         torch.ones(c4.d_I, device=dev), rn(c4.H_I, c4.D, std=c4.D ** -0.5)]
    wg = rn(c4.H_q, c4.d, std=c4.d ** -0.5)
    steps = 64
    xs, qs, ks, vs = rn(steps, 1, c4.D), rn(steps, 1, c4.H_q, c4.d), rn(steps, 1, c4.H_kv, c4.d), rn(steps, 1, c4.H_kv, c4.d)
    es = torch.empty((1,), dtype=torch.int32, device=dev)
    o = torch.empty((1, c4.H_q, c4.d), device=dev)

    def stream_steps():
        for t in range(steps):
            api.kvm_stream_evict(xs[t], qs[t], *W, kh, Ip, pos, npos, Kc, Vc, M, bv, c4.lam, c4.R, evict_slot=es)
            api.kvm_decode_attn_mem(qs[t], Kc, Vc, lens, k_new=ks[t], v_new=vs[t], append_slot=es, M=M, bvec=bv,
                                    w_g=wg, o=o)
    stream_steps()
    st = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(gr, stream=st):
            stream_steps()
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    with torch.cuda.stream(st):
        gr.replay()   # warm replay; the state keeps evolving, as it would in decode
        e0.record(st)
        gr.replay()
        e1.record(st)
    torch.cuda.synchronize()
    rows["A7_stream_step_us"] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
    rows["A7_workload"] = f"1 sequence, pool {P} slots, D {c4.D}, stream step + decode per token, HIP graph"
    # V1 / V3: MomentKV at the Qwen3-4B shape
    c5 = WORKLOADS["qwen3_4b_momentkv_32k"]
    Q = rn(c5.b, c5.W, c5.H_q, c5.d)
    K5, V5 = rn(c5.b, c5.L, c5.H_kv, c5.d), rn(c5.b, c5.L, c5.H_kv, c5.d)
    mom = dict(n_e=torch.full((c5.b, c5.H_kv), 1000, dtype=torch.int32, device=dev),
               s_k=torch.randn((c5.b, c5.H_kv, c5.d), generator=g, device=dev),
               s_v=torch.randn((c5.b, c5.H_kv, c5.d), generator=g, device=dev),
               S=torch.randn((c5.b, c5.H_kv, c5.d, c5.d), generator=g, device=dev))
    al = api.kvm_moment_alpha(Q, K5)
    sc = api.kvm_moment_score(K5, V5, al, mom)
    q5 = rn(c5.b, c5.H_q, c5.d)
    oR = torch.randn((c5.b, c5.H_q, c5.d), generator=g, device=dev)
    lR = torch.randn((c5.b, c5.H_q), generator=g, device=dev)
    o5 = api.kvm_moment_readout(q5, oR, lR, mom)
    torch.cuda.synchronize()
    reps = 10
    for name, fn in (("V1_alpha_ms", lambda: api.kvm_moment_alpha(Q, K5, alpha=al)),
                     ("V1_score_round_ms", lambda: api.kvm_moment_score(K5, V5, al, mom, score=sc)),
                     ("V3_readout_ms", lambda: api.kvm_moment_readout(q5, oR, lR, mom, o=o5))):
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        rows[name] = round(e0.elapsed_time(e1) / reps, 4)
    rows["V_workload"] = (f"MomentKV, batch {c5.b}, {c5.L} tokens, {c5.H_q}/{c5.H_kv} heads, d {c5.d}, window {c5.W}: "
                          "alpha (two passes), first score round over all tokens, read-out")
    # N1: MomentKV eviction step + decode over the pool, per token, at the budget and at 1024
    for Pn in (c5.B, 1024):
        capn = api.cache_cap(Pn)
        Kn, Vn = rn(c5.b, c5.H_kv, capn, c5.d), rn(c5.b, c5.H_kv, c5.d, capn)
        posn = (torch.arange(Pn, device=dev, dtype=torch.int32) * 4).expand(c5.b, c5.H_kv, Pn).contiguous()
        nextn = torch.full((c5.b,), 4 * Pn, dtype=torch.int32, device=dev)
        momn = {k: v.clone() for k, v in mom.items()}
        lensn = torch.full((c5.b,), Pn, dtype=torch.int32, device=dev)
        qn, kn, vn = rn(steps, c5.b, c5.H_q, c5.d), rn(steps, c5.b, c5.H_kv, c5.d), rn(steps, c5.b, c5.H_kv, c5.d)
        esn = torch.empty((c5.b, c5.H_kv), dtype=torch.int32, device=dev)
        on = torch.empty((c5.b, c5.H_q, c5.d), device=dev)

        def mstream_steps():
            for t in range(steps):
                api.kvm_moment_stream_evict(qn[t], kn[t], vn[t], Kn, Vn, posn, nextn, momn, 0, evict_slot=esn)
                api.kvm_decode_attn_mem(qn[t], Kn, Vn, lensn, moments=momn, o=on)
        mstream_steps()
        grn = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            with torch.cuda.graph(grn, stream=st):
                mstream_steps()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        with torch.cuda.stream(st):
            grn.replay()
            e0.record(st)
            grn.replay()
            e1.record(st)
        torch.cuda.synchronize()
        rows[f"N1_moment_stream_step_us_P{Pn}"] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
    rows["N1_workload"] = (f"MomentKV, batch {c5.b}, {c5.H_q}/{c5.H_kv} heads, d {c5.d}, pool of P slots per KV head: "
                           "eviction step + decode with the NC mix per token, HIP graph")
    # N2: the read-out projection: decode layer-steps at the 16K workload's shapes, with and
    # without the projected query (kvm_mem_query + decode reading q_mem)
    c3 = WORKLOADS["llama8b_32L_16k_b8"]
    cap3, n3 = api.cache_cap(c3.keep + 512), c3.keep + 256
    K3, V3 = rn(c3.b, c3.H_kv, cap3, c3.d), rn(c3.b, c3.H_kv, c3.d, cap3)
    q3, kn3, vn3 = rn(steps, c3.b, c3.H_q, c3.d), rn(steps, c3.b, c3.H_kv, c3.d), rn(steps, c3.b, c3.H_kv, c3.d)
    M3 = torch.randn((c3.b, c3.H_kv, c3.d, c3.d), generator=g, device=dev) * 0.01
    b3 = torch.rand((c3.b, c3.H_kv, c3.d), generator=g, device=dev) + 1
    wg3 = rn(c3.H_q, c3.d, std=c3.d ** -0.5)
    Wm = rn(c3.d, c3.d, std=c3.d ** -0.5)
    lens3 = torch.full((c3.b,), n3, dtype=torch.int32, device=dev)
    qm3 = torch.empty((c3.b, c3.H_q, c3.d), dtype=bf, device=dev)
    o3 = torch.empty((c3.b, c3.H_q, c3.d), device=dev)
    for proj in (False, True):
        def dsteps():
            for t in range(steps):
                if proj:
                    api.kvm_mem_query(q3[t], Wm, q_mem=qm3)
                api.kvm_decode_attn_mem(q3[t], K3, V3, lens3, k_new=kn3[t], v_new=vn3[t], M=M3, bvec=b3, w_g=wg3,
                                        o=o3, q_mem=qm3 if proj else None)
        dsteps()
        gr3 = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            with torch.cuda.graph(gr3, stream=st):
                dsteps()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        with torch.cuda.stream(st):
            gr3.replay()
            e0.record(st)
            gr3.replay()
            e1.record(st)
        torch.cuda.synchronize()
        rows["N2_decode_step_us_" + ("projected" if proj else "plain")] = round(e0.elapsed_time(e1) * 1e3 / steps, 2)
    rows["N2_workload"] = (f"decode layer-step, batch {c3.b}, {c3.H_q}/{c3.H_kv} heads, d {c3.d}, {n3} cached slots: "
                           "plain read-out vs read-out addressed with W_m q (one extra kernel), HIP graph")
    # N3: the attention-state memory at the 8B shapes, a 16K-token prefix
    Nc, Lp, Kc, iters = 4096, 16384, 256, 10
    Qc = rn(Nc, c3.H_q, c3.d)
    Kp, Vp = rn(Lp, c3.H_kv, c3.d), rn(Lp, c3.H_kv, c3.d)
    a_c, l_c = api.kvm_asm_prefix_states(Qc, Kp, Vp)
    C0 = Qc[:Kc].float().transpose(0, 1).contiguous()
    torch.cuda.synchronize()

    def timed(fn, reps):
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    t_ps = timed(lambda: api.kvm_asm_prefix_states(Qc, Kp, Vp, a=a_c, lse=l_c), 3)
    flops = 4.0 * Nc * Lp * c3.d * c3.H_q
    rows["N3_prefix_states_ms"] = round(t_ps, 3)
    rows["N3_prefix_states_tflops"] = round(flops / t_ps / 1e9, 1)
    Cw = C0.clone()
    idx_c = api.kvm_asm_kmeans(Qc, Cw, iters)
    t_km = timed(lambda: api.kvm_asm_kmeans(Qc, C0.clone(), iters, idx=idx_c), 3)
    rows["N3_kmeans_ms"] = round(t_km, 3)
    ab_c, lb_c = api.kvm_asm_cluster_states(a_c, l_c, idx_c, Kc)
    rows["N3_cluster_states_ms"] = round(timed(lambda: api.kvm_asm_cluster_states(a_c, l_c, idx_c, Kc, a_bar=ab_c,
                                                                                     lse_bar=lb_c), 5), 4)
    qd = rn(c3.b, c3.H_q, c3.d)
    o_l = torch.randn((c3.b, c3.H_q, c3.d), generator=g, device=dev)
    l_l = torch.randn((c3.b, c3.H_q), generator=g, device=dev)
    o_m = torch.empty_like(o_l)
    i_m = torch.empty((c3.b, c3.H_q), dtype=torch.int32, device=dev)
    rows["N3_lookup_merge_us"] = round(1e3 * timed(lambda: api.kvm_asm_lookup(qd, Cw, ab_c, lb_c, o_l, l_l, o=o_m,
                                                                             idx_out=i_m), 20), 2)
    rows["N3_workload"] = (f"ASM, {c3.H_q}/{c3.H_kv} heads, d {c3.d}: {Nc} calibration queries per head over a "
                           f"{Lp}-token prefix (4 N L d H_q flops), K-means with {Kc} centroids x {iters} iterations "
                           f"(+ the cluster states), retrieval + merge for {c3.b} decode queries")
    # N4: one layer's 16K prefill pre-evicted in chunks of 4096 tokens (the pool never holds
    # more than keep + 4096 rows) against the one-shot index + evict of the same tokens
    Cn = 4096
    nck = c3.L // Cn
    Xs = [rn(c3.b, Cn, c3.D) for _ in range(nck)]
    Qs = [rn(c3.b, c3.W, c3.H_q, c3.d) for _ in range(nck)]
    Ks = [rn(c3.b, Cn, c3.H_kv, c3.d) for _ in range(nck)]
    Vs = [rn(c3.b, Cn, c3.H_kv, c3.d) for _ in range(nck)]
    Wt = [rn(c3.d_I, c3.D, std=c3.D ** -0.5), torch.ones(c3.d_I, device=dev),
          rn(c3.H_I, c3.d_I, c3.d, std=c3.d ** -0.5), torch.ones(c3.d_I, device=dev),
          rn(c3.H_I, c3.D, std=c3.D ** -0.5)]
    Mn = torch.zeros((c3.b, c3.H_kv, c3.d, c3.d), device=dev)
    bn = torch.zeros((c3.b, c3.H_kv, c3.d), device=dev)
    cap_f = api.cache_cap(c3.keep + c3.T)
    lam3 = float(c3.lam)

    def chunked():
        P, pool = 0, dict(K=Ks[0].new_empty((c3.b, c3.H_kv, Cn, c3.d)), V=Vs[0].new_empty((c3.b, c3.H_kv, Cn, c3.d)),
                          khat=torch.empty((c3.b, Cn, c3.d_I), device=dev), I=torch.empty((c3.b, Cn), device=dev),
                          pos=torch.empty((c3.b, Cn), dtype=torch.int32, device=dev))
        for c in range(nck):
            last = c == nck - 1
            cap_out = cap_f if last else min(P + Cn, c3.B) + Cn
            pool, P = api.kvm_index_evict_chunk(Xs[c], Qs[c], Ks[c], Vs[c], *Wt, pool, P, c * Cn, c3.B, c3.R, lam3,
                                                cap_out, last, Mn, bn, eps=c3.eps_rms)
        return P
    assert chunked() == c3.keep
    Xf, Kf, Vf = torch.cat(Xs, 1), torch.cat(Ks, 1), torch.cat(Vs, 1)
    If = torch.empty((c3.b, c3.L), device=dev)
    idf = torch.empty((c3.b, c3.keep), dtype=torch.int32, device=dev)
    smf = torch.empty((c3.b, c3.L), dtype=torch.int32, device=dev)
    Kcf = torch.empty((c3.b, c3.H_kv, cap_f, c3.d), dtype=bf, device=dev)
    Vcf = torch.empty((c3.b, c3.H_kv, c3.d, cap_f), dtype=bf, device=dev)

    def one_shot():
        api.kvm_index_score(Xf, Qs[-1], *Wt, I=If, eps=c3.eps_rms)
        api.kvm_topk_select(If, c3.B, c3.R, True, idx=idf, slot_map=smf)
        api.kvm_compact_kv(Kf, Vf, smf, idf, c3.keep, cap_f, Kc=Kcf, Vc=Vcf, M=Mn, bvec=bn, lam=lam3)
    one_shot()
    torch.cuda.synchronize()
    rows["N4_chunked_index_evict_ms"] = round(timed(chunked, 5), 3)

    # the same with each chunk's K/V already in the pool's tail (written there, head-major, by
    # the chunk's attention; here a copy outside the timed calls): only the calls are timed
    def chunked_in_place(evs):
        P, pool = 0, dict(K=Ks[0].new_empty((c3.b, c3.H_kv, Cn, c3.d)), V=Vs[0].new_empty((c3.b, c3.H_kv, Cn, c3.d)),
                          khat=torch.empty((c3.b, Cn, c3.d_I), device=dev), I=torch.empty((c3.b, Cn), device=dev),
                          pos=torch.empty((c3.b, Cn), dtype=torch.int32, device=dev))
        for c in range(nck):
            last = c == nck - 1
            cap_out = cap_f if last else min(P + Cn, c3.B) + Cn
            pool["K"][:, :, P:P + Cn] = Ks[c].transpose(1, 2)
            pool["V"][:, :, P:P + Cn] = Vs[c].transpose(1, 2)
            e0, e1 = ev(), ev()
            e0.record()
            pool, P = api.kvm_index_evict_chunk(Xs[c], Qs[c], None, None, *Wt, pool, P, c * Cn, c3.B, c3.R, lam3,
                                                cap_out, last, Mn, bn, eps=c3.eps_rms)
            e1.record()
            evs.append((e0, e1))
    chunked_in_place([])
    torch.cuda.synchronize()
    evs = []
    for _ in range(5):
        chunked_in_place(evs)
    torch.cuda.synchronize()
    rows["N4_chunked_in_place_index_evict_ms"] = round(sum(a.elapsed_time(b) for a, b in evs) / 5, 3)
    rows["N4_one_shot_index_evict_ms"] = round(timed(one_shot, 5), 3)
    rows["N4_pool_rows_peak"] = c3.keep + Cn
    rows["N4_workload"] = (f"one layer at the 16K workload's shapes (batch {c3.b}, {c3.L} tokens, budget {c3.B}, "
                           f"recent {c3.R}): {nck} chunks of {Cn} tokens, each scored by its own {c3.W}-query window "
                           f"against pool + chunk, vs the one-shot index + evict holding all {c3.L} rows")
    # each row's fraction of the roofline that bounds it, from its algorithmic work
    kv5 = c5.b * c5.L * c5.H_kv * c5.d * 2 * 2                       # K and V of the 32K-token batch
    alpha_flop = 2 * 2.0 * (c5.W * c5.H_q // c5.H_kv) * c5.L * c5.d * c5.b * c5.H_kv   # two passes of logits
    pre_bytes = prefill_bytes(c3, c3.keep)                           # one layer of index+evict
    frac = lambda bound, achieved, peak, unit: {"bound": bound, "achieved": round(achieved, 1), "peak": peak,
                                                "unit": unit, "frac": round(achieved / peak, 4)}
    rows["roofline"] = {
        "N3_prefix_states": frac("mfma", rows["N3_prefix_states_tflops"], MFMA_BF16_PEAK_TFS, "TFLOP/s"),
        "V1_alpha": frac("mfma", alpha_flop / (rows["V1_alpha_ms"] * 1e-3) / 1e12, MFMA_BF16_PEAK_TFS, "TFLOP/s"),
        "V1_score_round": frac("hbm", kv5 / (rows["V1_score_round_ms"] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
        "N4_chunked_index_evict": frac("hbm", pre_bytes / (rows["N4_chunked_index_evict_ms"] * 1e-3) / 1e9,
                                       HBM_PEAK_GBS, "GB/s"),
        "N4_chunked_in_place_index_evict": frac("hbm", pre_bytes / (rows["N4_chunked_in_place_index_evict_ms"] * 1e-3)
                                                / 1e9, HBM_PEAK_GBS, "GB/s"),
        "N4_one_shot_index_evict": frac("hbm", pre_bytes / (rows["N4_one_shot_index_evict_ms"] * 1e-3) / 1e9,
                                        HBM_PEAK_GBS, "GB/s"),
        "latency_bound": ["A7_stream_step", "N1_moment_stream_step", "N2_decode_step", "N3_lookup_merge",
                          "V3_readout"],
    }
    return rows


def source_sha16():
    """Hash of the library sources, the header and this script (a machine that runs the
    benchmark need not have the git history)."""
    import glob
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    files = sorted(glob.glob(os.path.join(root, "learned_kv_cache_mqa_amd", "csrc", "*")))
    files += [os.path.join(root, "include", "kvm.h"), os.path.abspath(__file__)]
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_peaks(torch, dev):
    """Achievable figures measured on this device, beside the datasheet peaks: a plain 1 GiB
    device copy (read + write bytes over its time, best of 5) and a large bf16 GEMM through
    torch.matmul (the vendor library; best of 5)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    best = 1e9
    for _ in range(6):
        e0, e1 = ev(), ev()
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    copy_gbs = 2 * n / (best * 1e-3) / 1e9
    del a, b
    m = 8192
    x = torch.randn((m, m), device=dev, dtype=torch.bfloat16)
    y = torch.randn((m, m), device=dev, dtype=torch.bfloat16)
    best = 1e9
    for _ in range(6):
        e0, e1 = ev(), ev()
        e0.record()
        torch.matmul(x, y)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    gemm_tfs = 2.0 * m ** 3 / (best * 1e-3) / 1e12
    del x, y
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": round(copy_gbs, 1), "bf16_gemm_TFLOPs": round(gemm_tfs, 1),
            "how": "1 GiB device copy (2 x bytes / time) and an 8192^3 bf16 torch.matmul, best of 5 each"}


def time_prefill_pieces(torch, api, cfg, li, I, idx, sm, Kc, Vc, M, bvec, keep, cap, lam, ws_i, ws_c, reps=10):
    """One layer of the stack's index+evict split into its three calls, each replayed `reps`
    times from a HIP graph: indexer keys + queries + scores (A1-A3), top-k (A4), compaction +
    memory build (A5-A6), each with the roofline that bounds it (algorithmic work only)."""
    stream = torch.cuda.Stream()
    calls = {
        "A1_A3_index_score": lambda: api.kvm_index_score(li["X"], li["Q"], li["W_kI"], li["gk"], li["W_qI"], li["gq"],
                                                         li["W_g"], I=I, eps=cfg.eps_rms, ws=ws_i, stream=stream),
        "A4_topk": lambda: api.kvm_topk_select(I, cfg.B, cfg.R, True, idx=idx, slot_map=sm, stream=stream),
        "A5_A6_compact_build": lambda: api.kvm_compact_kv(li["K"], li["V"], sm, idx, keep, cap, Kc=Kc, Vc=Vc, M=M,
                                                          bvec=bvec, lam=lam, ws=ws_c, stream=stream),
    }
    us = {}
    for name, fn in calls.items():
        with torch.cuda.stream(stream):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for _ in range(reps):
                    fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            g.replay()
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        us[name] = e0.elapsed_time(e1) * 1e3 / reps
    tok = cfg.b * cfg.L
    x_bytes = tok * cfg.D * 2
    kv_bytes = tok * cfg.H_kv * cfg.d * 2 * 2
    kept_bytes = cfg.b * keep * cfg.H_kv * cfg.d * 2 * 2
    score_flops = 2 * cfg.W * cfg.H_I * cfg.d_I * tok
    build_flops = (tok - cfg.b * keep) * 2 * cfg.H_kv * cfg.d * (cfg.d + 1)
    build_bytes = kv_bytes + kept_bytes
    ai = build_flops / build_bytes
    attain = min(MFMA_BF16_PEAK_TFS, ai * HBM_PEAK_GBS / 1e3)   # TFLOP/s the build can reach
    t1, t2, t3 = us["A1_A3_index_score"], us["A4_topk"], us["A5_A6_compact_build"]
    return {
        "workload": f"one layer of the stack (batch {cfg.b}, {cfg.L} tokens), each call replayed {reps} times from a "
                    f"HIP graph",
        "A1_A3_index_score": {"us": round(t1, 2), "bound": "hbm", "bytes": x_bytes,
                              "hbm_frac": round(x_bytes / (t1 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                              "score_flops": score_flops},
        "A4_topk": {"us": round(t2, 2), "bound": "lds/alu latency (4 B read per token)"},
        "A5_A6_compact_build": {"us": round(t3, 2), "bound": "hbm", "bytes": build_bytes,
                                "hbm_frac": round(build_bytes / (t3 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "flops": build_flops, "arith_intensity": round(ai, 2),
                                "attainable_tflops": round(attain, 1),
                                "frac_of_attainable": round(build_flops / (t3 * 1e-6) / 1e12 / attain, 4)},
    }


def time_long_prefill(torch, api, dev):
    """The 131072-token workload's one-shot index + evict (batch 1): indexer scores over the
    whole prefill, the top 1024 plus a recent window of 64, compaction + memory build, and
    the top-k of the 131072-token row on its own; mean of 5 after a warm-up."""
    from synth import WORKLOADS
    c4 = WORKLOADS["llama8b_layer_131k_stream"]
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(5_000_000)
    rn = lambda *sh, std=1.0: (torch.randn(*sh, generator=g, device=dev) * std).to(bf)
    X = torch.empty((1, c4.L, c4.D), dtype=bf, device=dev)
    for r0 in range(0, c4.L, 16384):
        X[0, r0:r0 + 16384] = rn(16384, c4.D)
    Q, K4, V4 = rn(1, c4.W, c4.H_q, c4.d), rn(1, c4.L, c4.H_kv, c4.d), rn(1, c4.L, c4.H_kv, c4.d)
    Wt = [rn(c4.d_I, c4.D, std=c4.D ** -0.5), torch.ones(c4.d_I, device=dev),
          rn(c4.H_I, c4.d_I, c4.d, std=c4.d ** -0.5), torch.ones(c4.d_I, device=dev),
          rn(c4.H_I, c4.D, std=c4.D ** -0.5)]
    keep = api.kvm_topk_keep(c4.L, c4.B, c4.R, False)
    cap = api.cache_cap(keep)
    I = torch.empty((1, c4.L), device=dev)
    idx = torch.empty((1, keep), dtype=torch.int32, device=dev)
    sm = torch.empty((1, c4.L), dtype=torch.int32, device=dev)
    Kc = torch.empty((1, c4.H_kv, cap, c4.d), dtype=bf, device=dev)
    Vc = torch.empty((1, c4.H_kv, c4.d, cap), dtype=bf, device=dev)
    M = torch.zeros((1, c4.H_kv, c4.d, c4.d), device=dev)
    bv = torch.zeros((1, c4.H_kv, c4.d), device=dev)
    lam = float(c4.lam)

    def run():
        api.kvm_index_score(X, Q, *Wt, I=I, eps=c4.eps_rms)
        api.kvm_topk_select(I, c4.B, c4.R, False, idx=idx, slot_map=sm)
        api.kvm_compact_kv(K4, V4, sm, idx, keep, cap, Kc=Kc, Vc=Vc, M=M, bvec=bv, lam=lam)

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    ms = timed(run, 5)
    topk_us = 1e3 * timed(lambda: api.kvm_topk_select(I, c4.B, c4.R, False, idx=idx, slot_map=sm), 20)
    nbytes = prefill_bytes(c4, keep)
    out = {"ms": round(ms, 4), "topk_us": round(topk_us, 2), "bytes": nbytes,
           "roofline": {"bound": "hbm", "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
           "workload": f"1 sequence, {c4.L}-token prefill, {c4.D} hidden, {c4.H_q}/{c4.H_kv} heads: indexer "
                       f"scores ({c4.H_I}x{c4.d_I}, window {c4.W}), top {c4.B} + recent {c4.R} ({keep} slots), "
                       f"compaction + memory build; bytes = X + K + V read once + kept rows written"}
    del X, K4, V4
    torch.cuda.empty_cache()
    return out


def time_momentkv_decode(torch, api, dev, steps=32):
    """MomentKV decode at the Qwen3-4B shape (36 layers, batch 4, 32/8 heads, d 128) for each
    budget: `steps` decode steps x 36 layers replayed from a HIP graph, each layer with its own
    cache of B retained slots (plus the appended tokens) and its own moment sums; the step is
    the attention over the retained cache with the NC mix.  tok/s = batch x steps / time."""
    from synth import WORKLOADS
    c5 = WORKLOADS["qwen3_4b_momentkv_32k"]
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(6_000_000)
    rn = lambda *sh: torch.randn(*sh, generator=g, device=dev).to(bf)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    out = {}
    pairs = c5.b * c5.H_kv
    for B in c5.budgets:
        cap = api.cache_cap(B + steps)
        Ks = [rn(c5.b, c5.H_kv, cap, c5.d) for _ in range(c5.layers)]
        Vs = [rn(c5.b, c5.H_kv, c5.d, cap) for _ in range(c5.layers)]
        moms = [dict(n_e=torch.full((c5.b, c5.H_kv), c5.L - B, dtype=torch.int32, device=dev),
                     s_k=torch.randn((c5.b, c5.H_kv, c5.d), generator=g, device=dev),
                     s_v=torch.randn((c5.b, c5.H_kv, c5.d), generator=g, device=dev),
                     S=torch.randn((c5.b, c5.H_kv, c5.d, c5.d), generator=g, device=dev))
                for _ in range(c5.layers)]
        qs = rn(steps, c5.layers, c5.b, c5.H_q, c5.d)
        kn, vn = rn(steps, c5.layers, c5.b, c5.H_kv, c5.d), rn(steps, c5.layers, c5.b, c5.H_kv, c5.d)
        lens = torch.full((c5.b,), B, dtype=torch.int32, device=dev)
        o = torch.empty((c5.b, c5.H_q, c5.d), device=dev)
        ws = torch.zeros(1 << 22, dtype=torch.uint8, device=dev)

        def dsteps():
            for t in range(steps):
                for l in range(c5.layers):
                    api.kvm_decode_attn_mem(qs[t, l], Ks[l], Vs[l], lens, k_new=kn[t, l], v_new=vn[t, l],
                                            moments=moms[l], o=o, ws=ws)
                api.kvm_len_add(lens, 1)
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            dsteps()
            lens.fill_(B)
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=st):
                dsteps()
        torch.cuda.synchronize()
        lens.fill_(B)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        with torch.cuda.stream(st):
            e0.record(st)
            gr.replay()
            e1.record(st)
        torch.cuda.synchronize()
        t_ms = e0.elapsed_time(e1)
        n_avg = B + (steps + 1) / 2.0
        nbytes = (pairs * n_avg * c5.d * 2 * 2 + pairs * (c5.d * c5.d + 2 * c5.d + 1) * 4
                  + c5.b * c5.H_q * c5.d * (2 + 4) + pairs * c5.d * 2 * 2 * 2) * c5.layers
        launch_s = t_ms * 1e-3 / steps
        out[f"B{B}"] = {"tok_s": round(c5.b * steps / (t_ms * 1e-3), 1),
                        "layer_step_us": round(launch_s / c5.layers * 1e6, 2),
                        "hbm_frac": round(nbytes / launch_s / 1e9 / HBM_PEAK_GBS, 4)}
        del Ks, Vs, moms, gr
        torch.cuda.empty_cache()
    out["workload"] = (f"MomentKV decode, {c5.layers} layers, batch {c5.b}, {c5.H_q}/{c5.H_kv} heads, d {c5.d}, "
                       f"retained B slots per KV head + appended tokens, {steps} steps from a HIP graph; bytes = "
                       "K/V of the attended slots + S, s_k, s_v, n_e + q, o, new K/V")
    return out


def cpu_baseline(cfg, decode_steps):
    """The fp64 oracle on one (layer, sequence) of the workload: prefill index+evict and
    `decode_steps` decode steps, scaled to the workload's units."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import indexmem as im
    from synth import gen
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    one = cfg.with_(b=1)   # sequence 0 of layer 0, with the workload's planted needles
    p = gen.make_prefill(one, layer=0)
    f = lambda x: gen.from_storage(x, one.dtype)
    X, Q, K, V = f(p["X"][0]), f(p["Qwin"][0]), f(p["K"][0]), f(p["V"][0])
    Wk, Wq, Wg, wg = f(p["W_kI"]), f(p["W_qI"]), f(p["W_g"]), f(p["w_g"])
    t0 = time.perf_counter()
    lam = float(np.float32(cfg.lam))   # the value the library takes (fp32)
    pre = im.prefill(X, Q, K, V, Wk, p["gamma_k"], Wq, p["gamma_q"], Wg, cfg.B, cfg.R, lam,
                     cap=cfg.keep + decode_steps)
    t_pre = time.perf_counter() - t0
    dec = gen.make_decode(one, layer=0, steps=decode_steps)
    t0 = time.perf_counter()
    o_ref, _, _, _ = im.decode(f(dec["q"][:, 0]), f(dec["k_new"][:, 0]), f(dec["v_new"][:, 0]), pre["Kc"],
                               pre["Vc"], cfg.keep, pre["M"], pre["b"], wg)
    t_dec = (time.perf_counter() - t0) / decode_steps
    index_evict_ms = t_pre * cfg.layers * cfg.b * 1e3
    tok_s = 1.0 / (t_dec * cfg.layers)
    parity = _sample_parity(one, p, pre, dec, o_ref)
    return dict(value=round(tok_s, 3), unit="tok/s", cores=threads, kind="oracle",
                sample=f"1 layer x 1 sequence of the workload: prefill index+evict ({t_pre:.2f} s) and "
                       f"{decode_steps} decode steps ({t_dec * 1e3:.2f} ms each); decode tok/s = "
                       f"1/(32 layers x step time), sequences run one after another",
                cpu_model=_cpu_model(),
                index_evict_ms_estimate=round(index_evict_ms, 1),
                index_evict_estimate_from=f"one layer x one sequence measured ({t_pre * 1e3:.1f} ms) x "
                                          f"{cfg.layers} layers x {cfg.b} sequences",
                single_thread_4k_layer=_oracle_4k_one_thread(),
                parity_sample=parity)


def _sample_parity(one, p, pre, dec, o_ref):
    """The GPU path (index, top-k, compaction with the memory fold, then the decode steps over
    its own caches) on the oracle's sample, compared as the tests compare it: parity
    statistics and needle recall for the record (the tests hold the bars)."""
    import numpy as np
    import torch
    from learned_kv_cache_mqa_amd import api
    from oracle import indexmem as im
    dev = torch.device("cuda", 0)

    def up(a):   # storage array (uint16 holds bf16 bits) -> device tensor
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    I = api.kvm_index_score(up(p["X"]), up(p["Qwin"]), up(p["W_kI"]), up(p["gamma_k"]), up(p["W_qI"]),
                            up(p["gamma_q"]), up(p["W_g"]), eps=one.eps_rms)
    idx, sm = api.kvm_topk_select(I, one.B, one.R, one.recent_inclusive)
    keep = idx.shape[1]
    T = dec["q"].shape[0]
    cap = api.cache_cap(keep + T)
    M = torch.zeros((1, one.H_kv, one.d, one.d), device=dev)
    bv = torch.zeros((1, one.H_kv, one.d), device=dev)
    Kc, Vc = api.kvm_compact_kv(up(p["K"]), up(p["V"]), sm, idx, keep, cap, M=M, bvec=bv,
                                lam=float(np.float32(one.lam)))
    lens = torch.full((1,), keep, dtype=torch.int32, device=dev)
    outs = []
    for t in range(T):
        outs.append(api.kvm_decode_attn_mem(up(dec["q"][t]), Kc, Vc, lens, k_new=up(dec["k_new"][t]),
                                            v_new=up(dec["v_new"][t]), M=M, bvec=bv, w_g=up(p["w_g"])))
        api.kvm_len_add(lens, 1)
    torch.cuda.synchronize()
    gI, gidx = I.cpu().numpy()[0].astype(np.float64), idx.cpu().numpy()[0]
    Iref = pre["I"]
    # kept sets: positions where the GPU and the oracle differ, and those outside the 1e-5
    # band around the oracle's threshold (the decision taken on its scores rounded to fp32)
    I32 = Iref.astype(np.float32).astype(np.float64)
    ref_idx, _ = im.topk_select(I32, one.B, one.R, one.recent_inclusive)
    n_cand = one.L - min(one.R, one.L)
    sel = [t for t in ref_idx.tolist() if t < n_cand]
    tau = min(I32[t] for t in sel)
    band = np.abs(I32 - tau) <= 1e-5 * abs(tau)
    diff = set(gidx.tolist()) ^ set(ref_idx.tolist())
    same = not diff
    gK, gV = Kc.cpu().view(torch.int16).numpy()[0], Vc.cpu().view(torch.int16).numpy()[0]
    K0, V0 = p["K"][0].view(np.int16), p["V"][0].view(np.int16)
    caches_exact = (gK[:, :keep].tobytes() == np.ascontiguousarray(K0[gidx].transpose(1, 0, 2)).tobytes()
                    and gV[:, :, :keep].tobytes() == np.ascontiguousarray(V0[gidx].transpose(1, 2, 0)).tobytes())
    nw = lambda a, r: float(np.linalg.norm(a - r) / max(np.linalg.norm(r), 1e-300))
    rec = {"workload": f"layer 0, sequence 0 of the workload ({one.L} tokens, {len(p['needles'])} planted needles)",
           "I_max_rel_err": float(np.max(np.abs(gI - Iref) / np.maximum(np.abs(Iref), 1e-3))),
           "kept_set_diff": len(diff), "kept_set_diff_outside_band": sum(1 for t in diff if not band[t]),
           "band_positions": int(band.sum()), "caches_bit_exact": bool(caches_exact)}
    if same:   # equal kept sets: the memory and the decode see the oracle's own state
        rec["M_normwise_err"] = nw(M.cpu().numpy()[0].astype(np.float64), pre["M"])
        rec["b_normwise_err"] = nw(bv.cpu().numpy()[0].astype(np.float64), pre["b"])
        go = torch.stack(outs).cpu().numpy()[:, 0].astype(np.float64)
        rec["decode_steps"] = T
        rec["decode_o_max_abs_err"] = float(np.max(np.abs(go - o_ref)))
        rec["decode_o_normwise_err"] = nw(go, o_ref)
    needles = np.asarray(p["needles"])
    if len(needles):
        rec["needle_recall_gpu"] = float(np.isin(needles, gidx).mean())
        rec["needle_recall_oracle"] = float(np.isin(needles, pre["idx"]).mean())
    return rec


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_4k_one_thread(decode_steps=8):
    """The oracle on the Llama-3.1-8B-shaped 4K layer (batch 1, budget 410) with one BLAS
    thread: prefill index+evict and `decode_steps` decode steps, for a per-core figure."""
    from threadpoolctl import threadpool_limits
    from oracle import indexmem as im
    from synth import WORKLOADS, gen
    c2 = WORKLOADS["llama8b_layer_4k"].with_(needles=0)
    p = gen.make_prefill(c2)
    dec = gen.make_decode(c2, steps=decode_steps)
    f = lambda x: gen.from_storage(x, c2.dtype)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        pre = im.prefill(f(p["X"][0]), f(p["Qwin"][0]), f(p["K"][0]), f(p["V"][0]), f(p["W_kI"]), p["gamma_k"],
                         f(p["W_qI"]), p["gamma_q"], f(p["W_g"]), c2.B, c2.R, c2.lam, cap=c2.keep + decode_steps)
        t_pre = time.perf_counter() - t0
        t0 = time.perf_counter()
        im.decode(f(dec["q"][:, 0]), f(dec["k_new"][:, 0]), f(dec["v_new"][:, 0]), pre["Kc"], pre["Vc"], c2.keep,
                  pre["M"], pre["b"], f(p["w_g"]))
        t_dec = (time.perf_counter() - t0) / decode_steps
    return {"threads": 1, "prefill_index_evict_ms": round(t_pre * 1e3, 1),
            "decode_step_ms": round(t_dec * 1e3, 3),
            "workload": f"{c2.L}-token layer, batch 1, {c2.H_q}/{c2.H_kv} heads, budget {c2.B} (recent {c2.R})"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the path shards "
              "by sequence with no communication; see the design notes)", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        return calibrate_copy()
    import torch
    from synth import WORKLOADS
    from learned_kv_cache_mqa_amd import api
    from learned_kv_cache_mqa_amd import _lib as KL

    cfg = WORKLOADS["llama8b_32L_16k_b8"].with_(layers=args.layers, T=args.decode_steps)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    T, layers = cfg.T, cfg.layers
    keep = api.kvm_topk_keep(cfg.L, cfg.B, cfg.R, True)
    cap = api.cache_cap(keep + T)
    lam = float(cfg.lam)
    log(f"workload: {layers} layers, b={cfg.b}, L={cfg.L}, keep={keep}, cap={cap}, T={T}")
    L_in = make_inputs(cfg, layers, T, torch, dev)

    bf = torch.bfloat16
    Kc = [torch.zeros((cfg.b, cfg.H_kv, cap, cfg.d), dtype=bf, device=dev) for _ in range(layers)]
    Vc = [torch.zeros((cfg.b, cfg.H_kv, cfg.d, cap), dtype=bf, device=dev) for _ in range(layers)]
    Ms = [torch.zeros((cfg.b, cfg.H_kv, cfg.d, cfg.d), dtype=torch.float32, device=dev) for _ in range(layers)]
    bs = [torch.zeros((cfg.b, cfg.H_kv, cfg.d), dtype=torch.float32, device=dev) for _ in range(layers)]
    I = torch.empty((cfg.b, cfg.L), dtype=torch.float32, device=dev)
    idx = torch.empty((cfg.b, keep), dtype=torch.int32, device=dev)
    sm = torch.empty((cfg.b, cfg.L), dtype=torch.int32, device=dev)
    o = torch.empty((layers, cfg.b, cfg.H_q, cfg.d), dtype=torch.float32, device=dev)
    lens = torch.full((cfg.b,), keep, dtype=torch.int32, device=dev)

    import ctypes as C
    L0 = L_in[0]
    idesc = KL.IndexDesc(b=cfg.b, L=cfg.L, D=cfg.D, H_q=cfg.H_q, d=cfg.d, H_I=cfg.H_I, d_I=cfg.d_I, W=cfg.W,
                         dtype=KL.KVM_BF16, eps_rms=cfg.eps_rms)
    cdesc = KL.CompactDesc(b=cfg.b, L=cfg.L, H_kv=cfg.H_kv, d=cfg.d, cap=cap, keep=keep, dtype=KL.KVM_BF16,
                           per_head=0, kv_head_major=0, flags=KL.KVM_FUSE_MEM, lam=lam)
    ddesc = api.decode_desc(L0["q"][0], Kc[0], KL.KVM_READ_MEMORY, args.n_split)
    ws_i = torch.zeros(KL.lib().kvm_index_workspace_size(C.byref(idesc)), dtype=torch.uint8, device=dev)
    ws_c = torch.zeros(KL.lib().kvm_compact_workspace_size(C.byref(cdesc)), dtype=torch.uint8, device=dev)
    ws_d = torch.zeros(KL.lib().kvm_decode_workspace_size(C.byref(ddesc)), dtype=torch.uint8, device=dev)

    def prefill():
        for l in range(layers):
            li = L_in[l]
            api.kvm_index_score(li["X"], li["Q"], li["W_kI"], li["gk"], li["W_qI"], li["gq"], li["W_g"], I=I,
                                eps=cfg.eps_rms, ws=ws_i)
            api.kvm_topk_select(I, cfg.B, cfg.R, True, idx=idx, slot_map=sm)
            api.kvm_compact_kv(li["K"], li["V"], sm, idx, keep, cap, Kc=Kc[l], Vc=Vc[l], M=Ms[l], bvec=bs[l], lam=lam,
                               ws=ws_c)

    def decode_steps(t0, t1):
        for t in range(t0, t1):
            for l in range(layers):
                li = L_in[l]
                api.kvm_decode_attn_mem(li["q"][t], Kc[l], Vc[l], lens, k_new=li["kn"][t], v_new=li["vn"][t],
                                        M=Ms[l], bvec=bs[l], w_g=li["w_g"], o=o[l], n_split=args.n_split, ws=ws_d)
            api.kvm_len_add(lens, 1)

    graphs = []
    pgraph = None
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    if not args.no_graph:
        # capture the prefill (every layer's index, selection and compaction) and the decode
        # loop in chunks; the kernels never allocate or memset
        with torch.cuda.stream(stream):
            prefill()      # fill caches once so capture-time launches see valid data
            pgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(pgraph, stream=stream):
                prefill()
            for c0 in range(0, T, args.graph_chunk):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    decode_steps(c0, min(T, c0 + args.graph_chunk))
                graphs.append(g)
        torch.cuda.synchronize()
        lens.fill_(keep)
        torch.cuda.synchronize()
        log(f"captured the prefill ({layers} layers) and {len(graphs)} decode graphs of {args.graph_chunk} steps")

    def step(ev):
        with torch.cuda.stream(stream):
            ev[0].record(stream)
            if pgraph is not None:
                pgraph.replay()
            else:
                prefill()
            ev[1].record(stream)
            if graphs:
                for g in graphs:
                    g.replay()
            else:
                decode_steps(0, T)
            api.kvm_len_add(lens, -T)
            ev[2].record(stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for w in range(args.warmup):
        step(mk())
        torch.cuda.synchronize()
        log(f"warmup step {w + 1}/{args.warmup} done")
    evs = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    log(f"timed {args.steps} steps: prefill {sum(pre_ms) / len(pre_ms):.3f} ms, decode {sum(dec_ms) / len(dec_ms):.3f} ms")

    dec_mean = sum(dec_ms) / len(dec_ms)
    pre_mean = sum(pre_ms) / len(pre_ms)
    tok_s = cfg.b * T / (dec_mean / 1e3)
    launch_us = dec_mean * 1e3 / (T * layers)
    avg_bytes = sum(decode_bytes(cfg, keep + t + 1) for t in range(T)) / T
    achieved = avg_bytes / (launch_us * 1e-6) / 1e9
    pbytes = prefill_bytes(cfg, keep) * layers
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "kernel": "kvm_decode_attn_mem layer-step: decode_mfma_kernel<4,false> (split-K attention + "
                          "memory read-out rows) then decode_merge_kernel<bf16,128,4,false>; launch_us = decode phase time / "
                          "(steps x layers), HIP events on the launch stream",
                "bytes_per_launch": round(avg_bytes), "launch_us": round(launch_us, 3)}
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"Llama-3.1-8B-shaped {layers}-layer stack, batch {cfg.b}, {cfg.L}-token prefill "
                               f"evicted to {cfg.B} (recent {cfg.R} inside), {T} decode steps",
                   "layers": layers, "batch": cfg.b, "prefill_len": cfg.L, "budget": cfg.B, "recent": cfg.R,
                   "decode_steps": T, "indexer": f"{cfg.H_I}x{cfg.d_I}, window {cfg.W}", "lam": cfg.lam,
                   "hip_graphs": not args.no_graph},
        "index_evict_ms": round(pre_mean, 3),
        "index_evict_hbm_frac": round(pbytes / (pre_mean / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_ms_per_step": round(dec_mean / T, 4),
        "roofline": roofline,
    }
    out["index_evict_pieces"] = time_prefill_pieces(torch, api, cfg, L_in[0], I, idx, sm, Kc[0], Vc[0], Ms[0], bs[0],
                                                   keep, cap, lam, ws_i, ws_c)
    peaks = measured_peaks(torch, dev)
    roofline["measured_peak"] = peaks["hbm_copy_GBps"]
    roofline["frac_of_measured"] = round(achieved / peaks["hbm_copy_GBps"], 4)
    out["measured_peaks"] = peaks
    out["index_evict_frac_of_measured_hbm"] = round(pbytes / (pre_mean / 1e3) / 1e9 / peaks["hbm_copy_GBps"], 4)
    out["src_sha16"] = source_sha16()
    out["seeds"] = "device torch.Generator: 3000000 + layer (stack inputs), 4000000 (rows), 5000000 (long prefill), " \
                   "6000000 (MomentKV decode)"
    if not args.no_rows:
        log("long prefill: 131072 tokens one-shot ...")
        out["long_prefill_131k"] = time_long_prefill(torch, api, dev)
        log("MomentKV decode per budget ...")
        out["momentkv_decode"] = time_momentkv_decode(torch, api, dev)
        log("rows: streaming step and MomentKV timings ...")
        out["rows"] = time_rows(torch, api, KL, dev)
        for k in ("N3_prefix_states", "V1_alpha"):
            r = out["rows"]["roofline"][k]
            r["frac_of_measured"] = round(r["achieved"] / peaks["bf16_gemm_TFLOPs"], 4)
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on one layer x one sequence ...")
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_decode_steps)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
