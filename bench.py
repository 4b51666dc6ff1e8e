"""Benchmark of SANTA++ decode attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--layers R] [--scale NAMES]

A step is one SANTA++ decode-attention call (representative scoring, team
softmax, draws, inclusion probabilities, split-K gather, combine) for one
layer of the workload. The workload is the Qwen2.5-7B-shaped 32K-context
layer with M = 31 by default. Its cache is replicated R times ("layers",
about 1 GiB in total) and the steps cycle through them, so every step reads
HBM rather than the 256 MB last-level cache, as a real decode step does when
it moves from one layer's cache to the next. Inputs are resident in HBM
before timing starts. Each call is timed as GPU time per call from HIP-graph
replays (one call per layer captured, graph replayed; the median of three
timed loops), with the eager-launch figure reported alongside. The same is timed for the dense decode kernel, and
for the gather + combine stage alone (the kernels that move the bytes), whose
algorithmic bytes give the roofline figure. Two larger configurations (batch
8 at 32K, batch 4 at 128K) are then measured the same way with fewer steps
and reported compactly under "at_scale". The CPU oracle is timed first (its
worker processes fork before the GPU is used) on bounded samples of the
headline workload, on one thread and on every core, each the median of three
runs. "team_mass" reports how concentrated the team softmax is (the share of
teams with probability under 1 %, the mean largest probability).

Prints one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, AMD public specification
LLC_BYTES = 256 << 20         # MI355X Infinity Cache

METRIC = "decode-attn µs/layer + HBM GB/s (% peak), 32K ctx M=31, vs own dense decode"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="qwen7b_32k_b1_m31")
    ap.add_argument("--layers", type=int, default=0, help="cache copies to cycle through (0 = enough for 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate", action="store_true", help="also run plain 64 MiB device copies (counter scale)")
    ap.add_argument("--scale", default="qwen7b_32k_b8_m32,mixture_128k_b4_t256_m64",
                    help="workloads also measured, compactly, after the headline one ('' = none)")
    ap.add_argument("--scale-steps", type=int, default=100)
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the decode path (no draw schemes, hashed or k-means teams or representative builds)")
    return ap.parse_args()


def union_stats(w, sampled):
    """Per (b, g) union of the query heads' drawn teams, from the returned sets."""
    G = w.group
    T = w.page_size
    stats = []
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        K = (L + T - 1) // T
        for g in range(w.num_kv_heads):
            u = set()
            per_head = []
            for h in range(g * G, (g + 1) * G):
                s = [int(t) for t in sampled[b, h] if t >= 0]
                per_head.append(s)
                u.update(s)
            stats.append((b, g, L, K, sorted(u), per_head))
    return stats


def team_tokens(L, T, t):
    return min(T, L - t * T)


def algorithmic_bytes(w, stats):
    """Bytes the hot path must move, by the definition in the design notes.

    attend (gather + combine): K and V of every union team once per (b, g),
    the G queries, and out + lse. select: every representative once per
    (b, g) plus the queries. dense: K and V of every token, queries, out + lse.
    """
    e, d, G, T = w.elem_bytes, w.head_dim, w.group, w.page_size
    attend = select = dense = 0
    head_reads = dense_head_reads = 0
    for b, g, L, K, u, per_head in stats:
        kv_union = sum(2 * team_tokens(L, T, t) * d * e for t in u)
        io = G * d * e + G * (d + 1) * 4
        attend += kv_union + io
        select += K * d * e + G * d * e
        dense += 2 * L * d * e + io
        for s in per_head:
            head_reads += K * d * e + sum(2 * team_tokens(L, T, t) * d * e for t in s)
            dense_head_reads += 2 * L * d * e
    return dict(attend=attend, select=select, step=attend + select, dense=dense,
                frac_head=head_reads / dense_head_reads, frac_hbm=(attend + select) / dense)


def value_sampled_bytes(w, stats, positions):
    """Bytes of the value-sampled call beyond the selection: the keys of every
    union team once per (b, g), and the values of the distinct sampled tokens
    of the group (row grain: d values per token), plus queries and outputs.
    Also the value bytes at the cache's grain (a sampled token's values lie
    across its 32-token chunk of the tile, [channel][token]) and the
    per-query-head fraction of the dense bytes (keys of the head's drawn
    teams, representatives, values of its distinct sampled tokens)."""
    e, d, G, T = w.elem_bytes, w.head_dim, w.group, w.page_size
    C = min(T, 32)
    total = chunk_v = head_reads = dense_head_reads = 0
    for b, g, L, K, u, per_head in stats:
        pos_g = set()
        for i, s in enumerate(per_head):
            ph = set(int(x) for x in positions[b, g * G + i] if x >= 0)
            pos_g |= ph
            head_reads += K * d * e + sum(team_tokens(L, T, t) * d * e for t in s) + len(ph) * d * e
            dense_head_reads += 2 * L * d * e
        total += sum(team_tokens(L, T, t) * d * e for t in u) + len(pos_g) * d * e + G * d * e + G * (d + 1) * 4
        chunk_v += len(set(x // C for x in pos_g)) * C * d * e
    return dict(step=total, chunk_v=chunk_v, frac_head=head_reads / dense_head_reads)


def time_stream(fn, steps, warmup, torch):
    """Eager launches: HIP events around ``steps`` calls (includes host launch cost if it dominates)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / steps       # microseconds per call


def median_graph(fn, R, steps, warmup, torch, loops=3):
    """Median over `loops` timed replay loops of time_graph; returns (us, calls per loop)."""
    runs = [time_graph(fn, R, steps, warmup, torch) for _ in range(loops)]
    return sorted(t for t, _ in runs)[loops // 2], runs[0][1]


def time_graph(fn, R, steps, warmup, torch):
    """GPU time per call: one call per layer captured in a HIP graph, replayed;
    HIP events around the replays on the stream they run on."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(R):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(R):
            fn(i)
    replays = max(1, -(-steps // R))              # whole replays, at least `steps` calls
    for _ in range(max(1, warmup // R)):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / (replays * R), replays * R


def recorded_traffic(workload_name):
    """HBM bytes per launch of the gather + combine stage from the committed
    rocprofv3 counter summary, if the kernel source is unchanged since; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    csrc = os.path.join(ROOT, "sampled_sparse_decode_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read()
                   for f in ("gather.hip", "selection.h", "device_common.h"))
    if hashlib.sha256(src).hexdigest() != rec["kernel_source_sha256"]:
        return None
    return int(rec["read_bytes"] + rec["write_bytes"])


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_ORACLE = {}


def _oracle_state(name, w=None):
    """Per-process oracle inputs of workload `name` (built once per process;
    forked workers inherit them)."""
    if name not in _ORACLE:
        from oracle import numerics, santa as osanta
        from sampled_sparse_decode_amd import workloads as W
        w = w if w is not None else W.FULL_SIZE[name]()
        kv = osanta.PagedKV(w.dtype, w.k_pages, w.v_pages, w.page_table, w.seq_lens)
        reps = osanta.build_reps(w.k_pages, w.page_table, w.seq_lens, w.page_size, w.dtype)
        heads = [(b, h) for b in range(w.batch) for h in range(w.num_q_heads)]
        qs = {bh: numerics.decode(w.q[bh], w.dtype) for bh in heads}
        _ORACLE[name] = (w, kv, reps, heads, qs)
    return _ORACLE[name]


def _one_thread():
    """Holds this process's BLAS / OpenMP pools to one thread from here on."""
    from threadpoolctl import threadpool_limits
    global _LIMIT
    _LIMIT = threadpool_limits(limits=1)


def _oracle_eval(task):
    """One oracle evaluation (kind, workload, index)."""
    from oracle import santa as osanta
    kind, name, i = task
    w, kv, reps, heads, qs = _oracle_state(name)
    b, h = heads[i % len(heads)]
    if kind == "santa":
        osanta.santa_head(kv, qs[(b, h)], reps, b, h, w.num_q_heads, w.M, w.seed, i // len(heads))
    else:
        osanta.dense_head(kv, qs[(b, h)], b, h, w.num_q_heads)


def cpu_baseline(w, name, budget_s):
    """The CPU oracle, as it stands, on bounded samples of the same step:
    SANTA++ and dense (sequence, query head) evaluations, on one thread and on
    every core this process may use (capped at 16, one single-threaded worker
    process each, started before the GPU is touched), each the median of three
    timed runs, scaled to one layer. A one-thread run covers one layer; an
    all-cores run covers one layer per worker. A kind's repeats stop early
    once it has taken half of `budget_s` seconds."""
    import multiprocessing as mp
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    heads_per_layer = w.batch * w.num_q_heads
    _oracle_state(name, w)
    from threadpoolctl import threadpool_limits
    runs = {}
    with threadpool_limits(limits=1), mp.get_context("fork").Pool(cores, initializer=_one_thread) as pool:
        pool.map(_oracle_eval, [("santa", name, i) for i in range(cores)], chunksize=1)   # warm every worker
        _oracle_eval(("santa", name, 0))
        for kind in ("santa", "dense"):
            t_begin = time.perf_counter()
            one, many = [], []
            for rep in range(3):
                n1 = heads_per_layer
                t0 = time.perf_counter()
                for i in range(n1):
                    _oracle_eval((kind, name, rep * n1 + i))
                one.append((time.perf_counter() - t0) / n1 * heads_per_layer * 1e6)
                nm = heads_per_layer * cores
                t0 = time.perf_counter()
                pool.map(_oracle_eval, [(kind, name, rep * nm + i) for i in range(nm)], chunksize=1)
                many.append((time.perf_counter() - t0) / nm * heads_per_layer * 1e6)
                if time.perf_counter() - t_begin > budget_s / 2:
                    break
            runs[kind] = (sorted(one)[len(one) // 2], sorted(many)[len(many) // 2], len(one))
    santa1, santaN, n = runs["santa"]
    dense1, denseN, _ = runs["dense"]
    return {"value": round(santaN, 1), "unit": "us/layer", "cores": cores, "kind": "oracle",
            "value_1thread": round(santa1, 1), "dense_value": round(denseN, 1), "dense_value_1thread": round(dense1, 1),
            "cpu": cpu_model(),
            "sample": f"{name}: per kind, the median of {n} runs of one layer ({heads_per_layer} (sequence, query "
                      f"head) evaluations) on one thread and of {cores} layers on {cores} single-threaded "
                      f"processes; float64 Python/numpy oracle, representatives precomputed; scaled to one layer"}


def team_mass(w, q, reps, torch):
    """How concentrated the team softmax is: over (sequence, query head), the
    share of a sequence's teams whose probability p_t = softmax_t(q . rep_t /
    sqrt(d)) is below 1 %, and the mean largest p_t (float32, from the
    representatives the decode call uses)."""
    B, Hq, d = q.shape
    G = Hq // reps.shape[2]
    qf = q.float().reshape(B, reps.shape[2], G, d)
    rt = reps.float().permute(0, 2, 3, 1).contiguous()                          # [B, Hkv, d, P]
    s = torch.matmul(qf.contiguous(), rt) / math.sqrt(d)                        # [B, Hkv, G, P]
    K = torch.as_tensor([-(-int(L) // w.page_size) for L in w.seq_lens], device=q.device)
    valid = torch.arange(reps.shape[1], device=q.device)[None, :] < K[:, None]  # [B, P]
    s = s.masked_fill(~valid[:, None, None, :], float("-inf"))
    pt = torch.softmax(s, dim=-1)
    low = ((pt < 0.01) & valid[:, None, None, :]).sum(-1).float() / K.clamp(min=1)[:, None, None].float()
    return {"share_p_below_1pct": round(low.mean().item(), 4), "mean_max_p": round(pt.amax(-1).mean().item(), 4)}


def measure(w, steps, warmup, layers, torch, S, calibrate=False, extras=True):
    """Times SANTA++, dense and the attend stage on workload w (inputs resident,
    the layer's cache cycled over R copies). Returns a dict of results."""
    dev = torch.device("cuda:0")
    kv0, q = S.kv_from_workload(w, dev)
    kv_bytes = 2 * kv0.k_pages.numel() * kv0.k_pages.element_size()
    R = layers or max(4, math.ceil(4 * LLC_BYTES / kv_bytes))
    cache = [kv0]
    for _ in range(R - 1):
        cache.append(S.KVCache(kv0.k_pages.clone(), kv0.v_pages.clone(), kv0.page_table, kv0.seq_lens,
                               w.num_q_heads, w.page_size))
    reps = [S.santa_build_reps(kv) for kv in cache]
    M = w.M
    wss = [S.make_workspace(kv, M) for kv in cache]
    out = torch.empty((w.batch, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    # Sets of this step (identical on every layer copy) for the byte count.
    _, _, sampled, _ = S.santa_decode_attention(kv0, q, reps[0], M, w.seed, w.offset, wss[0], return_sets=True)
    torch.cuda.synchronize()
    ab = algorithmic_bytes(w, union_stats(w, sampled.cpu().numpy()))
    r_mass = team_mass(w, q, reps[0], torch)

    def santa_step(i):
        j = i % R
        S.santa_decode_attention(cache[j], q, reps[j], M, w.seed, w.offset, wss[j], out, lse)

    def dense_step(i):
        j = i % R
        S.dense_decode_attention(cache[j], q, wss[j], out, lse)

    def attend_step(i):
        j = i % R
        S.santa_attend_selected(cache[j], q, M, wss[j], out, lse)

    # Eager (stream) timings, then HIP-graph replay timings of the same calls.
    r = dict(R=R, ab=ab, mass=r_mass)
    r["santa_stream_us"] = time_stream(santa_step, steps, warmup, torch)
    r["dense_stream_us"] = time_stream(dense_step, steps, warmup, torch)
    r["santa_us"], r["timed_steps"] = median_graph(santa_step, R, steps, warmup, torch)
    r["dense_us"], _ = median_graph(dense_step, R, steps, warmup, torch)
    for j in range(R):
        S.santa_select_teams(cache[j], q, reps[j], M, w.seed, w.offset, wss[j])
    torch.cuda.synchronize()
    r["attend_us"], _ = median_graph(attend_step, R, steps, warmup, torch)

    r["schemes"], r["hashed"], r["kmeans"], r["value_sampled"] = None, None, None, None
    if extras:
        # The variance-reduced draw schemes: whole decode call, and the bytes of
        # their (larger: fewer repeated teams) unions.
        r["schemes"] = {}
        for name in ("systematic", "stratified"):
            _, _, smp, _ = S.santa_decode_attention_ex(kv0, q, reps[0], M, name, w.seed, w.offset, wss[0],
                                                       return_sets=True)
            torch.cuda.synchronize()
            abs_ = algorithmic_bytes(w, union_stats(w, smp.cpu().numpy()))

            def scheme_step(i, name=name):
                j = i % R
                S.santa_decode_attention_ex(cache[j], q, reps[j], M, name, w.seed, w.offset, wss[j], out, lse)

            us, _ = median_graph(scheme_step, R, steps, warmup, torch)
            r["schemes"][name] = {"us_per_layer": round(us, 3),
                                  "kv_read_fraction": {"per_query_head": round(abs_["frac_head"], 4),
                                                       "hbm": round(abs_["frac_hbm"], 4)}}

        # Re-partitioned teams (sign-hash and k-means): the pack that writes
        # them (from plain pages), SANTA++ on them, their bytes, and the
        # estimate's error against dense attention for contiguous, hashed and
        # k-means teams (mean over heads of ||out - dense|| / ||dense||, over
        # 16 draw offsets).
        from sampled_sparse_decode_amd import workloads as W
        K = max(1, -(-int(w.seq_lens.max()) // w.page_size))
        bits = min(10, max(1, math.ceil(math.log2(K))))
        dirs = torch.from_numpy(W.hash_directions(hkv=w.num_kv_heads, bits=bits, d=w.head_dim)).to(dev)
        k_src = S.storage_tensor(w.k_pages, w.dtype, dev)
        v_src = S.storage_tensor(w.v_pages, w.dtype, dev)
        codes = torch.empty((w.batch, w.num_kv_heads, w.max_pages_per_seq * w.page_size), dtype=torch.int32,
                            device=dev)
        token_of = torch.empty_like(codes)

        def fresh_caches():
            return [S.KVCache(torch.empty_like(kv.k_pages), torch.empty_like(kv.v_pages), kv.page_table,
                              kv.seq_lens, w.num_q_heads, w.page_size) for kv in cache]

        def santa_on(pcache):
            preps = [S.santa_build_reps(kv) for kv in pcache]
            _, _, smp, _ = S.santa_decode_attention(pcache[0], q, preps[0], M, w.seed, w.offset, wss[0],
                                                    return_sets=True)
            torch.cuda.synchronize()
            abp = algorithmic_bytes(w, union_stats(w, smp.cpu().numpy()))

            def step(i):
                j = i % R
                S.santa_decode_attention(pcache[j], q, preps[j], M, w.seed, w.offset, wss[j], out, lse)

            us, _ = median_graph(step, R, steps, warmup, torch)
            return preps, us, {"per_query_head": round(abp["frac_head"], 4), "hbm": round(abp["frac_hbm"], 4)}

        hcache = fresh_caches()

        def hpack_step(i):
            S.santa_pack_pages_hashed(hcache[i % R], k_src, v_src, dirs, codes, token_of)

        hp_us, _ = median_graph(hpack_step, R, max(R, steps // 4), max(R, warmup // 4), torch)
        for j in range(R):
            hpack_step(j)
        hreps, hs_us, hfrac = santa_on(hcache)

        # k-means: one cluster per team, 10 assignments; the pack is timed
        # eagerly over a few calls (it is milliseconds long).
        km_iters = 10
        kcache = fresh_caches()
        kws = torch.empty(S.santa_kmeans_workspace_size(kcache[0], 0), dtype=torch.uint8, device=dev)
        for j in range(R):
            S.santa_pack_pages_kmeans(kcache[j], k_src, v_src, 0, km_iters, codes, token_of, kws)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for j in range(3):
            S.santa_pack_pages_kmeans(kcache[j % R], k_src, v_src, 0, km_iters, codes, token_of, kws)
        ev1.record()
        torch.cuda.synchronize()
        kp_us = ev0.elapsed_time(ev1) * 1000.0 / 3
        del k_src, v_src, kws
        kreps, ks_us, kfrac = santa_on(kcache)

        dense_out, _ = S.dense_decode_attention(kv0, q, wss[0])

        # Value samples inside the drawn teams, S per head: the whole call,
        # its bytes and the estimate's error against dense attention (as
        # below, over 16 draw offsets).
        vws = S.make_value_sampled_workspace(kv0, M)
        r["value_sampled"] = {}
        for Sn in (64, 256):
            _, _, smp, _, pos = S.santa_decode_attention_value_sampled(
                kv0, q, reps[0], M, Sn, seed=w.seed, offset=w.offset, workspace=vws, return_sets=True,
                return_positions=True)
            torch.cuda.synchronize()
            vb = value_sampled_bytes(w, union_stats(w, smp.cpu().numpy()), pos.cpu().numpy())

            def vs_step(i, Sn=Sn):
                j = i % R
                S.santa_decode_attention_value_sampled(cache[j], q, reps[j], M, Sn, seed=w.seed, offset=w.offset,
                                                       workspace=vws, out=out, lse=lse)

            us, _ = median_graph(vs_step, R, steps, warmup, torch)
            verr = []
            for off in range(16):
                o, _ = S.santa_decode_attention_value_sampled(kv0, q, reps[0], M, Sn, seed=w.seed,
                                                              offset=w.offset + 1000 + off, workspace=vws)
                verr.append(((o - dense_out).norm(dim=-1) / dense_out.norm(dim=-1)).mean().item())
            r["value_sampled"][str(Sn)] = {
                "us_per_layer": round(us, 3), "bytes_row_grain": int(vb["step"] + ab["select"]),
                "value_bytes_chunk_grain": int(vb["chunk_v"]),
                "kv_read_fraction_per_query_head": round(vb["frac_head"], 4),
                "estimate_rel_error": round(float(np.mean(verr)), 4)}
        del vws

        errs = {"contiguous": [], "hashed": [], "kmeans": []}
        for off in range(16):
            for name, kv, rp in (("contiguous", kv0, reps[0]), ("hashed", hcache[0], hreps[0]),
                                 ("kmeans", kcache[0], kreps[0])):
                o, _ = S.santa_decode_attention(kv, q, rp, M, w.seed, w.offset + 1000 + off, wss[0])
                errs[name].append(((o - dense_out).norm(dim=-1) / dense_out.norm(dim=-1)).mean().item())
        rel = {k: round(float(np.mean(v)), 4) for k, v in errs.items()}
        r["hashed"] = {"bits": bits, "pack_us": round(hp_us, 2), "santa_us_per_layer": round(hs_us, 3),
                       "kv_read_fraction": hfrac,
                       "estimate_rel_error": {"contiguous": rel["contiguous"], "hashed": rel["hashed"]}}
        r["kmeans"] = {"clusters_per_seq": "one per team", "iters": km_iters, "pack_us": round(kp_us, 1),
                       "santa_us_per_layer": round(ks_us, 3), "kv_read_fraction": kfrac,
                       "estimate_rel_error": {"contiguous": rel["contiguous"], "kmeans": rel["kmeans"]}}
        del hcache, hreps, kcache, kreps

    # Representative upkeep of one decode step: every sequence's last token is
    # taken as just appended (lengths one less before), its team refreshed.
    prev = (kv0.seq_lens - 1).clamp(min=0)

    def update_step(i):
        j = i % R
        S.santa_update_reps(cache[j], reps[j], prev, 1)

    r["update_reps_us"], _ = median_graph(update_step, R, steps, warmup, torch)

    # A full build of each kind of representative over one layer's cache (the
    # cost after prefill), into a scratch buffer so the decode reps stay.
    scratch = torch.empty_like(reps[0])
    r["build_reps_us"] = {}
    for kind in (("mean", "medoid", "random") if extras else ()):
        def build_step(i, kind=kind):
            S.santa_build_reps_ex(cache[i % R], kind, reps=scratch, seed=1)

        r["build_reps_us"][kind], _ = median_graph(build_step, R, max(R, steps // 4), warmup // 4, torch)
    if calibrate:
        # Plain device copies of a known size, so rocprofv3 FETCH_SIZE / WRITE_SIZE
        # counters can be scaled (bytes per counter unit).
        src = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
    del cache, reps, wss
    return r


def gbps(nbytes, us):
    return nbytes / (us * 1e-6) / 1e9


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU layout is a "
              f"design note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    import torch
    from sampled_sparse_decode_amd import santa as S, workloads as W

    w = W.FULL_SIZE[args.workload]()
    # The CPU oracle first: its worker processes fork before the GPU is used.
    cpu = None if args.no_cpu else cpu_baseline(w, args.workload, args.cpu_seconds)
    torch.cuda.set_device(torch.device("cuda:0"))
    r = measure(w, args.steps, args.warmup, args.layers, torch, S, args.calibrate, not args.no_extras)
    ab = r["ab"]
    santa_us, dense_us, attend_us = r["santa_us"], r["dense_us"], r["attend_us"]
    attend_gbps = gbps(ab["attend"], attend_us)
    step_gbps = gbps(ab["step"], santa_us)
    dense_gbps = gbps(ab["dense"], dense_us)
    result = {
        "metric": METRIC,
        "value": round(santa_us, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": r["timed_steps"],
        "warmup": args.warmup,
        "ms_per_step": round(santa_us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": int(w.seq_lens.max()),
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "team_size": w.page_size, "M": w.M, "layers_cycled": r["R"]},
        "timing": "HIP-graph replay of one call per layer, median of 3 timed loops of `steps` calls; "
                  "eager stream figures alongside",
        "santa": {"us_per_layer": round(santa_us, 3), "us_per_layer_stream": round(r["santa_stream_us"], 3),
                  "hbm_gbps": round(step_gbps, 1), "pct_peak": round(100 * step_gbps / HBM_PEAK_GBPS, 2),
                  "bytes": ab["step"]},
        "dense": {"us_per_layer": round(dense_us, 3), "us_per_layer_stream": round(r["dense_stream_us"], 3),
                  "hbm_gbps": round(dense_gbps, 1), "pct_peak": round(100 * dense_gbps / HBM_PEAK_GBPS, 2),
                  "bytes": ab["dense"]},
        "speedup_vs_dense": round(dense_us / santa_us, 3),
        "kv_read_fraction": {"per_query_head": round(ab["frac_head"], 4), "hbm": round(ab["frac_hbm"], 4)},
        "team_mass": r["mass"],
        "update_reps_us": round(r["update_reps_us"], 3),
        "build_reps_us": {k: round(v, 2) for k, v in r["build_reps_us"].items()},
        "draw_schemes": r["schemes"],
        "hashed_teams": r["hashed"],
        "kmeans_teams": r["kmeans"],
        "value_sampled": r["value_sampled"],
        "roofline": {"kernel": "gather+combine (santa_attend_selected)", "bound": "hbm",
                     "achieved": round(attend_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(attend_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": recorded_traffic(args.workload),
                     "us_per_launch": round(attend_us, 3), "bytes_per_launch": ab["attend"]},
    }
    # The other configurations, compactly: same timing method, fewer steps.
    scale = {}
    for name in [x for x in args.scale.split(",") if x and x != args.workload]:
        ws = W.FULL_SIZE[name]()
        rs = measure(ws, args.scale_steps, max(10, args.scale_steps // 10), 0, torch, S, extras=not args.no_extras)
        a = rs["ab"]
        scale[name] = {"santa_us": round(rs["santa_us"], 2), "dense_us": round(rs["dense_us"], 2),
                       "speedup_vs_dense": round(rs["dense_us"] / rs["santa_us"], 3),
                       "attend_us": round(rs["attend_us"], 2),
                       "attend_frac_of_peak": round(gbps(a["attend"], rs["attend_us"]) / HBM_PEAK_GBPS, 4),
                       "dense_frac_of_peak": round(gbps(a["dense"], rs["dense_us"]) / HBM_PEAK_GBPS, 4),
                       "kv_read_fraction_hbm": round(a["frac_hbm"], 4), "team_mass": rs["mass"],
                       "build_reps_us": {k: round(v, 2) for k, v in rs["build_reps_us"].items()},
                       "draw_schemes": rs["schemes"],
                       "hashed_teams": rs["hashed"], "kmeans_teams": rs["kmeans"],
                       "value_sampled": rs["value_sampled"]}
        del ws
        torch.cuda.empty_cache()
    if scale:
        result["at_scale"] = scale
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
