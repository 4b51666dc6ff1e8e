"""Seeded synthetic decode workloads (inputs only).

This module builds the inputs that both the HIP path and the CPU oracle are
run on: paged key/value caches, queries, page tables and sequence lengths.
It holds none of the attention method's arithmetic; it only draws random
numbers (numpy's default_rng, seeded) and stores them as plain arrays (the
binding packs pages into the library's tile order on the device).

Layout:
  k_pages           [num_pages][Hkv][T][d]  bfloat16 bit patterns (uint16) or float32
  v_pages           [num_pages][Hkv][T][d]  same type, token-major
  q                 [B][Hq][d]               same storage type as the cache
  page_table        [B][max_pages_per_seq]   int32 physical page of each logical team
  seq_lens          [B]                      int32 tokens per sequence

The workloads stand in for the KV caches of the model the SANTA++ abstract
evaluates (Qwen2.5-7B-Instruct at 32K context: 28 query heads over 4 KV
heads, head dimension 128); no model weights or evaluation data are used.
"""
import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np


@dataclass
class Workload:
    name: str
    dtype: str                 # 'bf16' or 'f32'
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    max_pages_per_seq: int
    k_pages: np.ndarray
    v_pages: np.ndarray
    q: np.ndarray
    page_table: np.ndarray
    seq_lens: np.ndarray
    M: int
    seed: int = 0              # Philox key for the team draws
    offset: int = 0            # Philox counter word 3 (decode step / layer)
    notes: dict = field(default_factory=dict)

    @property
    def num_pages(self):
        return self.k_pages.shape[0]

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self):
        return 2 if self.dtype == "bf16" else 4


def to_storage(x, dtype):
    """float32 array -> storage array: bfloat16 bit patterns (round to nearest even) or float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def storage_to_f32(a, dtype):
    """Storage array -> float32 values (exact)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class _PagedBuilder:
    """Identity-mapped paged cache filled one (sequence, KV head) at a time.

    Sequence b's team t sits at physical page b * P + t, P = ceil(L / T); a
    ragged tail is zero-padded (padding slots are never read).
    """

    def __init__(self, B, hkv, L, T, d, dtype):
        self.B, self.hkv, self.L, self.T, self.d, self.dtype = B, hkv, L, T, d, dtype
        self.P = (L + T - 1) // T
        esz = np.uint16 if dtype == "bf16" else np.float32
        self.k = np.zeros((B * self.P, hkv, T, d), dtype=esz)
        self.v = np.zeros((B * self.P, hkv, T, d), dtype=esz)

    def put(self, which, b, g, x):
        """Store float32 rows x [L][d] of sequence b, KV head g; returns the stored values as float32."""
        P, T, d = self.P, self.T, self.d
        buf = np.zeros((P * T, d), dtype=np.float32)
        buf[:self.L] = x
        st = to_storage(buf, self.dtype)
        (self.k if which == "k" else self.v)[b * P:(b + 1) * P, g] = st.reshape(P, T, d)
        return storage_to_f32(st[:self.L], self.dtype)

    def workload(self, name, q, M, seed=0, offset=0, notes=None):
        B, P = self.B, self.P
        page_table = (np.arange(B, dtype=np.int32)[:, None] * P + np.arange(P, dtype=np.int32)[None, :])
        return Workload(name=name, dtype=self.dtype, batch=B, num_q_heads=q.shape[1], num_kv_heads=self.hkv,
                        head_dim=self.d, page_size=self.T, max_pages_per_seq=P, k_pages=self.k,
                        v_pages=self.v, q=to_storage(q, self.dtype), page_table=page_table.astype(np.int32),
                        seq_lens=np.full(B, self.L, dtype=np.int32), M=M, seed=seed, offset=offset,
                        notes=notes or {})


def _per_chunk(data_seed, B, hkv, fill):
    """Run fill(b, g, rng) for every (sequence, KV head) chunk, in parallel.

    Each chunk draws from its own generator, spawned from ``data_seed`` by
    numpy's SeedSequence, so the result does not depend on thread timing.
    """
    seqs = np.random.SeedSequence(data_seed).spawn(B * hkv)
    jobs = [(b, g, np.random.default_rng(seqs[b * hkv + g])) for b in range(B) for g in range(hkv)]
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda j: fill(*j), jobs))


def _contiguous(name, dtype, keys, vals, q, T, M, seed=0, offset=0, notes=None):
    """Pack logical caches keys, vals [B][Hkv][L][d] (float32) into identity-mapped pages."""
    B, hkv, L, d = keys.shape
    pb = _PagedBuilder(B, hkv, L, T, d, dtype)
    for b in range(B):
        for g in range(hkv):
            pb.put("k", b, g, keys[b, g])
            pb.put("v", b, g, vals[b, g])
    return pb.workload(name, q, M, seed, offset, notes)


def tiny_planted(data_seed=1, n=1024, d=64, T=32, M=8, dtype="f32", philox_seed=0):
    """One query head over N tokens; three planted key rows concentrate attention.

    Keys and values i.i.d. N(0,1); q = 0.5 z + 2 (k_a + k_b + k_c) for three
    distinct uniformly chosen rows a, b, c. Teams of T contiguous tokens.
    """
    rng = np.random.default_rng(data_seed)
    keys = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    vals = rng.standard_normal((1, 1, n, d), dtype=np.float32)
    keys = storage_to_f32(to_storage(keys, dtype), dtype)
    rows = rng.choice(n, size=3, replace=False)
    q = 0.5 * rng.standard_normal((1, 1, d), dtype=np.float32) + 2.0 * keys[0, 0, rows].sum(0)[None, None]
    return _contiguous(f"tiny_{dtype}_n{n}_t{T}_m{M}", dtype, keys, vals, q.astype(np.float32), T, M,
                       seed=philox_seed, notes={"planted_rows": rows.tolist()})


def _channel_scales(rng, hkv, d):
    """Per (KV head, channel) key scale, log-uniform in [0.5, 4]."""
    return np.exp(rng.uniform(np.log(0.5), np.log(4.0), size=(hkv, d))).astype(np.float32)


def qwen_planted(data_seed=2, batch=1, seq_len=32768, T=128, M=31, hq=28, hkv=4, d=128,
                 plants=8, dtype="bf16", philox_seed=0):
    """Qwen2.5-7B-shaped decode layer with planted high-similarity tokens.

    Keys N(0,1) times a per-(KV head, channel) log-uniform [0.5, 4] scale;
    values N(0,1); queries N(0,1). Each query head h gets ``plants`` tokens at
    distinct random positions (distinct across its KV group too) whose key is
    2 q_h + 0.5 z.
    """
    rng = np.random.default_rng(data_seed)
    G = hq // hkv
    scale = _channel_scales(rng, hkv, d)
    q = storage_to_f32(to_storage(rng.standard_normal((batch, hq, d), dtype=np.float32), dtype), dtype)
    pb = _PagedBuilder(batch, hkv, seq_len, T, d, dtype)
    planted = {}

    def fill(b, g, r):
        keys = r.standard_normal((seq_len, d), dtype=np.float32) * scale[g][None, :]
        pos = r.choice(seq_len, size=min(G * plants, seq_len), replace=False)
        for i in range(G):
            h = g * G + i
            ps = pos[i * plants:(i + 1) * plants]
            keys[ps] = 2.0 * q[b, h][None, :] + 0.5 * r.standard_normal((len(ps), d), dtype=np.float32)
            planted[(b, h)] = sorted(int(x) for x in ps)
        pb.put("k", b, g, keys)
        pb.put("v", b, g, r.standard_normal((seq_len, d), dtype=np.float32))

    _per_chunk(data_seed, batch, hkv, fill)
    return pb.workload(f"qwen7b_{dtype}_b{batch}_n{seq_len}_t{T}_m{M}", q, M, seed=philox_seed,
                       notes={"planted": planted})


def qwen_mixed_query(data_seed=3, batch=8, seq_len=32768, T=128, M=32, hq=28, hkv=4, d=128,
                     mix=0.3, dtype="bf16", philox_seed=0):
    """Batch of Qwen2.5-7B-shaped layers with heavy-tailed attention.

    Keys as in qwen_planted (no planted tokens); values N(0,1). Each query is
    (1 - mix) z + mix k_j with z ~ N(0, I) and k_j a uniformly chosen cached
    key of its own sequence and KV head.
    """
    rng = np.random.default_rng(data_seed)
    G = hq // hkv
    scale = _channel_scales(rng, hkv, d)
    q = (1.0 - mix) * rng.standard_normal((batch, hq, d), dtype=np.float32)
    pb = _PagedBuilder(batch, hkv, seq_len, T, d, dtype)

    def fill(b, g, r):
        stored = pb.put("k", b, g, r.standard_normal((seq_len, d), dtype=np.float32) * scale[g][None, :])
        picks = r.integers(0, seq_len, size=G)
        for i in range(G):
            q[b, g * G + i] += mix * stored[picks[i]]
        pb.put("v", b, g, r.standard_normal((seq_len, d), dtype=np.float32))

    _per_chunk(data_seed, batch, hkv, fill)
    return pb.workload(f"qwen7b_mixq_{dtype}_b{batch}_n{seq_len}_t{T}_m{M}", q.astype(np.float32), M,
                       seed=philox_seed)


def gaussian_mixture(data_seed=4, batch=4, seq_len=131072, T=256, M=64, hq=28, hkv=4, d=128,
                     components=64, run_min=64, run_max=2048, dtype="bf16", philox_seed=0):
    """Long-context layer whose keys form semantically coherent runs.

    Per KV head, ``components`` means drawn N(0, 4 I); each sequence is cut
    into contiguous runs of uniform length in [run_min, run_max], each run
    drawn from one uniformly chosen component: key = mean + N(0, I). Values
    and queries N(0,1).
    """
    rng = np.random.default_rng(data_seed)
    means = 2.0 * rng.standard_normal((hkv, components, d), dtype=np.float32)
    q = rng.standard_normal((batch, hq, d), dtype=np.float32)
    pb = _PagedBuilder(batch, hkv, seq_len, T, d, dtype)

    def fill(b, g, r):
        keys = r.standard_normal((seq_len, d), dtype=np.float32)
        pos = 0
        while pos < seq_len:
            run = int(r.integers(run_min, run_max + 1))
            c = int(r.integers(0, components))
            keys[pos:pos + run] += means[g, c][None, :]
            pos += run
        pb.put("k", b, g, keys)
        pb.put("v", b, g, r.standard_normal((seq_len, d), dtype=np.float32))

    _per_chunk(data_seed, batch, hkv, fill)
    return pb.workload(f"mixture_{dtype}_b{batch}_n{seq_len}_t{T}_m{M}", q, M, seed=philox_seed)


def paged_ragged(data_seed=5, num_seqs=16, len_min=4096, len_max=65536, T=128, M=48, hq=28, hkv=4,
                 d=128, sinks=4, sink_scale=8.0, dtype="bf16", philox_seed=0):
    """Ragged batch in a paged cache whose physical pages are in random order.

    Lengths uniform in [len_min, len_max]; keys as in qwen_planted (no planted
    tokens) except that the first ``sinks`` tokens of each sequence have
    their keys multiplied by ``sink_scale``; values and queries N(0,1).
    Teams are pages.
    """
    rng = np.random.default_rng(data_seed)
    scale = _channel_scales(rng, hkv, d)
    lens = rng.integers(len_min, len_max + 1, size=num_seqs).astype(np.int32)
    kb = (lens + T - 1) // T
    total = int(kb.sum())
    P = int(kb.max())
    perm = rng.permutation(total).astype(np.int32)
    page_table = np.zeros((num_seqs, P), dtype=np.int32)
    esz = np.uint16 if dtype == "bf16" else np.float32
    k_pages = np.zeros((total, hkv, T, d), dtype=esz)
    v_pages = np.zeros((total, hkv, T, d), dtype=esz)
    starts = np.concatenate([[0], np.cumsum(kb)[:-1]])
    for b in range(num_seqs):
        page_table[b, :kb[b]] = perm[starts[b]:starts[b] + kb[b]]

    def fill(b, g, r):
        L, K = int(lens[b]), int(kb[b])
        ids = page_table[b, :K]
        keys = r.standard_normal((K * T, d), dtype=np.float32) * scale[g][None, :]
        keys[:sinks] *= sink_scale
        keys[L:] = 0.0
        vals = r.standard_normal((K * T, d), dtype=np.float32)
        vals[L:] = 0.0
        k_pages[ids, g] = to_storage(keys, dtype).reshape(K, T, d)
        v_pages[ids, g] = to_storage(vals, dtype).reshape(K, T, d)

    _per_chunk(data_seed, num_seqs, hkv, fill)
    q = rng.standard_normal((num_seqs, hq, d), dtype=np.float32)
    return Workload(name=f"paged_ragged_{dtype}_s{num_seqs}_t{T}_m{M}", dtype=dtype, batch=num_seqs,
                    num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=T, max_pages_per_seq=P,
                    k_pages=k_pages, v_pages=v_pages, q=to_storage(q, dtype), page_table=page_table,
                    seq_lens=lens, M=M, seed=philox_seed)


# The five workloads at their full sizes, by name.
def hash_directions(data_seed=7, hkv=4, bits=8, d=128):
    """Directions of a hash partition: float32 N(0, 1), [Hkv][bits][d]."""
    return np.random.default_rng(data_seed).standard_normal((hkv, bits, d), dtype=np.float32)


def permuted_workload(w, k_pages, v_pages, suffix="hashed"):
    """A copy of workload w whose pages are replaced (same page table and lengths)."""
    return dataclasses.replace(w, name=f"{w.name}_{suffix}", k_pages=k_pages, v_pages=v_pages)


def kv_head_slice(w, g):
    """A copy of workload w reduced to KV head g and its query heads."""
    G = w.group
    return dataclasses.replace(w, name=f"{w.name}_kvhead{g}", num_q_heads=G, num_kv_heads=1,
                               k_pages=np.ascontiguousarray(w.k_pages[:, g:g + 1]),
                               v_pages=np.ascontiguousarray(w.v_pages[:, g:g + 1]),
                               q=np.ascontiguousarray(w.q[:, g * G:(g + 1) * G]))


FULL_SIZE = {
    "tiny_f32_n1024_m8": lambda: tiny_planted(),
    "qwen7b_32k_b1_m31": lambda: qwen_planted(),
    "qwen7b_32k_b8_m32": lambda: qwen_mixed_query(M=32),
    "qwen7b_32k_b8_m64": lambda: qwen_mixed_query(M=64),
    "mixture_128k_b4_t256_m64": lambda: gaussian_mixture(),
    "paged_ragged_16seq_m48": lambda: paged_ragged(),
}
