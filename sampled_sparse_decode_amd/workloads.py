"""Seeded synthetic decode workloads (inputs only).

This module builds the inputs that both the HIP path and the CPU oracle are
run on: paged key/value caches, queries, page tables and sequence lengths.
It holds none of the attention method's arithmetic; it only draws random
numbers (numpy's default_rng, seeded) and stores them in the library's
layout.

Layout (shared by every entry point of the library):
  k_pages, v_pages  [num_pages][Hkv][T][d]  bfloat16 bit patterns (uint16) or float32
  q                 [B][Hq][d]               same storage type as the cache
  page_table        [B][max_pages_per_seq]   int32 physical page of each logical team
  seq_lens          [B]                      int32 tokens per sequence

The workloads stand in for the KV caches of the model the SANTA++ abstract
evaluates (Qwen2.5-7B-Instruct at 32K context: 28 query heads over 4 KV
heads, head dimension 128); no model weights or evaluation data are used.
"""
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


def _contiguous(name, dtype, keys, vals, q, T, M, seed=0, offset=0, notes=None):
    """Pack logical caches [B][Hkv][L][d] into identity-mapped pages.

    Sequence b's team t sits at physical page b * P + t, P = ceil(L / T); a
    ragged tail is zero-padded (padding slots are never read).
    """
    B, hkv, L, d = keys.shape
    P = (L + T - 1) // T
    pad = P * T - L
    if pad:
        z = np.zeros((B, hkv, pad, d), dtype=np.float32)
        keys = np.concatenate([keys, z], axis=2)
        vals = np.concatenate([vals, z], axis=2)

    def pages(x):
        x = x.reshape(B, hkv, P, T, d).transpose(0, 2, 1, 3, 4)
        return to_storage(x.reshape(B * P, hkv, T, d), dtype)

    page_table = (np.arange(B, dtype=np.int32)[:, None] * P + np.arange(P, dtype=np.int32)[None, :]).astype(np.int32)
    return Workload(name=name, dtype=dtype, batch=B, num_q_heads=q.shape[1], num_kv_heads=hkv,
                    head_dim=d, page_size=T, max_pages_per_seq=P, k_pages=pages(keys),
                    v_pages=pages(vals), q=to_storage(q, dtype), page_table=page_table,
                    seq_lens=np.full(B, L, dtype=np.int32), M=M, seed=seed, offset=offset,
                    notes=notes or {})


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
    keys = rng.standard_normal((batch, hkv, seq_len, d), dtype=np.float32) * scale[None, :, None, :]
    vals = rng.standard_normal((batch, hkv, seq_len, d), dtype=np.float32)
    q = storage_to_f32(to_storage(rng.standard_normal((batch, hq, d), dtype=np.float32), dtype), dtype)
    planted = {}
    for b in range(batch):
        for g in range(hkv):
            pos = rng.choice(seq_len, size=min(G * plants, seq_len), replace=False)
            for i in range(G):
                h = g * G + i
                ps = pos[i * plants:(i + 1) * plants]
                keys[b, g, ps] = 2.0 * q[b, h][None, :] + 0.5 * rng.standard_normal((len(ps), d), dtype=np.float32)
                planted[(b, h)] = sorted(int(x) for x in ps)
    return _contiguous(f"qwen7b_{dtype}_b{batch}_n{seq_len}_t{T}_m{M}", dtype, keys, vals, q, T, M,
                       seed=philox_seed, notes={"planted": planted})


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
    keys = rng.standard_normal((batch, hkv, seq_len, d), dtype=np.float32) * scale[None, :, None, :]
    keys = storage_to_f32(to_storage(keys, dtype), dtype)
    vals = rng.standard_normal((batch, hkv, seq_len, d), dtype=np.float32)
    q = (1.0 - mix) * rng.standard_normal((batch, hq, d), dtype=np.float32)
    picks = rng.integers(0, seq_len, size=(batch, hq))
    for b in range(batch):
        for h in range(hq):
            q[b, h] += mix * keys[b, h // G, picks[b, h]]
    return _contiguous(f"qwen7b_mixq_{dtype}_b{batch}_n{seq_len}_t{T}_m{M}", dtype, keys, vals,
                       q.astype(np.float32), T, M, seed=philox_seed)


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
    keys = rng.standard_normal((batch, hkv, seq_len, d), dtype=np.float32)
    for b in range(batch):
        for g in range(hkv):
            pos = 0
            while pos < seq_len:
                run = int(rng.integers(run_min, run_max + 1))
                c = int(rng.integers(0, components))
                keys[b, g, pos:pos + run] += means[g, c][None, :]
                pos += run
    vals = rng.standard_normal((batch, hkv, seq_len, d), dtype=np.float32)
    q = rng.standard_normal((batch, hq, d), dtype=np.float32)
    return _contiguous(f"mixture_{dtype}_b{batch}_n{seq_len}_t{T}_m{M}", dtype, keys, vals, q, T, M,
                       seed=philox_seed)


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
    start = 0
    for b in range(num_seqs):
        L, K = int(lens[b]), int(kb[b])
        ids = perm[start:start + K]
        start += K
        page_table[b, :K] = ids
        keys = rng.standard_normal((hkv, K * T, d), dtype=np.float32) * scale[:, None, :]
        keys[:, :sinks] *= sink_scale
        keys[:, L:] = 0.0
        vals = rng.standard_normal((hkv, K * T, d), dtype=np.float32)
        vals[:, L:] = 0.0
        k_pages[ids] = to_storage(keys.reshape(hkv, K, T, d).transpose(1, 0, 2, 3), dtype)
        v_pages[ids] = to_storage(vals.reshape(hkv, K, T, d).transpose(1, 0, 2, 3), dtype)
    q = rng.standard_normal((num_seqs, hq, d), dtype=np.float32)
    return Workload(name=f"paged_ragged_{dtype}_s{num_seqs}_t{T}_m{M}", dtype=dtype, batch=num_seqs,
                    num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=T, max_pages_per_seq=P,
                    k_pages=k_pages, v_pages=v_pages, q=to_storage(q, dtype), page_table=page_table,
                    seq_lens=lens, M=M, seed=philox_seed)


# The five workloads at their full sizes, by name.
FULL_SIZE = {
    "tiny_f32_n1024_m8": lambda: tiny_planted(),
    "qwen7b_32k_b1_m31": lambda: qwen_planted(),
    "qwen7b_32k_b8_m32": lambda: qwen_mixed_query(M=32),
    "qwen7b_32k_b8_m64": lambda: qwen_mixed_query(M=64),
    "mixture_128k_b4_t256_m64": lambda: gaussian_mixture(),
    "paged_ragged_16seq_m48": lambda: paged_ragged(),
}
