"""ctypes binding of libsanta (include/santa.h), same names as the C ABI.

Argument marshalling only: torch tensors become device pointers, the
current torch stream becomes the HIP stream, and a non-zero status becomes a
``SantaError``. Every step of the computation runs in the library's HIP
kernels; there is no fallback path, and a missing library raises.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsanta.so")

SANTA_F32 = 0
SANTA_BF16 = 1
_DTYPES = {torch.float32: SANTA_F32, torch.bfloat16: SANTA_BF16}

EXPORTED = (
    "santa_workspace_size",
    "santa_value_sampled_workspace_size",
    "santa_build_reps",
    "santa_update_reps",
    "santa_append_kv",
    "santa_build_reps_ex",
    "santa_decode_attention",
    "santa_decode_attention_ex",
    "santa_decode_attention_noalloc",
    "santa_decode_attention_value_sampled",
    "santa_select_teams",
    "santa_select_teams_ex",
    "santa_attend_selected",
    "dense_decode_attention",
    "santa_attention_given_teams",
    "santa_pack_pages",
    "santa_pack_pages_hashed",
    "santa_kmeans_workspace_size",
    "santa_pack_pages_kmeans",
    "santa_status_string",
    "santa_version",
)


class SantaError(RuntimeError):
    """A libsanta entry point returned a non-zero status."""

    def __init__(self, func, status, text):
        super().__init__(f"{func} failed with status {status}: {text}")
        self.status = status


class santa_kv(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
    ]


_lib = None


def load():
    """Load libsanta.so (built in-tree) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m sampled_sparse_decode_amd.build")
    _lib = declare_signatures(ctypes.CDLL(LIB_PATH))
    return _lib


def declare_signatures(lib):
    """Set the argument and result types of every exported entry point on a
    ctypes handle of a libsanta build; returns it."""
    P = ctypes.c_void_p
    kvp = ctypes.POINTER(santa_kv)
    i32, u32, u64, sz = ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t
    sigs = {
        "santa_workspace_size": (i32, [kvp, i32, ctypes.POINTER(sz)]),
        "santa_value_sampled_workspace_size": (i32, [kvp, i32, ctypes.POINTER(sz)]),
        "santa_build_reps": (i32, [kvp, P, P]),
        "santa_update_reps": (i32, [kvp, P, P, i32, P]),
        "santa_append_kv": (i32, [kvp, P, P, P, i32, P]),
        "santa_build_reps_ex": (i32, [kvp, P, i32, u64, P, i32, P]),
        "santa_decode_attention": (i32, [kvp, P, P, i32, u64, u32, P, P, P, P, P, sz, P]),
        "santa_decode_attention_ex": (i32, [kvp, P, P, i32, u64, u32, i32, P, P, P, P, P, sz, P]),
        "santa_decode_attention_noalloc": (i32, [kvp, P, P, i32, u64, u32, P, P, P, P, P]),
        "santa_decode_attention_value_sampled": (i32, [kvp, P, P, i32, i32, i32, i32, u64, u32, P, P, P, P, P,
                                                       P, sz, P]),
        "santa_select_teams": (i32, [kvp, P, P, i32, u64, u32, P, P, P, sz, P]),
        "santa_select_teams_ex": (i32, [kvp, P, P, i32, u64, u32, i32, P, P, P, sz, P]),
        "santa_attend_selected": (i32, [kvp, P, i32, P, P, P, sz, P]),
        "dense_decode_attention": (i32, [kvp, P, P, P, P, sz, P]),
        "santa_attention_given_teams": (i32, [kvp, P, i32, P, P, P, P, P, sz, P]),
        "santa_pack_pages": (i32, [i32, ctypes.c_int64, i32, i32, i32, P, P, P, P, P]),
        "santa_pack_pages_hashed": (i32, [kvp, P, P, P, i32, P, P, P]),
        "santa_kmeans_workspace_size": (i32, [kvp, i32, ctypes.POINTER(sz)]),
        "santa_pack_pages_kmeans": (i32, [kvp, P, P, i32, i32, P, P, P, sz, P]),
        "santa_status_string": (ctypes.c_char_p, [i32]),
        "santa_version": (i32, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def santa_status_string(status):
    return load().santa_status_string(int(status)).decode()


def santa_version():
    return load().santa_version()


def _check(func, status):
    if status != 0:
        raise SantaError(func, status, santa_status_string(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class KVCache:
    """A paged KV cache on the device, in the layout of include/santa.h.

    k_pages, v_pages: [num_pages][Hkv][T * d] tiles in the library's tile
    order (write them with pack_pages), bfloat16 or float32; page_table
    [B][max_pages_per_seq] int32; seq_lens [B] int32.
    """

    def __init__(self, k_pages, v_pages, page_table, seq_lens, num_q_heads, page_size):
        for t in (k_pages, v_pages, page_table, seq_lens):
            if not t.is_contiguous():
                raise ValueError("KV cache tensors must be contiguous")
        if k_pages.dtype not in _DTYPES or v_pages.dtype != k_pages.dtype:
            raise ValueError("k_pages / v_pages must both be bfloat16 or float32")
        if page_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
            raise ValueError("page_table and seq_lens must be int32")
        if k_pages.dim() != 3 or v_pages.shape != k_pages.shape or k_pages.shape[2] % int(page_size):
            raise ValueError("k_pages and v_pages must both be [num_pages][Hkv][T * d] tiles")
        self.k_pages, self.v_pages = k_pages, v_pages
        self.page_table, self.seq_lens = page_table, seq_lens
        self.num_q_heads = int(num_q_heads)
        self.num_pages, self.num_kv_heads = int(k_pages.shape[0]), int(k_pages.shape[1])
        self.page_size = int(page_size)
        self.head_dim = int(k_pages.shape[2]) // self.page_size
        self.batch, self.max_pages_per_seq = (int(x) for x in page_table.shape)
        self.dtype = k_pages.dtype
        self.device = k_pages.device

    def desc(self):
        return santa_kv(_DTYPES[self.dtype], self.batch, self.num_q_heads, self.num_kv_heads,
                        self.head_dim, self.page_size, self.max_pages_per_seq, 0, self.num_pages,
                        self.k_pages.data_ptr(), self.v_pages.data_ptr(),
                        self.page_table.data_ptr(), self.seq_lens.data_ptr())


def pack_pages(k_src, v_src, k_dst=None, v_dst=None):
    """Pages [num_pages][Hkv][T][d] -> tiles [num_pages][Hkv][T * d] in the cache's tile order."""
    if k_src.dim() != 4 or v_src.shape != k_src.shape or k_src.dtype not in _DTYPES or v_src.dtype != k_src.dtype:
        raise ValueError("k_src and v_src must be [num_pages][Hkv][T][d] of one cache dtype")
    if not (k_src.is_contiguous() and v_src.is_contiguous()):
        raise ValueError("k_src and v_src must be contiguous")
    n, hkv, T, d = (int(x) for x in k_src.shape)
    if k_dst is None:
        k_dst = torch.empty((n, hkv, T * d), dtype=k_src.dtype, device=k_src.device)
    if v_dst is None:
        v_dst = torch.empty((n, hkv, T * d), dtype=k_src.dtype, device=k_src.device)
    _check("santa_pack_pages", load().santa_pack_pages(_DTYPES[k_src.dtype], n, hkv, T, d, _ptr(k_src), _ptr(v_src),
                                                      _ptr(k_dst), _ptr(v_dst), _stream()))
    return k_dst, v_dst


def _partition_outputs(kv, k_src, v_src, codes, token_of):
    """Checks the plain source pages of a re-partitioning pack and returns the
    (codes, token_of) output tensors, allocated when not given."""
    if k_src.shape != (kv.num_pages, kv.num_kv_heads, kv.page_size, kv.head_dim) or v_src.shape != k_src.shape:
        raise ValueError("k_src and v_src must be [num_pages][Hkv][T][d]")
    if k_src.dtype != kv.dtype or v_src.dtype != kv.dtype or not (k_src.is_contiguous() and v_src.is_contiguous()):
        raise ValueError("k_src and v_src must be contiguous tensors of the cache dtype")
    if k_src.device != kv.device or v_src.device != kv.device:
        raise ValueError("k_src and v_src must be on the cache's device")
    shape = (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq * kv.page_size)
    _check_tensor("codes", codes, shape, torch.int32, kv.device)
    _check_tensor("token_of", token_of, shape, torch.int32, kv.device)
    if codes is None:
        codes = torch.empty(shape, dtype=torch.int32, device=kv.device)
    if token_of is None:
        token_of = torch.empty(shape, dtype=torch.int32, device=kv.device)
    return codes, token_of


def santa_pack_pages_hashed(kv, k_src, v_src, directions, codes=None, token_of=None):
    """Write kv's pages from plain pages k_src / v_src [num_pages][Hkv][T][d]
    in hash-partition order for directions [Hkv][bits][d] (float32).
    Returns (codes, token_of), each [B][Hkv][P*T] int32."""
    if (directions.dtype != torch.float32 or directions.dim() != 3 or not directions.is_contiguous()
            or directions.shape[0] != kv.num_kv_heads or directions.shape[2] != kv.head_dim):
        raise ValueError("directions must be a contiguous float32 [Hkv][bits][d] tensor")
    if directions.device != kv.device:
        raise ValueError("directions must be on the cache's device")
    codes, token_of = _partition_outputs(kv, k_src, v_src, codes, token_of)
    d = kv.desc()
    _check("santa_pack_pages_hashed",
           load().santa_pack_pages_hashed(ctypes.byref(d), _ptr(k_src), _ptr(v_src), _ptr(directions),
                                          int(directions.shape[1]), _ptr(codes), _ptr(token_of), _stream()))
    return codes, token_of


def santa_kmeans_workspace_size(kv, clusters=0):
    """Bytes of workspace santa_pack_pages_kmeans needs for `clusters`."""
    n = ctypes.c_size_t(0)
    d = kv.desc()
    _check("santa_kmeans_workspace_size", load().santa_kmeans_workspace_size(ctypes.byref(d), int(clusters), ctypes.byref(n)))
    return n.value


def santa_pack_pages_kmeans(kv, k_src, v_src, clusters=0, iters=10, codes=None, token_of=None, workspace=None):
    """Write kv's pages from plain pages k_src / v_src [num_pages][Hkv][T][d]
    in the order of a k-means partition of each sequence's keys (`clusters`
    per sequence, 0 for one per team; `iters` assignments). Returns (codes,
    token_of), each [B][Hkv][P*T] int32; codes are cluster ids."""
    codes, token_of = _partition_outputs(kv, k_src, v_src, codes, token_of)
    need = santa_kmeans_workspace_size(kv, clusters)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=kv.device)
    elif (workspace.device != kv.device or not workspace.is_contiguous()
          or workspace.numel() * workspace.element_size() < need):
        raise ValueError(f"workspace must be a contiguous buffer of at least {need} bytes on the cache's device")
    d = kv.desc()
    _check("santa_pack_pages_kmeans",
           load().santa_pack_pages_kmeans(ctypes.byref(d), _ptr(k_src), _ptr(v_src), int(clusters), int(iters),
                                          _ptr(codes), _ptr(token_of), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream()))
    return codes, token_of


def kv_from_workload_kmeans(w, clusters=0, iters=10, device="cuda"):
    """Upload a workload and pack its pages in k-means order.
    Returns (KVCache, q tensor, codes, token_of)."""
    k_src = storage_tensor(w.k_pages, w.dtype, device)
    v_src = storage_tensor(w.v_pages, w.dtype, device)
    kv = _empty_cache_like(w, k_src, device)
    codes, token_of = santa_pack_pages_kmeans(kv, k_src, v_src, clusters, iters)
    torch.cuda.current_stream().synchronize()
    del k_src, v_src
    return kv, storage_tensor(w.q, w.dtype, device), codes, token_of


def _empty_cache_like(w, k_src, device):
    """A zeroed destination cache with the workload's page table and lengths."""
    n, hkv, T, d = (int(x) for x in k_src.shape)
    return KVCache(torch.zeros((n, hkv, T * d), dtype=k_src.dtype, device=device),
                   torch.zeros((n, hkv, T * d), dtype=k_src.dtype, device=device),
                   torch.from_numpy(np.ascontiguousarray(w.page_table, dtype=np.int32)).to(device),
                   torch.from_numpy(np.ascontiguousarray(w.seq_lens, dtype=np.int32)).to(device),
                   w.num_q_heads, w.page_size)


def kv_from_workload_hashed(w, directions, device="cuda"):
    """Upload a workload and pack its pages in hash-partition order.
    Returns (KVCache, q tensor, codes, token_of)."""
    k_src = storage_tensor(w.k_pages, w.dtype, device)
    v_src = storage_tensor(w.v_pages, w.dtype, device)
    kv = _empty_cache_like(w, k_src, device)
    dirs = torch.from_numpy(np.ascontiguousarray(directions, dtype=np.float32)).to(device)
    codes, token_of = santa_pack_pages_hashed(kv, k_src, v_src, dirs)
    torch.cuda.current_stream().synchronize()
    del k_src, v_src
    return kv, storage_tensor(w.q, w.dtype, device), codes, token_of


def storage_tensor(arr, dtype, device):
    """numpy storage array (uint16 bfloat16 bits or float32) -> torch tensor on ``device``."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def kv_from_workload(w, device="cuda"):
    """Upload a workloads.Workload (pages [num_pages][Hkv][T][d]) and pack its
    pages into the cache's tile order; returns (KVCache, q tensor)."""
    k_src = storage_tensor(w.k_pages, w.dtype, device)
    v_src = storage_tensor(w.v_pages, w.dtype, device)
    k_pages, v_pages = pack_pages(k_src, v_src)
    torch.cuda.current_stream().synchronize()
    del k_src, v_src
    kv = KVCache(k_pages, v_pages,
                 torch.from_numpy(np.ascontiguousarray(w.page_table, dtype=np.int32)).to(device),
                 torch.from_numpy(np.ascontiguousarray(w.seq_lens, dtype=np.int32)).to(device),
                 w.num_q_heads, w.page_size)
    return kv, storage_tensor(w.q, w.dtype, device)


def santa_workspace_size(kv, M):
    n = ctypes.c_size_t(0)
    d = kv.desc()
    _check("santa_workspace_size", load().santa_workspace_size(ctypes.byref(d), int(M), ctypes.byref(n)))
    return n.value


def make_workspace(kv, M=1):
    return torch.empty(santa_workspace_size(kv, M), dtype=torch.uint8, device=kv.device)


def santa_value_sampled_workspace_size(kv, M):
    d = kv.desc()
    n = ctypes.c_size_t(0)
    _check("santa_value_sampled_workspace_size",
           load().santa_value_sampled_workspace_size(ctypes.byref(d), int(M), ctypes.byref(n)))
    return n.value


def make_value_sampled_workspace(kv, M):
    return torch.empty(santa_value_sampled_workspace_size(kv, M), dtype=torch.uint8, device=kv.device)


def santa_build_reps(kv, reps=None):
    """Mean key per (sequence, team, KV head), rounded to the cache dtype: [B][P][Hkv][d]."""
    if reps is None:
        reps = torch.zeros((kv.batch, kv.max_pages_per_seq, kv.num_kv_heads, kv.head_dim), dtype=kv.dtype,
                           device=kv.device)
    _check_reps(kv, reps)
    d = kv.desc()
    _check("santa_build_reps", load().santa_build_reps(ctypes.byref(d), _ptr(reps), _stream()))
    return reps


def santa_update_reps(kv, reps, prev_seq_lens, max_new_tokens):
    """Refresh the representatives of the teams that received tokens since the
    sequence lengths were ``prev_seq_lens`` (device int32 [B])."""
    if prev_seq_lens.dtype != torch.int32 or tuple(prev_seq_lens.shape) != (kv.batch,):
        raise ValueError("prev_seq_lens must be an int32 [B] tensor")
    _check_reps(kv, reps)
    d = kv.desc()
    _check("santa_update_reps", load().santa_update_reps(ctypes.byref(d), _ptr(reps), _ptr(prev_seq_lens),
                                                        int(max_new_tokens), _stream()))
    return reps


def santa_append_kv(kv, prev_seq_lens, k_new, v_new):
    """Write appended tokens into the cache's tile layout: for each sequence
    b, the tokens at positions prev_seq_lens[b] .. kv.seq_lens[b] - 1 come
    from rows 0, 1, ... of k_new[b] / v_new[b] ([B][max_new][Hkv][d], the
    cache dtype). kv.seq_lens must already hold the new lengths."""
    if prev_seq_lens.dtype != torch.int32 or tuple(prev_seq_lens.shape) != (kv.batch,):
        raise ValueError("prev_seq_lens must be an int32 [B] tensor")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if (t.dim() != 4 or t.shape[0] != kv.batch or t.shape[2] != kv.num_kv_heads or t.shape[3] != kv.head_dim
                or t.dtype != kv.dtype or t.device != kv.device or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous [B, max_new, Hkv, d] tensor of the cache's dtype "
                             f"on its device")
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must have the same shape")
    d = kv.desc()
    _check("santa_append_kv", load().santa_append_kv(ctypes.byref(d), _ptr(prev_seq_lens), _ptr(k_new),
                                                    _ptr(v_new), int(k_new.shape[1]), _stream()))


REP_MEAN, REP_MEDOID, REP_RANDOM = 0, 1, 2
_REP_KINDS = {"mean": REP_MEAN, "medoid": REP_MEDOID, "random": REP_RANDOM}


def santa_build_reps_ex(kv, kind, reps=None, seed=0, prev_seq_lens=None, max_new_tokens=0):
    """Representatives of kind "mean", "medoid" or "random" (or its integer
    code): [B][P][Hkv][d]. With ``prev_seq_lens`` only the teams that received
    tokens since those lengths are refreshed, as in santa_update_reps."""
    code = _REP_KINDS.get(kind, kind) if isinstance(kind, str) else int(kind)
    if isinstance(code, str):
        raise ValueError(f"unknown representative kind {kind!r}")
    if reps is None:
        reps = torch.zeros((kv.batch, kv.max_pages_per_seq, kv.num_kv_heads, kv.head_dim), dtype=kv.dtype,
                           device=kv.device)
    if prev_seq_lens is not None and (prev_seq_lens.dtype != torch.int32
                                      or tuple(prev_seq_lens.shape) != (kv.batch,)):
        raise ValueError("prev_seq_lens must be an int32 [B] tensor")
    _check_reps(kv, reps)
    d = kv.desc()
    _check("santa_build_reps_ex",
           load().santa_build_reps_ex(ctypes.byref(d), _ptr(reps), code, int(seed) & (2**64 - 1),
                                      _ptr(prev_seq_lens) if prev_seq_lens is not None else None,
                                      int(max_new_tokens), _stream()))
    return reps


def _check_tensor(name, t, shape, dtype, device):
    """A caller-provided buffer must match exactly: the library reads and
    writes through its pointer with the sizes of the cache descriptor."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _check_reps(kv, reps):
    if reps is None:
        raise ValueError("reps is required")
    _check_tensor("reps", reps, (kv.batch, kv.max_pages_per_seq, kv.num_kv_heads, kv.head_dim), kv.dtype, kv.device)


def _check_outputs(kv, out=None, lse=None):
    _check_tensor("out", out, (kv.batch, kv.num_q_heads, kv.head_dim), torch.float32, kv.device)
    _check_tensor("lse", lse, (kv.batch, kv.num_q_heads), torch.float32, kv.device)


def _check_sets(kv, M, sampled, inv_pi):
    _check_tensor("sampled", sampled, (kv.batch, kv.num_q_heads, int(M)), torch.int32, kv.device)
    _check_tensor("inv_pi", inv_pi, (kv.batch, kv.num_q_heads, int(M)), torch.float32, kv.device)


def _check_workspace(workspace, kv):
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()
                                  or workspace.device != kv.device):
        raise ValueError("workspace must be a contiguous uint8 tensor on the cache's device")


def _check_q(kv, q):
    if (q.dtype != kv.dtype or not q.is_contiguous() or tuple(q.shape) != (kv.batch, kv.num_q_heads, kv.head_dim)
            or q.device != kv.device):
        raise ValueError("q must be a contiguous [B][Hq][d] tensor of the cache dtype on the cache's device")


DRAW_IID, DRAW_SYSTEMATIC, DRAW_STRATIFIED = 0, 1, 2
_SCHEMES = {"iid": DRAW_IID, "systematic": DRAW_SYSTEMATIC, "stratified": DRAW_STRATIFIED}


def _scheme_code(scheme):
    if isinstance(scheme, str):
        if scheme not in _SCHEMES:
            raise ValueError(f"unknown draw scheme {scheme!r}")
        return _SCHEMES[scheme]
    return int(scheme)


def santa_decode_attention(kv, q, reps, M, seed=0, offset=0, workspace=None, out=None, lse=None,
                           return_sets=False):
    """SANTA++ decode attention. Returns (out, lse) or (out, lse, sampled, inv_pi)."""
    return _decode(kv, q, reps, M, seed, offset, None, workspace, out, lse, return_sets)


def santa_decode_attention_ex(kv, q, reps, M, scheme, seed=0, offset=0, workspace=None, out=None, lse=None,
                              return_sets=False):
    """santa_decode_attention with a draw scheme: "iid", "systematic" or "stratified"."""
    return _decode(kv, q, reps, M, seed, offset, _scheme_code(scheme), workspace, out, lse, return_sets)


def _decode(kv, q, reps, M, seed, offset, scheme, workspace, out, lse, return_sets):
    _check_q(kv, q)
    _check_reps(kv, reps)
    _check_outputs(kv, out, lse)
    _check_workspace(workspace, kv)
    B, Hq, d = kv.batch, kv.num_q_heads, kv.head_dim
    dev = kv.device
    if workspace is None:
        workspace = make_workspace(kv, M)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    sampled = inv_pi = None
    if return_sets:
        sampled = torch.empty((B, Hq, M), dtype=torch.int32, device=dev)
        inv_pi = torch.empty((B, Hq, M), dtype=torch.float32, device=dev)
    desc = kv.desc()
    if scheme is None:
        st = load().santa_decode_attention(ctypes.byref(desc), _ptr(q), _ptr(reps), int(M), int(seed), int(offset),
                                           _ptr(out), _ptr(lse), _ptr(sampled), _ptr(inv_pi),
                                           _ptr(workspace), workspace.numel(), _stream())
        _check("santa_decode_attention", st)
    else:
        st = load().santa_decode_attention_ex(ctypes.byref(desc), _ptr(q), _ptr(reps), int(M), int(seed),
                                              int(offset), scheme, _ptr(out), _ptr(lse), _ptr(sampled),
                                              _ptr(inv_pi), _ptr(workspace), workspace.numel(), _stream())
        _check("santa_decode_attention_ex", st)
    if return_sets:
        return out, lse, sampled, inv_pi
    return out, lse


def santa_decode_attention_value_sampled(kv, q, reps, M, S, scheme="iid", value_scheme="iid", seed=0, offset=0,
                                         workspace=None, out=None, lse=None, return_sets=False,
                                         return_positions=False):
    """SANTA++ team draws, then S value samples inside the drawn teams (the
    mean of the sampled tokens' values). Returns (out, lse), followed by
    (sampled, inv_pi) when return_sets and by positions [B][Hq][S] when
    return_positions."""
    _check_q(kv, q)
    _check_reps(kv, reps)
    _check_outputs(kv, out, lse)
    _check_workspace(workspace, kv)
    B, Hq, d = kv.batch, kv.num_q_heads, kv.head_dim
    dev = kv.device
    if workspace is None:
        workspace = make_value_sampled_workspace(kv, M)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    sampled = inv_pi = positions = None
    if return_sets:
        sampled = torch.empty((B, Hq, M), dtype=torch.int32, device=dev)
        inv_pi = torch.empty((B, Hq, M), dtype=torch.float32, device=dev)
    if return_positions:
        positions = torch.empty((B, Hq, max(int(S), 1)), dtype=torch.int32, device=dev)
    desc = kv.desc()
    st = load().santa_decode_attention_value_sampled(
        ctypes.byref(desc), _ptr(q), _ptr(reps), int(M), _scheme_code(scheme), int(S), _scheme_code(value_scheme),
        int(seed), int(offset), _ptr(out), _ptr(lse), _ptr(sampled), _ptr(inv_pi), _ptr(positions),
        _ptr(workspace), workspace.numel(), _stream())
    _check("santa_decode_attention_value_sampled", st)
    res = (out, lse)
    if return_sets:
        res += (sampled, inv_pi)
    if return_positions:
        res += (positions,)
    return res


def santa_decode_attention_noalloc(kv, q, reps, M, seed=0, offset=0, out=None, lse=None, sampled=None,
                                   inv_pi=None):
    """santa_decode_attention on the library's own device scratch (no workspace
    argument; the call allocates nothing). Outputs not given are allocated
    here, before the call. Returns (out, lse, sampled, inv_pi); the last two
    are None unless given."""
    _check_q(kv, q)
    _check_reps(kv, reps)
    _check_outputs(kv, out, lse)
    _check_sets(kv, M, sampled, inv_pi)
    B, Hq, d = kv.batch, kv.num_q_heads, kv.head_dim
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=kv.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=kv.device)
    desc = kv.desc()
    st = load().santa_decode_attention_noalloc(ctypes.byref(desc), _ptr(q), _ptr(reps), int(M), int(seed),
                                               int(offset), _ptr(out), _ptr(lse), _ptr(sampled), _ptr(inv_pi),
                                               _stream())
    _check("santa_decode_attention_noalloc", st)
    return out, lse, sampled, inv_pi


def santa_select_teams(kv, q, reps, M, seed, offset, workspace, sampled=None, inv_pi=None):
    """Steps 1-4 of SANTA++ into ``workspace`` (and sampled / inv_pi when given)."""
    _check_q(kv, q)
    _check_reps(kv, reps)
    _check_sets(kv, M, sampled, inv_pi)
    _check_workspace(workspace, kv)
    desc = kv.desc()
    st = load().santa_select_teams(ctypes.byref(desc), _ptr(q), _ptr(reps), int(M), int(seed), int(offset),
                                   _ptr(sampled), _ptr(inv_pi), _ptr(workspace), workspace.numel(), _stream())
    _check("santa_select_teams", st)


def santa_select_teams_ex(kv, q, reps, M, scheme, seed, offset, workspace, sampled=None, inv_pi=None):
    """santa_select_teams with a draw scheme: "iid", "systematic" or "stratified"."""
    _check_q(kv, q)
    _check_reps(kv, reps)
    _check_sets(kv, M, sampled, inv_pi)
    _check_workspace(workspace, kv)
    desc = kv.desc()
    st = load().santa_select_teams_ex(ctypes.byref(desc), _ptr(q), _ptr(reps), int(M), int(seed), int(offset),
                                      _scheme_code(scheme), _ptr(sampled), _ptr(inv_pi), _ptr(workspace),
                                      workspace.numel(), _stream())
    _check("santa_select_teams_ex", st)


def santa_attend_selected(kv, q, M, workspace, out, lse=None):
    """Step 5 of SANTA++ over the teams the last santa_select_teams left in ``workspace``."""
    _check_q(kv, q)
    _check_outputs(kv, out, lse)
    _check_workspace(workspace, kv)
    desc = kv.desc()
    st = load().santa_attend_selected(ctypes.byref(desc), _ptr(q), int(M), _ptr(out), _ptr(lse),
                                      _ptr(workspace), workspace.numel(), _stream())
    _check("santa_attend_selected", st)
    return out, lse


def dense_decode_attention(kv, q, workspace=None, out=None, lse=None):
    """Dense decode attention over every cached token. Returns (out, lse)."""
    _check_q(kv, q)
    _check_outputs(kv, out, lse)
    _check_workspace(workspace, kv)
    B, Hq, d = kv.batch, kv.num_q_heads, kv.head_dim
    if workspace is None:
        workspace = make_workspace(kv, 1)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=kv.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=kv.device)
    desc = kv.desc()
    st = load().dense_decode_attention(ctypes.byref(desc), _ptr(q), _ptr(out), _ptr(lse),
                                       _ptr(workspace), workspace.numel(), _stream())
    _check("dense_decode_attention", st)
    return out, lse


def santa_attention_given_teams(kv, q, teams, weights, workspace=None, out=None, lse=None):
    """Estimator over caller-chosen teams [B][Hq][M] (int32, -1 unused) and weights (float32)."""
    _check_q(kv, q)
    _check_outputs(kv, out, lse)
    _check_workspace(workspace, kv)
    B, Hq, d = kv.batch, kv.num_q_heads, kv.head_dim
    M = int(teams.shape[-1])
    if teams.dtype != torch.int32 or weights.dtype != torch.float32 or tuple(teams.shape) != (B, Hq, M) \
            or tuple(weights.shape) != (B, Hq, M):
        raise ValueError("teams must be int32 [B][Hq][M] and weights float32 [B][Hq][M]")
    if workspace is None:
        workspace = make_workspace(kv, M)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=kv.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=kv.device)
    desc = kv.desc()
    st = load().santa_attention_given_teams(ctypes.byref(desc), _ptr(q), M, _ptr(teams.contiguous()),
                                            _ptr(weights.contiguous()), _ptr(out), _ptr(lse),
                                            _ptr(workspace), workspace.numel(), _stream())
    _check("santa_attention_given_teams", st)
    return out, lse
