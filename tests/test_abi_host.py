"""Host-side checks of the C ABI: the library loads, exports every function
include/santa.h declares, sizes its workspace, and rejects bad arguments
with the documented status before making any HIP call (so these run
without a GPU; no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from sampled_sparse_decode_amd import santa as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "santa.h")

OK, NULL, SHAPE, UNSUP, WS = 0, 1, 2, 3, 4
S_F32 = 0
FAKE = 0x10000      # non-NULL pointer value; never dereferenced by validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


# SANTA_TEST_LIB names another build of the same C ABI to check (the
# host-only sanitizer build of tests/test_host_sanitized.py); default: the
# library the binding loads.
TEST_LIB = os.environ.get("SANTA_TEST_LIB")


@pytest.fixture(scope="module")
def lib():
    if TEST_LIB:
        return S.declare_signatures(ctypes.CDLL(TEST_LIB))
    if not os.path.exists(S.LIB_PATH):
        pytest.skip("libsanta.so not built")
    return S.load()


def kv(**over):
    d = dict(dtype=S.SANTA_BF16, batch=2, num_q_heads=28, num_kv_heads=4, head_dim=128, page_size=128,
             max_pages_per_seq=256, reserved=0, num_pages=512, k_pages=FAKE, v_pages=FAKE,
             page_table=FAKE, seq_lens=FAKE)
    d.update(over)
    return S.santa_kv(**d)


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == set(S.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.santa_version() == 260
    for code in range(6):
        assert S.santa_status_string(code)
    assert S.santa_status_string(99) == "unknown status"


def test_workspace_size_layout(lib):
    k = kv()
    n = ctypes.c_size_t(0)
    assert lib.santa_workspace_size(ctypes.byref(k), 31, ctypes.byref(n)) == OK
    B, Hq, P, d = 2, 28, 256, 128

    def a(x):
        return (x + 255) // 256 * 256
    words = (P + 31) // 32
    S = max(P, 256)                      # partial slots per head of a bfloat16 cache
    expect = a(B * Hq * words * 4) + a(B * Hq * P * 4) + a(B * Hq * S * 8) + a(B * Hq * S * d * 4) + a(B * 4 * 4)
    assert n.value == expect
    # Few pages: the spread gather's 256 slots per head; float32 keeps P.
    k = kv(max_pages_per_seq=8)
    assert lib.santa_workspace_size(ctypes.byref(k), 31, ctypes.byref(n)) == OK
    assert n.value == a(B * Hq * 4) + a(B * Hq * 8 * 4) + a(B * Hq * 256 * 8) + a(B * Hq * 256 * d * 4) + a(B * 4 * 4)
    k = kv(max_pages_per_seq=8, dtype=S_F32)
    assert lib.santa_workspace_size(ctypes.byref(k), 31, ctypes.byref(n)) == OK
    assert n.value == a(B * Hq * 4) + a(B * Hq * 8 * 4) + a(B * Hq * 8 * 8) + a(B * Hq * 8 * d * 4) + a(B * 4 * 4)


@pytest.mark.parametrize("over,code", [
    (dict(dtype=7), UNSUP),
    (dict(batch=0), SHAPE),
    (dict(batch=70000), SHAPE),
    (dict(num_q_heads=30), SHAPE),              # 30 % 4 != 0
    (dict(num_q_heads=68), UNSUP),              # group of 17
    (dict(head_dim=96), UNSUP),
    (dict(page_size=48), UNSUP),
    (dict(max_pages_per_seq=0), SHAPE),
    (dict(max_pages_per_seq=4096), SHAPE),
    (dict(reserved=1), SHAPE),
    (dict(num_pages=0), SHAPE),
    (dict(k_pages=None), NULL),
    (dict(page_table=None), NULL),
    (dict(seq_lens=None), NULL),
])
def test_validation_rejects(lib, over, code):
    k = kv(**over)
    n = ctypes.c_size_t(0)
    assert lib.santa_workspace_size(ctypes.byref(k), 8, ctypes.byref(n)) == code
    assert lib.santa_build_reps(ctypes.byref(k), FAKE, None) == code
    assert lib.dense_decode_attention(ctypes.byref(k), FAKE, FAKE, None, FAKE, 1 << 40, None) == code
    assert lib.santa_decode_attention(ctypes.byref(k), FAKE, FAKE, 8, 0, 0, FAKE, None, None, None,
                                      FAKE, 1 << 40, None) == code


def test_null_descriptor(lib):
    n = ctypes.c_size_t(0)
    assert lib.santa_workspace_size(None, 8, ctypes.byref(n)) == NULL
    assert lib.santa_decode_attention(None, FAKE, FAKE, 8, 0, 0, FAKE, None, None, None, FAKE, 1, None) == NULL


def test_decode_argument_checks(lib):
    k = kv()
    big = 1 << 40
    call = lib.santa_decode_attention
    assert call(ctypes.byref(k), None, FAKE, 8, 0, 0, FAKE, None, None, None, FAKE, big, None) == NULL
    assert call(ctypes.byref(k), FAKE, None, 8, 0, 0, FAKE, None, None, None, FAKE, big, None) == NULL
    assert call(ctypes.byref(k), FAKE, FAKE, 8, 0, 0, None, None, None, None, FAKE, big, None) == NULL
    assert call(ctypes.byref(k), FAKE, FAKE, 0, 0, 0, FAKE, None, None, None, FAKE, big, None) == SHAPE
    # sampled and inv_pi come together
    assert call(ctypes.byref(k), FAKE, FAKE, 8, 0, 0, FAKE, None, FAKE, None, FAKE, big, None) == NULL
    # workspace missing or short
    assert call(ctypes.byref(k), FAKE, FAKE, 8, 0, 0, FAKE, None, None, None, None, big, None) == WS
    n = ctypes.c_size_t(0)
    lib.santa_workspace_size(ctypes.byref(k), 8, ctypes.byref(n))
    assert call(ctypes.byref(k), FAKE, FAKE, 8, 0, 0, FAKE, None, None, None, FAKE, n.value - 1, None) == WS
    assert lib.dense_decode_attention(ctypes.byref(k), FAKE, FAKE, None, FAKE, n.value - 1, None) == WS
    assert lib.santa_attention_given_teams(ctypes.byref(k), FAKE, 8, FAKE, FAKE, FAKE, None, FAKE,
                                           n.value - 1, None) == WS
    assert lib.santa_attention_given_teams(ctypes.byref(k), FAKE, 8, None, FAKE, FAKE, None, FAKE,
                                           big, None) == NULL
    assert lib.santa_attention_given_teams(ctypes.byref(k), FAKE, 0, FAKE, FAKE, FAKE, None, FAKE,
                                           big, None) == SHAPE
    assert lib.santa_build_reps(ctypes.byref(k), None, None) == NULL


def test_noalloc_decode_argument_checks(lib):
    # Every rejection happens before the scratch lookup (no HIP call).
    f = lib.santa_decode_attention_noalloc
    k = kv()
    assert f(ctypes.byref(k), None, FAKE, 31, 0, 0, FAKE, None, None, None, None) == NULL
    assert f(ctypes.byref(k), FAKE, None, 31, 0, 0, FAKE, None, None, None, None) == NULL
    assert f(ctypes.byref(k), FAKE, FAKE, 31, 0, 0, None, None, None, None, None) == NULL
    assert f(ctypes.byref(k), FAKE, FAKE, 0, 0, 0, FAKE, None, None, None, None) == SHAPE
    assert f(ctypes.byref(k), FAKE, FAKE, 31, 0, 0, FAKE, None, FAKE, None, None) == NULL
    assert f(None, FAKE, FAKE, 31, 0, 0, FAKE, None, None, None, None) == NULL
    bad = kv(head_dim=96)
    assert f(ctypes.byref(bad), FAKE, FAKE, 31, 0, 0, FAKE, None, None, None, None) == UNSUP
    # A shape whose single-call workspace exceeds the 64 MiB device array:
    # the log-weights alone are 4096 * 28 * 2048 * 4 bytes.
    big = kv(batch=4096, max_pages_per_seq=2048)
    assert f(ctypes.byref(big), FAKE, FAKE, 31, 0, 0, FAKE, None, None, None, None) == WS


def test_pack_pages_validation(lib):
    """santa_pack_pages rejects bad arguments on the host, before any launch."""
    F = ctypes.c_void_p
    a, b, c, d = (F(0x10000000 * i) for i in (1, 2, 3, 4))
    ok = dict(dtype=S.SANTA_BF16, n=8, hkv=4, T=128, d=128)

    def call(**over):
        x = dict(ok, **over)
        ptrs = over.get("ptrs", (a, b, c, d))
        return lib.santa_pack_pages(x["dtype"], x["n"], x["hkv"], x["T"], x["d"], *ptrs, None)

    assert call(dtype=7) == UNSUP
    assert call(d=96) == UNSUP
    assert call(T=48) == UNSUP
    assert call(hkv=0) == SHAPE
    assert call(n=-1) == SHAPE
    assert call(n=1 << 40) == SHAPE
    assert call(n=0, ptrs=(None, None, None, None)) == OK          # nothing to do, nothing enqueued
    assert call(ptrs=(a, b, None, d)) == NULL
    # 8 pages x 4 heads x 128 x 128 bf16 = 1 MiB per buffer: destinations may
    # not overlap any buffer; the two sources may
    assert call(ptrs=(a, b, F(a.value + 4096), d)) == SHAPE
    assert call(ptrs=(a, b, c, F(c.value + (1 << 20) - 2))) == SHAPE


def test_update_reps_validation(lib):
    """santa_update_reps checks its arguments on the host; 0 new tokens enqueues nothing."""
    k = kv()
    F = ctypes.c_void_p(FAKE)
    assert lib.santa_update_reps(ctypes.byref(k), None, F, 1, None) == NULL
    assert lib.santa_update_reps(ctypes.byref(k), F, None, 1, None) == NULL
    assert lib.santa_update_reps(ctypes.byref(k), F, F, -1, None) == SHAPE
    assert lib.santa_update_reps(ctypes.byref(k), F, F, 0, None) == OK
    assert lib.santa_update_reps(ctypes.byref(kv(page_size=48)), F, F, 1, None) == UNSUP


def test_value_sampled_validation(lib):
    """santa_decode_attention_value_sampled: sample counts, schemes and the
    drawn-token bound are checked on the host."""
    k = kv(batch=1)
    F = ctypes.c_void_p(FAKE)
    big = 1 << 40
    call = lib.santa_decode_attention_value_sampled

    def go(kvx=k, M=31, scheme=0, S=32, vscheme=0, sampled=None, inv_pi=None, reps=F, out=F):
        return call(ctypes.byref(kvx), F, reps, M, scheme, S, vscheme, 1, 2, out, F, sampled, inv_pi, None, F, big, None)
    assert go(reps=None) == NULL
    assert go(out=None) == NULL
    assert go(sampled=F) == NULL                         # sets come in pairs
    assert go(S=0) == SHAPE
    assert go(S=257) == SHAPE
    assert go(scheme=3) == SHAPE
    assert go(vscheme=-1) == SHAPE
    assert go(M=0) == SHAPE
    assert go(M=129) == UNSUP                            # 129 teams x 128 tokens > 16384
    assert go(kvx=kv(batch=1, page_size=256, max_pages_per_seq=65), M=500) == UNSUP   # 65 x 256 > 16384
    n = ctypes.c_size_t(0)
    assert lib.santa_value_sampled_workspace_size(ctypes.byref(k), 31, ctypes.byref(n)) == OK
    small = n.value
    assert small >= lib_workspace(lib, k, 31)
    # selection sections, then 31 x 128 tokens -> 8 chunks of 512 running sums per head, and 8 (max, sum) pairs
    assert lib.santa_value_sampled_workspace_size(ctypes.byref(k), 128, ctypes.byref(n)) == OK
    assert n.value >= small
    assert lib.santa_value_sampled_workspace_size(ctypes.byref(k), 129, ctypes.byref(n)) == UNSUP
    assert lib.santa_value_sampled_workspace_size(ctypes.byref(k), 0, ctypes.byref(n)) == SHAPE
    # a workspace big enough for the decode but not for the running sums
    # (64 teams x 256 tokens x 8 bytes per head exceed the d = 64 partials)
    k2 = kv(batch=1, head_dim=64, page_size=256, max_pages_per_seq=64)
    ws = lib_workspace(lib, k2, 64)
    assert lib.santa_value_sampled_workspace_size(ctypes.byref(k2), 64, ctypes.byref(n)) == OK and n.value > ws
    assert call(ctypes.byref(k2), F, F, 64, 0, 32, 0, 1, 2, F, F, None, None, None, F, ws, None) == WS


def lib_workspace(lib, k, M):
    n = ctypes.c_size_t(0)
    assert lib.santa_workspace_size(ctypes.byref(k), M, ctypes.byref(n)) == OK
    return n.value


def test_append_kv_validation(lib):
    """santa_append_kv checks its arguments on the host; 0 new tokens enqueues nothing."""
    k = kv()
    F = ctypes.c_void_p(FAKE)
    assert lib.santa_append_kv(ctypes.byref(k), None, F, F, 1, None) == NULL
    assert lib.santa_append_kv(ctypes.byref(k), F, None, F, 1, None) == NULL
    assert lib.santa_append_kv(ctypes.byref(k), F, F, None, 1, None) == NULL
    assert lib.santa_append_kv(ctypes.byref(k), F, F, F, -1, None) == SHAPE
    assert lib.santa_append_kv(ctypes.byref(k), F, F, F, 0, None) == OK
    assert lib.santa_append_kv(ctypes.byref(kv(page_size=48)), F, F, F, 1, None) == UNSUP
    assert lib.santa_append_kv(ctypes.byref(kv(batch=65535)), F, F, F, 1 << 30, None) == SHAPE


def test_build_reps_ex_validation(lib):
    """santa_build_reps_ex: unknown kinds and bad update bounds are rejected
    on the host; an update with 0 new tokens enqueues nothing."""
    k = kv()
    F = ctypes.c_void_p(FAKE)
    assert lib.santa_build_reps_ex(ctypes.byref(k), None, 1, 0, None, 0, None) == NULL
    assert lib.santa_build_reps_ex(ctypes.byref(k), F, 3, 0, None, 0, None) == SHAPE
    assert lib.santa_build_reps_ex(ctypes.byref(k), F, -1, 0, None, 0, None) == SHAPE
    assert lib.santa_build_reps_ex(ctypes.byref(k), F, 2, 0, F, -1, None) == SHAPE
    assert lib.santa_build_reps_ex(ctypes.byref(k), F, 1, 0, F, 0, None) == OK
    assert lib.santa_build_reps_ex(ctypes.byref(kv(head_dim=96)), F, 1, 0, None, 0, None) == UNSUP
    with pytest.raises(ValueError):
        S.santa_build_reps_ex(None, "centroid")


def test_draw_scheme_validation(lib):
    """The _ex entry points reject unknown draw schemes on the host and check
    their other arguments as the plain calls do."""
    k = kv()
    big = 1 << 40
    dec, sel = lib.santa_decode_attention_ex, lib.santa_select_teams_ex
    for bad in (3, -1):
        assert dec(ctypes.byref(k), FAKE, FAKE, 8, 0, 0, bad, FAKE, None, None, None, FAKE, big, None) == SHAPE
        assert sel(ctypes.byref(k), FAKE, FAKE, 8, 0, 0, bad, None, None, FAKE, big, None) == SHAPE
    assert dec(ctypes.byref(k), FAKE, FAKE, 0, 0, 0, 1, FAKE, None, None, None, FAKE, big, None) == SHAPE
    assert dec(ctypes.byref(k), FAKE, FAKE, 8, 0, 0, 2, None, None, None, None, FAKE, big, None) == NULL
    assert sel(ctypes.byref(k), FAKE, FAKE, 8, 0, 0, 1, None, None, None, big, None) == WS
    with pytest.raises(ValueError):
        S.santa_decode_attention_ex(None, None, None, 8, "poisson")


def test_pack_pages_hashed_validation(lib):
    """santa_pack_pages_hashed checks its arguments on the host."""
    k = kv(v_pages=FAKE + (3 << 40))          # distinct destination buffers
    call = lib.santa_pack_pages_hashed
    far = ctypes.c_void_p(FAKE + (1 << 40))
    far2 = ctypes.c_void_p(FAKE + (2 << 40))
    F = ctypes.c_void_p(FAKE)
    assert call(ctypes.byref(k), None, far2, F, 4, F, F, None) == NULL
    assert call(ctypes.byref(k), far, far2, None, 4, F, F, None) == NULL
    assert call(ctypes.byref(k), far, far2, F, 4, None, F, None) == NULL
    assert call(ctypes.byref(k), far, far2, F, 0, F, F, None) == SHAPE
    assert call(ctypes.byref(k), far, far2, F, 11, F, F, None) == SHAPE
    assert call(ctypes.byref(k), F, far2, F, 4, F, F, None) == SHAPE          # source overlaps destination
    assert call(ctypes.byref(kv()), far, far2, F, 4, F, F, None) == SHAPE     # destinations overlap
    assert call(ctypes.byref(kv(head_dim=80)), far, far2, F, 4, F, F, None) == UNSUP


def test_plain_c_consumer(lib, tmp_path):
    """tests/c_consumer.c, built with gcc as C99 against include/santa.h and
    linked with libsanta.so, runs its host-only checks."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "c_consumer"
    libdir = os.path.dirname(S.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_consumer.c"),
                    "-o", str(exe), f"-L{libdir}", "-lsanta", f"-Wl,-rpath,{libdir}"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert "c consumer ok" in res.stdout


def test_kmeans_workspace_size(lib):
    """Centroids [B][Hkv][cmax][d] float64, |mu|^2 [B][Hkv][cmax] float64 and
    the sort offsets [B][Hkv][2^bits + 1] int32, each section 256-aligned."""
    n = ctypes.c_size_t(0)
    size = lib.santa_kmeans_workspace_size
    a = lambda x: (x + 255) // 256 * 256
    B, Hkv, P, d = 2, 4, 256, 128
    assert size(ctypes.byref(kv()), 0, ctypes.byref(n)) == OK              # one cluster per team: cmax = P
    assert n.value == a(B * Hkv * P * d * 8) + a(B * Hkv * P * 8) + a(B * Hkv * (256 + 1) * 4)
    assert size(ctypes.byref(kv()), 100, ctypes.byref(n)) == OK            # bits = 7
    assert n.value == a(B * Hkv * 100 * d * 8) + a(B * Hkv * 100 * 8) + a(B * Hkv * (128 + 1) * 4)
    assert size(ctypes.byref(kv(max_pages_per_seq=2, num_pages=4)), 1000, ctypes.byref(n)) == OK   # capped at P*T
    assert n.value == a(B * Hkv * 256 * d * 8) + a(B * Hkv * 256 * 8) + a(B * Hkv * (256 + 1) * 4)
    assert size(ctypes.byref(kv()), 1025, ctypes.byref(n)) == SHAPE
    assert size(ctypes.byref(kv(max_pages_per_seq=1025, num_pages=4096)), 0, ctypes.byref(n)) == SHAPE
    assert size(ctypes.byref(kv()), -1, ctypes.byref(n)) == SHAPE
    assert size(ctypes.byref(kv()), 0, None) == NULL


def test_pack_pages_kmeans_validation(lib):
    """santa_pack_pages_kmeans checks its arguments on the host."""
    k = kv(v_pages=FAKE + (3 << 40))
    call = lib.santa_pack_pages_kmeans
    far = ctypes.c_void_p(FAKE + (1 << 40))
    far2 = ctypes.c_void_p(FAKE + (2 << 40))
    F = ctypes.c_void_p(FAKE)
    big = 1 << 40
    assert call(ctypes.byref(k), None, far2, 0, 5, F, F, F, big, None) == NULL
    assert call(ctypes.byref(k), far, far2, 0, 5, None, F, F, big, None) == NULL
    assert call(ctypes.byref(k), far, far2, 0, 5, F, None, F, big, None) == NULL
    assert call(ctypes.byref(k), far, far2, 0, 0, F, F, F, big, None) == SHAPE          # iters
    assert call(ctypes.byref(k), far, far2, 0, 1001, F, F, F, big, None) == SHAPE
    assert call(ctypes.byref(k), far, far2, 1025, 5, F, F, F, big, None) == SHAPE       # clusters
    assert call(ctypes.byref(k), far, far2, -3, 5, F, F, F, big, None) == SHAPE
    assert call(ctypes.byref(k), far, far2, 0, 5, F, F, None, big, None) == WS
    assert call(ctypes.byref(k), far, far2, 0, 5, F, F, F, 1024, None) == WS
    assert call(ctypes.byref(k), far, far2, 0, 5, F, F, ctypes.c_void_p(FAKE + 4), big, None) == WS   # alignment
    assert call(ctypes.byref(k), F, far2, 0, 5, F, F, F, big, None) == SHAPE            # source overlaps destination
    assert call(ctypes.byref(kv()), far, far2, 0, 5, F, F, F, big, None) == SHAPE       # destinations overlap
    assert call(ctypes.byref(kv(head_dim=80)), far, far2, 0, 5, F, F, F, big, None) == UNSUP


def test_binding_rejects_mismatched_buffers():
    """The binding checks caller-provided tensors against the cache
    descriptor before any library call (no GPU needed: CPU tensors)."""
    import torch
    B, P, Hkv, G, T, d = 2, 4, 2, 3, 16, 64
    kv = S.KVCache(torch.zeros((8, Hkv, T * d), dtype=torch.bfloat16), torch.zeros((8, Hkv, T * d), dtype=torch.bfloat16),
                   torch.zeros((B, P), dtype=torch.int32), torch.zeros((B,), dtype=torch.int32), Hkv * G, T)
    q = torch.zeros((B, Hkv * G, d), dtype=torch.bfloat16)
    good = torch.zeros((B, P, Hkv, d), dtype=torch.bfloat16)
    for bad in (torch.zeros((B, P, Hkv, d), dtype=torch.float32), torch.zeros((B, P + 1, Hkv, d), dtype=torch.bfloat16),
                torch.zeros((B, P, Hkv, 2 * d), dtype=torch.bfloat16)[..., ::2]):
        with pytest.raises(ValueError):
            S.santa_decode_attention(kv, q, bad, 4)
        with pytest.raises(ValueError):
            S.santa_build_reps(kv, bad)
        with pytest.raises(ValueError):
            S.santa_update_reps(kv, bad, torch.zeros((B,), dtype=torch.int32), 1)
        with pytest.raises(ValueError):
            S.santa_build_reps_ex(kv, "medoid", reps=bad)
    with pytest.raises(ValueError):
        S.santa_decode_attention(kv, q, good, 4, out=torch.zeros((B, Hkv * G, d + 1)))
    with pytest.raises(ValueError):
        S.santa_decode_attention(kv, q, good, 4, lse=torch.zeros((B, Hkv * G), dtype=torch.float64))
    with pytest.raises(ValueError):
        S.santa_select_teams(kv, q, good, 4, 0, 0, torch.zeros(16, dtype=torch.uint8),
                             torch.zeros((B, Hkv * G, 5), dtype=torch.int32), torch.zeros((B, Hkv * G, 5)))
    with pytest.raises(ValueError):
        S.dense_decode_attention(kv, q, torch.zeros(16, dtype=torch.float32))
    prev = torch.zeros((B,), dtype=torch.int32)
    new = torch.zeros((B, 1, Hkv, d), dtype=torch.bfloat16)
    for kb, vb in ((new.float(), new.float()), (new[:, :, :1], new[:, :, :1]), (new, new[:1]),
                   (torch.zeros((B, 2, Hkv, 2 * d), dtype=torch.bfloat16)[..., ::2], new)):
        with pytest.raises(ValueError):
            S.santa_append_kv(kv, prev, kb, vb)
    with pytest.raises(ValueError):
        S.santa_append_kv(kv, prev.long(), new, new)
