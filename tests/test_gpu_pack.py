"""santa_pack_pages against the tile order that include/santa.h states,
written out here element by element with numpy (bit-exact: a permutation)."""
import numpy as np
import pytest
import torch

from sampled_sparse_decode_amd import santa as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load()


def expected_tiles(src, kind):
    """[n][hkv][T][d] -> [n][hkv][T*d] in the header's chunked order."""
    n, hkv, T, d = src.shape
    C = min(T, 32)
    out = np.empty((n, hkv, T * d), dtype=src.dtype)
    tok = np.arange(T)[:, None]
    ch = np.arange(d)[None, :]
    c, i = tok // C, tok % C
    if kind == "k":
        idx = c * C * d + (ch // 32) * C * 32 + i * 32 + (ch % 32)
    else:
        idx = c * C * d + ch * C + i
    out[:, :, idx.reshape(-1)] = src.reshape(n, hkv, T * d)
    return out


@pytest.mark.parametrize("dtype,T,d", [("bf16", 16, 64), ("bf16", 128, 128), ("bf16", 256, 64),
                                       ("f32", 32, 128), ("f32", 16, 128), ("f32", 64, 64)])
def test_pack_pages_tile_order(dtype, T, d):
    print(f"[pack] {dtype} T={T} d={d}", flush=True)
    rng = np.random.default_rng(T * 1000 + d)
    n, hkv = 5, 3
    if dtype == "bf16":
        raw = rng.integers(0, 1 << 16, size=(2, n, hkv, T, d), dtype=np.uint16)
        tdt = torch.bfloat16
        dev = [torch.from_numpy(x.view(np.int16)).view(tdt).cuda() for x in raw]
    else:
        raw = rng.standard_normal((2, n, hkv, T, d)).astype(np.float32)
        dev = [torch.from_numpy(x).cuda() for x in raw]
    kt, vt = S.pack_pages(dev[0], dev[1])
    torch.cuda.synchronize()

    def host(t):
        a = t.cpu()
        return a.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else a.numpy()

    assert np.array_equal(host(kt), expected_tiles(raw[0], "k"))
    assert np.array_equal(host(vt), expected_tiles(raw[1], "v"))
