"""The achievable-peak probes do the work their rates are computed from: the
matrix-core loop's products (summed over a wave, which does not depend on the
instruction's lane layout) equal the products written out in float64, and the
streaming read's outputs xor to the xor of every word of the buffer."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _hash_unit(x):
    x = x.astype(np.uint64) & 0xFFFFFFFF
    x ^= x >> 16
    x = (x * 0x7FEB352D) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * 0x846CA68B) & 0xFFFFFFFF
    x ^= x >> 16
    return x.astype(np.uint32).view(np.int32).astype(np.float32) * np.float32(1.0 / 2147483648.0)


def _bf16(v):
    return torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()


def test_mfma_probe_does_the_counted_products():
    from sparse_long_context_pool_amd import probe
    n_wg, iters = 3, 37
    _, sink = probe.mfma_bf16(n_wg, iters, reps=1)
    got = sink.cpu().numpy().astype(np.float64).reshape(n_wg * 4, 64).sum(axis=1)
    # lane l of a wave holds A[l % 32][8 (l / 32) + e] and B[8 (l / 32) + e][l % 32]
    # (e = 0..7) of each 32 x 32 x 16 product; chain c multiplies a[c % 4] by b[c / 2]
    gid = np.arange(n_wg * 256, dtype=np.uint64)
    u, e = np.arange(4, dtype=np.uint64), np.arange(8, dtype=np.uint64)
    idx = gid[:, None, None] * 64 + 8 * u[None, :, None] + e[None, None, :]
    a = _bf16(_hash_unit(idx))                        # [thread][u][e]
    b = _bf16(_hash_unit(idx + 0x9E3779B9))
    want = np.zeros(n_wg * 4)
    for w in range(n_wg * 4):
        aw, bw = a[64 * w:64 * w + 64], b[64 * w:64 * w + 64]
        # sum over i, j of (A B)[i][j] = sum over k of (sum_i A[i][k]) (sum_j B[k][j])
        col_a = np.stack([aw[32 * h:32 * h + 32].sum(axis=0) for h in range(2)])  # [h][u][e]
        row_b = np.stack([bw[32 * h:32 * h + 32].sum(axis=0) for h in range(2)])
        tot = 0.0
        for c in range(8):
            tot += float((col_a[:, c % 4, :] * row_b[:, c // 2, :]).sum())
        want[w] = iters * tot
    scale = np.abs(want).max() + 1.0
    assert np.all(np.abs(got - want) <= 1e-4 * scale), (got[:4], want[:4])


def test_read_probe_reads_every_word_once():
    from sparse_long_context_pool_amd import probe
    g = torch.Generator().manual_seed(7)
    n_words = (1 << 22) + 4 * 1000  # not a multiple of the grid's stride
    host = torch.randint(0, 2 ** 31 - 1, (n_words,), generator=g, dtype=torch.int32)
    buf = host.cuda()
    gbs, sink = probe.hbm_read(buf, 40, reps=1)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want
    assert gbs > 0


@pytest.mark.parametrize("mode", [0, 1])
def test_lds_probe_reads_what_it_counts(mode):
    from sparse_long_context_pool_amd import probe
    n_wg, iters = 2, 19
    tbs, per_clk, sink = probe.lds_read(mode, n_wg, iters, reps=1)
    s = sink.cpu().numpy().view(np.uint32).reshape(n_wg, 8, 64, 2)
    # the array: 16-byte element i = (i, 3i + 1, 5i + 2, 7i + 3)
    words = np.zeros(65536 // 4, dtype=np.uint32)
    i = np.arange(65536 // 16, dtype=np.uint32)
    words[0::4], words[1::4], words[2::4], words[3::4] = i, 3 * i + 1, 5 * i + 2, 7 * i + 3
    halves = words.view(np.int16).astype(np.int64)
    for w in range(8):
        want = 0
        for it in range(iters):
            for u in range(8):
                row = (it * 9 + u * 8 + w) & 63
                if mode == 0:  # lane l: the four words at row * 1024 + 16 l
                    want += int(words[row * 256:row * 256 + 256].astype(np.int64).sum())
                else:          # the wave together reads the 256 halves at row * 1024
                    want += int(halves[row * 512:row * 512 + 256].sum())
        for g in range(n_wg):
            assert int(s[g, w, :, 0].astype(np.int64).sum()) % 2 ** 32 == want % 2 ** 32, (g, w)
    assert tbs > 0 and per_clk > 0
