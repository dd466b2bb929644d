"""Seeded random shapes against the oracle: each case draws its own sizes and
options (compression rates, overlap, widths, RoPE, gates and slot biases,
window sizes, index-row lengths, query positions, head counts, dtype) from a
seeded generator, so the parity checks reach combinations the hand-picked
cases do not.  The bars are those of the hand-picked stage tests: one bf16 ulp
(2^-7 relative) or 1e-5 relative for the compressor, the summation-order bound
for index scores, bit-exact top-k on identical scores, and 2e-2 (bf16) /
1e-4 (fp32) for attention."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import BF16_ATOL, F32_ATOL, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from sparse_long_context_pool_amd import csa
    assert torch.cuda.is_available()
    csa.lib()
    return csa


def _data(r, shape, bf16, scale=1.0):
    a = (r.standard_normal(shape) * scale).astype(np.float32)
    return oracle.round_bf16(a) if bf16 else a


@pytest.mark.parametrize("seed", range(24))
def test_random_compress(ops, seed):
    r = np.random.default_rng(1000 + seed)
    m = int(r.choice([1, 2, 3, 4, 8, 16, 128]))
    overlap = int(r.integers(0, 2)) if m > 1 else 0
    D = int(r.choice([64, 128, 256, 512, 576]))
    rope = int(r.choice([0, 16, 64]))
    gate, bias = bool(r.integers(0, 2)), bool(r.integers(0, 2))
    if m == 1 and not (gate or bias):
        gate = bool(seed % 2)
    bf16 = bool(r.integers(0, 2))
    B = int(r.integers(1, 4))
    S = int(r.integers(m, m * 9 + 7))
    pos0 = int(r.integers(0, 5000))
    theta = 160000.0
    x = _data(r, (B, S, D), bf16)
    g = _data(r, (B, S, D), bf16) if gate else None
    sb = _data(r, ((1 + overlap) * m, D), False) if bias else None
    dt = torch.bfloat16 if bf16 else torch.float32
    cs = ops.csa_rope_table(pos0 + S + 1, max(rope, 2), theta) if rope else None
    out = host(ops.csa_compress(dev(x, dt), None if g is None else dev(g, dt),
                                None if sb is None else dev(sb, torch.float32), m=m,
                                overlap=overlap, rope_dim=rope, cs=cs, pos0=pos0))
    rel = 2.0 ** -7 if bf16 else 1e-5
    for b in range(B):
        ref = oracle.compress(x[b], None if g is None else g[b], sb, m=m, overlap=overlap,
                              rope_dim=rope, theta=theta, pos0=pos0, round_bf16=bf16)
        np.testing.assert_allclose(out[b], ref, rtol=rel, atol=1e-5,
                                   err_msg=f"m={m} ov={overlap} D={D} rope={rope}")


@pytest.mark.parametrize("seed", range(20))
def test_random_index_scores_and_topk(ops, seed):
    r = np.random.default_rng(2000 + seed)
    mfma = seed % 2 == 0                      # the bf16 64 x 128 shape, else generic fp32
    nI, cI = (64, 128) if mfma else (int(r.integers(1, 9)), int(r.choice([16, 32, 40])))
    bf16 = mfma
    m = int(r.choice([1, 2, 4]))
    T = int(r.integers(20, 3000))
    B = int(r.integers(1, 4))
    S = int(r.choice([1, 3, int(r.integers(16, 70))]))
    k = int(r.choice([8, 64, 512, 2048]))
    qp = [int(r.integers(0, T * m + 50)) for _ in range(B)]
    dt = torch.bfloat16 if bf16 else torch.float32
    q = _data(r, (B, S, nI, cI), bf16, 0.5)
    w = _data(r, (B, S, nI), False, 0.5)
    kk = _data(r, (B, T, cI), bf16, 0.5)
    q_pos = torch.tensor(qp, dtype=torch.int32, device="cuda")
    sc_d = ops.csa_index_scores(dev(q, dt), dev(w, torch.float32), dev(kk, dt), q_pos, m=m)
    idx = host(ops.csa_topk(sc_d, q_pos, k=k, m=m)).astype(np.int32)
    sc = host(sc_d)
    for b in range(B):
        t = qp[b] + np.arange(S)
        ref = oracle.index_scores(q[b], w[b], t, kk[b], m=m)
        bound = 1e-5 * np.einsum("nj,njw->nw", np.abs(w[b]).astype(np.float64),
                                 np.einsum("njc,wc->njw", np.abs(q[b]).astype(np.float64),
                                           np.abs(kk[b]).astype(np.float64))) + 1e-6
        for i in range(S):
            R = oracle.ready_count(int(t[i]), m, T)
            assert np.all(np.abs(sc[b, i, :R] - ref[i, :R]) <= bound[i, :R]), (b, i)
        # the selection over the GPU's own scores equals the oracle's selection
        # over those same scores (entries past R are never read)
        g_sc = np.where(np.arange(T)[None, :] < np.array(
            [oracle.ready_count(int(x), m, T) for x in t])[:, None], sc[b], -np.inf)
        assert np.array_equal(idx[b], oracle.topk(g_sc.astype(np.float32), t, k=k, m=m)), b


@pytest.mark.parametrize("seed", range(24))
def test_random_attention(ops, seed):
    r = np.random.default_rng(3000 + seed)
    mfma = seed % 3 != 0
    if mfma:      # the matrix-core shapes (H multiple of 64, D = 512 or 576)
        dsa = seed % 4 == 1
        H, D, rope = (128, 576, 64) if dsa else (64, 512, 64)
        dv = 512
        bf16 = True
    else:         # the generic kernel
        H = int(r.choice([1, 3, 4, 8, 16]))
        D = int(r.choice([32, 40, 64, 96]))
        rope = int(r.choice([8, 16]))
        dv = int(r.choice([D, D - rope]))
        bf16 = bool(r.integers(0, 2))
    m = int(r.choice([1, 2, 4])) if not (mfma and dsa) else 1
    T = int(r.integers(8, 400))
    B = int(r.integers(1, 3))
    S = int(r.choice([1, 2, int(r.integers(3, 40))]))
    k = int(r.choice([1, 16, 48, 200]))
    window = 0 if (mfma and dsa) else int(r.choice([0, 5, 32, 128]))
    sink = bool(r.integers(0, 2)) and not (mfma and dsa)
    qp = [int(r.integers(0, T * m + 20)) for _ in range(B)]
    theta = 160000.0
    q = _data(r, (B, S, H, D), bf16)
    L = max(qp) + S if window else 0
    kv = _data(r, (B, L, D), bf16) if window else None
    pool = _data(r, (B, T, D), bf16)
    z = _data(r, (H,), False) if sink else None
    idx = np.full((B, S, k), -1, np.int32)
    for b in range(B):
        for i in range(S):
            R = oracle.ready_count(qp[b] + i, m, T)
            sel = np.sort(r.choice(R, size=min(k, R), replace=False)) if R else []
            idx[b, i, :len(sel)] = sel
    dt = torch.bfloat16 if bf16 else torch.float32
    cs = ops.csa_rope_table(max(qp) + S + 1, rope, theta)
    q_pos = torch.tensor(qp, dtype=torch.int32, device="cuda")
    win_pos0 = torch.zeros(B, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    out = host(ops.csa_sparse_attn(dev(q, dt), None if kv is None else dev(kv, dt), win_pos0,
                                   dev(pool, dt), dev(idx, torch.int32),
                                   None if z is None else dev(z, torch.float32), q_pos,
                                   rope_dim=rope, cs=cs, window=window, scale=scale, dv=dv))
    tol = BF16_ATOL if bf16 else F32_ATOL
    for b in range(B):
        t = qp[b] + np.arange(S)
        ref = oracle.attention(q[b], t, kv_win=None if kv is None else kv[b], win_pos0=0,
                               window=window, pool=pool[b], idx=idx[b], m=m, sink=z,
                               rope_dim=rope, theta=theta, scale=scale, dv=dv)
        err = float(np.abs(out[b] - ref).max())
        assert err <= tol, (dict(H=H, D=D, dv=dv, m=m, T=T, S=S, k=k, window=window), b, err)


@pytest.mark.parametrize("seed", range(16))
def test_random_hca_attention(ops, seed):
    """Dense attention over every ready entry (HCA), including layers with no
    pool (sliding window only), on the matrix-core and generic kernels."""
    r = np.random.default_rng(4000 + seed)
    mfma = seed % 2 == 0
    if mfma:
        H, D, rope, dv, bf16 = 64, 512, 64, 512, True
    else:
        H = int(r.choice([1, 2, 4, 8]))
        D = int(r.choice([32, 64, 96]))
        rope = int(r.choice([8, 16]))
        dv = int(r.choice([D, D - rope]))
        bf16 = bool(r.integers(0, 2))
    m = int(r.choice([4, 8, 16, 128]))
    T = 0 if seed % 5 == 4 else int(r.integers(1, 40))
    B = int(r.integers(1, 3))
    S = int(r.choice([1, 2, int(r.integers(3, 60))]))
    window = int(r.choice([8, 32, 128])) if T == 0 else int(r.choice([0, 5, 32, 128]))
    sink = bool(r.integers(0, 2))
    qp = [int(r.integers(0, max(T, 1) * m + 30)) for _ in range(B)]
    theta = 160000.0
    q = _data(r, (B, S, H, D), bf16)
    L = max(qp) + S if window else 0
    kv = _data(r, (B, L, D), bf16) if window else None
    pool = _data(r, (B, T, D), bf16)
    z = _data(r, (H,), False) if sink else None
    dt = torch.bfloat16 if bf16 else torch.float32
    cs = ops.csa_rope_table(max(qp) + S + 1, rope, theta)
    q_pos = torch.tensor(qp, dtype=torch.int32, device="cuda")
    win_pos0 = torch.zeros(B, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    out = host(ops.hca_attn(dev(q, dt), None if kv is None else dev(kv, dt), win_pos0,
                            dev(pool, dt) if T else None,
                            None if z is None else dev(z, torch.float32), q_pos, m=m,
                            rope_dim=rope, cs=cs, window=window, scale=scale, dv=dv))
    tol = BF16_ATOL if bf16 else F32_ATOL
    for b in range(B):
        t = qp[b] + np.arange(S)
        ref = oracle.attention(q[b], t, kv_win=None if kv is None else kv[b], win_pos0=0,
                               window=window, pool=pool[b], idx=None, m=m, sink=z,
                               rope_dim=rope, theta=theta, scale=scale, dv=dv)
        err = float(np.abs(out[b] - ref).max())
        assert err <= tol, (dict(H=H, D=D, dv=dv, m=m, T=T, S=S, window=window), b, err)
