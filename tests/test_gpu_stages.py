"""GPU parity, stage by stage, against the CPU oracle on the same seeded
inputs.  Each GPU stage receives the ORACLE's upstream tensors, so a stage is
judged on its own.  Sizes span several tiles and end in ragged tails."""
import math
import zlib

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


def rng(s):
    return np.random.default_rng(s)


def rnd(shape, seed, bf16, scale=1.0):
    a = (rng(seed).standard_normal(shape) * scale).astype(np.float32)
    return oracle.round_bf16(a) if bf16 else a


# ------------------------------------------------------------------ RoPE table
@pytest.mark.parametrize("theta,rope_dim", [(160000.0, 64), (10000.0, 64), (160000.0, 16)])
def test_rope_table(ops, theta, rope_dim):
    n = 131073
    g = host(ops.csa_rope_table(n, rope_dim, theta))
    o = oracle.rope_table(n, rope_dim, theta)
    assert np.max(np.abs(g - o)) <= 1.2e-7


@pytest.mark.parametrize("factor,orig,theta,rope_dim", [
    (16.0, 65536, 160000.0, 64), (4.0, 4096, 10000.0, 64), (1.0, 65536, 160000.0, 64),
    (40.0, 4096, 10000.0, 128)])
def test_rope_table_yarn(ops, factor, orig, theta, rope_dim):
    n = 131073
    g = host(ops.csa_rope_table_yarn(n, rope_dim, theta, factor, orig, 32.0, 1.0))
    o = oracle.rope_table(n, rope_dim, theta,
                          freqs=oracle.yarn_freqs(rope_dim, theta, factor, orig, 32.0, 1.0))
    assert np.max(np.abs(g - o)) <= 1.2e-7


def test_attention_with_yarn_table(ops):
    """The attention kernels take every angle from the table: a CSA case on the
    matrix-core kernel with a YaRN table (16x extension) against the oracle
    with the same frequencies."""
    B, S, H, D, dv, rope, T, k, window, m, qp, sink, bf16, dense = ATTN_CASES["csa_mfma"]
    # (inputs drawn for rows at t >= 400, where all T entries are ready, as at
    # the positions used below)
    q, kv, pool, z, idx = _attn_case(411, B, S, H, D, dv, rope, T, k, window, m, [400, 400],
                                     sink, bf16, dense)
    qp = [70000, 100000]
    theta, factor, orig = 160000.0, 16.0, 65536
    cs = ops.csa_rope_table_yarn(max(qp) + S + 1, rope, theta, factor, orig)
    fr = oracle.yarn_freqs(rope, theta, factor, orig)
    dt = torch.bfloat16
    # the window rows of positions qp - window .. qp + S - 1
    lo = [p - window for p in qp]
    kvw = np.ascontiguousarray(kv[:, :S + window])
    out = host(ops.csa_sparse_attn(dev(q, dt), dev(kvw, dt),
                                   torch.tensor(lo, dtype=torch.int32, device="cuda"),
                                   dev(pool, dt), dev(idx, torch.int32), dev(z, torch.float32),
                                   torch.tensor(qp, dtype=torch.int32, device="cuda"),
                                   rope_dim=rope, cs=cs, window=window,
                                   scale=1.0 / math.sqrt(D), dv=dv))
    for b in range(B):
        t = qp[b] + np.arange(S)
        ref = oracle.attention(q[b], t, kv_win=kvw[b], win_pos0=lo[b], window=window,
                               pool=pool[b], idx=idx[b], m=m, sink=z, rope_dim=rope,
                               theta=theta, scale=1.0 / math.sqrt(D), dv=dv, freqs=fr)
        err = np.abs(out[b] - ref).max()
        assert err <= BF16_ATOL, (b, float(err))


# ------------------------------------------------------------------ compressor
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("m,ov,D,rope,gate,bias", [
    (4, 1, 512, 64, True, False), (4, 1, 64, 16, True, True), (128, 0, 512, 64, True, False),
    (1, 0, 576, 64, False, False), (1, 0, 128, 0, False, False), (1, 0, 64, 16, True, False),
    (8, 0, 96, 32, False, True),
    (4, 1, 128, 0, True, False)])
def test_compress(ops, bf16, m, ov, D, rope, gate, bias):
    B = 2
    S = 3 * m * 4 + 3 if m < 128 else 5 * 128 + 17       # ragged tail
    x = rnd((B, S, D), 1, bf16)
    g = rnd((B, S, D), 2, bf16) if gate else None
    sb = rnd(((1 + ov) * m, D), 3, False) if bias else None
    theta, pos0 = 160000.0, 12
    dt = torch.bfloat16 if bf16 else torch.float32
    cs = ops.csa_rope_table(pos0 + S + 1, max(rope, 2), theta) if rope else None
    out = host(ops.csa_compress(dev(x, dt), None if g is None else dev(g, dt),
                                None if sb is None else dev(sb, torch.float32), m=m,
                                overlap=ov, rope_dim=rope, cs=cs, pos0=pos0))
    for b in range(B):
        ref = oracle.compress(x[b], None if g is None else g[b], sb, m=m, overlap=ov,
                              rope_dim=rope, theta=theta, pos0=pos0, round_bf16=bf16)
        rel = 2.0 ** -7 if bf16 else 1e-5
        np.testing.assert_allclose(out[b], ref, rtol=rel, atol=1e-5)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("mix", ["prefill", "dsa", "hca", "five"])
def test_compress_many(ops, bf16, mix):
    """csa_compress_many gives exactly what separate csa_compress calls give
    (the passes batched into one launch, the rest on their own kernels), and
    the prefill trio matches the oracle."""
    dt = torch.bfloat16 if bf16 else torch.float32
    theta = 160000.0
    B, S, D, Di, rope = 2, 4 * 37 + 3, 512, 128, 64
    x = rnd((B, S, D), 11, bf16)
    g = rnd((B, S, D), 12, bf16)
    xi = rnd((B, S, Di), 13, bf16)
    gi = rnd((B, S, Di), 14, bf16)
    cs = ops.csa_rope_table(S + 40, rope, theta)
    X, G, XI, GI = (dev(a, dt) for a in (x, g, xi, gi))
    win = dict(x=X, m=1, overlap=0, rope_dim=rope, cs=cs, pos0=5)
    kv = dict(x=X, gate=G, m=4, overlap=1, rope_dim=rope, cs=cs, pos0=5)
    ki = dict(x=XI, gate=GI, m=4, overlap=1)
    if mix == "prefill":
        passes = [win, kv, ki]
    elif mix == "dsa":
        passes = [win, dict(x=XI, m=1, overlap=0)]
    elif mix == "hca":        # m = 128: not batchable, runs on its own kernel between batched ones
        passes = [win, dict(x=X, gate=G, m=128, overlap=0, rope_dim=rope, cs=cs, pos0=5), ki]
    else:                     # more passes than one launch takes, with a slot bias and m = 8
        sb = dev(rnd((8, Di), 15, False), torch.float32)
        passes = [win, kv, ki, dict(x=XI, gate=GI, slot_bias=sb, m=8, overlap=0),
                  dict(x=XI, gate=GI, m=2, overlap=1)]
    many = [host(o) for o in ops.csa_compress_many(passes)]
    torch.cuda.synchronize()
    for q, p in enumerate(passes):
        one = host(ops.csa_compress(p["x"], p.get("gate"), p.get("slot_bias"), m=p["m"],
                                    overlap=p["overlap"], rope_dim=p.get("rope_dim", 0),
                                    cs=p.get("cs"), pos0=p.get("pos0", 0)))
        assert np.array_equal(many[q].view(np.uint8), one.view(np.uint8)), (mix, q)
    if mix == "prefill":
        rel = 2.0 ** -7 if bf16 else 1e-5
        for b in range(B):
            refs = [oracle.compress(x[b], None, None, m=1, overlap=0, rope_dim=rope,
                                    theta=theta, pos0=5, round_bf16=bf16),
                    oracle.compress(x[b], g[b], None, m=4, overlap=1, rope_dim=rope,
                                    theta=theta, pos0=5, round_bf16=bf16),
                    oracle.compress(xi[b], gi[b], None, m=4, overlap=1, round_bf16=bf16)]
            for q in range(3):
                np.testing.assert_allclose(many[q][b], refs[q], rtol=rel, atol=1e-5)


def test_compress_many_empty_and_degenerate_passes(ops):
    """No passes, and passes with no whole window, enqueue nothing; a valid
    pass beside them is still computed."""
    assert ops.csa_compress_many([]) == []
    x = dev(rnd((1, 3, 64), 16, True), torch.bfloat16)
    y = dev(rnd((2, 16, 64), 17, True), torch.bfloat16)
    a, b = ops.csa_compress_many([dict(x=x, m=4, overlap=1), dict(x=y, m=4, overlap=1)])
    assert a.shape == (1, 0, 64)
    ref = host(ops.csa_compress(y, m=4, overlap=1))
    assert np.array_equal(host(b).view(np.uint8), ref.view(np.uint8))


# ------------------------------------------------------------------ index scores
def _score_bound(q, w, k):
    tot = np.einsum("nj,njw->nw", np.abs(w).astype(np.float64),
                    np.einsum("njc,wc->njw", np.abs(q).astype(np.float64),
                              np.abs(k).astype(np.float64)))
    return 1e-5 * tot + 1e-6


@pytest.mark.parametrize("case", [
    # (dtype, B, S, nI, cI, T, m, q_pos): the 64x128 bf16 shape runs on matrix cores
    ("bf16", 2, 61, 64, 128, 300, 4, [0, 700]),     # prefill mode, ragged rows
    ("bf16", 5, 1, 64, 128, 3000, 4, [12000, 11999, 3, 0, 40000]),  # decode mode
    # few rows per sequence, many blocks per wave (several rounds, ragged ends)
    ("bf16", 16, 8, 64, 128, 3000, 4, [11990 + 13 * b - 4000 * (b % 3) for b in range(16)]),
    ("bf16", 1, 200, 64, 128, 200, 1, [0]),         # token level (m=1)
    # token level at a position that is not a multiple of 4: rows of one 4-row
    # block end on both sides of a chunk start (a row's range within a chunk
    # can be empty)
    ("bf16", 1, 20, 64, 128, 5000, 1, [4990]),
    ("f32", 2, 33, 2, 32, 64, 4, [0, 100]),         # generic kernel
    ("bf16", 1, 20, 4, 64, 50, 4, [150]),           # generic kernel, bf16
])
def test_index_scores(ops, case):
    dt_s, B, S, nI, cI, T, m, qp = case
    bf16 = dt_s == "bf16"
    dt = torch.bfloat16 if bf16 else torch.float32
    q = rnd((B, S, nI, cI), 10, bf16, 0.5)
    w = rnd((B, S, nI), 11, False, 0.5)
    k = rnd((B, T, cI), 12, bf16, 0.5)
    q_pos = torch.tensor(qp, dtype=torch.int32, device="cuda")
    sc = ops.csa_index_scores(dev(q, dt), dev(w, torch.float32), dev(k, dt), q_pos, m=m)
    sc = host(sc)
    for b in range(B):
        t = qp[b] + np.arange(S)
        ref = oracle.index_scores(q[b], w[b], t, k[b], m=m)
        bound = _score_bound(q[b], w[b], k[b])
        for i in range(S):
            R = oracle.ready_count(int(t[i]), m, T)
            if not bf16:  # fp32: same order, no fused multiply-add -> identical bits
                assert np.array_equal(sc[b, i, :R], ref[i, :R]), (b, i)
            d = np.abs(sc[b, i, :R] - ref[i, :R])
            assert np.all(d <= bound[i, :R]), (b, i, float(d.max()))
            assert not np.any(np.signbit(sc[b, i, :R]) & (sc[b, i, :R] == 0))


# ------------------------------------------------------------------ top-k
@pytest.mark.parametrize("T,k,m,qp,S", [
    # T <= 2048: one wave per row (8, 16 or 32 keys per lane)
    (64, 16, 4, [0, 120], 37), (2048, 512, 4, [0, 6000], 70), (2048, 512, 1, [1000, 1500], 20),
    (1000, 128, 1, [900, 10], 33), (1536, 700, 4, [5000, 2100], 11),
    (32768, 2048, 4, [131071, 90000], 3), (40000, 2048, 1, [39990, 20000], 4),
    (300, 300, 1, [0, 100], 9), (12000, 1024, 1, [11000, 6000], 130),
    # 2048 < T <= 8192: the 512-thread register kernel with 16 keys per thread
    (6000, 512, 4, [23000, 3000], 40), (8192, 2048, 1, [8000, 500], 10)])
def test_topk_bit_exact(ops, T, k, m, qp, S):
    B = 2
    r = rng(T + k)
    sc = r.standard_normal((B, S, T)).astype(np.float32)
    # ties: exact zeros, signed zeros, repeated values, an all-equal row
    sc[:, :, ::5] = 0.0
    sc[:, :, 2::7] = -0.0
    sc[:, :, 3::9] = 0.75
    sc[0, S // 2, :] = -1.25
    q_pos = torch.tensor(qp, dtype=torch.int32, device="cuda")
    idx = host(ops.csa_topk(dev(sc, torch.float32), q_pos, k=k, m=m)).astype(np.int32)
    for b in range(B):
        t = qp[b] + np.arange(S)
        ref = oracle.topk(sc[b], t, k=k, m=m)
        assert np.array_equal(idx[b], ref), b


@pytest.mark.parametrize("T,k,crowd", [
    # the k-th largest key lies in a crowded bin of the first 11-bit radix
    # digit (hundreds to thousands of distinct values and ties), so the second
    # and third digits decide the selection
    (32768, 2048, 5000), (32768, 2048, 1500), (12000, 1024, 3000), (6000, 512, 2500),
    (2048, 512, 900)])
def test_topk_crowded_top_digit(ops, T, k, crowd):
    B, S, m = 1, 6, 1
    r = rng(T + crowd)
    sc = np.minimum(r.standard_normal((B, S, T)), 1.99).astype(np.float32)
    for i in range(S):
        sel = r.choice(T, crowd, replace=False)
        # [2, 2.5): one bin of the first digit (sign, exponent, two mantissa bits)
        sc[0, i, sel] = (2.0 + 0.5 * r.random(crowd)).astype(np.float32)
        sc[0, i, sel[: crowd // 4]] = 2.25  # and ties inside it
    qp = [T - S]
    q_pos = torch.tensor(qp, dtype=torch.int32, device="cuda")
    idx = host(ops.csa_topk(dev(sc, torch.float32), q_pos, k=k, m=m)).astype(np.int32)
    t = qp[0] + np.arange(S)
    ref = oracle.topk(sc[0], t, k=k, m=m)
    assert np.array_equal(idx[0], ref)


# ------------------------------------------------------------------ attention
def _attn_case(seed, B, S, H, D, dv, rope, T, k, window, m, qp, sink, bf16, dense):
    r = rng(seed)
    q = rnd((B, S, H, D), seed + 1, bf16)
    L = max(qp) + S if window else 0
    kv = rnd((B, L, D), seed + 2, bf16) if window else None
    pool = rnd((B, T, D), seed + 3, bf16)
    z = rnd((H,), seed + 4, False) if sink else None
    idx = None
    if not dense:
        idx = np.full((B, S, k), -1, np.int32)
        for b in range(B):
            for i in range(S):
                R = oracle.ready_count(qp[b] + i, m, T)
                sel = np.sort(r.choice(R, size=min(k, R), replace=False)) if R else []
                idx[b, i, :len(sel)] = sel
    return q, kv, pool, z, idx


ATTN_CASES = {
    # name: (B, S, H, D, dv, rope, T, k, window, m, q_pos, sink, bf16, dense)
    # >= 256 query rows x head groups run unsplit; fewer rows split their keys
    "csa_mfma": (2, 150, 64, 512, 512, 64, 100, 48, 32, 4, [0, 300], True, True, False),
    "csa_mfma_split": (2, 1, 64, 512, 512, 64, 700, 600, 128, 4, [2900, 5000], True, True,
                       False),
    "hca_mfma": (1, 300, 64, 512, 512, 64, 12, 0, 32, 8, [40], True, True, True),
    "hca_mfma_split": (1, 2, 64, 512, 512, 64, 520, 0, 128, 128, [70000], True, True, True),
    "dsa_mfma": (1, 150, 128, 576, 512, 64, 160, 40, 0, 1, [10], False, True, False),
    "dsa_mfma_split": (1, 24, 128, 576, 512, 64, 80, 40, 0, 1, [40], False, True, False),
    # sliding-window-only layers (no pool): hca_attn with T = 0
    "swa_mfma": (1, 300, 64, 512, 512, 64, 0, 0, 128, 128, [5000], True, True, True),
    "swa_mfma_split": (2, 1, 64, 512, 512, 64, 0, 0, 128, 128, [3000, 3], True, True, True),
    "generic_swa_f32": (1, 40, 4, 64, 64, 16, 0, 0, 16, 4, [0], True, False, True),
    # head counts and widths without a matrix-core kernel (H % 64 != 0, D = 64 / 96)
    "generic_small_bf16": (1, 300, 16, 64, 64, 16, 40, 20, 16, 4, [0], True, True, False),
    "generic_small_b2_bf16": (2, 50, 16, 64, 64, 16, 30, 20, 16, 4, [0, 64], True, True, False),
    "generic_small_latent_bf16": (1, 33, 32, 96, 64, 32, 40, 12, 0, 1, [5], False, True, False),
    "generic_f32": (2, 45, 4, 64, 64, 16, 64, 16, 32, 4, [0, 200], True, False, False),
    "generic_bf16": (1, 30, 6, 40, 40, 8, 20, 8, 8, 4, [60], True, True, False),
    "generic_hca_f32": (1, 40, 3, 32, 24, 8, 10, 0, 5, 4, [0], False, False, True),
    # more index slots than the matrix-core kernel keeps in LDS: generic kernel
    "generic_bigk_bf16": (1, 2, 64, 512, 512, 64, 3200, 3000, 32, 4, [20000], True, True, False),
}


@pytest.mark.parametrize("name", sorted(ATTN_CASES))
def test_attention(ops, name):
    B, S, H, D, dv, rope, T, k, window, m, qp, sink, bf16, dense = ATTN_CASES[name]
    q, kv, pool, z, idx = _attn_case(zlib.crc32(name.encode()) % 1000, B, S, H, D, dv, rope, T, k, window,
                                     m, qp, sink, bf16, dense)
    theta = 160000.0
    dt = torch.bfloat16 if bf16 else torch.float32
    n_pos = max(qp) + S + 1
    cs = ops.csa_rope_table(n_pos, rope, theta)
    q_pos = torch.tensor(qp, dtype=torch.int32, device="cuda")
    win_pos0 = torch.zeros(B, dtype=torch.int32, device="cuda")
    kvd = dev(kv, dt) if kv is not None else None
    zd = dev(z, torch.float32) if z is not None else None
    scale = 1.0 / math.sqrt(D)
    if dense:
        # (T = 0: a sliding-window-only layer, no pool at all)
        out = ops.hca_attn(dev(q, dt), kvd, win_pos0, dev(pool, dt) if T else None, zd, q_pos,
                           m=m, rope_dim=rope, cs=cs, window=window, scale=scale, dv=dv)
    else:
        out = ops.csa_sparse_attn(dev(q, dt), kvd, win_pos0, dev(pool, dt), dev(idx, torch.int32),
                                  zd, q_pos, rope_dim=rope, cs=cs, window=window, scale=scale,
                                  dv=dv)
    out = host(out)
    tol = BF16_ATOL if bf16 else F32_ATOL
    for b in range(B):
        t = qp[b] + np.arange(S)
        ref = oracle.attention(q[b], t, kv_win=None if kv is None else kv[b], win_pos0=0,
                               window=window, pool=pool[b], idx=None if dense else idx[b],
                               m=m, sink=z, rope_dim=rope, theta=theta, scale=scale, dv=dv)
        err = np.abs(out[b] - ref).max()
        assert err <= tol, (name, b, float(err))


@pytest.mark.parametrize("name", ["csa_mfma", "csa_mfma_split", "hca_mfma_split", "dsa_mfma",
                                  "dsa_mfma_split"])
def test_attention_large_logits(ops, name):
    """Logits that grow by far more than the kernel's lazy-rescale margin from
    one key tile to the next: window keys are tiny, pool keys large, and the
    score scale is 12, so the running maximum jumps by ~2^7 (log2 units) when
    the first pool tile arrives and again, now and then, between pool tiles.
    The query's RoPE channels are zero so that its rotation is exact and the
    large scale does not amplify the rounding of the rotated query."""
    B, S, H, D, dv, rope, T, k, window, m, qp, sink, bf16, dense = ATTN_CASES[name]
    q, kv, pool, z, idx = _attn_case(zlib.crc32(name.encode()) % 1000 + 17, B, S, H, D, dv, rope,
                                     T, k, window, m, qp, sink, bf16, dense)
    q[..., D - rope:] = 0.0
    pool *= 0.25                       # powers of two: still bf16 values
    if kv is not None:
        kv *= 1.0 / 64.0
    theta, scale = 160000.0, 12.0
    cs = ops.csa_rope_table(max(qp) + S + 1, rope, theta)
    dt = torch.bfloat16
    q_pos = torch.tensor(qp, dtype=torch.int32, device="cuda")
    win_pos0 = torch.zeros(B, dtype=torch.int32, device="cuda")
    kvd = dev(kv, dt) if kv is not None else None
    zd = dev(z, torch.float32) if z is not None else None
    if dense:
        out = ops.hca_attn(dev(q, dt), kvd, win_pos0, dev(pool, dt), zd, q_pos, m=m,
                           rope_dim=rope, cs=cs, window=window, scale=scale, dv=dv)
    else:
        out = ops.csa_sparse_attn(dev(q, dt), kvd, win_pos0, dev(pool, dt), dev(idx, torch.int32),
                                  zd, q_pos, rope_dim=rope, cs=cs, window=window, scale=scale,
                                  dv=dv)
    out = host(out)
    for b in range(B):
        t = qp[b] + np.arange(S)
        ref = oracle.attention(q[b], t, kv_win=None if kv is None else kv[b], win_pos0=0,
                               window=window, pool=pool[b], idx=None if dense else idx[b],
                               m=m, sink=z, rope_dim=rope, theta=theta, scale=scale, dv=dv)
        assert np.all(np.isfinite(out[b]))
        err = np.abs(out[b] - ref).max()
        assert err <= BF16_ATOL, (name, b, float(err))


def test_attention_edge_rows(ops):
    """Rows with nothing visible and no sink give zeros; a query position past
    the RoPE table gives NaN; both on the matrix-core and the generic kernel."""
    for (H, D, dv, rope, bf16) in [(64, 512, 512, 64, True), (4, 64, 64, 16, False)]:
        B, S, T, k = 1, 3, 8, 4
        dt = torch.bfloat16 if bf16 else torch.float32
        q = dev(rnd((B, S, H, D), 5, bf16), dt)
        pool = dev(rnd((B, T, D), 6, bf16), dt)
        idx = torch.full((B, S, k), -1, dtype=torch.int32, device="cuda")
        cs = ops.csa_rope_table(10, rope, 1e4)
        q_pos = torch.tensor([2], dtype=torch.int32, device="cuda")
        out = host(ops.csa_sparse_attn(q, None, None, pool, idx, None, q_pos, rope_dim=rope,
                                       cs=cs, window=0, scale=0.1, dv=dv))
        assert np.all(out == 0)
        q_pos = torch.tensor([8], dtype=torch.int32, device="cuda")   # rows at t = 8, 9, 10
        idx[..., 0] = 1
        out = host(ops.csa_sparse_attn(q, None, None, pool, idx, None, q_pos, rope_dim=rope,
                                       cs=cs, window=0, scale=0.1, dv=dv))
        assert np.all(np.isfinite(out[0, :2])) and np.all(np.isnan(out[0, 2]))
    # unsplit launch (many rows): rows past the table are NaN, the rest finite
    H, D, rope = 64, 512, 64
    S = 300
    q = dev(rnd((1, S, H, D), 8, True), torch.bfloat16)
    pool = dev(rnd((1, 8, D), 9, True), torch.bfloat16)
    idx = torch.full((1, S, 4), -1, dtype=torch.int32, device="cuda")
    idx[..., 0] = 2
    cs = ops.csa_rope_table(250, rope, 1e4)
    q_pos = torch.tensor([0], dtype=torch.int32, device="cuda")
    out = host(ops.csa_sparse_attn(q, None, None, pool, idx, None, q_pos, rope_dim=rope, cs=cs,
                                   window=0, scale=0.1))
    assert np.all(np.isfinite(out[0, :250])) and np.all(np.isnan(out[0, 250:]))


def test_attention_deterministic(ops):
    B, S, H, D, dv, rope, T, k, window, m, qp, sink, bf16, dense = ATTN_CASES["csa_mfma_split"]
    q, kv, pool, z, idx = _attn_case(7, B, S, H, D, dv, rope, T, k, window, m, qp, sink, bf16,
                                     dense)
    cs = ops.csa_rope_table(max(qp) + S + 1, rope, 160000.0)
    args = (dev(q, torch.bfloat16), dev(kv, torch.bfloat16),
            torch.zeros(B, dtype=torch.int32, device="cuda"), dev(pool, torch.bfloat16),
            dev(idx, torch.int32), dev(z, torch.float32),
            torch.tensor(qp, dtype=torch.int32, device="cuda"))
    a = ops.csa_sparse_attn(*args, rope_dim=rope, cs=cs, window=window, scale=0.05)
    b = ops.csa_sparse_attn(*args, rope_dim=rope, cs=cs, window=window, scale=0.05)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
