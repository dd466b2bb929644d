"""The whole CSA step captured in one HIP graph (as the benchmark times it):
every replay gives exactly the eager result, with unrelated eager work and
synchronisations between the replays.  Two sizes: one whose attention runs
unsplit, one (few rows) whose attention splits its keys and merges them.  The
eager reference of the compression is also checked against separate
csa_compress calls."""
import pytest
import torch

from parity import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    from sparse_long_context_pool_amd import csa
    assert torch.cuda.is_available()
    csa.lib()
    return csa


def _pipeline(ops, S, ctx, q_pos0):
    g = torch.Generator().manual_seed(S + ctx)

    def rn(*shape, scale=0.5, dtype=torch.bfloat16):
        return dev((torch.randn(*shape, generator=g) * scale).numpy(), dtype)

    B, H, D, R, m, nI, cI, topk, win = 1, 64, 512, 64, 4, 64, 128, 512, 128
    T = ctx // m
    cs = ops.csa_rope_table(max(q_pos0 + S, ctx), R, 160000.0)
    x, gate = rn(B, ctx, D), rn(B, ctx, D)
    xi, gi = rn(B, ctx, cI), rn(B, ctx, cI)
    q, q_idx = rn(B, S, H, D), rn(B, S, nI, cI)
    w_idx = rn(B, S, nI, dtype=torch.float32)
    sink = rn(H, scale=1.0, dtype=torch.float32)
    q_pos = torch.full((B,), q_pos0, dtype=torch.int32, device="cuda")
    win_pos0 = torch.zeros((B,), dtype=torch.int32, device="cuda")
    kv_win = torch.empty_like(x)
    pool = torch.empty((B, T, D), dtype=torch.bfloat16, device="cuda")
    k_idx = torch.empty((B, T, cI), dtype=torch.bfloat16, device="cuda")
    scores = torch.zeros((B, S, T), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, S, topk), dtype=torch.int32, device="cuda")
    out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
    need = ops.lib().csa_sparse_attn_workspace_size(B, S, H, D, D, R, topk, win, 1)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    passes = [dict(x=x, m=1, overlap=0, rope_dim=R, cs=cs, pos0=0, out=kv_win),
              dict(x=x, gate=gate, m=m, overlap=1, rope_dim=R, cs=cs, pos0=0, out=pool),
              dict(x=xi, gate=gi, m=m, overlap=1, out=k_idx)]

    def step():
        # the three compression passes in one launch, as the benchmark's step runs them
        ops.csa_compress_many(passes)
        ops.csa_index_scores(q_idx, w_idx, k_idx, q_pos, m=m, out=scores)
        ops.csa_topk(scores, q_pos, k=topk, m=m, out=idx)
        ops.csa_sparse_attn(q, kv_win, win_pos0, pool, idx, sink, q_pos, rope_dim=R, cs=cs,
                            window=win, scale=D ** -0.5, out=out, workspace=ws)

    def separate():
        return (ops.csa_compress(x, m=1, overlap=0, rope_dim=R, cs=cs, pos0=0),
                ops.csa_compress(x, gate, m=m, overlap=1, rope_dim=R, cs=cs, pos0=0),
                ops.csa_compress(xi, gi, m=m, overlap=1))

    return step, (kv_win, pool, k_idx, scores, idx, out), separate


@pytest.mark.parametrize("S,ctx,q_pos0", [(1024, 4096, 3072), (4, 8192, 8188)])
def test_step_graph_replays(ops, S, ctx, q_pos0):
    step, outs, separate = _pipeline(ops, S, ctx, q_pos0)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    for name, a, b in zip(("kv_win", "pool", "k_idx"), separate(), ref[:3]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    junk = torch.ones(1 << 20, device="cuda")
    for rep in range(4):
        for t in outs:          # stale results must not survive a replay
            t.view(torch.uint8).fill_(0xFF)
        junk.mul_(1.5).sum()    # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("kv_win", "pool", "k_idx", "scores", "idx", "out"), outs, ref):
            if name == "scores":    # only entries w < R(t) are written
                continue
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rep, name)
        # the scores the top-k read: the ready entries of every row
        m, T = 4, ctx // 4
        for i in (0, S // 2, S - 1):
            r = min(T, (q_pos0 + i + 1) // m)
            assert torch.equal(outs[3][0, i, :r], ref[3][0, i, :r]), (rep, i)
