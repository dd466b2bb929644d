"""csa_sparse_attn_noalloc (the entry point that allocates nothing: its split
partials live in the library's own device array) against csa_sparse_attn with
a caller workspace, through the C ABI: two calls in a row, the second on a
smaller input, both bit-identical to the workspace entry point and within the
bf16 bar of the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import BF16_ATOL, dev, host

pytestmark = pytest.mark.gpu


def _case(seed, B, T, k, window, qpos):
    r = np.random.default_rng(seed)
    H, D = 64, 512

    def bf(shape):
        return oracle.round_bf16(r.standard_normal(shape).astype(np.float32))
    q = bf((B, 1, H, D))
    L = window
    kv = bf((B, L, D))
    pool = bf((B, T, D))
    z = r.standard_normal(H).astype(np.float32)
    idx = np.full((B, 1, k), -1, np.int32)
    for b in range(B):
        R = oracle.ready_count(qpos[b], 4, T)
        sel = np.sort(r.choice(R, size=min(k, R), replace=False))
        idx[b, 0, :len(sel)] = sel
    return q, kv, pool, z, idx


@pytest.mark.parametrize("first,second", [((6, 3000, 2048), (2, 1500, 1024))])
def test_noalloc_matches_workspace_entry(first, second):
    from sparse_long_context_pool_amd import csa
    assert torch.cuda.is_available()
    window, rope, theta = 128, 64, 160000.0
    for call, (B, T, k) in enumerate((first, second)):
        qpos = [4 * T + 7 * b + call for b in range(B)]
        q, kv, pool, z, idx = _case(100 + call, B, T, k, window, qpos)
        cs = csa.csa_rope_table(max(qpos) + 2, rope, theta)
        args = (dev(q, torch.bfloat16), dev(kv, torch.bfloat16),
                torch.tensor([p - window + 1 for p in qpos], dtype=torch.int32, device="cuda"),
                dev(pool, torch.bfloat16), dev(idx, torch.int32), dev(z, torch.float32),
                torch.tensor(qpos, dtype=torch.int32, device="cuda"))
        kw = dict(rope_dim=rope, cs=cs, window=window, scale=1.0 / math.sqrt(512))
        need = csa.lib().csa_sparse_attn_workspace_size(B, 1, 64, 512, 512, rope, k, window, 1)
        assert need > 0, "the shape must split its keys over workgroups"
        a = csa.csa_sparse_attn_noalloc(*args, **kw)
        ref = csa.csa_sparse_attn(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), ref.view(torch.int16)), call
        out = host(a)
        for b in (0, B - 1):
            o = oracle.attention(q[b], np.array([qpos[b]]), kv_win=kv[b],
                                 win_pos0=qpos[b] - window + 1, window=window, pool=pool[b],
                                 idx=idx[b], m=4, sink=z, rope_dim=rope, theta=theta,
                                 scale=1.0 / math.sqrt(512))
            err = float(np.abs(out[b] - o).max())
            assert err <= BF16_ATOL, (call, b, err)


def test_noalloc_rejects_shapes_beyond_its_array():
    """255 query rows of 64 heads split in two need about 32 MiB of partials,
    more than the library's 24 MiB array: a clear error, nothing launched."""
    from sparse_long_context_pool_amd import csa
    B, T, k, window = 255, 256, 64, 0
    need = csa.lib().csa_sparse_attn_workspace_size(B, 1, 64, 512, 512, 64, k, window, 1)
    assert need > (24 << 20)
    q = torch.zeros((B, 1, 64, 512), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((B, T, 512), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((B, 1, k), dtype=torch.int32, device="cuda")
    cs = csa.csa_rope_table(2048, 64, 1e4)
    q_pos = torch.full((B,), 1024, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="scratch"):
        csa.csa_sparse_attn_noalloc(q, None, None, pool, idx, None, q_pos, rope_dim=64, cs=cs,
                                    window=0, scale=0.05)
