"""GPU parity of the grouped low-rank output projection (csa_grouped_out_proj)
against the oracle, stage by stage: mid against the oracle's grouped product,
then out against the oracle's second product of the GPU's own stored mid.

Bounds: a sum of K fp32 products in any order is within K 2^-24 sum |a b| of
the exact sum; a bf16 store rounds to within 2^-8 relative, and two roundings
of nearby sums land at most one bf16 ulp (2^-7 relative) apart."""
import numpy as np
import pytest
import torch

import oracle
from parity import dev, host

pytestmark = pytest.mark.gpu

CASES = {
    # name: (dtype, M, G, Kg, rank, hidden)
    "v4_prefill_rows_bf16": ("bf16", 300, 8, 4096, 1024, 4096),   # 8 groups of 8 heads x 512
    "v4_decode_bf16": ("bf16", 64, 8, 4096, 1024, 4096),
    "small_groups_bf16": ("bf16", 50, 4, 64, 256, 256),
    # K steps of 32 in the matrix-core kernel: 5 then 16 (whole rounds of its
    # 5-stage ring, then one extra step), 1 then 8, 4 then 24
    "ksteps_5_bf16": ("bf16", 70, 2, 160, 256, 256),
    "ksteps_1_bf16": ("bf16", 33, 1, 32, 256, 256),
    "ksteps_4_bf16": ("bf16", 129, 3, 128, 256, 512),
    "generic_bf16": ("bf16", 20, 2, 40, 24, 16),
    "generic_f32": ("f32", 37, 2, 48, 40, 24),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_grouped_out_proj(name):
    from sparse_long_context_pool_amd import csa
    dt_s, M, G, Kg, rank, hidden = CASES[name]
    bf16 = dt_s == "bf16"
    r = np.random.default_rng(len(name) * 7919 + M)

    def draw(shape, scale):
        a = (r.standard_normal(shape) * scale).astype(np.float32)
        return oracle.round_bf16(a) if bf16 else a
    o = draw((M, G * Kg), 1.0)
    w_a = draw((G, rank, Kg), 1.0 / np.sqrt(Kg))
    w_b = draw((hidden, G * rank), 1.0 / np.sqrt(G * rank))
    dt = torch.bfloat16 if bf16 else torch.float32
    mid_g, out_g = csa.csa_grouped_out_proj(dev(o, dt), dev(w_a, dt), dev(w_b, dt))
    mid_g, out_g = host(mid_g), host(out_g)
    u = 2.0 ** -24
    # stage 1
    mid_o, _ = oracle.grouped_out_proj(o, w_a, w_b, round_mid_bf16=bf16)
    absum = np.concatenate([np.abs(o[:, g * Kg:(g + 1) * Kg]).astype(np.float64)
                            @ np.abs(w_a[g]).astype(np.float64).T for g in range(G)], axis=1)
    b1 = Kg * u * absum + (2.0 ** -7 * np.abs(mid_o) if bf16 else 0.0) + 1e-30
    d1 = np.abs(mid_g - mid_o)
    assert np.all(d1 <= b1), (name, float((d1 / b1).max()))
    # stage 2, from the GPU's stored mid
    _, out_o = oracle.grouped_out_proj(None, None, w_b, mid=mid_g)
    K2 = G * rank
    absum2 = np.abs(mid_g).astype(np.float64) @ np.abs(w_b).astype(np.float64).T
    b2 = K2 * u * absum2 + (2.0 ** -8 * np.abs(out_o) if bf16 else 0.0) + 1e-30
    d2 = np.abs(out_g - out_o)
    assert np.all(d2 <= b2), (name, float((d2 / b2).max()))
    # and the result is not trivially small
    assert np.abs(out_o).mean() > 0.1


def test_grouped_out_proj_full_size_sampled():
    """The prefill workload's projection at its full size, in the launch the
    benchmark times ([8192, 64 x 512] -> 8 groups x 1024 -> 4096, bf16, the
    benchmark's seeded inputs), checked on 24 token rows: both ends, both
    sides of 256-row tile seams, and 12 seeded random rows."""
    from sparse_long_context_pool_amd import csa, synth
    S, H, dv, G, rank, hidden = 8192, 64, 512, 8, 1024, 4096
    Kg = H * dv // G
    bf = torch.bfloat16
    o = synth.normal_torch(0, "attn_out", S, (H * dv,), scale=0.5, dtype=bf).to("cuda")
    w_a = synth.normal_torch(0, "o_a_proj", G * rank, (Kg,), scale=Kg ** -0.5,
                             dtype=bf).to("cuda").view(G, rank, Kg)
    w_b = synth.normal_torch(0, "o_b_proj", hidden, (G * rank,), scale=(G * rank) ** -0.5,
                             dtype=bf).to("cuda")
    mid_g, out_g = csa.csa_grouped_out_proj(o, w_a, w_b)
    rng = np.random.default_rng(8192)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095, 4096, 7935, 7936, 8190, 8191],
                                     [2047, 6144], rng.integers(0, S, 12)]))
    ri = torch.tensor(rows, device="cuda")
    o_s = host(o.index_select(0, ri))
    mid_s, out_s = host(mid_g.index_select(0, ri)), host(out_g.index_select(0, ri))
    wa_h, wb_h = host(w_a), host(w_b)
    del o, mid_g, out_g
    torch.cuda.empty_cache()
    u = 2.0 ** -24
    mid_o, _ = oracle.grouped_out_proj(o_s, wa_h, wb_h, round_mid_bf16=True)
    absum = np.concatenate([np.abs(o_s[:, g * Kg:(g + 1) * Kg]).astype(np.float64)
                            @ np.abs(wa_h[g]).astype(np.float64).T for g in range(G)], axis=1)
    b1 = Kg * u * absum + 2.0 ** -7 * np.abs(mid_o) + 1e-30
    d1 = np.abs(mid_s - mid_o)
    assert np.all(d1 <= b1), float((d1 / b1).max())
    _, out_o = oracle.grouped_out_proj(None, None, wb_h, mid=mid_s)
    absum2 = np.abs(mid_s).astype(np.float64) @ np.abs(wb_h).astype(np.float64).T
    b2 = G * rank * u * absum2 + 2.0 ** -8 * np.abs(out_o) + 1e-30
    d2 = np.abs(out_s - out_o)
    assert np.all(d2 <= b2), float((d2 / b2).max())
    assert np.abs(out_o).mean() > 0.01
