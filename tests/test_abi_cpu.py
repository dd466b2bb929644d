"""The C-ABI library loads, exports every entry point include/csa.h declares,
and rejects invalid arguments on the host -- all without touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:csa_status_t|size_t|const char \*)\s*\**\s*(\w+)\s*\(",
                                 text)))


@pytest.fixture(scope="module")
def L():
    from sparse_long_context_pool_amd import csa
    return csa.lib()


def test_header_declares_the_hot_path():
    names = declared_functions()
    for n in ("csa_rope_table", "csa_compress", "csa_index_scores", "csa_topk",
              "csa_sparse_attn", "hca_attn", "csa_last_error"):
        assert n in names


def test_library_resolves_every_symbol():
    # immediate binding: a kernel whose launch stub the compiler failed to emit
    # shows up here as an undefined symbol rather than at first use on a GPU
    from sparse_long_context_pool_amd import csa
    ctypes.CDLL(csa._LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    from sparse_long_context_pool_amd import csa
    assert set(csa.EXPORTS) == set(declared_functions())
    assert b"gfx950" in L.csa_version()


def test_debug_build_loads_and_exports_the_same_entry_points():
    from sparse_long_context_pool_amd import csa
    D = csa.load(csa.DEBUG_LIB_PATH)
    for name in declared_functions():
        assert hasattr(D, name), name
    assert b"debug" in D.csa_version()
    assert b"debug" not in csa.lib().csa_version()
    # host-side checks are the same in both builds
    nul = None
    assert D.csa_compress(nul, nul, nul, nul, 1, 8, 12, 4, 1, 0, nul, 0, 0, 1, nul) == 1


def test_invalid_arguments_are_rejected_on_the_host(L):
    nul = None
    # YaRN table: factor below 1, beta_fast not above beta_slow
    dummy = ctypes.c_void_p(16)
    assert L.csa_rope_table_yarn(dummy, 10, 64, 1e4, 0.5, 4096, 32.0, 1.0, nul) == 1
    assert b"factor" in L.csa_last_error()
    assert L.csa_rope_table_yarn(dummy, 10, 64, 1e4, 4.0, 4096, 1.0, 1.0, nul) == 1
    # unknown dtype
    assert L.csa_compress(nul, nul, nul, nul, 1, 8, 8, 4, 1, 0, nul, 0, 0, 7, nul) == 1
    assert b"dtype" in L.csa_last_error()
    # D not a multiple of 8
    assert L.csa_compress(nul, nul, nul, nul, 1, 8, 12, 4, 1, 0, nul, 0, 0, 1, nul) == 1
    # odd rope_dim
    assert L.csa_compress(nul, nul, nul, nul, 1, 8, 16, 4, 1, 3, nul, 0, 0, 1, nul) == 1
    # missing tensors
    assert L.csa_compress(nul, nul, nul, nul, 1, 8, 16, 4, 1, 0, nul, 0, 0, 1, nul) == 1
    assert b"required" in L.csa_last_error()
    # RoPE positions beyond the table
    fake = ctypes.c_void_p(0x10000)
    assert L.csa_compress(fake, nul, nul, fake, 1, 64, 16, 4, 1, 8, fake, 10, 0, 1, nul) == 1
    assert b"RoPE table" in L.csa_last_error()
    # misaligned pointer
    odd = ctypes.c_void_p(0x10002)
    assert L.csa_compress(odd, nul, nul, fake, 1, 64, 16, 4, 1, 0, nul, 0, 0, 1, nul) == 1
    assert b"aligned" in L.csa_last_error()
    # index scores: k must be >= 1 for top-k, bad sizes
    assert L.csa_topk(nul, nul, nul, 1, 4, 16, 0, 4, nul) == 1
    assert L.csa_index_scores(nul, nul, nul, nul, nul, 1, 4, 16, 0, 32, 4, 1, nul) == 1
    assert L.csa_index_scores(nul, nul, nul, nul, nul, 1, 4, 16, 2, 30, 4, 1, nul) == 1
    # attention: dv must be D or D - rope_dim
    args = [fake, fake, fake, 8, fake, 4, fake, 2, nul, fake, fake, 1, 4, 4, 64, 50, 16,
            fake, 100, 8, ctypes.c_float(0.125), nul, ctypes.c_size_t(0), 1, nul]
    assert L.csa_sparse_attn(*args) == 1
    assert b"dv" in L.csa_last_error()
    args[15] = 48          # D - rope_dim: accepted shape-wise, but a zero scale is not
    args[20] = ctypes.c_float(0.0)
    assert L.csa_sparse_attn(*args) == 1
    assert b"scale" in L.csa_last_error()
    # hca: m must be >= 1
    hargs = [fake, fake, fake, 8, fake, 4, 0, nul, fake, fake, 1, 4, 4, 64, 64, 16, fake, 100,
             8, ctypes.c_float(0.125), nul, ctypes.c_size_t(0), 1, nul]
    assert L.hca_attn(*hargs) == 1
    # empty work is OK and enqueues nothing
    assert L.csa_topk(nul, nul, nul, 0, 4, 16, 2, 4, nul) == 0
    assert L.csa_compress(nul, nul, nul, nul, 1, 3, 16, 4, 1, 0, nul, 0, 0, 1, nul) == 0


def test_compress_many_checks_every_pass_before_enqueueing(L):
    from sparse_long_context_pool_amd.csa import CompressPass
    arr = (CompressPass * 17)()
    for c in arr:
        c.x = c.pool = 0x10000
        c.B, c.S, c.D, c.m, c.overlap = 1, 64, 16, 4, 1
    arr[1].D = 12                   # pass 1 invalid: nothing may be enqueued for pass 0
    assert L.csa_compress_many(arr, 2, 1, None) == 1
    assert b"pass 1" in L.csa_last_error()
    arr[1].D = 16
    arr[1].rope_dim, arr[1].cs, arr[1].n_pos = 8, 0x10000, 10   # table too short
    assert L.csa_compress_many(arr, 2, 1, None) == 1
    assert b"RoPE table" in L.csa_last_error()
    assert L.csa_compress_many(arr, 17, 1, None) == 1           # too many passes
    assert L.csa_compress_many(arr, 1, 7, None) == 1            # unknown dtype
    assert L.csa_compress_many(None, 0, 1, None) == 0           # nothing to do
    arr[0].S = 3                                                # no whole window: no work
    assert L.csa_compress_many(arr, 1, 1, None) == 0


def test_cache_append_many_checks_every_pass_before_enqueueing(L):
    from sparse_long_context_pool_amd.csa import CachePass
    arr = (CachePass * 17)()
    for c in arr:
        c.x = c.ring_x = c.pool = c.count = 0x10000
        c.B, c.n, c.D, c.m, c.overlap, c.T_cap = 2, 1, 64, 4, 1, 8
    arr[1].win = 0x10000                 # pass 1: a window buffer but W = 0
    assert L.csa_cache_append_many(arr, 2, 1, None) == 1
    assert b"pass 1" in L.csa_last_error()
    arr[1].win = None
    arr[1].D = 2048                      # beyond the supported width
    assert L.csa_cache_append_many(arr, 2, 1, None) == 2
    assert L.csa_cache_append_many(arr, 17, 1, None) == 1      # too many passes
    assert L.csa_cache_append_many(arr, 1, 9, None) == 1       # unknown dtype
    assert L.csa_cache_append_many(None, 0, 1, None) == 0      # nothing to do
    arr[0].n = 0                                               # no token: no work
    assert L.csa_cache_append_many(arr, 1, 1, None) == 0


def test_cache_append_rejects_bad_arguments_on_the_host(L):
    nul = None
    fake = ctypes.c_void_p(0x10000)

    def call(x=fake, gate=nul, ring_x=fake, ring_g=nul, pool=fake, win=nul, count=fake, B=2,
             n=1, D=64, m=4, ov=1, T_cap=8, W=0, R=0, cs=nul, n_pos=0, dt=1):
        return L.csa_cache_append(x, gate, nul, ring_x, ring_g, pool, win, count, B, n, D, m,
                                  ov, T_cap, W, R, cs, n_pos, dt, nul)
    assert call(dt=5) == 1 and b"dtype" in L.csa_last_error()
    assert call(D=60) == 1                                   # D % 8
    assert call(m=0) == 1 and b"bad sizes" in L.csa_last_error()
    assert call(m=200, ov=1) == 2                            # window of 400 rows
    assert call(gate=fake) == 1 and b"gate and ring_g" in L.csa_last_error()
    assert call(W=8) == 1 and b"win" in L.csa_last_error()
    assert call(count=nul) == 1 and b"required" in L.csa_last_error()
    assert call(R=16) == 1 and b"RoPE table" in L.csa_last_error()
    assert call(pool=ctypes.c_void_p(0x10004)) == 1 and b"aligned" in L.csa_last_error()
    assert call(n=0) == 0                                    # nothing to append


def test_ring_window_must_cover_every_row(L):
    fake = ctypes.c_void_p(0x10000)
    # window 8, S = 4 query rows: a ring (win_pos0 NULL) needs L_win >= 11
    args = [fake, fake, None, 10, fake, 4, fake, 2, None, fake, fake, 1, 4, 4, 64, 64, 16,
            fake, 100, 8, ctypes.c_float(0.125), None, ctypes.c_size_t(0), 1, None]
    assert L.csa_sparse_attn(*args) == 1
    assert b"ring window" in L.csa_last_error()


def test_workspace_plans(L):
    # decode shape: few rows, many keys -> split over workgroups, workspace > 0
    ws = L.csa_sparse_attn_workspace_size(64, 1, 64, 512, 512, 64, 2048, 128, 1)
    # (per split and row: fp32 max and sum, and bf16 partial outputs, for 64 heads)
    assert ws > 0 and ws % (64 * 64 * (2 * 4 + 512 * 2)) == 0
    # prefill shape: enough rows -> no split
    assert L.csa_sparse_attn_workspace_size(1, 8192, 64, 512, 512, 64, 512, 128, 1) == 0
    # fp32 never splits
    assert L.csa_sparse_attn_workspace_size(1, 4, 4, 64, 64, 16, 16, 32, 0) == 0
    assert L.hca_attn_workspace_size(1, 2, 64, 512, 512, 64, 512, 128, 1) > 0


# ------------------------------------------------------------------ probe library
PROBE_HEADER = os.path.join(ROOT, "include", "csa_probe.h")


def probe_declared_functions():
    text = open(PROBE_HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|double)\s+(\w+)\s*\(", text)))


def test_probe_library_exports_its_header():
    from sparse_long_context_pool_amd import probe
    P = probe.lib()
    names = probe_declared_functions()
    assert names == sorted(probe.EXPORTS)
    for n in names:
        assert hasattr(P, n), n
    ctypes.CDLL(probe._LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_probe_arguments_are_checked_on_the_host():
    from sparse_long_context_pool_amd import probe
    P = probe.lib()
    assert P.csa_probe_mfma_bf16(None, 4, 10, None) != 0
    assert P.csa_probe_mfma_bf16(ctypes.c_void_p(16), 0, 10, None) != 0
    assert P.csa_probe_read(None, 1024, ctypes.c_void_p(16), 4, None) != 0
    assert P.csa_probe_read(ctypes.c_void_p(16), 1000, ctypes.c_void_p(16), 4, None) != 0
    assert P.csa_probe_read(ctypes.c_void_p(8), 1024, ctypes.c_void_p(16), 4, None) != 0
    # 4 waves x 8 chains x 32768 flop per round
    assert P.csa_probe_mfma_flops(3, 7) == 3 * 4 * 8 * 32768 * 7
