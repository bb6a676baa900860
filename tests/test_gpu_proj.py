"""GPU parity of mla_ctx_kv_proj (bf16 MFMA GEMM, fp32 accumulation) against
the CPU oracle (float64 accumulation, one bf16 rounding).

Tolerance: |gpu - oracle| <= 2e-2 * |oracle| + 2e-2 element-wise (rtol 2e-2
for the projection; the absolute term covers outputs near zero, whose
relative error is unbounded).  The one-hot weight test is bit-exact: each
output is a single product x * 1.

Shapes: ragged ones, strided X and Y, a grid with more tiles than compute
units; the full fused context-KV projection (X [4096, 7168], W [7168, 2880])
is checked on every output in tests/test_gpu_context_chain.py.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_insert_amd import synth
from gpu_util import DEV, announce, bf16_ulps, requires_gpu, run_sliced, u16

pytestmark = [pytest.mark.gpu, requires_gpu]


def f32(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def gpu_proj(mk, x, w_kn, y_stride=None):
    T = x.shape[0]
    N = w_kn.shape[1]
    w_nk = w_kn.t().contiguous().to(DEV)
    if y_stride is None:
        y = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    else:
        y = torch.zeros(T, y_stride, dtype=torch.bfloat16, device=DEV)[:, :N]
    mk.mla_ctx_kv_proj(x.to(DEV) if x.device.type == "cpu" else x, w_nk, y)
    torch.cuda.synchronize()
    return y


def check_close(got_bits, ref_bits, what):
    g = f32(got_bits).astype(np.float64)
    r = f32(ref_bits).astype(np.float64)
    err = np.abs(g - r)
    tol = 2e-2 * np.abs(r) + 2e-2
    assert np.all(err <= tol), f"{what}: max err {err.max()} (tol at that point {tol[np.argmax(err - tol)]})"
    ulps = bf16_ulps(got_bits, ref_bits)
    announce(f"{what}: {np.mean(ulps == 0):.4f} exact, max {ulps.max()} bf16 ulp")
    return ulps


@pytest.mark.parametrize("T,K,N", [(1, 64, 16), (300, 128, 208), (256, 192, 192),
                                   (513, 640, 400), (37, 64, 2880),
                                   (200, 320, 192), (129, 384, 96), (64, 448, 2880)])
def test_proj_ragged_shapes(mk, T, K, N):
    """Ragged row and column tiles; K from 1 to 10 stages of 64 (the K loop
    is unrolled by six stages over a three-buffer X ring and a two-buffer W
    ring, so 5, 6 and 7 stages end the loop at each buffer phase)."""
    announce("proj", T, K, N)
    g = torch.Generator().manual_seed(T + K + N)
    x = synth.bf16_normal((T, K), g)
    w = synth.bf16_normal((K, N), g, std=0.05)
    y = gpu_proj(mk, x, w)
    ref = oracle.gemm_rows(u16(x), u16(w))
    check_close(u16(y), ref, f"proj {T}x{K}x{N}")


def test_proj_one_hot_columns_exact(mk):
    announce("proj one-hot")
    g = torch.Generator().manual_seed(9)
    T, K, N = 300, 256, 400
    x = synth.bf16_normal((T, K), g)
    perm = torch.randint(0, K, (N,), generator=g)
    w = torch.zeros(K, N)
    w[perm, torch.arange(N)] = 1.0
    y = gpu_proj(mk, x, w.to(torch.bfloat16))
    assert np.array_equal(u16(y), u16(x)[:, perm.numpy()])


@pytest.mark.parametrize("K", [128, 512])
def test_proj_strided_rows(mk, K):
    """X with a padded row stride (two and eight K stages: the three-buffer X
    ring wraps at K = 512)."""
    announce("proj strided", K)
    g = torch.Generator().manual_seed(10)
    T, N = 200, 96
    xb = synth.bf16_normal((T, K + 64), g)
    x = xb.to(DEV)[:, 32:32 + K]           # row stride K + 64, offset 64 bytes
    w = synth.bf16_normal((K, N), g, std=0.05)
    y = gpu_proj(mk, x, w, y_stride=N + 16)
    ref = oracle.gemm_rows(u16(xb[:, 32:32 + K]), u16(w))
    check_close(u16(y), ref, "proj strided")


def test_proj_more_tiles_than_compute_units(mk):
    """4400 x 256 . 256 x 2880: 18 x 15 = 270 tiles, more than the 256 compute
    units, so some tiles start in a second round; the last tile row is ragged
    (4400 = 17 * 256 + 48).  Every output against the oracle."""
    announce("proj 270 tiles")
    g = torch.Generator().manual_seed(12)
    T, K, N = 4400, 256, 2880
    x = synth.bf16_normal((T, K), g)
    w = synth.bf16_normal((K, N), g, std=0.05)
    y = gpu_proj(mk, x, w)
    xn, wn = u16(x), u16(w)
    ref = np.concatenate(run_sliced(
        lambda a, b: oracle.gemm_rows(xn, wn, np.arange(a, b, dtype=np.int64)), T))
    check_close(u16(y), ref, "proj 270 tiles")


def test_proj_then_epilogue_chain(mk):
    """Projection -> epilogue on the GPU: the projection is within tolerance
    of the oracle, and the epilogue reading the [T, L, 576] projection output
    through strides gives the same caches as on a contiguous copy of it (the
    epilogue's own parity is tested on seeded inputs)."""
    announce("proj -> epilogue chain")
    d = synth.context_epilogue("cpu", num_tokens=256, hidden=1024, num_blocks=8)
    L, T = d["num_layers"], d["num_tokens"]
    y = gpu_proj(mk, d["x"], d["w_kn"])
    ref_y = oracle.gemm_rows(u16(d["x"]), u16(d["w_kn"]))
    check_close(u16(y), ref_y, "chain projection")
    all_kv = y.view(T, L, 576)
    cs = torch.empty(T, 2 * 64, dtype=torch.float32, device=DEV)
    mk.mla_rope_cos_sin_cache(cs, T, 64, 10000.0)
    caches = [c.to(DEV) for c in d["caches"]]
    rows = torch.empty(L, T, 576, dtype=torch.bfloat16, device=DEV)
    mk.mla_ctx_kv_epilogue(all_kv, d["gamma"].to(DEV), d["eps"], d["positions"].to(DEV), cs,
                           caches, d["slot_mapping"].to(DEV), 64, caches[0].stride(0),
                           caches[0].stride(1), d["scales"].to(DEV), "fp8", dbg_rows=rows)
    caches2 = [c.to(DEV) for c in d["caches"]]
    mk.mla_ctx_kv_epilogue(all_kv.contiguous(), d["gamma"].to(DEV), d["eps"],
                           d["positions"].to(DEV), cs, caches2, d["slot_mapping"].to(DEV), 64,
                           caches2[0].stride(0), caches2[0].stride(1), d["scales"].to(DEV), "fp8")
    torch.cuda.synchronize()
    for a, b in zip(caches, caches2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("rows,cols,pad", [(8, 8, 0), (72, 136, 8), (520, 64, 24), (64, 2880, 0)])
def test_transpose_bf16_matches_oracle(mk, rows, cols, pad):
    """mla_transpose_bf16 bit for bit against the oracle's transpose, with
    padded source and destination rows and partial edge tiles."""
    announce("transpose", rows, cols, pad)
    g = torch.Generator().manual_seed(rows + cols + pad)
    srcb = synth.random_bf16_bits((rows, cols + pad), g)
    src = srcb.to(DEV)[:, :cols]
    dstb = torch.zeros(cols, rows + pad, dtype=torch.bfloat16, device=DEV)
    mk.mla_transpose_bf16(src, dstb[:, :rows])
    torch.cuda.synchronize()
    ref = oracle.transpose(u16(srcb)[:, :cols])
    got = u16(dstb)
    assert np.array_equal(got[:, :rows], ref)
    assert not got[:, rows:].any()                 # padding untouched


def test_transpose_of_the_context_weight(mk):
    """The fused context-KV weight as the workload states it, [7168, 2880]
    (the [K, N] matrix), into the [2880, 7168] storage the projection reads:
    every element against the oracle."""
    announce("transpose C3 weight")
    d = synth.context_epilogue("cpu")
    w = d["w_kn"]
    out = torch.empty(w.shape[1], w.shape[0], dtype=torch.bfloat16, device=DEV)
    mk.mla_transpose_bf16(w.to(DEV), out)
    torch.cuda.synchronize()
    assert np.array_equal(u16(out), oracle.transpose(u16(w)))
