"""The fused context-KV epilogue workload end to end on the GPU, checked stage
by stage against the CPU oracle at its full size.

Page: "PR #50585 完整报告", 关键源码片段 (_precompute_fused_context_kv): one
KV-only projection of the context hidden states for all draft layers, its
output viewed as [T, L, 576] and split into kv_c and k_pe, the grouped
RMSNorm of kv_c, RoPE of k_pe at the context positions, then the grouped
insert of "PR #55356 完整报告" (关键源码片段, the grouped path).

Workload: X [4096, 7168] ~ N(0, 1), W [7168, 5 * 576] ~ N(0, 0.02) (the
[K, N] matrix, converted on the GPU into the projection's [N, K] storage
with mla_transpose_bf16), gamma
~ U(0.8, 1.2), eps 1e-6, positions 0..4095, per-layer fp8 scales ~ U(0.5, 2),
5 e4m3fn caches [512, 64, 576] of random bytes, per-layer distinct slots.

Stages, each against the oracle:
  1. projection: every one of the 4096 x 2880 outputs against the oracle's
     float64 product of the same seeded X and W (|d| <= 2e-2 |ref| + 2e-2);
  2. RMSNorm + RoPE: the oracle's norm and RoPE fed the projection output the
     GPU epilogue read (the GPU's Y, through the same [T, L, 576] strides):
     every bf16 row value within 1 ulp of the GPU's rows (dbg_rows);
  3. quantise + scatter: the oracle's grouped insert fed the GPU's rows:
     the five caches equal the GPU's bit for bit;
  4. both together: the caches of the oracle's epilogue of the GPU's Y within
     one fp8 code of the GPU's, and identical wherever the rows agree.
Each oracle stage takes the GPU's output of the stage before, as a check of
that stage alone: the projection's tolerance is many bf16 ulps, so an
end-to-end comparison from X would hide a one-ulp or one-code error in the
stages after it.  Stage 1 compares that input itself with the oracle's own.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_insert_amd import synth
from gpu_util import (DEV, announce, bf16_ulps, check_slots, fp8_codes_apart, requires_gpu,
                      run_sliced, u16, u8)

pytestmark = [pytest.mark.gpu, requires_gpu]


def f32(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


@pytest.mark.timeout(600)
def test_context_kv_projection_epilogue_chain_full(mk):
    announce("context KV chain: projection -> epilogue, 4096 tokens x 5 layers")
    d = synth.context_epilogue("cpu")
    L, T = d["num_layers"], d["num_tokens"]
    x, w_kn = d["x"], d["w_kn"]
    check_slots(d["slot_mapping"], d["caches"][0].shape[0] * d["block_size"])

    # --- GPU: the weight as stated ([K, N]) into the projection's [N, K]
    # storage, the projection, then the epilogue reading its output through
    # strides
    w_nk = torch.empty(L * 576, x.shape[1], dtype=torch.bfloat16, device=DEV)
    mk.mla_transpose_bf16(w_kn.to(DEV), w_nk)
    y = torch.empty(T, L * 576, dtype=torch.bfloat16, device=DEV)
    mk.mla_ctx_kv_proj(x.to(DEV), w_nk, y)
    cs = torch.empty(T, 2 * 64, dtype=torch.float32, device=DEV)
    mk.mla_rope_cos_sin_cache(cs, T, 64, d["rope_base"])
    caches = [c.to(DEV) for c in d["caches"]]
    rows = torch.empty(L, T, 576, dtype=torch.bfloat16, device=DEV)
    mk.mla_ctx_kv_epilogue(y.view(T, L, 576), d["gamma"].to(DEV), d["eps"],
                           d["positions"].to(DEV), cs, caches, d["slot_mapping"].to(DEV),
                           d["block_size"], caches[0].stride(0), caches[0].stride(1),
                           d["scales"].to(DEV), "fp8", dbg_rows=rows)
    torch.cuda.synchronize()
    y_np = u16(y)
    rows_np = u16(rows)
    got_caches = [u8(c) for c in caches]

    # --- 1. projection, every output against the oracle (row slices on threads)
    xn, wn = u16(x), u16(w_kn)
    ref_y = np.concatenate(run_sliced(
        lambda a, b: oracle.gemm_rows(xn, wn, np.arange(a, b, dtype=np.int64)), T))
    g, r = f32(y_np).astype(np.float64), f32(ref_y).astype(np.float64)
    err = np.abs(g - r)
    tol = 2e-2 * np.abs(r) + 2e-2
    assert np.all(err <= tol), f"projection: worst error {err.max()} beyond tolerance"
    ul = bf16_ulps(y_np, ref_y)
    announce(f"projection: {np.mean(ul == 0):.4f} of outputs identical, "
             f"{np.mean(ul <= 1):.6f} within 1 ulp, max {ul.max()} ulp, "
             f"worst error / tolerance {float((err / tol).max()):.4f}")

    # --- 2 + 4. the oracle's epilogue of the GPU's Y (rows and caches)
    ref_caches = [u8(c).copy() for c in d["caches"]]
    sm = d["slot_mapping"].numpy()
    ref_rows = oracle.ctx_kv_epilogue(y_np.reshape(T, L, 576), u16(d["gamma"]), d["eps"],
                                      d["positions"].numpy(), sm, ref_caches,
                                      d["scales"].numpy(), rope_base=d["rope_base"])
    ulps = bf16_ulps(rows_np, ref_rows)
    announce(f"rows: norm part {np.mean(ulps[..., :512] == 0):.6f} identical "
             f"(max {ulps[..., :512].max()} ulp), rope part "
             f"{np.mean(ulps[..., 512:] == 0):.6f} identical (max {ulps[..., 512:].max()} ulp)")
    if ulps.max() > 1:
        for l, t, i in np.argwhere(ulps > 1)[:8]:
            announce(f"  layer {l} token {t} element {i}: gpu 0x{rows_np[l, t, i]:04x} "
                     f"oracle 0x{ref_rows[l, t, i]:04x} input 0x{y_np[t, l * 576 + i]:04x}")
    assert ulps.max() <= 1, f"rows differ by up to {ulps.max()} bf16 ulp"
    for l in range(L):
        gr, rr = got_caches[l].reshape(-1, 576)[sm[l]], ref_caches[l].reshape(-1, 576)[sm[l]]
        assert fp8_codes_apart(gr, rr).max() <= 1, f"layer {l}: codes more than one apart"
        agree = rows_np[l] == ref_rows[l]
        assert np.array_equal(gr[agree], rr[agree]), f"layer {l}: codes differ where rows agree"
        touched = np.zeros(got_caches[l].reshape(-1, 576).shape[0], bool)
        touched[sm[l]] = True
        init = u8(d["caches"][l]).reshape(-1, 576)
        assert np.array_equal(got_caches[l].reshape(-1, 576)[~touched], init[~touched]), \
            f"layer {l}: stray writes"
    announce(f"rows: {np.mean(ulps == 0):.5f} identical to the oracle's")

    # --- 3. quantise + scatter of the GPU's rows, bit for bit
    dbg = [u8(c).copy() for c in d["caches"]]
    oracle.insert_grouped(rows_np[:, :, :512], rows_np[:, :, 512:], sm, dbg,
                          d["scales"].numpy())
    for l in range(L):
        if not np.array_equal(got_caches[l], dbg[l]):
            bad = np.argwhere(got_caches[l] != dbg[l])
            raise AssertionError(f"layer {l}: {len(bad)} cache bytes differ from the "
                                 f"oracle's insert of the GPU rows, first at {bad[0]}")
