"""GPU parity of mla_ctx_merge_chunk and mla_ctx_neutralize_partials against
the CPU oracle.

Page: "PR #51772 完整报告", 实现拆解 item 3 (accumulate_mla_context_chunk with
output_written; neutralize_empty_context_partials).  Tolerance, from the
arithmetic (fp32 expf / logf and one bf16 rounding on the GPU against float64
and one rounding in the oracle): a single merge within 1 bf16 ulp per output,
or within 2^-20 of the magnitude of the two weighted terms where they cancel
(an fp32-sized difference is then many ulps of the tiny result), and 1e-6
relative (or absolute below 1) for the lse; a chain of n merges
within n bf16 rounding steps (2^-8 relative) of the larger of the values
merged.  The neutral-partial identities, INIT modes and neutralize are exact.

Workloads: random partials over the pages' test-matrix head counts and
several head sizes, partials with -inf entries, strided layouts, the
chunk loop of the long-context stress test (16 chunks), and the full-size
accumulator (16384 query tokens x 64 heads x 128), every token.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_paged_insert_amd import synth
from gpu_util import DEV, announce, bf16_ulps, requires_gpu, run_sliced, u16

pytestmark = [pytest.mark.gpu, requires_gpu]


def f32np(t):
    return t.detach().cpu().numpy().astype(np.float32)


def lse_close(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf) and np.array_equal(got[inf], ref[inf])
    err = np.abs(got[~inf] - ref[~inf])
    assert np.all(err <= 1e-6 * np.maximum(1.0, np.abs(ref[~inf]))), err.max()


def merge_close(got_bits, ref_bits, a, b, la, lb):
    """got within 1 bf16 ulp of ref, or within 2^-20 of |w_a a| + |w_b b| / (w_a + w_b)."""
    ulps = bf16_ulps(got_bits, ref_bits)
    A = np.asarray(la, np.float64).T[:, :, None]
    B = np.asarray(lb, np.float64).T[:, :, None]
    m = np.maximum(A, B)
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isinf(A), 0.0, np.exp(A - m))
        wb = np.where(np.isinf(B), 0.0, np.exp(B - m))
        s = np.where(wa + wb > 0, wa + wb, 1.0)
    fa = oracle.bf16_to_f32(u16(a)).astype(np.float64)
    fb = oracle.bf16_to_f32(u16(b)).astype(np.float64)
    terms = (wa * np.abs(fa) + wb * np.abs(fb)) / s
    err = np.abs(oracle.bf16_to_f32(got_bits).astype(np.float64) -
                 oracle.bf16_to_f32(ref_bits).astype(np.float64))
    ok = (ulps <= 1) | (err <= 2.0 ** -20 * terms)
    assert ok.all(), f"{(~ok).sum()} outputs off; worst {ulps[~ok].max()} ulp"
    return ulps


def gpu_merge(mk, out, lse, part, plse, mode):
    o, l = out.to(DEV).clone(), lse.to(DEV).clone()
    mk.mla_ctx_merge_chunk(o, l, part.to(DEV), plse.to(DEV), mode)
    torch.cuda.synchronize()
    return o, l


def oracle_merge(out, lse, part, plse, mode):
    o, l = u16(out).copy(), f32np(lse).copy()
    oracle.merge_chunk(o, l, u16(part), f32np(plse), mode)
    return o, l


@pytest.mark.parametrize("T,H,D", [(1, 3, 128), (37, 4, 128), (300, 64, 128), (45, 3, 8),
                                   (20, 4, 512), (33, 2, 136)])
def test_single_merge_random(mk, T, H, D):
    announce("merge random", T, H, D)
    d = synth.attention_partials(seed=T + H + D, num_tokens=T, heads=H, head_dim=D, chunks=2,
                                 empty_frac=0.1)
    (oa, ob), (la, lb) = d["outs"], d["lses"]
    go, gl = gpu_merge(mk, oa, la, ob, lb, mk.MLA_MERGE_ACCUMULATE)
    ro, rl = oracle_merge(oa, la, ob, lb, oracle.MERGE_ACCUMULATE)
    ulps = merge_close(u16(go), ro, oa, ob, f32np(la), f32np(lb))
    lse_close(f32np(gl), rl)
    announce(f"outputs identical: {np.mean(ulps == 0):.5f}")



@pytest.mark.parametrize("stretch,offset", [(40.0, 0.0), (1.0, 1.0e5), (0.01, -3.0e4)])
def test_merge_wide_lse_range(mk, stretch, offset):
    """lse values far outside the workload's N(8, 3^2): spread 40x (most
    pairs differ by hundreds, so one weight underflows to 0 and the other
    partial passes through), shifted to 1e5 (exp(lse) itself overflows fp32;
    only differences may be exponentiated), and squeezed to 1/100 of the
    spread around -3e4 (weights nearly equal); 10% of the entries -inf.
    Outputs and lse against the oracle as in the other merge tests."""
    announce("merge wide lse", stretch, offset)
    d = synth.attention_partials(seed=77, num_tokens=300, heads=8, head_dim=128, chunks=2,
                                 empty_frac=0.1)
    (oa, ob), (la, lb) = d["outs"], d["lses"]
    la = la * stretch + offset
    lb = lb * stretch + offset
    go, gl = gpu_merge(mk, oa, la, ob, lb, mk.MLA_MERGE_ACCUMULATE)
    ro, rl = oracle_merge(oa, la, ob, lb, oracle.MERGE_ACCUMULATE)
    ulps = merge_close(u16(go), ro, oa, ob, f32np(la), f32np(lb))
    lse_close(f32np(gl), rl)
    announce(f"outputs identical: {np.mean(ulps == 0):.5f}")


def test_identities_and_edge_cases(mk):
    announce("merge identities")
    T, H, D = 16, 4, 128
    d = synth.attention_partials(seed=11, num_tokens=T, heads=H, head_dim=D, chunks=1)
    o, l = d["outs"][0], d["lses"][0]
    zero, ninf = torch.zeros_like(o), torch.full_like(l, float("-inf"))
    A = mk.MLA_MERGE_ACCUMULATE
    x, lx = gpu_merge(mk, o, l, zero, ninf, A)                 # X + neutral
    assert torch.equal(x.cpu(), o) and torch.equal(lx.cpu(), l)
    y, ly = gpu_merge(mk, zero, ninf, o, l, A)                 # neutral + X
    assert torch.equal(y.cpu(), o) and torch.equal(ly.cpu(), l)
    nan = torch.full_like(o, float("nan"))
    z, lz = gpu_merge(mk, o, l, nan, ninf, A)                  # no keys: output ignored
    assert torch.equal(z.cpu(), o) and torch.equal(lz.cpu(), l)
    w, lw = gpu_merge(mk, nan, ninf, zero, ninf, A)            # neutral + neutral
    assert not u16(w).any() and torch.all(lw.cpu() == float("-inf"))
    big = torch.full_like(l, 300.0)
    v, lv = gpu_merge(mk, o, l, zero, big, A)                  # dominant partial wins
    assert not u16(v).any() and torch.equal(lv.cpu(), big)
    half = torch.full_like(o, 1.5)
    q, lq = gpu_merge(mk, half, l, torch.full_like(o, -0.25), l, A)   # equal lse
    assert torch.all(q.cpu() == 0.625)
    lse_close(f32np(lq), f32np(l).astype(np.float64) + np.log(2.0))


def test_init_modes(mk):
    announce("merge init modes")
    T, H, D = 40, 3, 128
    d = synth.attention_partials(seed=12, num_tokens=T, heads=H, head_dim=D, chunks=1)
    o, l = d["outs"][0].to(DEV), d["lses"][0].to(DEV)
    acc = torch.zeros_like(o)
    lacc = torch.zeros_like(l)
    mk.mla_ctx_merge_chunk(acc, lacc, o, l, mk.MLA_MERGE_INIT_COPY)
    torch.cuda.synchronize()
    assert torch.equal(acc, o) and torch.equal(lacc, l)
    acc2 = o.clone()
    lacc2 = torch.zeros_like(l)
    mk.mla_ctx_merge_chunk(acc2, lacc2, None, l, mk.MLA_MERGE_INIT_WRITTEN)
    torch.cuda.synchronize()
    assert torch.equal(acc2, o) and torch.equal(lacc2, l)
    with pytest.raises(mk.MlaError, match="continuation chunk"):
        mk.mla_ctx_merge_chunk(acc2, lacc2, acc2, l, mk.MLA_MERGE_ACCUMULATE)


def test_strided_layouts(mk):
    """The accumulator as a head-slice of a wider buffer and the lse stored
    [T, H] (viewed as [H, T]): same result as contiguous arrays."""
    announce("merge strided")
    T, H, D = 50, 4, 128
    d = synth.attention_partials(seed=13, num_tokens=T, heads=H, head_dim=D, chunks=2)
    (oa, ob), (la, lb) = d["outs"], d["lses"]
    ro, rl = oracle_merge(oa, la, ob, lb, oracle.MERGE_ACCUMULATE)
    wide = torch.zeros(T, H + 2, D + 64, dtype=torch.bfloat16, device=DEV)
    acc = wide[:, 1:H + 1, 32:32 + D]
    acc.copy_(oa.to(DEV))
    lse_th = la.t().contiguous().to(DEV)            # [T, H] storage
    pw = torch.zeros(T, H, 2 * D, dtype=torch.bfloat16, device=DEV)
    part = pw[:, :, D:]
    part.copy_(ob.to(DEV))
    mk.mla_ctx_merge_chunk(acc, lse_th.t(), part, lb.to(DEV), mk.MLA_MERGE_ACCUMULATE)
    torch.cuda.synchronize()
    merge_close(u16(acc), ro, oa, ob, f32np(la), f32np(lb))
    lse_close(f32np(lse_th.t()), rl)
    assert not u16(wide[:, 0]).any() and not u16(wide[:, H + 1]).any()   # untouched


def test_sixteen_chunk_loop(mk):
    """The long-context loop's 16 chunks on 512 query tokens: init copy, then
    15 merges, GPU chain against the oracle chain on the same partials."""
    announce("merge 16-chunk loop")
    d = synth.attention_partials(seed=14, num_tokens=512, heads=8, head_dim=128, chunks=16,
                                 empty_frac=0.05)
    acc = torch.empty_like(d["outs"][0], device=DEV)
    lacc = torch.empty_like(d["lses"][0], device=DEV)
    ro = np.empty(u16(d["outs"][0]).shape, np.uint16)
    rl = np.empty(f32np(d["lses"][0]).shape, np.float32)
    mag = np.zeros(ro.shape)
    for c in range(16):
        mode = mk.MLA_MERGE_INIT_COPY if c == 0 else mk.MLA_MERGE_ACCUMULATE
        mk.mla_ctx_merge_chunk(acc, lacc, d["outs"][c].to(DEV), d["lses"][c].to(DEV), mode)
        oracle.merge_chunk(ro, rl, u16(d["outs"][c]), f32np(d["lses"][c]), mode)
        mag = np.maximum(mag, np.abs(oracle.bf16_to_f32(u16(d["outs"][c]))))
    torch.cuda.synchronize()
    got = oracle.bf16_to_f32(u16(acc)).astype(np.float64)
    ref = oracle.bf16_to_f32(ro).astype(np.float64)
    tol = 16 * 2.0 ** -8 * np.maximum(mag, np.abs(ref))
    assert np.all(np.abs(got - ref) <= tol)
    lse_close(f32np(lacc), rl)
    announce(f"16-chunk loop: {np.mean(got == ref):.4f} outputs identical")


@pytest.mark.timeout(300)
def test_full_size_accumulate(mk):
    """16384 query tokens x 64 heads x 128: one merge at full size, every
    token against the oracle (token slices on host threads)."""
    announce("merge full size")
    d = synth.attention_partials(num_tokens=16384, heads=64, head_dim=128, chunks=2)
    (oa, ob), (la, lb) = d["outs"], d["lses"]
    go, gl = gpu_merge(mk, oa, la, ob, lb, mk.MLA_MERGE_ACCUMULATE)
    ro, rl = u16(oa).copy(), f32np(la).copy()
    obn, lbn = u16(ob), f32np(lb)
    run_sliced(lambda a, b: oracle.merge_chunk(ro[a:b], rl[:, a:b], obn[a:b], lbn[:, a:b],
                                               oracle.MERGE_ACCUMULATE), 16384)
    ulps = merge_close(u16(go), ro, oa, ob, f32np(la), f32np(lb))
    announce(f"full size: {np.mean(ulps == 0):.5f} identical, {np.mean(ulps <= 1):.6f} within 1 ulp")
    lse_close(f32np(gl), rl)


def test_neutralize(mk):
    announce("neutralize")
    T, H, D = 300, 4, 128
    d = synth.attention_partials(seed=16, num_tokens=T, heads=H, head_dim=D, chunks=1)
    o, l = d["outs"][0], d["lses"][0]
    flags = (torch.arange(T) % 7 == 3)
    go, gl = o.to(DEV).clone(), l.to(DEV).clone()
    mk.mla_ctx_neutralize_partials(go, gl, flags.to(DEV))
    torch.cuda.synchronize()
    ro, rl = u16(o).copy(), f32np(l).copy()
    oracle.neutralize_partials(ro, rl, flags.numpy().astype(np.uint8))
    assert np.array_equal(u16(go), ro) and np.array_equal(f32np(gl), rl)
