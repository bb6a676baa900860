"""Pins for the oracle's merge of chunked-context attention partials.

Page: "PR #51772 完整报告", 实现拆解 item 3 (accumulate_mla_context_chunk with
output_written; neutralize_empty_context_partials for prefills without
context).  The pages name the steps, not their arithmetic; the reading is the
log-sum-exp merge of partial softmax results.  What pins it to something
other than itself:
  * brute force: attention over all keys at once (float64, scipy's
    logsumexp) equals the merge of per-chunk partials, chunk by chunk, within
    the bf16 rounding of the partials and of each merge;
  * the neutral partial (0, -inf) is an identity on either side, bit for
    bit, and neutral + neutral stays neutral;
  * merging is symmetric bit for bit; equal lse gives the exact average and
    lse + ln 2; a partial that covers no keys contributes nothing even if its
    output holds NaN;
  * INIT_COPY / INIT_WRITTEN take the partial (output and lse, or lse only).
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def f32(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def chunk_partial(s, v, keys):
    """Float64 attention of all queries over the key subset `keys`:
    s [T, H, N] scores, v [N, H, D] values -> (O [T, H, D] bf16 bits, lse [H, T] f32)."""
    T, H, _ = s.shape
    D = v.shape[2]
    if len(keys) == 0:
        return np.zeros((T, H, D), np.uint16), np.full((H, T), -np.inf, np.float32)
    sc = s[:, :, keys]
    lse = logsumexp(sc, axis=2)                                   # [T, H]
    p = np.exp(sc - lse[:, :, None])                              # [T, H, n]
    o = np.einsum("thn,nhd->thd", p, v[keys])
    return bf16_bits(o), lse.T.astype(np.float32).copy()


@pytest.mark.parametrize("splits", [[0, 7, 19, 40], [0, 40], [0, 0, 13, 13, 40], [0, 1, 2, 40]])
def test_chunk_by_chunk_equals_attention_over_all_keys(orc, splits):
    rng = np.random.default_rng(len(splits) * 7 + splits[1])
    T, H, N, D = 9, 3, 40, 16
    s = rng.normal(0, 3, (T, H, N))
    v = f32(bf16_bits(rng.normal(0, 1, (N, H, D))))               # bf16-exact values
    out, lse = None, None
    mag = np.zeros((T, H, D))              # largest |partial| seen per element
    for c in range(len(splits) - 1):
        o_c, l_c = chunk_partial(s, v, np.arange(splits[c], splits[c + 1]))
        mag = np.maximum(mag, np.abs(f32(o_c)))
        if out is None:
            out, lse = o_c.copy(), np.empty((H, T), np.float32)
            orc.merge_chunk(out, lse, o_c, l_c, orc.MERGE_INIT_COPY)
        else:
            orc.merge_chunk(out, lse, o_c, l_c, orc.MERGE_ACCUMULATE)
    o_ref, l_ref = chunk_partial(s, v, np.arange(N))
    ref = f32(o_ref)
    got = f32(out)
    # each partial and each merge rounds once to bf16 (half an ulp, 2^-9
    # relative, of values no larger than the largest partial)
    n_chunks = len(splits) - 1
    tol = (2 * n_chunks) * 2.0 ** -9 * np.maximum(mag, np.abs(ref)) + 1e-12
    assert np.all(np.abs(got - ref) <= tol), np.max(np.abs(got - ref) - tol)
    assert np.allclose(lse, l_ref, rtol=1e-6, atol=1e-6)


def random_partial(rng, T, H, D, lse_scale=4.0):
    return bf16_bits(rng.normal(0, 1, (T, H, D))), rng.normal(0, lse_scale, (H, T)).astype(np.float32)


def test_neutral_partial_is_an_identity_on_both_sides(orc):
    rng = np.random.default_rng(3)
    T, H, D = 7, 4, 32
    o, l = random_partial(rng, T, H, D)
    zero, ninf = np.zeros_like(o), np.full_like(l, -np.inf)
    a, la = o.copy(), l.copy()
    orc.merge_chunk(a, la, zero, ninf)                       # X + neutral
    assert np.array_equal(a, o) and np.array_equal(la, l)
    b, lb = zero.copy(), ninf.copy()
    orc.merge_chunk(b, lb, o, l)                             # neutral + X
    assert np.array_equal(b, o) and np.array_equal(lb, l)
    c, lc = np.full_like(o, 0x3F80), ninf.copy()             # garbage output, no keys
    orc.merge_chunk(c, lc, zero, ninf)
    assert not c.any() and np.all(lc == -np.inf)


def test_merge_is_symmetric(orc):
    rng = np.random.default_rng(4)
    T, H, D = 11, 3, 24
    oa, la = random_partial(rng, T, H, D)
    ob, lb = random_partial(rng, T, H, D)
    x, lx = oa.copy(), la.copy()
    orc.merge_chunk(x, lx, ob, lb)
    y, ly = ob.copy(), lb.copy()
    orc.merge_chunk(y, ly, oa, la)
    assert np.array_equal(x, y) and np.array_equal(lx, ly)


def test_equal_lse_gives_the_average_and_ln2(orc):
    T, H, D = 2, 2, 8
    oa = bf16_bits(np.full((T, H, D), 1.5))
    ob = bf16_bits(np.full((T, H, D), -0.25))
    l = np.array([[0.0, 3.0], [-2.0, 10.0]], np.float32)
    orc.merge_chunk(oa, l, ob, l.copy())
    assert np.all(f32(oa) == 0.625)
    assert np.allclose(l, np.array([[0.0, 3.0], [-2.0, 10.0]]) + math.log(2.0), rtol=0, atol=1e-6)


def test_partial_without_keys_ignores_its_output(orc):
    rng = np.random.default_rng(5)
    T, H, D = 5, 2, 8
    o, l = random_partial(rng, T, H, D)
    nan_out = np.full_like(o, 0x7FC0)
    a, la = o.copy(), l.copy()
    orc.merge_chunk(a, la, nan_out, np.full_like(l, -np.inf))
    assert np.array_equal(a, o) and np.array_equal(la, l)


def test_dominant_partial_wins(orc):
    """A partial whose lse is 200 above the other's carries all the weight."""
    T, H, D = 3, 2, 8
    oa = bf16_bits(np.full((T, H, D), 3.0))
    ob = bf16_bits(np.full((T, H, D), -7.0))
    la = np.zeros((H, T), np.float32)
    orc.merge_chunk(oa, la, ob, np.full((H, T), 200.0, np.float32))
    assert np.all(f32(oa) == -7.0) and np.all(la == 200.0)


def test_init_modes(orc):
    rng = np.random.default_rng(6)
    T, H, D = 4, 3, 16
    o, l = random_partial(rng, T, H, D)
    acc, lacc = np.zeros_like(o), np.zeros_like(l)
    orc.merge_chunk(acc, lacc, o, l, orc.MERGE_INIT_COPY)
    assert np.array_equal(acc, o) and np.array_equal(lacc, l)
    acc2, lacc2 = o.copy(), np.zeros_like(l)
    orc.merge_chunk(acc2, lacc2, o, l, orc.MERGE_INIT_WRITTEN)   # output already there
    assert np.array_equal(acc2, o) and np.array_equal(lacc2, l)
    acc3 = np.full_like(o, 0x1234)
    orc.merge_chunk(acc3, np.zeros_like(l), o, l, orc.MERGE_INIT_WRITTEN)
    assert np.all(acc3 == 0x1234)                                # output untouched


def test_strided_views(orc):
    """lse given as a [T, H] array viewed as [H, T], outputs as strided views
    of a wider buffer: same result as contiguous arrays."""
    rng = np.random.default_rng(7)
    T, H, D = 6, 4, 16
    oa, la = random_partial(rng, T, H, D)
    ob, lb = random_partial(rng, T, H, D)
    x, lx = oa.copy(), la.copy()
    orc.merge_chunk(x, lx, ob, lb)
    wide = np.zeros((T, H, D + 16), np.uint16)
    wide[:, :, 8:8 + D] = oa
    la_t = np.ascontiguousarray(la.T)                 # [T, H] storage
    orc.merge_chunk(wide[:, :, 8:8 + D], la_t.T, ob, lb)
    assert np.array_equal(wide[:, :, 8:8 + D], x) and np.array_equal(la_t.T, lx)


def test_neutralize_sets_only_flagged_tokens(orc):
    rng = np.random.default_rng(8)
    T, H, D = 6, 2, 8
    o, l = random_partial(rng, T, H, D)
    flags = np.array([1, 0, 0, 1, 0, 1], np.uint8)
    a, la = o.copy(), l.copy()
    orc.neutralize_partials(a, la, flags)
    f = flags.astype(bool)
    assert not a[f].any() and np.all(la[:, f] == -np.inf)
    assert np.array_equal(a[~f], o[~f]) and np.array_equal(la[:, ~f], l[:, ~f])
