"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

DEV = torch.device("cuda:0")

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def u16(t):
    """bf16 tensor (any device, any strides) -> contiguous numpy uint16 bits."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def u8(t):
    return t.detach().contiguous().cpu().view(torch.uint8).numpy()


def ordered_bf16(bits):
    b = np.asarray(bits).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def bf16_ulps(a, b):
    return np.abs(ordered_bf16(a) - ordered_bf16(b))


def ordered_e4m3(codes):
    c = np.asarray(codes).astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def fp8_codes_apart(a, b):
    return np.abs(ordered_e4m3(a) - ordered_e4m3(b))


def tensor_to_dev(v):
    """Copy to the GPU keeping the layout: permuted views keep their strides
    and a layer-broadcast (stride 0) mapping stays a broadcast."""
    if v.dim() == 2 and v.stride(0) == 0 and v.shape[0] > 1:
        return v[0].to(DEV).unsqueeze(0).expand(v.shape[0], v.shape[1])
    return v.to(DEV)


def to_dev(d):
    out = {}
    for k, v in d.items():
        if isinstance(v, torch.Tensor):
            out[k] = tensor_to_dev(v)
        elif isinstance(v, list) and v and isinstance(v[0], torch.Tensor):
            out[k] = [x.to(DEV) for x in v]
        else:
            out[k] = v
    return out


def announce(*what):
    print("[gpu-case]", *what, flush=True)


def check_slots(slot_mapping, num_slots):
    """Host-side precondition check before a launch: every valid slot lies in
    the cache and no layer names a slot twice."""
    sm = slot_mapping.detach().cpu()
    sm = sm.reshape(-1, sm.shape[-1]) if sm.dim() > 1 else sm.reshape(1, -1)
    assert int(sm.max()) < num_slots if sm.numel() else True, "slot beyond the cache"
    for row in sm:
        v = row[row >= 0]
        assert v.unique().numel() == v.numel(), "duplicate slot in one layer"


def host_threads():
    """Host threads for slicing oracle work: the CPUs this process may use,
    at most 16 (one GPU's share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def run_sliced(fn, n, parts=None):
    """fn(lo, hi) over disjoint consecutive slices of range(n), run on host
    threads (the oracle's C calls release the GIL, so slices run in
    parallel); the results come back in slice order.  Only the work is
    split: each slice is the oracle's own call on that slice."""
    parts = parts or 4 * host_threads()
    edges = np.linspace(0, n, max(1, min(parts, n)) + 1).astype(np.int64)
    spans = [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]
    with ThreadPoolExecutor(host_threads()) as ex:
        futs = [ex.submit(fn, a, b) for a, b in spans]
        return [f.result() for f in futs]
