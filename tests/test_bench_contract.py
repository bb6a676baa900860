"""CPU checks of bench.py's contract: the algorithmic byte counts it divides
by are the figures derived from the workloads' shapes, and a request for more
than one GPU is refused before anything touches a device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("fn,args,want", [
    # fp8 pack of 8192 tokens x 64 heads: k_nope + v read (2 x 128 bf16), k_pe read once per
    # token (64 bf16); key (192 codes) and V (128 codes) written
    (bench.pack_fp8_bytes, (8192, 64), 8192 * 64 * (512 + 192 + 128) + 8192 * 128),
    (bench.pack_bf16_bytes, (8192, 64), 8192 * 64 * (256 + 384) + 8192 * 128),
    # gather: 576 codes read, 576 bf16 written, one int64 slot per token, the fp32 scale
    (bench.gather_bytes, (8192,), 8192 * (576 + 1152 + 8) + 4),
    # merge: accumulator read + write and the partial read (bf16 rows), three fp32 lse
    (bench.merge_bytes, (16384, 64), 16384 * 64 * (3 * 256 + 3 * 4)),
    # small-batch grouped fp8 insert, 5 layers x 4 tokens, one skipped: 15 rows read and
    # written, 4 shared slots, 5 scales and 5 cache pointers
    (bench.small_insert_bytes, (15, 4, 5, True), 26012),
    # single-layer bf16 insert of 16 tokens: 16 rows read and written, 16 slots
    (bench.small_insert_bytes, (16, 16, 1, False), 36992),
])
def test_byte_formulas(fn, args, want):
    assert fn(*args) == want


def test_long_context_insert_bytes_match_the_workload():
    # 5 layers x 16384 rows: bf16 kv_c + k_pe read (1152 B), one slot each, 576 codes
    # written per row, plus the per-layer pointer and scale
    assert bench.insert_bytes(5, 16384) == 5 * 16384 * (1152 + 8 + 576) + 5 * 12


def test_new_token_bytes_are_mode_specific_sums():
    T, H = 8192, 64
    # per token: latent row, position, slot and the fp32 cos/sin row (256 B)
    fp8 = T * H * (384 + 256 + 256 + 192 + 192 + 128) + T * (1152 + 8 + 8 + 256) + (T - 1) * 576
    bf16 = T * H * (384 + 256 + 384 + 384) + T * (1152 + 8 + 8 + 256) + (T - 1) * 576
    assert bench.new_token_bytes(T, H, True, T - 1) == fp8
    assert bench.new_token_bytes(T, H, False, T - 1) == bf16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_oracle_timed_beside_each_component():
    """Every component outside the timed step gets the oracle's own figure on
    a bounded sample, in the component's unit, with the sample stated."""
    import torch

    import bench

    # the multi-threaded whole projection on a few rows here (the bench runs
    # all 4096)
    r = bench.oracle_components(torch, projection_rows=64)
    assert set(r) == {"small_batch_insert", "context_kv_proj", "context_epilogue", "chunk_merge",
                      "new_token_epilogue"}
    for name, o in r.items():
        assert o["value"] > 0 and o["cores"] == 1 and o["unit"] and o["sample"], name
    mt = r["context_kv_proj"]["all_cores"]
    assert mt["value"] > 0 and mt["cores"] >= 1 and "64 of the 4096 rows" in mt["sample"]
