"""HIP-graph capture of the library's launches.

A serving loop captures its per-step kernels once and replays them with new
inputs copied into the same buffers.  The captured step here is a KV-only
projection (300 x 512 . 512 x 576: eight K stages, so its three-buffer
LDS ring wraps), a grouped fp8 insert (5 layers x 4 tokens), a new-token
epilogue (4 tokens x 8 heads, fp8 outputs, fp8 cache) and a chunk merge
(4 tokens x 8 heads x 128).  Every
replay runs on fresh inputs written eagerly between replays, and its results
(caches, query / key / V rows, accumulator and lse) must equal bit for bit
the same calls run eagerly from the same starting state.  The library records
no memset into the graph: every kernel writes its outputs directly.
"""
import pytest
import torch

from fp8_paged_insert_amd import synth
from gpu_util import DEV, announce, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

L, T, H, NB, BS = 5, 4, 8, 64, 64


def test_captured_step_replays_match_eager_runs(mk):
    announce("graph capture: projection + grouped insert + new-token epilogue + merge")
    g = synth.gen(77)
    bf = torch.bfloat16
    # static buffers the graph is captured on
    kv = torch.zeros(T, L, 576, dtype=bf, device=DEV)          # token-major latent rows
    caches = [synth.random_bytes((NB, BS, 576), g).to(DEV) for _ in range(L)]
    ptrs = mk.cache_ptr_table(caches)
    scales = synth.f32_uniform((L,), 0.5, 2.0, g).to(DEV)
    slots = torch.zeros(L, T, dtype=torch.int64, device=DEV)
    q = torch.zeros(T, H, 192, dtype=bf, device=DEV)
    kvb = torch.zeros(T, H, 256, dtype=bf, device=DEV)
    lat = torch.zeros(T, 576, dtype=bf, device=DEV)
    pos = torch.zeros(T, dtype=torch.int64, device=DEV)
    cs = torch.empty(4096, 2 * 64, dtype=torch.float32, device=DEV)
    mk.mla_rope_cos_sin_cache(cs, 4096, 64, 10000.0)
    nt_cache = synth.random_bytes((16, BS, 576), g).to(DEV)
    nt_slots = torch.zeros(T, dtype=torch.int64, device=DEV)
    nt_scale = torch.tensor([0.75], dtype=torch.float32, device=DEV)
    q_out = torch.empty(T, H, 192, dtype=torch.uint8, device=DEV)
    k_out = torch.empty(T, H, 192, dtype=torch.uint8, device=DEV)
    v_out = torch.empty(T, H, 128, dtype=torch.uint8, device=DEV)
    acc = synth.bf16_normal((T, H, 128), g).to(DEV)
    lacc = torch.randn(H, T, generator=g).to(DEV)
    part = torch.zeros(T, H, 128, dtype=bf, device=DEV)
    plse = torch.zeros(H, T, dtype=torch.float32, device=DEV)
    px = torch.zeros(300, 512, dtype=bf, device=DEV)
    pw = torch.zeros(576, 512, dtype=bf, device=DEV)
    py = torch.empty(300, 576, dtype=bf, device=DEV)

    def step():
        mk.mla_ctx_kv_proj(px, pw, py)
        mk.mla_kv_insert_grouped(kv[:, :, :512].permute(1, 0, 2), kv[:, :, 512:].permute(1, 0, 2),
                                 ptrs, slots, BS, BS * 576, 576, scales, "fp8")
        mk.mla_new_token_epilogue(q[..., :128], q[..., 128:], kvb[..., :128], lat[:, :512],
                                  lat[:, 512:], pos, cs, q_out, k_out, v=kvb[..., 128:],
                                  v_out=v_out, mode=mk.MLA_PACK_KEY_V_FP8, cache=nt_cache,
                                  slot_mapping=nt_slots, kv_cache_dtype="fp8",
                                  cache_scale=nt_scale)
        mk.mla_ctx_merge_chunk(acc, lacc, part, plse, mk.MLA_MERGE_ACCUMULATE)

    def fill(seed):
        """Fresh inputs for one step, written eagerly into the static buffers."""
        r = synth.gen(seed)
        kv.copy_(synth.bf16_normal((T, L, 576), r).to(DEV))
        s = torch.stack([synth.randperm(NB * BS, r)[:T] for _ in range(L)])
        s[:, T - 1] = -1
        slots.copy_(s.to(DEV))
        q.copy_(synth.bf16_normal((T, H, 192), r).to(DEV))
        kvb.copy_(synth.bf16_normal((T, H, 256), r).to(DEV))
        lat.copy_(synth.bf16_normal((T, 576), r).to(DEV))
        pos.copy_(torch.randint(0, 4096, (T,), generator=r).to(DEV))
        ns = synth.randperm(16 * BS, r)[:T].clone()
        ns[1] = -1
        nt_slots.copy_(ns.to(DEV))
        part.copy_(synth.bf16_normal((T, H, 128), r).to(DEV))
        plse.copy_((4.0 * torch.randn(H, T, generator=r)).to(DEV))
        px.copy_(synth.bf16_normal((300, 512), r).to(DEV))
        pw.copy_(synth.bf16_normal((576, 512), r, std=0.05).to(DEV))

    state = lambda: [*caches, nt_cache, acc, lacc]             # noqa: E731
    outputs = lambda: [*state(), q_out, k_out, v_out, py]     # noqa: E731

    # warm up eagerly on a side stream, then capture
    fill(1000)
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        fill(2000 + rep)
        before = [t.clone() for t in state()]
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outputs()]
        for t, b in zip(state(), before):                      # rewind, then run eagerly
            t.copy_(b)
        step()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, outputs())):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a,
                               b.view(torch.uint8) if b.dtype != torch.float32 else b), (rep, i)
        # the replay did write: the inserted rows changed the caches
        assert not all(torch.equal(a, b) for a, b in zip(got[:L], before[:L])), rep
