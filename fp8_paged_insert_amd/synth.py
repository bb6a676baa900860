"""Seeded synthetic inputs for the insert / epilogue / gather / pack workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no norm, rotation, quantisation or indexing of caches).
Both the HIP path's tests and the CPU oracle's tests take their inputs from
here, so the two sides always see identical bytes.

Every generator takes a seed and a torch device; bf16 values are float32
normal draws rounded to bf16 by torch, fp8 caches are pre-filled with random
finite e4m3fn codes or random bytes so that any stray write is visible.

Workload shapes (all quoted from the statement of the problem; the pages give
the model geometry: 5 draft layers, kv_lora_rank 512, rope dim 64):
  single_layer_bf16   L=1, T=16, bf16 cache [4, 16, 576]
  small_batch_fp8     L=5, T=4 token-major, fp8 caches [512, 64, 576], shared
                      slot mapping with one -1
  context_epilogue    X [4096, 7168], W [7168, 2880], gamma [5, 512], 5 fp8 caches
                      [512, 64, 576], per-layer slots
  context_pack        fp8 cache [512, 64, 576] (scale 0.5) holding 8192 tokens,
                      kv_b_proj output [8192, 64, 256]
  long_context        insert L=5 x 16384 tokens into [4096, 64, 576] caches;
                      16 pack chunks of 8192 tokens from a [4096, 64, 576] cache
  grouped_test_shape  L=5, T=42, block 16, 8 blocks, scales linspace(.05,.25)
"""
from __future__ import annotations

import torch

KV_LORA_RANK = 512
PE_DIM = 64
KV_WIDTH = KV_LORA_RANK + PE_DIM
NUM_LAYERS = 5


def gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def bf16_normal(shape, g, device="cpu", std=1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.bfloat16)


def f16_normal(shape, g, device="cpu", std=1.0) -> torch.Tensor:
    """N(0, std^2) rounded to IEEE fp16 (values beyond 65504 become inf)."""
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.float16)


def f32_uniform(shape, lo, hi, g, device="cpu") -> torch.Tensor:
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return lo + (hi - lo) * u


def bf16_uniform(shape, lo, hi, g, device="cpu") -> torch.Tensor:
    return f32_uniform(shape, lo, hi, g, device).to(torch.bfloat16)


def random_bytes(shape, g, device="cpu") -> torch.Tensor:
    return torch.randint(0, 256, shape, generator=g, device=device,
                         dtype=torch.int32).to(torch.uint8)


def random_bf16_bits(shape, g, device="cpu") -> torch.Tensor:
    """Random 16-bit patterns viewed as bf16 (cache pre-fill for bf16 caches)."""
    r = torch.randint(-32768, 32768, shape, generator=g, device=device,
                      dtype=torch.int32).to(torch.int16)
    return r.view(torch.bfloat16)


def finite_e4m3_codes(shape, g, device="cpu") -> torch.Tensor:
    """Uniform over the 254 finite e4m3fn codes (0x7F and 0xFF are NaN)."""
    r = torch.randint(0, 254, shape, generator=g, device=device, dtype=torch.int32)
    r = r + (r >= 0x7F).to(torch.int32)  # skip 0x7F
    return r.to(torch.uint8)             # 0..0xFE, never 0x7F or 0xFF


def randperm(n, g, device="cpu") -> torch.Tensor:
    return torch.randperm(n, generator=g, device=device, dtype=torch.int64)


def block_table_slots(blocks: torch.Tensor, block_size: int, num_tokens: int) -> torch.Tensor:
    """Flatten a sequence's block table into one slot per context token."""
    j = torch.arange(num_tokens, dtype=torch.int64, device=blocks.device)
    return blocks[j // block_size] * block_size + j % block_size


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------

def single_layer_bf16(device="cpu", seed=1):
    g = gen(seed, device)
    T = 16
    return dict(
        kv_c=bf16_normal((1, T, KV_LORA_RANK), g, device),
        k_pe=bf16_normal((1, T, PE_DIM), g, device),
        caches=[random_bf16_bits((4, 16, KV_WIDTH), g, device)],
        slot_mapping=randperm(64, g, device)[:T].reshape(1, T).contiguous(),
        scales=None, num_layers=1, num_tokens=T, block_size=16)


def small_batch_fp8(device="cpu", seed=2):
    g = gen(seed, device)
    L, T = NUM_LAYERS, 4
    kv_c_tm = bf16_normal((T, L, KV_LORA_RANK), g, device)
    k_pe_tm = bf16_normal((T, L, PE_DIM), g, device)
    caches = [random_bytes((512, 64, KV_WIDTH), g, device) for _ in range(L)]
    scales = f32_uniform((L,), 0.5, 2.0, g, device)
    slots = randperm(512 * 64, g, device)[:T].clone()
    slots[T - 1] = -1
    return dict(
        # token-major storage, exposed as [L, T, D] views (layer stride D)
        kv_c=kv_c_tm.permute(1, 0, 2), k_pe=k_pe_tm.permute(1, 0, 2),
        caches=caches, scales=scales,
        slot_mapping=slots.reshape(1, T).expand(L, T),  # shared: layer stride 0
        num_layers=L, num_tokens=T, block_size=64)


def grouped_test_shape(device="cpu", seed=42, shared=False, fp8=True):
    """The grouped-insert unit-test shape: 5 layers, 42 tokens, block 16, 8 blocks."""
    g = gen(seed, device)
    L, T, bs, nb = NUM_LAYERS, 42, 16, 8
    kv_c = bf16_normal((L, T, KV_LORA_RANK), g, device)
    k_pe = bf16_normal((L, T, PE_DIM), g, device)
    if fp8:
        caches = [random_bytes((nb, bs, KV_WIDTH), g, device) for _ in range(L)]
    else:
        caches = [random_bf16_bits((nb, bs, KV_WIDTH), g, device) for _ in range(L)]
    scales = torch.linspace(0.05, 0.25, L, dtype=torch.float32, device=device)
    slots = torch.stack([randperm(nb * bs, g, device)[:T] for _ in range(L)])
    slots[:, -1] = -1
    if shared:
        slots = slots[:1].expand(L, T)
    return dict(kv_c=kv_c, k_pe=k_pe, caches=caches,
                scales=scales if fp8 else None, slot_mapping=slots,
                num_layers=L, num_tokens=T, block_size=bs)


def context_epilogue(device="cpu", seed=3, num_tokens=4096, hidden=7168,
                     num_blocks=512, with_gemm=True, fp8=True, num_layers=NUM_LAYERS):
    g = gen(seed, device)
    L, T = num_layers, num_tokens
    N = L * KV_WIDTH
    d = {}
    if with_gemm:
        d["x"] = bf16_normal((T, hidden), g, device)
        d["w_kn"] = bf16_normal((hidden, N), g, device, std=0.02)
    d["gamma"] = bf16_uniform((L, KV_LORA_RANK), 0.8, 1.2, g, device)
    d["positions"] = torch.arange(T, dtype=torch.int64, device=device)
    d["scales"] = f32_uniform((L,), 0.5, 2.0, g, device)
    fill = random_bytes if fp8 else random_bf16_bits
    d["caches"] = [fill((num_blocks, 64, KV_WIDTH), g, device) for _ in range(L)]
    d["slot_mapping"] = torch.stack(
        [randperm(num_blocks * 64, g, device)[:T] for _ in range(L)])
    # Stand-in for the projection output when the epilogue is checked on its
    # own: a [T, L, 576] bf16 array with the spread of the projection output
    # (std ~ 0.02 * sqrt(hidden)).
    d["all_kv"] = bf16_normal((T, L, KV_WIDTH), g, device, std=0.02 * hidden ** 0.5)
    d.update(num_layers=L, num_tokens=T, block_size=64, eps=1e-6, rope_base=10000.0)
    return d


def context_cache(device="cpu", seed=4, num_blocks=512, num_ctx=8192, block_size=64):
    """An fp8 paged latent cache holding one sequence's context, plus its slot list."""
    g = gen(seed, device)
    cache = finite_e4m3_codes((num_blocks, block_size, KV_WIDTH), g, device)
    blocks = randperm(num_blocks, g, device)[: (num_ctx + block_size - 1) // block_size]
    src_slots = block_table_slots(blocks, block_size, num_ctx)
    return dict(cache=cache, cache_scale=0.5, src_slots=src_slots, g=g,
                block_size=block_size)


def kv_b_proj_output(num_tokens, g, device="cpu", heads=64, nope=128, vdim=128):
    """kv_b_proj output [T, H, nope + vdim]; k_nope and v are its strided halves."""
    return bf16_normal((num_tokens, heads, nope + vdim), g, device)


def context_pack(device="cpu", seed=4, num_ctx=8192, heads=64):
    d = context_cache(device, seed, num_blocks=512, num_ctx=num_ctx)
    g = d.pop("g")
    d["kvb"] = kv_b_proj_output(num_ctx, g, device, heads=heads)
    # A gather workspace stand-in for checking the pack on its own.
    d["workspace"] = bf16_normal((num_ctx, KV_WIDTH), g, device)
    d.update(num_tokens=num_ctx, num_heads=heads, nope=128, rope=PE_DIM, vdim=128)
    return d


def new_tokens(device="cpu", seed=8, num_tokens=8192, heads=64, num_blocks=512, requests=8,
               fp8_cache=True):
    """Inputs of the new-token epilogue for one layer: the query projection
    output q [T, H, 192] (q_nope | q_pe), the kv_b_proj output [T, H, 256]
    (k_nope | v), the normed latent and un-rotated k_pe [T, 576], positions of
    `requests` prefills of T / requests tokens each that continue a context
    of U[0, 4096) tokens, a seeded cache of num_blocks x 64 entries, distinct
    slots with one padded token (-1), and scales U(0.5, 2)."""
    g = gen(seed, device)
    T, H = num_tokens, heads
    q = bf16_normal((T, H, 192), g, device)
    kvb = kv_b_proj_output(T, g, device, heads=H)
    kv = bf16_normal((T, KV_WIDTH), g, device)
    per = max(1, T // requests)
    starts = torch.randint(0, 4096, (requests,), generator=g, device=device)
    idx = torch.arange(T, device=device)
    req = torch.clamp(idx // per, max=requests - 1)
    positions = starts[req] + (idx - req * per)
    if fp8_cache:
        cache = random_bytes((num_blocks, 64, KV_WIDTH), g, device)
    else:
        cache = random_bf16_bits((num_blocks, 64, KV_WIDTH), g, device)
    slots = randperm(num_blocks * 64, g, device)[:T].clone()
    if T > 5:
        slots[5] = -1
    sc = f32_uniform((4,), 0.5, 2.0, g, device)
    return dict(q=q, kvb=kvb, kv=kv, positions=positions.to(torch.int64), cache=cache,
                slots=slots, q_scale=sc[0:1], k_scale=sc[1:2], v_scale=sc[2:3],
                cache_scale=sc[3:4], num_tokens=T, num_heads=H, max_pos=8192 + T,
                block_size=64)


def attention_partials(device="cpu", seed=7, num_tokens=16384, heads=64, head_dim=128,
                       chunks=16, empty_frac=0.0):
    """Per-chunk attention partials of the chunked-context loop: outputs
    [chunks][T, H, D] ~ N(0, 1) in bf16 and natural-log lse [chunks][H, T]
    ~ N(8, 3^2) in fp32; a fraction empty_frac of the lse entries is -inf
    (chunks that hold no key for that query)."""
    g = gen(seed, device)
    outs = [bf16_normal((num_tokens, heads, head_dim), g, device) for _ in range(chunks)]
    lses = []
    for _ in range(chunks):
        l = 8.0 + 3.0 * torch.randn((heads, num_tokens), generator=g, device=device)
        if empty_frac > 0:
            u = torch.rand((heads, num_tokens), generator=g, device=device)
            l = torch.where(u < empty_frac, torch.full_like(l, float("-inf")), l)
        lses.append(l)
    return dict(outs=outs, lses=lses, num_tokens=num_tokens, heads=heads, head_dim=head_dim)


def long_context_insert(device="cpu", seed=5, num_tokens=16384, num_blocks=4096):
    g = gen(seed, device)
    L, T = NUM_LAYERS, num_tokens
    return dict(
        kv_c=bf16_normal((L, T, KV_LORA_RANK), g, device),
        k_pe=bf16_normal((L, T, PE_DIM), g, device),
        caches=[random_bytes((num_blocks, 64, KV_WIDTH), g, device) for _ in range(L)],
        scales=f32_uniform((L,), 0.5, 2.0, g, device),
        slot_mapping=torch.stack(
            [randperm(num_blocks * 64, g, device)[:T] for _ in range(L)]),
        num_layers=L, num_tokens=T, block_size=64)


def long_context_pack(device="cpu", seed=55, num_ctx=131072, chunk=8192,
                      num_blocks=4096, heads=64, num_chunks=None):
    """Cache with 131072 context tokens plus one kv_b_proj output per chunk."""
    d = context_cache(device, seed, num_blocks=num_blocks, num_ctx=num_ctx)
    g = d.pop("g")
    n = num_ctx // chunk if num_chunks is None else num_chunks
    d["kvb_chunks"] = [kv_b_proj_output(chunk, g, device, heads=heads) for _ in range(n)]
    d.update(num_tokens=num_ctx, chunk=chunk, num_heads=heads, nope=128,
             rope=PE_DIM, vdim=128)
    return d
