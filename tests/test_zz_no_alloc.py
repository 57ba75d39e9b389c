"""The allocation-free entry point (sparse_attn_fwd_noalloc) against sparse_attn_fwd, through the
C ABI: the same kernels on the same inputs, so the outputs must be bitwise equal. Two calls in a
row on the library's shared scratch array, the second smaller than the first (its partials
overwrite only part of what the first left), then the first shape again."""
import pytest
import torch

import top_sparse_attention_attn_amd as sa
from top_sparse_attention_attn_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _custom(B, S, H, D, T, K, seed, holes=0.1):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, T, D, generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g)
    idx = torch.stack([torch.randperm(T, generator=g)[:K] for _ in range(B * S)]).view(B, S, K).to(torch.int32)
    idx[torch.rand(B, S, K, generator=g) < holes] = -1
    return {"q": q.to(DEV), "kv": kv.to(DEV), "attn_sink": sink.to(DEV), "topk_idxs": idx.to(DEV), "scale": D ** -0.5}


def _both(inp, splits=0):
    args = (inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    a = sa.sparse_attn(*args, num_splits=splits)
    b = torch.full_like(a, 5.0)
    sa.sparse_attn_noalloc(*args, out=b, num_splits=splits)
    torch.cuda.synchronize()
    return a, b


def test_noalloc_equals_workspace_entry():
    big = wl.sparse_inputs("decode", 1004, DEV)        # 64 tokens x 4 splits: 33 MB of partials
    small = _custom(3, 2, 128, 512, 700, 400, seed=77)  # 6 tokens, library's split choice
    for inp in (big, small, big):
        a, b = _both(inp)
        assert torch.equal(a, b)
    # forced split counts, including a 64-head and a D = 64 shape
    for inp, splits in ((_custom(5, 1, 64, 512, 300, 250, seed=78), 3), (_custom(4, 2, 40, 64, 300, 200, seed=79), 5)):
        a, b = _both(inp, splits)
        assert torch.equal(a, b)
