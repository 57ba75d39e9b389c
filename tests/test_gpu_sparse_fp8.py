"""sparse_attn_fp8_fwd on the GPU: FP8 rows in the MODEL1 layout ("DeepSeek V4 源码剖析"
ch. 5, section 5.7) against the oracle over the exactly dequantized rows, and bitwise
against the bf16 kernel run on those dequantized rows."""
import numpy as np
import pytest
import torch

import top_sparse_attention_attn_amd as sa
from top_sparse_attention_attn_amd import workloads as wl
from gpu_util import assert_close, bits, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, S, H, T, K, seed, holes=0.05):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, H, 512, generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g)
    idx = torch.stack([torch.randperm(T, generator=g)[:K] for _ in range(B * S)]).view(B, S, K).to(torch.int32)
    idx[torch.rand(B, S, K, generator=g) < holes] = -1
    kv8 = wl.fp8_kv_rows(B, T, seed)
    return q, kv8, sink, idx


def _run(q, kv8, sink, idx, scale, **kw):
    out = sa.sparse_attn_fp8(q.to(DEV), kv8.to(DEV), sink.to(DEV), idx.to(DEV), scale, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("H", [16, 32, 64, 128])
def test_fp8_vs_oracle(oracle_impl, H):
    """Every head-block size, ragged slot count (K = 75: a partial last tile), empty slots."""
    B, S, T, K = 2, 3, 300, 75
    q, kv8, sink, idx = _case(B, S, H, T, K, seed=H)
    out = _run(q, kv8, sink, idx, 512 ** -0.5)
    ref = oracle_impl.sparse_attn_fp8(bits(q), kv8.numpy(), sink.numpy(), idx.numpy(), 512 ** -0.5)
    assert_close(to64(out).reshape(ref.shape), ref, f"fp8 H={H}")


@pytest.mark.parametrize("num_splits", [1, 2, 4])
def test_fp8_equals_bf16_kernel_on_dequantized_rows(oracle_impl, num_splits):
    """The FP8 path expands rows to bf16 before the unchanged score/softmax/PV code, so on the
    same (exactly representable) rows it must give the bf16 kernel's output bit for bit."""
    B, S, H, T, K = 4, 1, 128, 2000, 1152
    q, kv8, sink, idx = _case(B, S, H, T, K, seed=7)
    deq = torch.from_numpy(oracle_impl.fp8_dequant(kv8.numpy())).to(torch.bfloat16)
    a = _run(q, kv8, sink, idx, 512 ** -0.5, num_splits=num_splits)
    b = sa.sparse_attn(q.to(DEV), deq.to(DEV), sink.to(DEV), idx.to(DEV), 512 ** -0.5, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("H,num_splits", [(96, 0), (96, 2), (64, 3)])
def test_fp8_head_groups_with_padded_blocks(oracle_impl, H, num_splits):
    """Two head groups (96 heads: 48 per group in a padded 64-head block; 64: 32 per group): bit
    for bit the bf16 kernel's output on the dequantised rows, and within tolerance of the oracle."""
    B, S, T, K = 4, 1, 700, 500
    assert sa.sparse_attn_head_groups(B, S, H, 512, K, fp8=True) == 2
    q, kv8, sink, idx = _case(B, S, H, T, K, seed=17 + H)
    deq = torch.from_numpy(oracle_impl.fp8_dequant(kv8.numpy())).to(torch.bfloat16)
    a = _run(q, kv8, sink, idx, 512 ** -0.5, num_splits=num_splits)
    b = sa.sparse_attn(q.to(DEV), deq.to(DEV), sink.to(DEV), idx.to(DEV), 512 ** -0.5, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle_impl.sparse_attn_fp8(bits(q), kv8.numpy(), sink.numpy(), idx.numpy(), 512 ** -0.5)
    assert_close(to64(a).reshape(ref.shape), ref, f"fp8 H={H} splits={num_splits}")


def test_fp8_single_row_is_the_dequantized_row(oracle_impl):
    """One valid slot and sink -inf: each head's output is that row, dequantized (exactly, for
    these scale bytes) and rounded to bf16."""
    B, S, H, T, K = 2, 2, 32, 50, 40
    q, kv8, _, idx = _case(B, S, H, T, K, seed=9, holes=0.0)
    idx.fill_(-1)
    idx[:, :, 17] = torch.tensor([[3, 44], [0, 49]], dtype=torch.int32)
    sink = torch.full((H,), -float("inf"))
    out = _run(q, kv8, sink, idx, 512 ** -0.5)
    deq = oracle_impl.fp8_dequant(kv8.numpy())
    for b in range(B):
        for s in range(S):
            row = torch.from_numpy(deq[b, int(idx[b, s, 17])]).to(torch.bfloat16).to(DEV)
            assert torch.equal(out[b, s], row.expand(H, 512)), (b, s)


def test_fp8_all_slots_empty_is_zero():
    B, S, H, T, K = 1, 2, 16, 80, 64
    q, kv8, sink, idx = _case(B, S, H, T, K, seed=10, holes=0.0)
    idx.fill_(-1)
    out = _run(q, kv8, torch.full((H,), 0.5), idx, 512 ** -0.5)
    assert torch.count_nonzero(out).item() == 0


def test_fp8_decode_config_sampled(oracle_impl):
    """The decode shape (B=64, H=128, T=8320, K=1152, the library's default splits): sampled
    tokens against the oracle."""
    cfg = wl.SPARSE_CONFIGS["decode"]
    inp = wl.sparse_inputs(cfg, 2101, DEV)
    kv8 = wl.fp8_kv_rows(cfg.B, cfg.T, 2102, DEV)
    out = sa.sparse_attn_fp8(inp["q"], kv8, inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    torch.cuda.synchronize()
    toks = np.array([0, 1, 31, 63])
    q_s = inp["q"][toks].cpu()
    idx_s = inp["topk_idxs"][toks].cpu()
    ref = oracle_impl.sparse_attn_fp8(bits(q_s), kv8[toks].cpu().numpy(), inp["attn_sink"].cpu().numpy(),
                                      idx_s.numpy(), inp["scale"])
    assert_close(to64(out[toks]).reshape(ref.shape), ref, "fp8 decode")


@pytest.mark.parametrize("splits", [1, 2, 4])
def test_fp8_split_then_merge_equals_one_call(splits):
    """sparse_attn_fp8_split_fwd then sparse_attn_fp8_merge_fwd give exactly the one-call result."""
    B, S, H, T, K = 16, 1, 128, 600, 512
    q, kv8, sink, idx = _case(B, S, H, T, K, seed=61)
    q, kv8, sink, idx = q.to(DEV), kv8.to(DEV), sink.to(DEV), idx.to(DEV)
    ws = sa.new_workspace(sa.sparse_attn_workspace_bytes(B, S, H, 512, K, splits), DEV)
    a = sa.sparse_attn_fp8(q, kv8, sink, idx, 512 ** -0.5, num_splits=splits, workspace=ws)
    b = torch.full_like(a, 7.0)
    sa.sparse_attn_fp8_split(q, kv8, sink, idx, 512 ** -0.5, out=b, num_splits=splits, workspace=ws)
    sa.sparse_attn_fp8_merge(q, kv8, sink, idx, 512 ** -0.5, out=b, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("num_splits", [1, 4])
def test_fp8_padded_head_blocks(oracle_impl, num_splits):
    """H = 100 (eight head blocks, heads 100 .. 127 padded) over FP8 rows, one token per batch."""
    B, S, H, T, K = 3, 1, 100, 300, 200
    q, kv8, sink, idx = _case(B, S, H, T, K, seed=71)
    out = _run(q, kv8, sink, idx, 512 ** -0.5, num_splits=num_splits)
    ref = oracle_impl.sparse_attn_fp8(bits(q), kv8.numpy(), sink.numpy(), idx.numpy(), 512 ** -0.5)
    assert_close(to64(out).reshape(ref.shape), ref, f"fp8 H=100 splits={num_splits}")


@pytest.mark.parametrize("seed", range(4))
def test_fp8_random_shapes_equal_bf16_on_dequantized_rows(oracle_impl, seed):
    """Randomised batch, token, head, row and slot counts and split choices: the FP8 call is bitwise
    the bf16 call on the oracle's dequantized rows (6 cases per seed)."""
    rng = np.random.default_rng(3000 + seed)
    for _ in range(6):
        B, S, H = int(rng.integers(1, 4)), int(rng.integers(1, 3)), int(rng.choice([1, 16, 40, 100, 128]))
        T, K = int(rng.integers(1, 600)), int(rng.integers(0, 400))
        splits = int(rng.choice([0, 1, 3, 8]))
        q, kv8, sink, idx = _case(B, S, H, max(T, 1), 0, seed=int(rng.integers(1 << 30)))
        g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
        idx = torch.randint(-1, T, (B, S, K), generator=g, dtype=torch.int32)
        deq = torch.from_numpy(oracle_impl.fp8_dequant(kv8.numpy())).to(torch.bfloat16)
        a = _run(q, kv8, sink, idx, 512 ** -0.5, num_splits=splits)
        b = sa.sparse_attn(q.to(DEV), deq.to(DEV), sink.to(DEV), idx.to(DEV), 512 ** -0.5, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(a, b), (B, S, H, T, K, splits)
