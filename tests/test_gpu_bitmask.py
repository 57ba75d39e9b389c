"""topk_bitmask_build on the GPU: bit-exact against the CPU oracle, whole buffer."""
import json
import os

import numpy as np
import pytest
import torch

import top_sparse_attention_attn_amd as sa
from top_sparse_attention_attn_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "bitmask_worked_example.json")


def _u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def test_worked_example():
    with open(GOLDEN) as f:
        ex = json.load(f)["build"]
    idx = torch.tensor(ex["topk_idxs"], dtype=torch.int32, device=DEV)
    mask = sa.topk_bitmask_build(idx, ex["key_len"], q_lens=torch.tensor(ex["q_lens"], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    m = _u32(mask)
    assert m.shape == (1, 128, 8)
    assert m[0, 0].tolist() == ex["row0_expect"]
    assert not m[0, 1:].any()


@pytest.mark.parametrize("hole_prob", [0.0, 0.05])
def test_config_masks_bit_exact(oracle_impl, hole_prob):
    cfg = wl.MASKED_CONFIGS["masked"]
    idx = wl.topk_lists(cfg.B, cfg.Q, cfg.topk, cfg.KV, seed=1004, hole_prob=hole_prob)
    got = sa.topk_bitmask_build(idx.to(DEV), cfg.KV)
    torch.cuda.synchronize()
    ref = oracle_impl.topk_mask_build(idx.numpy(), cfg.KV)
    assert got.shape == ref.shape == (2, 2048, 256)
    assert np.array_equal(_u32(got), ref)


def test_messy_indices_q_lens_and_key_starts(oracle_impl):
    g = np.random.default_rng(5)
    B, Q, topk, key_len = 3, 150, 77, 1000
    idx = g.integers(-3, key_len + 50, size=(B, Q, topk)).astype(np.int32)
    idx[:, :, 5] = idx[:, :, 6]
    q_lens = np.array([150, 17, 0], dtype=np.int32)
    ks = np.array([12345, -7, 99], dtype=np.int32)
    got = sa.topk_bitmask_build(torch.from_numpy(idx).to(DEV), key_len, q_lens=torch.from_numpy(q_lens).to(DEV),
                                key_starts=torch.from_numpy(ks).to(DEV))
    torch.cuda.synchronize()
    ref = oracle_impl.topk_mask_build(idx, key_len, q_lens=q_lens, key_starts=ks)
    assert got.shape == ref.shape
    assert np.array_equal(_u32(got), ref)


def test_single_equals_batched():
    idx = torch.randint(-1, 500, (2, 40, 30), dtype=torch.int32, device=DEV)
    full = sa.topk_bitmask_build(idx, 500)
    one = sa.topk_bitmask_build(idx[1:2].contiguous(), 500)
    torch.cuda.synchronize()
    assert torch.equal(full[1:2], one)


def test_index_list_4byte_aligned(oracle_impl):
    """topk a multiple of 4 but the index list only 4-byte aligned (a view one int32 into a
    buffer): the mask builder reads it with 4-byte loads and gives the same bits as an aligned copy."""
    B, Q, topk, key_len = 2, 100, 64, 3000
    g = torch.Generator().manual_seed(77)
    src = torch.randint(-1, key_len + 5, (B, Q, topk), generator=g, dtype=torch.int32)
    buf = torch.zeros(B * Q * topk + 4, dtype=torch.int32, device=DEV)
    view = buf[1:1 + B * Q * topk].view(B, Q, topk)
    view.copy_(src.to(DEV))
    assert view.data_ptr() % 16 == 4
    got = sa.topk_bitmask_build(view, key_len)
    aligned = sa.topk_bitmask_build(src.to(DEV).contiguous(), key_len)
    torch.cuda.synchronize()
    ref = oracle_impl.topk_mask_build(src.numpy(), key_len)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref)
    assert torch.equal(got, aligned)


def test_overwrites_garbage_and_stays_in_bounds():
    """The whole buffer is written (no pre-zeroing needed) and nothing outside it."""
    idx = torch.randint(0, 300, (2, 9, 20), dtype=torch.int32, device=DEV)
    B, pq, W = sa.topk_bitmask_shape(2, 9, 300)
    n = B * pq * W
    buf = torch.full((n + 2048,), -1, dtype=torch.int32, device=DEV)
    out = buf[1024:1024 + n].view(B, pq, W)
    sa.topk_bitmask_build(idx, 300, out=out)
    clean = sa.topk_bitmask_build(idx, 300)
    torch.cuda.synchronize()
    assert torch.equal(out, clean)
    assert (buf[:1024] == -1).all() and (buf[1024 + n:] == -1).all()


def test_empty_batch_is_noop():
    idx = torch.zeros((0, 5, 4), dtype=torch.int32, device=DEV)
    m = sa.topk_bitmask_build(idx, 100)
    assert m.shape == (0, 128, 4)
