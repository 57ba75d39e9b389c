"""masked_attn_fwd on the GPU against the CPU oracle, and the two forms against each other."""
import numpy as np
import pytest
import torch

import top_sparse_attention_attn_amd as sa
from top_sparse_attention_attn_amd import workloads as wl
from gpu_util import assert_close, bits, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _small(seed=31):
    inp = wl.masked_inputs("masked_small", seed, DEV)
    cfg = inp["config"]
    mask = sa.topk_bitmask_build(inp["topk_idxs"], cfg.KV)
    return inp, cfg, mask


def _ref(orc, inp, mask, rows=None):
    m = None if mask is None else mask.cpu().numpy().view(np.uint32)
    return orc.masked_attn(bits(inp["q"]), bits(inp["k"]), bits(inp["v"]), m, inp["scale"], rows)


@pytest.mark.parametrize("bits_", [128, 32])
def test_small_topk_mask(oracle_impl, bits_):
    inp, cfg, mask = _small()
    out = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"], mask_load_bits=bits_)
    torch.cuda.synchronize()
    ref = _ref(oracle_impl, inp, mask).reshape(cfg.B, cfg.Q, cfg.H, cfg.Dv)
    assert_close(to64(out), ref, f"masked small {bits_}")


def test_small_dense_and_null_mask(oracle_impl):
    inp, cfg, _ = _small(32)
    B, pq, W = sa.topk_bitmask_shape(cfg.B, cfg.Q, cfg.KV)
    ones = torch.full((B, pq, W), -1, dtype=torch.int32, device=DEV)
    a = sa.masked_attn(inp["q"], inp["k"], inp["v"], ones, inp["scale"])
    b = sa.masked_attn(inp["q"], inp["k"], inp["v"], None, inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = _ref(oracle_impl, inp, None).reshape(cfg.B, cfg.Q, cfg.H, cfg.Dv)
    assert_close(to64(b), ref, "dense")


def test_load_widths_bitwise_identical():
    inp, cfg, mask = _small(33)
    a = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"], mask_load_bits=128)
    b = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"], mask_load_bits=32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_empty_and_single_key_rows():
    inp, cfg, mask = _small(34)
    mask = mask.clone()
    mask[0, 3].zero_()
    mask[1, 4].zero_()
    mask[1, 4, 2] = 1 << 5  # key 69 only
    out = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0, 3]).item() == 0
    assert torch.equal(out[1, 4], inp["v"][1, 69])


def test_two_forms_agree(oracle_impl):
    """Distinct top-k lists -> bitmask -> masked attention with one head and k = v = kv equals
    sparse attention with sink -inf over the same lists (D padded to the masked kernel's
    192/128 shape by zero columns, which change neither logits nor the first 128 outputs)."""
    g = torch.Generator().manual_seed(41)
    B, Q, KV, topk = 2, 70, 400, 50
    kv = torch.randn(B, KV, 128, generator=g).to(torch.bfloat16)
    q = torch.randn(B, Q, 1, 128, generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(KV, generator=g)[:topk] for _ in range(B * Q)]).view(B, Q, topk).to(torch.int32)
    mask = sa.topk_bitmask_build(idx.to(DEV), KV)
    kq = torch.zeros(B, KV, 1, 192, dtype=torch.bfloat16)
    kq[..., :128] = kv.unsqueeze(2)
    qq = torch.zeros(B, Q, 1, 192, dtype=torch.bfloat16)
    qq[..., :128] = q
    scale = 128 ** -0.5
    a = sa.masked_attn(qq.to(DEV), kq.to(DEV), kv.unsqueeze(2).contiguous().to(DEV), mask, scale)
    torch.cuda.synchronize()
    ref = oracle_impl.sparse_attn(bits(q), bits(kv), np.array([-np.inf], dtype=np.float32), idx.numpy(), scale)
    assert_close(to64(a).reshape(ref.shape), ref, "two forms")


def test_masked_config_sampled(oracle_impl):
    inp = wl.masked_inputs("masked", 1004, DEV)
    cfg = inp["config"]
    mask = sa.topk_bitmask_build(inp["topk_idxs"], cfg.KV)
    out = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"])
    out32 = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"], mask_load_bits=32)
    torch.cuda.synchronize()
    assert torch.equal(out, out32)
    rows = np.array([0, 1, 127, 128, 1000, 2047, 2048, 2049, 3000, 4095])
    ref = _ref(oracle_impl, inp, mask, rows)
    got = to64(out.reshape(cfg.B * cfg.Q, cfg.H, cfg.Dv)[torch.as_tensor(rows, device=DEV)])
    assert_close(got, ref, "masked config")
