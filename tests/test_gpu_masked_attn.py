"""masked_attn_fwd / masked_attn_offset_fwd on the GPU against the CPU oracle, and the forms
against each other. Masks that the oracle also reads are built by the oracle."""
import numpy as np
import pytest
import torch

import top_sparse_attention_attn_amd as sa
from top_sparse_attention_attn_amd import workloads as wl
from gpu_util import assert_close, bits, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _small(seed=31, orc=None):
    inp = wl.masked_inputs("masked_small", seed, DEV)
    cfg = inp["config"]
    if orc is None:
        mask = sa.topk_bitmask_build(inp["topk_idxs"], cfg.KV)
    else:
        mask = _oracle_mask(orc, inp["topk_idxs"], cfg.KV)
    return inp, cfg, mask


def _oracle_mask(orc, idx, key_len, key_starts=None):
    ks = None if key_starts is None else np.asarray(key_starts, dtype=np.int32)
    m = orc.topk_mask_build(idx.cpu().numpy(), key_len, key_starts=ks)
    return torch.from_numpy(m.view(np.int32)).to(DEV)


def _ref(orc, inp, mask, rows=None):
    m = None if mask is None else mask.cpu().numpy().view(np.uint32)
    return orc.masked_attn(bits(inp["q"]), bits(inp["k"]), bits(inp["v"]), m, inp["scale"], rows)


@pytest.mark.parametrize("bits_", [128, 32])
def test_small_topk_mask(oracle_impl, bits_):
    inp, cfg, mask = _small(orc=oracle_impl)
    out = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"], mask_load_bits=bits_)
    torch.cuda.synchronize()
    ref = _ref(oracle_impl, inp, mask).reshape(cfg.B, cfg.Q, cfg.H, cfg.Dv)
    assert_close(to64(out), ref, f"masked small {bits_}")


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.6])
@pytest.mark.parametrize("offset", [False, True])
def test_scale_signs(oracle_impl, scale, offset):
    """A positive scale takes the kernel form that finds each query's maximum on the raw scores
    and scales it once; zero and negative scales take the form that scales every score first.
    Zero gives equal weights over the visible keys, a negative scale reverses the order of the
    scores, and 0.6 makes the weights peaked. Both forms against the oracle, plain and chunked
    (key start 0, where the chunked form reads the same bits)."""
    inp, cfg, _ = _small(35, orc=oracle_impl)
    inp = dict(inp, scale=scale)
    mask = _oracle_mask(oracle_impl, inp["topk_idxs"], cfg.KV, key_starts=[0] * cfg.B)
    if offset:
        out = sa.masked_attn_offset(inp["q"], inp["k"], inp["v"], mask, scale)
    else:
        out = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, scale)
    torch.cuda.synchronize()
    ref = _ref(oracle_impl, inp, mask).reshape(cfg.B, cfg.Q, cfg.H, cfg.Dv)
    assert_close(to64(out), ref, f"masked scale {scale} offset {offset}")


def test_small_dense_and_null_mask(oracle_impl):
    inp, cfg, _ = _small(32, orc=oracle_impl)
    B, pq, W = sa.topk_bitmask_shape(cfg.B, cfg.Q, cfg.KV)
    ones = torch.full((B, pq, W), -1, dtype=torch.int32, device=DEV)
    a = sa.masked_attn(inp["q"], inp["k"], inp["v"], ones, inp["scale"])
    b = sa.masked_attn(inp["q"], inp["k"], inp["v"], None, inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = _ref(oracle_impl, inp, None).reshape(cfg.B, cfg.Q, cfg.H, cfg.Dv)
    assert_close(to64(b), ref, "dense")


@pytest.mark.parametrize("masked", [False, True])
def test_late_maximum_jump(oracle_impl, masked):
    """Each query's key row equals that query in a late key tile (past the first 64 keys, in
    either key half), so its logit maximum jumps after the first tiles and the accumulators of
    that key half must be rescaled; with N(0,1) data the maximum never moves that far."""
    inp, cfg, mask = _small(33, orc=oracle_impl)
    q, k = inp["q"].clone(), inp["k"].clone()
    for b in range(cfg.B):
        for i in range(cfg.Q):
            key = 64 + (i * 37 + b * 11) % (cfg.KV - 64)
            for h in range(cfg.H):
                k[b, key, h] = q[b, i, h]
    inp = dict(inp, q=q, k=k)
    if not masked:
        mask = None
    else:  # the jump key is visible in every row
        m = mask.clone().view(torch.int32)
        for b in range(cfg.B):
            for i in range(cfg.Q):
                key = 64 + (i * 37 + b * 11) % (cfg.KV - 64)
                w = m[b, i, key // 32].item() & 0xFFFFFFFF
                w |= 1 << (key % 32)
                m[b, i, key // 32] = w - (1 << 32) if w >= (1 << 31) else w
        mask = m
    out = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"])
    torch.cuda.synchronize()
    ref = _ref(oracle_impl, inp, mask).reshape(cfg.B, cfg.Q, cfg.H, cfg.Dv)
    assert_close(to64(out), ref, f"late jump masked={masked}")


@pytest.mark.parametrize("masked", [False, True])
def test_rising_maximum_every_tile(oracle_impl, masked):
    """Keys whose logit with every query rises by ~10 (log2 units) from one 64-key tile to the next,
    so each key half's reference maximum moves and its accumulators are rescaled at every tile."""
    inp, cfg, mask = _small(34, orc=oracle_impl)
    g = torch.Generator().manual_seed(34)
    D = cfg.Dqk
    u = torch.randn(D, generator=g)
    u = u / u.norm()
    q = (torch.randn(cfg.B, cfg.Q, cfg.H, D, generator=g) * 0.05 + 4.0 * u).to(torch.bfloat16)
    step = 10.0 / 1.4426950408889634 * D ** 0.5 / 4.0
    tiles = (torch.arange(cfg.KV) // 64).to(torch.float32)
    k = (torch.randn(cfg.B, cfg.KV, cfg.H, D, generator=g) * 0.05 + tiles[None, :, None, None] * step * u).to(torch.bfloat16)
    inp = dict(inp, q=q.to(DEV), k=k.to(DEV))
    out = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask if masked else None, inp["scale"])
    torch.cuda.synchronize()
    ref = _ref(oracle_impl, inp, mask if masked else None).reshape(cfg.B, cfg.Q, cfg.H, cfg.Dv)
    assert_close(to64(out), ref, f"rising maximum masked={masked}")


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
    mask = _oracle_mask(oracle_impl, inp["topk_idxs"], cfg.KV)
    out = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"])
    out32 = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"], mask_load_bits=32)
    torch.cuda.synchronize()
    assert torch.equal(out, out32)
    rows = np.array([0, 1, 127, 128, 1000, 2047, 2048, 2049, 3000, 4095])
    ref = _ref(oracle_impl, inp, mask, rows)
    got = to64(out.reshape(cfg.B * cfg.Q, cfg.H, cfg.Dv)[torch.as_tensor(rows, device=DEV)])
    assert_close(got, ref, "masked config")


def test_masked_config_no_mask_and_all_ones(oracle_impl):
    """The masked config's shape (B=2, Q=2048, KV=8192, H=8) with no mask and with an all-ones
    mask (the benchmark's mask-overhead forms): bitwise equal to each other (both 16- and 4-byte
    mask loads), and sampled rows of every 128-query tile against the oracle's dense attention."""
    inp = wl.masked_inputs("masked", 1006, DEV)
    cfg = inp["config"]
    mask = sa.topk_bitmask_build(inp["topk_idxs"], cfg.KV)
    ones = torch.full_like(mask, -1)
    none = sa.masked_attn(inp["q"], inp["k"], inp["v"], None, inp["scale"])
    all1 = sa.masked_attn(inp["q"], inp["k"], inp["v"], ones, inp["scale"])
    all1_32 = sa.masked_attn(inp["q"], inp["k"], inp["v"], ones, inp["scale"], mask_load_bits=32)
    torch.cuda.synchronize()
    assert torch.equal(none, all1) and torch.equal(all1, all1_32)
    rows = np.concatenate([np.arange(b * cfg.Q + 37, (b + 1) * cfg.Q, 128) for b in range(cfg.B)] + [[0, cfg.Q - 1]])
    ref = _ref(oracle_impl, inp, None, rows)
    got = to64(none.reshape(cfg.B * cfg.Q, cfg.H, cfg.Dv)[torch.as_tensor(rows, device=DEV)])
    assert_close(got, ref, "masked config, no mask")


# --------------------------------------------------------------------------- chunked-context (offset) form
def _chunk(inp, start, n, seed):
    """k, v of a chunk of n keys (fresh values: the chunk is any slice of a longer context)."""
    g = torch.Generator().manual_seed(seed)
    B, _, H, Dqk = inp["q"].shape
    Dv = inp["v"].shape[3]
    k = torch.randn(B, n, H, Dqk, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(B, n, H, Dv, generator=g).to(torch.bfloat16).to(DEV)
    return k, v


def _offset_ref(orc, inp, k, v, mask, rows=None):
    return orc.masked_attn_offset(bits(inp["q"]), bits(k), bits(v), mask.cpu().numpy().view(np.uint32), inp["scale"],
                                  rows)


@pytest.mark.parametrize("starts,n", [((0, 37), 130), ((96, 170), 64), ((250, 3), 130), ((31, 33), 1)],
                         ids=["s0-37", "s96-170", "past-reserved", "one-key"])
def test_offset_small_vs_oracle(oracle_impl, starts, n):
    """Global context of 300 keys (12 words, the last reserved), chunk of n keys at per-batch
    starts; (250, .) runs past the reserved word's position (352) and must see nothing there."""
    inp, cfg, _ = _small(51)
    mask = _oracle_mask(oracle_impl, inp["topk_idxs"], cfg.KV, key_starts=starts)
    assert mask.shape[2] == 12
    k, v = _chunk(inp, 0, n, 52)
    out = sa.masked_attn_offset(inp["q"], k, v, mask, inp["scale"])
    torch.cuda.synchronize()
    ref = _offset_ref(oracle_impl, inp, k, v, mask).reshape(cfg.B, cfg.Q, cfg.H, cfg.Dv)
    assert_close(to64(out), ref, f"offset {starts} n={n}")


def test_offset_start_zero_equals_plain():
    """Start 0 over the whole context: the same visible keys as the plain form, so the same
    arithmetic and bitwise-identical outputs."""
    inp, cfg, _ = _small(53)
    B = cfg.B
    mask = sa.topk_bitmask_build(inp["topk_idxs"], cfg.KV,
                                 key_starts=torch.zeros(B, dtype=torch.int32, device=DEV))
    a = sa.masked_attn_offset(inp["q"], inp["k"], inp["v"], mask, inp["scale"])
    b = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("cut", [150, 64, 1])
def test_offset_chunks_merged_by_lse_equal_global(oracle_impl, cut):
    """The fallback from one global mask to per-chunk masks (prhub summary of vLLM PR #48770,
    review discussion): the context cut at `cut` into two chunks, each run through the chunked
    form with its key_start, merged by the returned log-sum-exps, equals the oracle on the
    global mask and the global form."""
    inp, cfg, _ = _small(56)
    B, KV = cfg.B, cfg.KV
    gmask = _oracle_mask(oracle_impl, inp["topk_idxs"], KV)
    glob = sa.masked_attn(inp["q"], inp["k"], inp["v"], gmask, inp["scale"])
    outs, lses = [], []
    for start, end in ((0, cut), (cut, KV)):
        starts = torch.full((B,), start, dtype=torch.int32, device=DEV)
        cmask = sa.topk_bitmask_build(inp["topk_idxs"], KV, key_starts=starts)
        k = inp["k"][:, start:end].contiguous()
        v = inp["v"][:, start:end].contiguous()
        o, lse = sa.masked_attn_offset(inp["q"], k, v, cmask, inp["scale"], return_lse=True)
        outs.append(o.double().cpu())
        lses.append(lse.double().cpu())
    torch.cuda.synchronize()
    lse = torch.stack(lses)                                    # [chunk, B, Q, H]
    w = torch.nan_to_num(torch.exp(lse - torch.logsumexp(lse, dim=0)), nan=0.0)  # no visible key: 0
    merged = (w[0][..., None] * outs[0] + w[1][..., None] * outs[1]).numpy()
    ref = _ref(oracle_impl, inp, gmask).reshape(cfg.B, cfg.Q, cfg.H, cfg.Dv)
    assert_close(merged, ref, f"chunks cut at {cut}, merged by lse")
    assert_close(merged, to64(glob), f"chunks cut at {cut} vs the global form")


def test_offset_lse_closed_forms():
    """lse of a query with exactly one visible key is that key's scaled logit (the weight sum
    is exactly 1); without any visible key it is -inf."""
    inp, cfg, _ = _small(57)
    B, n = cfg.B, 100
    k, v = _chunk(inp, 0, n, 58)
    idx = torch.full_like(inp["topk_idxs"], -1)
    idx[:, 0::2, 0] = 7  # even queries see key 7 only, odd queries nothing
    mask = sa.topk_bitmask_build(idx, n, key_starts=torch.zeros(B, dtype=torch.int32, device=DEV))
    o, lse = sa.masked_attn_offset(inp["q"], k, v, mask, inp["scale"], return_lse=True)
    torch.cuda.synchronize()
    want = (inp["q"].double() * k[:, 7].double()[:, None]).sum(-1) * inp["scale"]  # [B, Q, H]
    got = lse.double()
    assert torch.isneginf(got[:, 1::2]).all()
    assert torch.allclose(got[:, 0::2], want[:, 0::2], atol=1e-3, rtol=1e-4)
    assert torch.equal(o[:, 0::2], v[:, 7][:, None].expand_as(o[:, 0::2]))
    assert torch.count_nonzero(o[:, 1::2]).item() == 0


@pytest.mark.parametrize("start", [37, 64, 200])
def test_offset_equals_plain_on_shifted_mask(start):
    """A chunk [start, start + n) read through the global mask's offset equals the plain form
    over a mask built from the indices shifted by -start (bitwise: same keys, same arithmetic)."""
    inp, cfg, _ = _small(54)
    B, n = cfg.B, 90
    starts = torch.full((B,), start, dtype=torch.int32, device=DEV)
    gmask = sa.topk_bitmask_build(inp["topk_idxs"], cfg.KV, key_starts=starts)
    k, v = _chunk(inp, start, n, 55)
    a = sa.masked_attn_offset(inp["q"], k, v, gmask, inp["scale"])
    shifted = inp["topk_idxs"] - start  # keys outside [0, n) are dropped by the builder
    lmask = sa.topk_bitmask_build(shifted, n)
    b = sa.masked_attn(inp["q"], k, v, lmask, inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_offset_start_past_context_is_zero():
    inp, cfg, _ = _small(56)
    starts = torch.tensor([5000, 352], dtype=torch.int32, device=DEV)  # 352 = first reserved position
    mask = sa.topk_bitmask_build(inp["topk_idxs"], cfg.KV, key_starts=starts)
    k, v = _chunk(inp, 0, 100, 57)
    out = sa.masked_attn_offset(inp["q"], k, v, mask, inp["scale"])
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_offset_masked_config_sampled(oracle_impl):
    """The masked config's queries and mask (8192-key context) with a 4096-key chunk at starts
    1000 and 2500 (neither a multiple of 32); sampled rows against the oracle."""
    inp = wl.masked_inputs("masked", 1005, DEV)
    cfg = inp["config"]
    starts = (1000, 2500)
    mask = _oracle_mask(oracle_impl, inp["topk_idxs"], cfg.KV, key_starts=starts)
    k, v = _chunk(inp, 0, 4096, 58)
    out = sa.masked_attn_offset(inp["q"], k, v, mask, inp["scale"])
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 1000, 2047, 2048, 2049, 3000, 4095])
    ref = _offset_ref(oracle_impl, inp, k, v, mask, rows)
    got = to64(out.reshape(cfg.B * cfg.Q, cfg.H, cfg.Dv)[torch.as_tensor(rows, device=DEV)])
    assert_close(got, ref, "offset masked config")


# --------------------------------------------------------------------------- bounds and graph replay
@pytest.mark.parametrize("offset", [False, True])
def test_masked_write_bounds_guard_band(offset):
    """Q = 80 (a partial 128-query tile): guard bands around out keep their sentinel, for the
    plain and the chunked form."""
    inp, cfg, _ = _small(61)
    starts = torch.tensor([5, 40], dtype=torch.int32, device=DEV) if offset else None
    mask = sa.topk_bitmask_build(inp["topk_idxs"], cfg.KV, key_starts=starts)
    n = cfg.B * cfg.Q * cfg.H * cfg.Dv
    buf = torch.full((n + 2 * 4096,), 3.0, dtype=torch.bfloat16, device=DEV)
    out = buf[4096:4096 + n].view(cfg.B, cfg.Q, cfg.H, cfg.Dv)
    fn = sa.masked_attn_offset if offset else sa.masked_attn
    fn(inp["q"], inp["k"], inp["v"], mask, inp["scale"], out=out)
    torch.cuda.synchronize()
    assert (buf[:4096] == 3.0).all() and (buf[4096 + n:] == 3.0).all()
    assert not (out == 3.0).all(dim=-1).any(), "a row of out was not written"


def test_masked_graph_replay_tracks_new_masks(oracle_impl):
    """Capture one call, replay it with new queries and new mask bits: every replay matches
    the oracle (the launch depends only on the shapes)."""
    inp, cfg, _ = _small(62)
    mask = _oracle_mask(oracle_impl, inp["topk_idxs"], cfg.KV)
    out = torch.empty((cfg.B, cfg.Q, cfg.H, cfg.Dv), dtype=torch.bfloat16, device=DEV)
    sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"], out=out)  # warm up outside the graph
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, inp["scale"], out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        new = wl.masked_inputs("masked_small", 200 + rep, DEV)
        inp["q"].copy_(new["q"])
        mask.copy_(_oracle_mask(oracle_impl, new["topk_idxs"], cfg.KV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = _ref(oracle_impl, inp, mask).reshape(cfg.B, cfg.Q, cfg.H, cfg.Dv)
        assert_close(to64(out), ref, f"masked replay {rep}")


@pytest.mark.parametrize("seed", range(4))
def test_random_shapes_and_data(oracle_impl, seed):
    """Randomised shapes, masks (top-k lists of random length, or none) and data modes (N(0,1),
    keys equal to queries, a large common logit offset) against the oracle; 16- and 4-byte mask
    loads bitwise equal. Fixed seeds, 6 cases each."""
    rng = np.random.default_rng(2000 + seed)
    for _ in range(6):
        B, Q, KV, H = int(rng.integers(1, 3)), int(rng.integers(1, 300)), int(rng.integers(1, 400)), int(rng.integers(1, 5))
        mode = rng.choice(["normal", "aligned", "offset"])
        g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
        q = torch.randn(B, Q, H, 192, generator=g)
        k = torch.randn(B, KV, H, 192, generator=g)
        v = torch.randn(B, KV, H, 128, generator=g)
        if mode == "aligned":
            for b in range(B):
                for i in range(Q):
                    k[b, int(rng.integers(KV))] = q[b, i]
        if mode == "offset":
            u = torch.randn(192, generator=g)
            q, k = q + 3.0 * u / u.norm(), k + 3.0 * u / u.norm()
        topk = int(rng.integers(0, KV + 1))
        idx = torch.stack([torch.randperm(KV, generator=g)[:topk] for _ in range(B * Q)]).view(B, Q, topk).to(torch.int32)
        mask = None if rng.random() < 0.25 else _oracle_mask(oracle_impl, idx, KV)
        scale = float(rng.choice([192 ** -0.5, 0.02, 0.3]))
        inp = {"q": q.to(torch.bfloat16).to(DEV), "k": k.to(torch.bfloat16).to(DEV), "v": v.to(torch.bfloat16).to(DEV),
               "scale": scale}
        out = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, scale)
        if mask is not None:
            out32 = sa.masked_attn(inp["q"], inp["k"], inp["v"], mask, scale, mask_load_bits=32)
            torch.cuda.synchronize()
            assert torch.equal(out, out32)
        torch.cuda.synchronize()
        ref = _ref(oracle_impl, inp, mask).reshape(B, Q, H, 128)
        assert_close(to64(out), ref, f"B={B} Q={Q} KV={KV} H={H} topk={topk} mode={mode} mask={mask is not None}")
