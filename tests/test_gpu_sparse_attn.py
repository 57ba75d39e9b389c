"""sparse_attn on the GPU against the CPU oracle (through the C ABI)."""
import math

import numpy as np
import pytest
import torch

import top_sparse_attention_attn_amd as sa
from top_sparse_attention_attn_amd import workloads as wl
from gpu_util import assert_close, sparse_reference, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(inp, **kw):
    return sa.sparse_attn(inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"], **kw)


def _custom(B, S, H, D, T, K, seed, holes=0.1):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, T, D, generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g)
    idx = torch.stack([torch.randperm(T, generator=g)[:K] for _ in range(B * S)]).view(B, S, K).to(torch.int32)
    idx[torch.rand(B, S, K, generator=g) < holes] = -1
    return {"q": q.to(DEV), "kv": kv.to(DEV), "attn_sink": sink.to(DEV), "topk_idxs": idx.to(DEV), "scale": D ** -0.5}


def test_tiny_config(oracle_impl):
    inp = wl.sparse_inputs("tiny", 1001, DEV)
    out = _run(inp)
    torch.cuda.synchronize()
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, "tiny")


@pytest.mark.parametrize("D,H", [(64, 1), (64, 8), (64, 40), (512, 1), (512, 16), (512, 128)])
@pytest.mark.parametrize("splits", [1, 3])
def test_shapes_and_splits(oracle_impl, D, H, splits):
    # K = 200 spans several 32-row tiles and ends in a ragged tile; splits > 1 exercise the combine.
    inp = _custom(2, 3, H, D, 300, 200, seed=7 + D + H)
    out = _run(inp, num_splits=splits)
    torch.cuda.synchronize()
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, f"D={D} H={H} splits={splits}")


@pytest.mark.parametrize("S,splits,H,D", [(1, 1, 128, 512), (1, 4, 128, 512), (2, 1, 128, 512), (1, 4, 40, 512),
                                         (2, 1, 16, 512), (1, 1, 100, 64)])
def test_late_maximum_jump_every_head(oracle_impl, S, splits, H, D):
    """Each head's query equals one gathered row that sits in a late tile, so that head's logit
    maximum jumps by ~33 (log2 units) after its first tiles and the accumulators must be rescaled
    (the lazily moved reference maximum). Every head position of a head block and both head
    blocks of a score wave take the jump, at tiles that differ between heads, and the output is
    then dominated by that one row. With N(0,1) data the reference maximum never moves after the
    first tile, so this is the only path that exercises the rescale."""
    B, T, K = 2, 600, 256  # 8 tiles: 2 per split at 4 splits
    g = torch.Generator().manual_seed(123 + S + splits + H + D)
    kv = torch.randn(B, T, D, generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(T, generator=g)[:K] for _ in range(B * S)]).view(B, S, K).to(torch.int32)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16)
    for b in range(B):
        for s_ in range(S):
            for h in range(H):
                tile = 1 + 2 * ((h + s_) % 4)              # the second tile of one of the 4 ranges
                slot = tile * 32 + (h * 7 + b) % 32
                q[b, s_, h] = kv[b, int(idx[b, s_, slot])]
    sink = torch.randn(H, generator=g)
    inp = {"q": q.to(DEV), "kv": kv.to(DEV), "attn_sink": sink.to(DEV), "topk_idxs": idx.to(DEV), "scale": D ** -0.5}
    out = _run(inp, num_splits=splits)
    torch.cuda.synchronize()
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, f"late jump S={S} splits={splits} H={H} D={D}")


@pytest.mark.parametrize("S,splits", [(1, 1), (2, 1), (1, 2)])
def test_rising_maximum_every_tile(oracle_impl, S, splits):
    """Rows whose logit with every head rises by ~10 (log2 units) from one 32-row tile to the next,
    so the reference maximum moves and the accumulators are rescaled at every tile (weights of the
    earlier tiles fall by 2^-10 each time)."""
    B, H, D, T, K = 1, 128, 512, 400, 256
    g = torch.Generator().manual_seed(131 + S + splits)
    u = torch.randn(D, generator=g)
    u = u / u.norm()
    q = (torch.randn(B, S, H, D, generator=g) * 0.05 + 4.0 * u).to(torch.bfloat16)
    kv = (torch.randn(B, T, D, generator=g) * 0.05).to(torch.float32)
    idx = torch.stack([torch.randperm(T, generator=g)[:K] for _ in range(B * S)]).view(B, S, K).to(torch.int32)
    # row of slot k: its component along u grows with the slot's tile, so logit ~ 4 * c_t / sqrt(D)
    step = 10.0 / 1.4426950408889634 * D ** 0.5 / 4.0  # ~10 log2 units per tile
    for s_ in range(S):
        for k in range(K):
            r = int(idx[0, s_, k])
            kv[0, r] = kv[0, r] * 0 + torch.randn(D, generator=g) * 0.05 + (k // 32) * step * u
    kv = kv.to(torch.bfloat16)
    sink = torch.randn(H, generator=g)
    inp = {"q": q.to(DEV), "kv": kv.to(DEV), "attn_sink": sink.to(DEV), "topk_idxs": idx.to(DEV), "scale": D ** -0.5}
    out = _run(inp, num_splits=splits)
    torch.cuda.synchronize()
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, f"rising maximum S={S} splits={splits}")


@pytest.mark.parametrize("scale", [0.0, -0.05, 0.3])
@pytest.mark.parametrize("S,splits", [(1, 4), (2, 1)])
def test_scale_signs(oracle_impl, scale, S, splits):
    """A zero scale (every valid slot weighs the same), a negative one (the order of the logits
    reversed) and a large one, with and without splits."""
    inp = _custom(2, S, 128, 512, 400, 300, seed=140 + S + splits)
    inp["scale"] = scale
    out = _run(inp, num_splits=splits)
    torch.cuda.synchronize()
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, f"scale={scale} S={S} splits={splits}")


@pytest.mark.parametrize("H", [72, 100])
@pytest.mark.parametrize("S,splits", [(1, 0), (1, 1), (2, 3)])
def test_padded_head_blocks(oracle_impl, H, S, splits):
    """Head counts that are not a multiple of 16 in the eight-head-block form: the padded heads
    (72 or 100 .. 127) have zero queries, are computed and never written; one token per batch
    (the decode form, queries staged per score wave) and two, with and without splits."""
    inp = _custom(3, S, H, 512, 400, 300, seed=90 + H + S + splits)
    out = _run(inp, num_splits=splits)
    torch.cuda.synchronize()
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, f"H={H} S={S} splits={splits}")


@pytest.mark.parametrize("H", [96, 64])
@pytest.mark.parametrize("S,splits", [(1, 0), (1, 2), (2, 1), (2, 3)])
def test_head_groups_with_padded_blocks(oracle_impl, H, S, splits):
    """Two head groups: 96 heads are groups of 48 in a 64-head block (the padded heads are never
    written), 64 heads groups of 32; each group's queries, sink entries and output rows are those
    of its own heads."""
    B = 4
    assert sa.sparse_attn_head_groups(B, S, H, 512, 300) == 2
    inp = _custom(B, S, H, 512, 400, 300, seed=130 + H + S + splits)
    out = torch.full_like(inp["q"], 5.0)
    _run(inp, out=out, num_splits=splits)
    torch.cuda.synchronize()
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, f"H={H} S={S} splits={splits}")


@pytest.mark.parametrize("K", [0, 1, 31, 33])
@pytest.mark.parametrize("splits", [0, 3])
def test_few_slots(oracle_impl, K, splits):
    """K = 0 (no slot: only the sink, so o = 0 exactly), one slot, a single ragged tile, one full
    tile plus one slot; with the library's split choice and with three forced splits (more
    splits than tiles for the small K)."""
    inp = _custom(3, 2, 128, 512, 64, K, seed=40 + K, holes=0.05)
    out = _run(inp, num_splits=splits)
    torch.cuda.synchronize()
    if K == 0:
        assert torch.count_nonzero(out).item() == 0
        return
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, f"K={K} splits={splits}")


@pytest.mark.parametrize("splits", [4, 10])
def test_empty_splits_leave_no_trace(oracle_impl, splits):
    """Tokens whose valid slots end early (0, 1, 33, ... of 320): the later slot ranges hold no
    gathered row. The workspace is filled with NaN bytes first, so a merge that read a block no
    slot range wrote would show in the output."""
    B, S, H, D, T, K = 8, 1, 128, 512, 600, 320
    inp = _custom(B, S, H, D, T, K, seed=91, holes=0.0)
    for bb, n in enumerate([0, 1, 33, 100, 160, 250, 319, 320]):
        inp["topk_idxs"][bb, :, n:] = -1
    ws = sa.new_workspace(sa.sparse_attn_workspace_bytes(B, S, H, D, K, splits), DEV)
    ws.fill_(0xFF)
    out = _run(inp, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, f"empty splits, {splits} splits")
    assert torch.count_nonzero(out[0]).item() == 0


def test_all_invalid_is_exactly_zero():
    inp = _custom(2, 2, 128, 512, 100, 70, seed=3)
    inp["topk_idxs"].fill_(-1)
    for splits in (1, 2):
        out = _run(inp, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0


def test_exact_mean_bit_exact():
    """q = 0, sink -inf, exactly 64 valid slots over {-1,0,1} rows: o is the plain mean,
    exactly representable in bf16; any wrong or missed row changes it."""
    g = torch.Generator().manual_seed(11)
    B, S, H, D, T, K = 2, 3, 128, 512, 500, 150
    kv = torch.randint(-1, 2, (B, T, D), generator=g).to(torch.bfloat16)
    q = torch.zeros(B, S, H, D, dtype=torch.bfloat16)
    idx = torch.full((B, S, K), -1, dtype=torch.int32)
    ref = torch.zeros(B, S, D, dtype=torch.float64)
    for b in range(B):
        for s in range(S):
            rows = torch.randperm(T, generator=g)[:64]
            idx[b, s, torch.randperm(K, generator=g)[:64]] = rows.to(torch.int32)
            ref[b, s] = kv[b, rows].double().mean(0)
    sink = torch.full((H,), float("-inf"))
    want = ref.unsqueeze(2).expand(B, S, H, D)
    # one workgroup per token, and three and four splits: a split's partial is its unnormalised
    # row sum (weights exactly 1 here, sums of at most 64 values in {-1, 0, 1}), exact in bf16,
    # so the merged result is the exact mean on every path.
    for splits in (1, 3, 4):
        out = sa.sparse_attn(q.to(DEV), kv.to(DEV), sink.to(DEV), idx.to(DEV), 1.0, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out.double().cpu(), want), f"{splits} splits"
    # the two phases apart
    args = (q.to(DEV), kv.to(DEV), sink.to(DEV), idx.to(DEV), 1.0)
    ws = sa.new_workspace(sa.sparse_attn_workspace_bytes(B, S, H, D, K, 4), DEV)
    out = torch.empty_like(args[0])
    sa.sparse_attn_split(*args, out=out, num_splits=4, workspace=ws)
    sa.sparse_attn_merge(*args, out=out, num_splits=4, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.double().cpu(), want)


@pytest.mark.parametrize("splits", [1, 3, 4])
def test_duplicate_slots(oracle_impl, splits):
    """Repeated indices each count (a row listed twice weighs double): lists with pairs and
    triples of one row, against the oracle, on every path."""
    inp = _custom(4, 2, 128, 512, 200, 160, seed=17, holes=0.05)
    idx = inp["topk_idxs"]
    g = torch.Generator().manual_seed(5)
    for t in range(8):
        b, s_ = t // 2, t % 2
        src = torch.randint(0, 160, (24,), generator=g)
        dst = torch.randint(0, 160, (24,), generator=g)
        idx[b, s_, dst.to(DEV)] = idx[b, s_, src.to(DEV)]
    idx[0, 0, :3] = 7  # one row three times
    out = _run(inp, num_splits=splits)
    torch.cuda.synchronize()
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], idx, inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, f"duplicates, {splits} splits")


def test_single_row_bit_exact():
    inp = _custom(1, 2, 128, 512, 90, 40, seed=5)
    inp["topk_idxs"].fill_(-1)
    inp["topk_idxs"][:, :, 17] = 33
    inp["attn_sink"].fill_(float("-inf"))
    for splits in (1, 2):
        out = _run(inp, num_splits=splits)
        torch.cuda.synchronize()
        row = inp["kv"][0, 33]
        assert torch.equal(out[0], row.expand_as(out[0]))


def test_sink_special_values(oracle_impl):
    inp = _custom(1, 2, 16, 64, 90, 40, seed=6)
    inp["attn_sink"][0] = float("inf")
    inp["attn_sink"][1] = float("nan")
    inp["attn_sink"][2] = float("-inf")
    inp["attn_sink"][3] = 100.0
    for splits in (1, 2):
        out = _run(inp, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out[:, :, 0]).item() == 0
        assert torch.isnan(out[:, :, 1]).all()
        ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
        assert_close(to64(out).reshape(ref.shape), ref, f"sink specials splits={splits}")


def test_sink_halves_mean():
    """q = 0 and sink = ln(n): o is half the mean of the n rows."""
    g = torch.Generator().manual_seed(8)
    T, D, n = 300, 512, 100
    kv = torch.randn(1, T, D, generator=g).to(torch.bfloat16)
    q = torch.zeros(1, 1, 128, D, dtype=torch.bfloat16)
    idx = torch.randperm(T, generator=g)[:n].view(1, 1, n).to(torch.int32)
    sink = torch.full((128,), math.log(n))
    out = sa.sparse_attn(q.to(DEV), kv.to(DEV), sink.to(DEV), idx.to(DEV), 1.0)
    torch.cuda.synchronize()
    ref = kv[0, idx[0, 0].long()].double().mean(0) / (1.0 + math.exp(float(sink[0])) / n)
    assert_close(out[0, 0].double().cpu().numpy(), ref.expand(128, D).numpy(), "sink halves")


def test_order_invariance():
    inp = _custom(2, 2, 128, 512, 400, 300, seed=9)
    a = _run(inp)
    perm = torch.randperm(300, generator=torch.Generator().manual_seed(1)).to(DEV)
    inp2 = dict(inp)
    inp2["topk_idxs"] = inp["topk_idxs"][:, :, perm].contiguous()
    b = _run(inp2)
    torch.cuda.synchronize()
    assert_close(to64(a), to64(b), "order invariance")


def test_out_of_range_indices_are_empty():
    inp = _custom(1, 2, 16, 64, 100, 48, seed=12)
    a_idx = inp["topk_idxs"].clone()
    a_idx[:, :, 0] = 100  # == T
    a_idx[:, :, 1] = -5
    a_idx[:, :, 2] = 2**30
    b_idx = a_idx.clone()
    b_idx[:, :, :3] = -1
    inp["topk_idxs"] = a_idx
    a = _run(inp)
    inp["topk_idxs"] = b_idx
    b = _run(inp)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_write_bounds_guard_band():
    """Guard bands around out keep their sentinel."""
    inp = _custom(2, 3, 128, 512, 200, 100, seed=13)
    B, S, H, D = inp["q"].shape
    n = B * S * H * D
    buf = torch.full((n + 2 * 4096,), 3.0, dtype=torch.bfloat16, device=DEV)
    out = buf[4096:4096 + n].view(B, S, H, D)
    for splits in (1, 2):
        _run(inp, out=out, num_splits=splits)
        torch.cuda.synchronize()
        assert (buf[:4096] == 3.0).all() and (buf[4096 + n:] == 3.0).all()


def test_decode_config_all_tokens(oracle_impl):
    """The decode shape (B=64, H=128, D=512, K=1152, 4 splits) as the benchmark runs it: every
    token against the oracle."""
    inp = wl.sparse_inputs("decode", 1002, DEV)
    out = _run(inp)
    torch.cuda.synchronize()
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    assert_close(to64(out).reshape(ref.shape), ref, "decode")


def test_prefill_config_sampled(oracle_impl):
    inp = wl.sparse_inputs("prefill", 1003, DEV)
    out = _run(inp)
    torch.cuda.synchronize()
    tokens = np.array([0, 1, 2, 127, 128, 129, 511, 1000, 2047, 3000, 4094, 4095])
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"], tokens)
    got = to64(out[0][torch.as_tensor(tokens, device=DEV)])
    assert_close(got, ref, "prefill")


def test_ragged_config_sampled(oracle_impl):
    inp = wl.sparse_inputs("ragged", 1005, DEV)
    out = _run(inp)
    torch.cuda.synchronize()
    tokens = np.arange(0, 32, 3)
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"], tokens)
    got = to64(out.reshape(32, *out.shape[2:])[torch.as_tensor(tokens, device=DEV)])
    assert_close(got, ref, "ragged")
    del inp


@pytest.mark.parametrize("D,B,S,splits", [(512, 2, 1, 0), (512, 1, 2, 1), (512, 1, 1, 4), (64, 2, 1, 0), (64, 1, 2, 1)])
def test_rows_past_4gb(oracle_impl, D, B, S, splits):
    """bf16 rows more than 4 GB into a batch (2^22 rows per 4 GB at D = 512, 2^25 at D = 64): rows
    on both sides of each 4 GB mark, the batch's last row and, with B = 2, a second batch that
    starts past 4 GB, against the oracle on the gathered rows."""
    H, K = 16, 320
    mark = (1 << 32) // (2 * D)
    T = mark + 3000
    gen = torch.Generator(device=DEV).manual_seed(77)
    kv = torch.randn(B, T, D, device=DEV, dtype=torch.bfloat16, generator=gen)
    g = torch.Generator().manual_seed(78)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).to(DEV)
    sink = torch.randn(H, generator=g).to(DEV)
    fixed = torch.tensor([0, mark - 2, mark - 1, mark, mark + 1, T - 1], dtype=torch.int64)
    idx = torch.empty(B * S, K, dtype=torch.int64)
    for t in range(B * S):
        lo = torch.randperm(mark - 2, generator=g)[: (K - 6) // 2] + 1
        hi = torch.randperm(T - mark - 2, generator=g)[: K - 6 - (K - 6) // 2] + mark + 2
        idx[t] = torch.cat([fixed, lo, hi])[torch.randperm(K, generator=g)]
    idx = idx.view(B, S, K).to(torch.int32).to(DEV)
    out = sa.sparse_attn(q, kv, sink, idx, D ** -0.5, num_splits=splits)
    torch.cuda.synchronize()
    tokens = np.arange(B * S)
    ref = sparse_reference(oracle_impl, q, kv, sink, idx, D ** -0.5, tokens)
    assert_close(to64(out.reshape(B * S, H, D)), ref, f"rows past 4 GB D={D} B={B} S={S}")
    del kv


def test_graph_replay_tracks_new_indices(oracle_impl):
    """Capture once, replay with new index lists (grid depends only on shapes)."""
    inp = _custom(4, 1, 128, 512, 600, 320, seed=21)
    out = torch.empty_like(inp["q"])
    ws = sa.new_workspace(sa.sparse_attn_workspace_bytes(4, 1, 128, 512, 320), DEV)
    _run(inp, out=out, workspace=ws)  # warm up outside the graph
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(inp, out=out, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        new = _custom(4, 1, 128, 512, 600, 320, seed=100 + rep, holes=0.3 * rep)
        inp["topk_idxs"].copy_(new["topk_idxs"])
        graph.replay()
        torch.cuda.synchronize()
        ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
        assert_close(to64(out).reshape(ref.shape), ref, f"replay {rep}")


# More tokens and splits: every split's partial goes through the merge kernel.
@pytest.mark.parametrize("D,H,B,S,splits", [(512, 128, 16, 1, 4), (512, 128, 8, 2, 2), (512, 16, 4, 2, 8),
                                            (64, 64, 16, 1, 4), (512, 40, 8, 1, 16), (512, 128, 64, 1, 4)])
def test_split_merge_shapes(oracle_impl, D, H, B, S, splits):
    inp = _custom(B, S, H, D, 700, 640, seed=31 + H + splits)
    ws = sa.new_workspace(sa.sparse_attn_workspace_bytes(B, S, H, D, 640, splits), DEV)
    out = _run(inp, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    tokens = np.arange(0, B * S, max(1, B * S // 6))
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"], tokens)
    got = to64(out.reshape(B * S, H, D)[torch.as_tensor(tokens, device=DEV)])
    assert_close(got, ref, f"merge D={D} H={H} B={B} S={S} splits={splits}")


def test_split_merge_special_cases():
    """All-invalid rows, a single row in the last split, sink specials (16 tokens, 4 splits)."""
    inp = _custom(16, 1, 128, 512, 300, 256, seed=41)
    inp["topk_idxs"][0].fill_(-1)                  # token 0: nothing valid
    inp["topk_idxs"][1].fill_(-1)
    inp["topk_idxs"][1, 0, 200] = 17               # token 1: one row in the last split only
    inp["attn_sink"][0] = float("inf")
    inp["attn_sink"][1] = float("nan")
    inp["attn_sink"][2:].fill_(float("-inf"))
    out = _run(inp, num_splits=4)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0, :, 2:]).item() == 0
    assert torch.equal(out[1, 0, 2:], inp["kv"][1, 17].expand(126, 512))
    assert torch.count_nonzero(out[:, :, 0]).item() == 0
    assert torch.isnan(out[:, :, 1]).all()


@pytest.mark.parametrize("splits", [1, 2, 4])
def test_split_then_merge_equals_one_call(splits):
    """The two phases called apart give exactly the one-call result."""
    inp = _custom(16, 1, 128, 512, 600, 512, seed=51)
    ws = sa.new_workspace(sa.sparse_attn_workspace_bytes(16, 1, 128, 512, 512, splits), DEV)
    a = _run(inp, num_splits=splits, workspace=ws)
    b = torch.full_like(a, 7.0)
    args = (inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
    sa.sparse_attn_split(*args, out=b, num_splits=splits, workspace=ws)
    sa.sparse_attn_merge(*args, out=b, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_split_merge_many_tokens(oracle_impl):
    """4100 tokens with 2 splits (8200 partial blocks, D = 64), tokens sampled at both ends."""
    B, S, H, D, T, K = 1, 4100, 16, 64, 300, 64
    inp = _custom(B, S, H, D, T, K, seed=53)
    out = _run(inp, num_splits=2)
    torch.cuda.synchronize()
    tokens = np.array([0, 1, 2047, 4095, 4096, 4099])
    ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"], tokens)
    got = to64(out.reshape(B * S, H, D)[torch.as_tensor(tokens, device=DEV)])
    assert_close(got, ref, "4100 tokens, 2 splits")



def _random_case(rng: np.random.Generator):
    """One random shape and data mode: N(0,1), queries equal to gathered rows (late maximum jumps),
    heavy duplicates, most slots empty, or all heads' logits shifted by a large common offset."""
    D = int(rng.choice([64, 512]))
    H = int(rng.choice([1, 5, 16, 33, 64, 100, 128]))
    B, S = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    T = int(rng.integers(1, 700))
    K = int(rng.integers(0, 400))
    splits = int(rng.choice([0, 1, 2, 3, 7, 16]))
    mode = rng.choice(["normal", "aligned", "dups", "holes", "offset"])
    g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    q = torch.randn(B, S, H, D, generator=g)
    kv = torch.randn(B, T, D, generator=g)
    idx = torch.randint(0, T, (B, S, K), generator=g, dtype=torch.int32)
    if mode == "dups" and K > 0:
        idx = idx % max(1, min(T, 3))
    if mode == "holes":
        idx[torch.rand(B, S, K, generator=g) < 0.9] = -1
    else:
        idx[torch.rand(B, S, K, generator=g) < 0.05] = -1
    if mode == "aligned" and K > 0:
        for b in range(B):
            for s_ in range(S):
                for h in range(H):
                    k = int(torch.randint(0, K, (1,), generator=g))
                    r = int(idx[b, s_, k])
                    if r >= 0:
                        q[b, s_, h] = kv[b, r]
    if mode == "offset":
        u = torch.randn(D, generator=g)
        kv = kv + 3.0 * u / u.norm()
        q = q + 3.0 * u / u.norm()
    sink = torch.randn(H, generator=g) * 2
    scale = float(rng.choice([D ** -0.5, 0.02, 0.3]))
    inp = {"q": q.to(torch.bfloat16).to(DEV), "kv": kv.to(torch.bfloat16).to(DEV), "attn_sink": sink.to(DEV),
           "topk_idxs": idx.to(DEV), "scale": scale}
    return inp, splits, f"B={B} S={S} H={H} D={D} T={T} K={K} splits={splits} mode={mode} scale={scale:.3g}"


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_and_data(oracle_impl, seed):
    """Randomised shapes, split counts and data modes against the oracle (fixed seeds, 8 cases each)."""
    rng = np.random.default_rng(1000 + seed)
    for _ in range(8):
        inp, splits, what = _random_case(rng)
        out = _run(inp, num_splits=splits)
        torch.cuda.synchronize()
        ref = sparse_reference(oracle_impl, inp["q"], inp["kv"], inp["attn_sink"], inp["topk_idxs"], inp["scale"])
        assert_close(to64(out).reshape(ref.shape), ref, what)
