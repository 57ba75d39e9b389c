"""candidate_mask_apply on the GPU against the oracle's whole-row rule.

The contract (prhub summary of vLLM PR #56628, its tests): bit-exact agreement on
[0, end) of every row, nothing written at or past end, and a captured graph that
replays correctly when the ends change."""
import numpy as np
import pytest
import torch

import top_sparse_attention_attn_amd as sa

pytestmark = pytest.mark.gpu
DEV = "cuda"
NARROW = 8192
WIDE = 262144


def _inputs(rows, width, ends, block_size=16, starts=None, col_stride=1, seed=0, keep=0.5, row_repeat=1):
    g = torch.Generator().manual_seed(seed)
    nb = -(-width // block_size)
    flags = (torch.rand((rows, nb + 1), generator=g) < keep).to(torch.uint8)
    base = torch.randn((rows, width * col_stride), generator=g)
    logits = base.to(DEV)[:, ::col_stride]
    e = torch.tensor(ends, dtype=torch.int32)
    s = None if starts is None else torch.tensor(starts, dtype=torch.int32)
    return logits, e, s, flags


def _oracle(orc, logits_before, ends, starts, flags, block_size, row_repeat=1):
    return orc.candidate_mask(logits_before.cpu().numpy(), ends.numpy(), flags.numpy(), block_size,
                              starts=None if starts is None else starts.numpy(), row_repeat=row_repeat)


def _assert_contract(got, before, ref, ends, row_repeat=1):
    """[0, end) equals the oracle bit for bit; [end, width) is what it was."""
    got, before = got.cpu().numpy(), before.cpu().numpy()
    for r in range(got.shape[0]):
        e = int(ends[r // row_repeat])
        lim = max(0, min(e, got.shape[1]))
        assert np.array_equal(got[r, :lim], ref[r, :lim]), f"row {r} differs within [0, {lim})"
        assert np.array_equal(got[r, lim:], before[r, lim:]), f"row {r} written at or past end {e}"


@pytest.mark.parametrize("width", [NARROW, WIDE])
@pytest.mark.parametrize("col_stride", [1, 2])
def test_matches_oracle_ragged_ends(oracle_impl, width, col_stride):
    # the page's test ends: empty, one column, the 1024-column tile edges, width - 1, width, width / 2
    ends = [0, 1, 1023, 1024, 1025, width - 1, width, width // 2]
    logits, e, s, flags = _inputs(len(ends), width, ends, col_stride=col_stride, seed=width + col_stride)
    before = logits.clone()
    ref = _oracle(oracle_impl, before, e, s, flags, 16)
    sa.candidate_mask_apply(logits, e.to(DEV), flags.to(DEV), 16)
    torch.cuda.synchronize()
    _assert_contract(logits, before, ref, e.numpy())


@pytest.mark.parametrize("block_size", [8, 16, 12])
def test_starts_row_repeat_and_block_sizes(oracle_impl, block_size):
    """Nonzero starts (one negative), row_repeat 2, a non-power-of-two block size, an end past
    the width, and the edge flag set on every row."""
    width = 5000
    ends = [4000, 5000, 6000, 37]
    starts = [0, 129, -40, 3]
    rows = 2 * len(ends)
    logits, e, s, flags = _inputs(rows, width, ends, block_size=block_size, starts=starts, seed=block_size)
    flags[:, -1] = 1
    before = logits.clone()
    ref = _oracle(oracle_impl, before, e, s, flags, block_size, row_repeat=2)
    sa.candidate_mask_apply(logits, e.to(DEV), flags.to(DEV), block_size, starts=s.to(DEV), row_repeat=2)
    torch.cuda.synchronize()
    _assert_contract(logits, before, ref, e.numpy(), row_repeat=2)


def test_leaves_columns_past_end_untouched():
    ends = [0, 1, 1025, WIDE // 2]
    logits, e, _, flags = _inputs(len(ends), WIDE, ends, seed=7, keep=0.0)
    logits.fill_(1.5)
    sa.candidate_mask_apply(logits, e.to(DEV), flags.to(DEV), 16)
    torch.cuda.synchronize()
    for r, end in enumerate(ends):
        row = logits[r]
        assert torch.all(row[end:] == 1.5), f"row {r} (end {end}) written past its end"
        assert torch.all(torch.isneginf(row[:end])), f"row {r}: a column below end kept with no flag"


def test_ends_past_width_and_nonpositive(oracle_impl):
    width = 3000
    ends = [-7, 0, width + 1, 2 ** 31 - 1]
    logits, e, _, flags = _inputs(len(ends), width, ends, seed=8)
    before = logits.clone()
    ref = _oracle(oracle_impl, before, e, None, flags, 16)
    sa.candidate_mask_apply(logits, e.to(DEV), flags.to(DEV), 16)
    torch.cuda.synchronize()
    _assert_contract(logits, before, ref, e.numpy())


def test_graph_replay_tracks_changing_ends(oracle_impl):
    """The launch is fixed by (rows, width); a captured call replayed with other ends (longer
    and shorter than at capture) still meets the contract on every replay."""
    rows = 4
    logits, e, _, flags = _inputs(rows, WIDE, [1024, 4096, 8192, 2048], seed=9)
    base = logits.clone()
    ends_dev, flags_dev = e.to(DEV), flags.to(DEV)
    sa.candidate_mask_apply(logits.clone(), ends_dev, flags_dev, 16)  # load the library outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sa.candidate_mask_apply(logits, ends_dev, flags_dev, 16)
    for replay_ends in ([1, 131072, WIDE, 0], [WIDE, 1025, 3, 65536], [1024, 4096, 8192, 2048]):
        ends_dev.copy_(torch.tensor(replay_ends, dtype=torch.int32))
        logits.copy_(base)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = _oracle(oracle_impl, base, torch.tensor(replay_ends, dtype=torch.int32), None, flags, 16)
        _assert_contract(logits, base, ref, replay_ends)


def test_config_shape_sampled_rows(oracle_impl):
    """The benchmark's shape (96 rows x 1M columns, ends ~ U[64, 192]): every row checked on
    [0, end) and on a window past it."""
    from top_sparse_attention_attn_amd import workloads as wl
    inp = wl.candidate_inputs("candidate", 3, DEV)
    logits, e, flags = inp["logits"], inp["ends"], inp["flags"]
    head = logits[:, :4096].clone()
    tail = logits[:, 4096:4096 + 8192].clone()
    sa.candidate_mask_apply(logits, e, flags, inp["block_size"])
    torch.cuda.synchronize()
    # the oracle on the first 4096 columns of each row: ends are below 4096, and the block
    # rule only reads flags of blocks below the end, so the narrow slice decides the same
    nb = 4096 // inp["block_size"]
    f_narrow = torch.cat([flags[:, :nb], torch.zeros_like(flags[:, :1])], dim=1).cpu()
    ref = oracle_impl.candidate_mask(head.cpu().numpy(), e.cpu().numpy(), f_narrow.numpy(), inp["block_size"])
    _assert_contract(logits[:, :4096], head, ref, e.cpu().numpy())
    assert torch.equal(logits[:, 4096:4096 + 8192], tail)


@pytest.mark.parametrize("block_size", [4, 16, 12])
@pytest.mark.parametrize("misaligned", [False, True])
def test_long_rows_both_store_forms(oracle_impl, block_size, misaligned):
    """Long rows with ends anywhere in the row (not multiples of 4), starts of mixed alignment
    (multiples of 4 take the 16-byte store form, the others the per-column form) and the edge
    flag set on half the rows. misaligned: the rows start 4 bytes past a 16-byte boundary, so
    the whole launch takes the per-column form. Every row is compared over its full width."""
    width = 65536 + 12
    ends = [width, width - 1, 3, 40001, 65535, 17, width - 2, 1027]
    starts = [0, 8, -12, 4, 129, 3, 62, 1024]
    g = torch.Generator().manual_seed(1000 + block_size + misaligned)
    nb = -(-width // block_size)
    flags = (torch.rand((len(ends), nb + 1), generator=g) < 0.5).to(torch.uint8)
    flags[::2, -1] = 1
    base = torch.randn((len(ends), width + 4), generator=g).to(DEV)
    logits = base[:, 1:width + 1] if misaligned else base[:, :width]
    e = torch.tensor(ends, dtype=torch.int32)
    s = torch.tensor(starts, dtype=torch.int32)
    before = logits.clone()
    ref = _oracle(oracle_impl, before, e, s, flags, block_size)
    sa.candidate_mask_apply(logits, e.to(DEV), flags.to(DEV), block_size, starts=s.to(DEV))
    torch.cuda.synchronize()
    _assert_contract(logits, before, ref, e.numpy())
