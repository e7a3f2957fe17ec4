"""GPU parity of the packed row gather (needs an MI355X).

[P1] "DFlash to DSpark in SGLang", section "Ragged verify under full CUDA
graphs": the per-row data of the scheduled verify tokens sits back to back,
with no padding, in a buffer of total-tokens rows. dspark_gather_rows moves per-position rows of
any width through the packed source rows of the compaction; the result must
be a byte-exact copy of the oracle's gather, with every row past the packed
total left untouched.
"""
import numpy as np
import pytest
import torch

import __graft_entry__  # noqa: F401
import confidence_scheduled_ragged_amd as dspark
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(B, g, row_shape, dtype, seed, full=False):
    rng = np.random.default_rng(seed)
    cap = B * (g + 1)
    src = rng.integers(0, 1 << 15, (cap,) + row_shape).astype(dtype)
    L = (np.full(B, g) if full else rng.integers(0, g + 1, B)).astype(np.int32)
    tok = rng.integers(0, 1000, (B, g + 1)).astype(np.int32)
    return src, L, tok


def _run(src, L, tok, offset=0):
    B, g1 = tok.shape
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    cu, ptok, psrc, _ = dspark.dspark_compact(t(L), t(tok))
    src_d = t(src)
    if offset:
        # a byte-offset copy of the rows: exercises the 4-byte and 1-byte paths
        raw = torch.zeros(src_d.numel() * src_d.element_size() + offset, dtype=torch.uint8,
                          device=DEV)
        raw[offset:] = src_d.view(torch.uint8).reshape(-1)
        src_d = raw[offset:].view(src.shape[0], -1)
        src = src.view(np.uint8).reshape(src.shape[0], -1)
    out = torch.full_like(src_d, 77)
    dspark.dspark_gather_rows(src_d, psrc, cu, out=out)
    torch.cuda.synchronize()
    o_cu, _, o_ps = oracle.compact(L, tok)
    want = oracle.gather_rows(src, o_ps, o_cu, dst=np.full_like(src, 77))
    got = out.cpu().numpy()
    assert np.array_equal(cu.cpu().numpy(), o_cu)
    assert np.array_equal(got, want)
    return int(o_cu[-1])


@pytest.mark.parametrize("B,g,row_shape,dtype", [
    (256, 16, (7168,), np.uint16),   # bf16 activations at a DeepSeek-V4 width (16-byte path)
    (64, 16, (4096,), np.uint16),
    (5, 3, (3,), np.int32),          # 12-byte rows: 4-byte path
    (7, 4, (13,), np.uint8),         # 13-byte rows: byte path
    (1, 1, (1,), np.uint8),
    (3, 64, (257,), np.uint16),      # odd bf16 width: 4-byte rows not possible, byte path
    (4200, 2, (8,), np.uint16),      # more rows than the grid's row stride
])
def test_gather_rows_matches_oracle(B, g, row_shape, dtype):
    src, L, tok = _case(B, g, row_shape, dtype, seed=B + g)
    _run(src, L, tok)


def test_gather_rows_full_block_and_misaligned():
    src, L, tok = _case(9, 5, (64,), np.uint16, seed=3, full=True)
    assert _run(src, L, tok) == 9 * 6
    src, L, tok = _case(9, 5, (64,), np.uint16, seed=4)
    _run(src, L, tok, offset=1)
    _run(src, L, tok, offset=4)


def test_gather_rows_out_of_range_source_is_skipped():
    B, g = 3, 2
    cap = B * (g + 1)
    src = torch.arange(cap * 4, dtype=torch.int32, device=DEV).view(cap, 4)
    cu = torch.tensor([0, 2, 3, 5], dtype=torch.int32, device=DEV)
    psrc = torch.tensor([0, 99, 3, -1, 7, 0, 0, 0, 0], dtype=torch.int32, device=DEV)
    out = torch.full_like(src, -5)
    dspark.dspark_gather_rows(src, psrc, cu, out=out)
    o = out.cpu().numpy()
    s = src.cpu().numpy()
    assert np.array_equal(o[0], s[0]) and np.array_equal(o[2], s[3]) and np.array_equal(o[4], s[7])
    assert np.all(o[1] == -5) and np.all(o[3] == -5) and np.all(o[5:] == -5)
