"""Host-side argument checks of the Python binding's decode() (no GPU).

The C ABI receives pointers and a shape descriptor only, so a tensor that is
smaller than the descriptor says would be indexed past its end on the
device.  check_decode_args must turn every such mismatch into a ValueError
before anything is launched; each case below breaks one property of an
otherwise valid call.
"""

import pytest
import torch

import decode_attention_paged_fp8pa_amd as fp

B, QL, HQ, HKV, D, BT, NB = 3, 2, 8, 2, 64, 16, 12


def _valid(**over):
    a = dict(
        q=torch.zeros((B, QL, HQ, D), dtype=torch.bfloat16),
        k_cache=torch.zeros((NB, BT, HKV, D), dtype=torch.uint8),
        v_cache=torch.zeros((NB, BT, HKV, D), dtype=torch.uint8),
        block_table=torch.zeros((B, 4), dtype=torch.int32),
        seq_lens=torch.full((B,), 40, dtype=torch.int32),
        k_scale=torch.ones(HKV, dtype=torch.float32),
        v_scale=torch.ones(1, dtype=torch.float32),
        sinks=torch.zeros(HQ, dtype=torch.float32),
        out=torch.empty((B, QL, HQ, D), dtype=torch.bfloat16),
        lse=torch.empty((B, QL, HQ), dtype=torch.float32),
    )
    a.update(over)
    return a


def _check(**over):
    a = _valid(**over)
    fp.check_decode_args(a.pop("q"), a.pop("k_cache"), a.pop("v_cache"), a.pop("block_table"),
                         a.pop("seq_lens"), a.pop("k_scale"), a.pop("v_scale"), a.pop("sinks"), **a)


def test_valid_call_passes():
    _check()
    _check(sinks=None, out=None, lse=None)
    _check(k_scale=torch.ones(1), v_scale=torch.ones(HKV))


BAD = {
    "q_dtype": dict(q=torch.zeros((B, QL, HQ, D), dtype=torch.float16)),
    "q_rank": dict(q=torch.zeros((B, HQ, D), dtype=torch.bfloat16)),
    "cache_dtype": dict(k_cache=torch.zeros((NB, BT, HKV, D), dtype=torch.int8)),
    "cache_shapes_differ": dict(v_cache=torch.zeros((NB + 1, BT, HKV, D), dtype=torch.uint8)),
    "head_dim_mismatch": dict(k_cache=torch.zeros((NB, BT, HKV, 2 * D), dtype=torch.uint8),
                              v_cache=torch.zeros((NB, BT, HKV, 2 * D), dtype=torch.uint8)),
    "hq_not_multiple": dict(k_cache=torch.zeros((NB, BT, 3, D), dtype=torch.uint8),
                            v_cache=torch.zeros((NB, BT, 3, D), dtype=torch.uint8),
                            k_scale=torch.ones(1)),
    "cache_not_contiguous": dict(k_cache=torch.zeros((NB, BT, D, HKV), dtype=torch.uint8).transpose(2, 3)),
    "table_dtype": dict(block_table=torch.zeros((B, 4), dtype=torch.int64)),
    "table_rows": dict(block_table=torch.zeros((B - 1, 4), dtype=torch.int32)),
    "table_column_stride": dict(block_table=torch.zeros((4, B), dtype=torch.int32).t()),
    "seq_lens_dtype": dict(seq_lens=torch.full((B,), 40, dtype=torch.int64)),
    "seq_lens_count": dict(seq_lens=torch.full((B + 1,), 40, dtype=torch.int32)),
    "seq_lens_rank": dict(seq_lens=torch.full((B, 1), 40, dtype=torch.int32)),
    "k_scale_dtype": dict(k_scale=torch.ones(HKV, dtype=torch.float64)),
    "v_scale_dtype": dict(v_scale=torch.ones(1, dtype=torch.float16)),
    "k_scale_count": dict(k_scale=torch.ones(HKV + 1)),
    "v_scale_count": dict(v_scale=torch.ones(3)),
    "sinks_dtype": dict(sinks=torch.zeros(HQ, dtype=torch.float64)),
    "sinks_count": dict(sinks=torch.zeros(HQ - 1)),
    "sinks_not_contiguous": dict(sinks=torch.zeros(2 * HQ)[::2]),
    "out_dtype": dict(out=torch.empty((B, QL, HQ, D), dtype=torch.float32)),
    "out_shape": dict(out=torch.empty((B, QL, HQ, D - 1), dtype=torch.bfloat16)),
    "out_short_batch": dict(out=torch.empty((B - 1, QL, HQ, D), dtype=torch.bfloat16)),
    "out_not_contiguous": dict(out=torch.empty((B, QL, D, HQ), dtype=torch.bfloat16).transpose(2, 3)),
    "lse_dtype": dict(lse=torch.empty((B, QL, HQ), dtype=torch.bfloat16)),
    "lse_shape": dict(lse=torch.empty((B, QL, HQ + 1))),
    "lse_not_contiguous": dict(lse=torch.empty((B, HQ, QL)).transpose(1, 2)),
    "workspace_not_contiguous": dict(workspace=torch.empty((64, 2), dtype=torch.uint8)[:, 0]),
    "tensor_on_other_device": dict(sinks=torch.zeros(HQ, device="meta")),
    "out_on_other_device": dict(out=torch.empty((B, QL, HQ, D), dtype=torch.bfloat16, device="meta")),
}


@pytest.mark.parametrize("case", sorted(BAD))
def test_bad_argument_is_rejected(case):
    with pytest.raises(ValueError):
        _check(**BAD[case])


def test_k_groups_scale_counts():
    fp.check_decode_args(*[_valid()[k] for k in ("q", "k_cache", "v_cache", "block_table", "seq_lens")],
                         torch.ones(HKV * 2), torch.ones(1), k_groups=2)
    fp.check_decode_args(*[_valid()[k] for k in ("q", "k_cache", "v_cache", "block_table", "seq_lens")],
                         torch.ones(2), torch.ones(1), k_groups=2)
    with pytest.raises(ValueError):
        fp.check_decode_args(*[_valid()[k] for k in ("q", "k_cache", "v_cache", "block_table", "seq_lens")],
                             torch.ones(HKV * 2 + 1), torch.ones(1), k_groups=2)


def test_blockscaled_page_bytes():
    per_row = D // 2 + D // 16
    page = BT * HKV * per_row
    a = _valid(k_cache=torch.zeros((NB, page), dtype=torch.uint8),
               v_cache=torch.zeros((NB, page), dtype=torch.uint8))
    args = [a[k] for k in ("q", "k_cache", "v_cache", "block_table", "seq_lens", "k_scale", "v_scale")]
    fp.check_decode_args(*args, kv_format="nvfp4", num_kv_heads=HKV, block_tokens=BT)
    short = torch.zeros((NB, page - 16), dtype=torch.uint8)
    with pytest.raises(ValueError):
        fp.check_decode_args(args[0], short, short, *args[3:], kv_format="nvfp4", num_kv_heads=HKV,
                             block_tokens=BT)
    with pytest.raises(ValueError):
        fp.check_decode_args(*args, kv_format="nvfp4")  # geometry missing


def test_e4m3_pages_interleaved_in_one_buffer():
    """K and V pages interleaved in one buffer ([blocks, 2, bt, Hkv, D]):
    each pool is dense inside a page, and the shape carries the page stride."""
    buf = torch.zeros((NB, 2, BT, HKV, D), dtype=torch.uint8)
    k, v = buf[:, 0], buf[:, 1]
    _check(k_cache=k, v_cache=v)
    a = _valid()
    shape = fp.shape_for(a["q"], k, a["block_table"], a["k_scale"], a["v_scale"], max_seq_len=40)
    assert shape.kv_page_stride == 2 * BT * HKV * D
    assert fp.shape_for(a["q"], a["k_cache"], a["block_table"], a["k_scale"], a["v_scale"],
                        max_seq_len=40).kv_page_stride == 0
    # V's pages must be laid out like K's
    with pytest.raises(ValueError):
        _check(k_cache=k, v_cache=torch.zeros((NB, BT, HKV, D), dtype=torch.uint8))


def test_size_one_dimensions_keep_any_stride():
    """A dimension of size 1 addresses nothing, so its stride does not count:
    head-major pools of one-token pages made by transposing token-major ones
    (torch keeps them as views with the old stride) are dense, and so are
    one-page pools sliced out of a wider buffer; a page that is really
    strided is still refused."""
    hnd = torch.zeros((NB, 1, HKV, D), dtype=torch.uint8).transpose(1, 2)
    assert hnd.is_contiguous() and hnd.stride(2) != D
    assert fp._e4m3_page_stride(hnd) == 0
    a = _valid(k_cache=hnd, v_cache=torch.zeros((NB, HKV, 1, D), dtype=torch.uint8),
               block_table=torch.zeros((B, 64), dtype=torch.int32))
    fp.check_decode_args(a.pop("q"), a.pop("k_cache"), a.pop("v_cache"), a.pop("block_table"),
                         a.pop("seq_lens"), a.pop("k_scale"), a.pop("v_scale"), a.pop("sinks"),
                         kv_layout="HND", **a)
    one_page = torch.zeros((2, BT, HKV, D), dtype=torch.uint8)[:1]
    assert fp._e4m3_page_stride(one_page) == 0
    wide = torch.zeros((1, 4096), dtype=torch.uint8)
    assert fp._row_stride(wide[:, :2048].t().contiguous().t()) == 0
    strided_rows = torch.zeros((NB, BT, HKV, 2 * D), dtype=torch.uint8)[..., :D]
    assert fp._e4m3_page_stride(strided_rows) is None
    with pytest.raises(ValueError):
        _check(k_cache=strided_rows, v_cache=strided_rows)


def test_overlapping_pages_are_refused():
    """Pools whose page stride is below one page (an expanded view, stride 0)
    would send the kernels past the storage: refused in every path that
    builds a shape from tensors, E4M3 and block-scaled."""
    one = torch.zeros((1, BT, HKV, D), dtype=torch.uint8)
    expanded = one.expand(NB, BT, HKV, D)
    assert expanded.stride(0) == 0
    assert fp._e4m3_page_stride(expanded) is None
    with pytest.raises(ValueError):
        _check(k_cache=expanded, v_cache=expanded)
    a = _valid()
    with pytest.raises(ValueError):
        fp.shape_for(a["q"], expanded, a["block_table"], a["k_scale"], a["v_scale"], max_seq_len=40)
    rows = torch.zeros((1, 4096), dtype=torch.uint8).expand(NB, 4096)
    assert fp._row_stride(rows) is None
    with pytest.raises(ValueError):
        fp.shape_for(a["q"], rows, a["block_table"], a["k_scale"], a["v_scale"], max_seq_len=40,
                     kv_format="nvfp4", num_kv_heads=HKV, block_tokens=BT)
    # rows that overlap partly (stride below the row length)
    base = torch.zeros(NB * 2048 + 2048, dtype=torch.uint8)
    partly = base.as_strided((NB, 4096), (2048, 1))
    assert fp._row_stride(partly) is None
    # a writer into such pools is refused before any launch
    key = torch.zeros((2, HKV, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fp.cache_write(key, key, torch.zeros(2, dtype=torch.int64), torch.ones(1), torch.ones(1),
                       expanded, expanded)


def test_table_width_against_max_seq_len():
    a = _valid()
    fp._check_table_width(a["block_table"], 4 * BT, a["k_cache"], "NHD", "e4m3", None)
    with pytest.raises(ValueError):
        fp._check_table_width(a["block_table"], 4 * BT + 1, a["k_cache"], "NHD", "e4m3", None)


def test_decode_refuses_host_tensors():
    a = _valid()
    with pytest.raises(ValueError):
        fp.decode(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seq_lens"], a["k_scale"],
                  a["v_scale"], max_seq_len=40)
