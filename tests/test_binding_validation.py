"""The Python binding checks every tensor against the shape and the layouts of
include/santa.h before anything reaches the library: a cache of another dtype,
shape or stride, a non-contiguous output or tensors on different devices raise
ValueError without a launch (no GPU needed; the tensors live on the CPU)."""
import pytest
import torch

import sampling_sparse_attention_amd as santa


def _good(paged=False, dtype=torch.bfloat16, S=16):
    B, Hq, Hkv, d, n = 2, 8, 2, 64, 96
    q = torch.zeros(B, Hq, d, dtype=dtype)
    if paged:
        ps, pages = 16, 16
        k = torch.zeros(pages, ps, Hkv, d, dtype=dtype)
        bt = torch.arange(B * (n // ps), dtype=torch.int32).reshape(B, n // ps)
    else:
        k = torch.zeros(B, n, Hkv, d, dtype=dtype)
        bt = None
    args = dict(q=q, k_cache=k, v_cache=torch.zeros_like(k), seq_lens=torch.full((B,), n, dtype=torch.int32),
                block_table=bt, num_samples=S, o=torch.zeros(B, Hq, d), idx=torch.zeros(B, Hq, S, dtype=torch.int32),
                workspace=torch.zeros(4096, dtype=torch.uint8))
    shape = santa.make_shape(q, k, bt, max_seq_len=n)
    return shape, args


def _check(shape, args):
    santa.validate(shape, **args)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_consistent_tensors_pass(paged, dtype):
    _check(*_good(paged, dtype))


def _mutations():
    def cache_dtype(shape, a):
        a["k_cache"] = a["k_cache"].float()
        a["v_cache"] = a["v_cache"].float()

    def v_dtype(shape, a):
        a["v_cache"] = a["v_cache"].to(torch.float16)

    def v_shape(shape, a):
        a["v_cache"] = a["v_cache"][:, :-16]

    def v_strides(shape, a):
        a["v_cache"] = a["v_cache"].transpose(1, 2).contiguous().transpose(1, 2)

    def k_last_stride(shape, a):
        k = a["k_cache"]
        a["k_cache"] = torch.zeros(k.shape[:-1] + (2 * k.shape[-1],), dtype=k.dtype)[..., ::2]
        a["v_cache"] = torch.zeros(k.shape[:-1] + (2 * k.shape[-1],), dtype=k.dtype)[..., ::2]

    def q_sliced(shape, a):
        a["q"] = torch.zeros(a["q"].shape[0], a["q"].shape[1], 2 * a["q"].shape[2], dtype=a["q"].dtype)[..., ::2]

    def q_dtype_vs_shape(shape, a):
        shape.dtype = 1

    def shape_heads(shape, a):
        shape.num_q_heads = 4

    def shape_kv_heads(shape, a):
        shape.num_kv_heads = 4

    def shape_strides(shape, a):
        shape.kv_stride_tok += 8

    def cache_too_short(shape, a):
        shape.max_seq_len = a["k_cache"].shape[1] + 16

    def o_dtype(shape, a):
        a["o"] = a["o"].to(torch.bfloat16)

    def o_not_contiguous(shape, a):
        a["o"] = torch.zeros(a["o"].shape[0], a["o"].shape[2], a["o"].shape[1]).transpose(1, 2)

    def idx_shape(shape, a):
        a["idx"] = a["idx"][..., :-1]

    def idx_dtype(shape, a):
        a["idx"] = a["idx"].long()

    def seq_lens_dtype(shape, a):
        a["seq_lens"] = a["seq_lens"].long()

    def seq_lens_shape(shape, a):
        a["seq_lens"] = torch.zeros(5, dtype=torch.int32)

    def block_table_given_for_contiguous(shape, a):
        a["block_table"] = torch.zeros(2, 6, dtype=torch.int32)

    def not_a_tensor(shape, a):
        a["o"] = None

    def other_device(shape, a):
        a["o"] = a["o"].to("meta")

    return {f.__name__: f for f in (cache_dtype, v_dtype, v_shape, v_strides, k_last_stride, q_sliced,
                                     q_dtype_vs_shape, shape_heads, shape_kv_heads, shape_strides,
                                     cache_too_short, o_dtype, o_not_contiguous, idx_shape, idx_dtype,
                                     seq_lens_dtype, seq_lens_shape, block_table_given_for_contiguous,
                                     not_a_tensor, other_device)}


@pytest.mark.parametrize("name", sorted(_mutations()))
def test_mismatch_raises_before_launch(name):
    shape, args = _good()
    _mutations()[name](shape, args)
    with pytest.raises(ValueError):
        _check(shape, args)


def _paged_mutations():
    def no_table(shape, a):
        a["block_table"] = None

    def table_dtype(shape, a):
        a["block_table"] = a["block_table"].long()

    def table_shape(shape, a):
        a["block_table"] = a["block_table"][:, :-1].contiguous()

    def pages_vs_shape(shape, a):
        shape.num_pages += 1

    def page_size_vs_shape(shape, a):
        shape.page_size = 32

    return {f.__name__: f for f in (no_table, table_dtype, table_shape, pages_vs_shape, page_size_vs_shape)}


@pytest.mark.parametrize("name", sorted(_paged_mutations()))
def test_paged_mismatch_raises_before_launch(name):
    shape, args = _good(paged=True)
    _paged_mutations()[name](shape, args)
    with pytest.raises(ValueError):
        _check(shape, args)


def test_decode_entry_points_validate_first(monkeypatch):
    """santa_decode and friends run the checks before asking for the library."""
    shape, args = _good()
    args["v_cache"] = args["v_cache"].float()
    monkeypatch.setattr(santa, "library", lambda: pytest.fail("library reached before validation"))
    for fn in (santa.santa_decode, santa.santa_decode_flash, santa.santa_score_pass, santa.santa_sample_pass):
        with pytest.raises(ValueError):
            fn(shape, args["q"], args["k_cache"], args["v_cache"], args["seq_lens"], args["block_table"],
               args["num_samples"], 2, 0, args["o"], args["idx"], args["workspace"])
