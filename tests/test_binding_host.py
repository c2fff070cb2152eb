"""Host-side checks of the Python binding (no GPU): the record-pool view
helper and the prefill epilogue's argument checks, which run before any
library call and so before any launch."""

import pytest
import torch

from head_latent_attention_sparse_amd import ops


@pytest.mark.parametrize("shape", [(7, 656), (7, 1, 656), (7, 1, 1, 656), (3, 64, 656), (1, 656), (1, 1, 656)])
@pytest.mark.parametrize("dtype", [torch.uint8, torch.int8, torch.float8_e4m3fn])
def test_record_pool_flat_views(shape, dtype):
    kv = torch.zeros(shape, dtype=dtype)
    ptr, n, pitch = ops._record_pool(kv)
    assert ptr == kv.data_ptr()
    assert n == kv.numel() // 656
    assert pitch == 656


def test_record_pool_slices_keep_their_base_and_count():
    base = torch.zeros((10, 656), dtype=torch.uint8)
    ptr, n, pitch = ops._record_pool(base[3:8])
    assert (ptr, n, pitch) == (base.data_ptr() + 3 * 656, 5, 656)


def test_record_pool_padded_pages_are_not_flat():
    # pages of 70 records of which 64 are used: the page pitch is not 64 * 656
    pages = torch.zeros((2, 70, 656), dtype=torch.uint8)[:, :64]
    assert ops._record_pool(pages)[2] == -1
    # a strided record dim (every other record) is a run of pitch 1312
    assert ops._record_pool(torch.zeros((8, 656), dtype=torch.uint8)[::2])[2] == 2 * 656


@pytest.mark.parametrize("make", [
    lambda: torch.zeros((4, 657), dtype=torch.uint8),            # not 656 bytes
    lambda: torch.zeros((4, 656), dtype=torch.int16),            # 2-byte dtype
    lambda: torch.zeros((656,), dtype=torch.uint8),              # rank 1
    lambda: torch.zeros((2, 2, 2, 2, 656), dtype=torch.uint8),   # rank 5
    lambda: torch.zeros((656, 4), dtype=torch.uint8).t(),        # record bytes not contiguous
])
def test_record_pool_rejects(make):
    with pytest.raises(ValueError):
        ops._record_pool(make())


def _prefill_tensors(tp=5, heads=3, nope=128):
    bf = torch.bfloat16
    return dict(q=torch.zeros((tp, heads, nope + 64), dtype=bf), k_nope=torch.zeros((tp, heads, nope), dtype=bf),
                k_pe=torch.zeros((tp, 64), dtype=bf), kv_c_normed=torch.zeros((tp, 512), dtype=bf),
                slot_mapping=torch.zeros(tp, dtype=torch.int64), positions=None, cos_sin_cache=None,
                k_out=torch.zeros((tp, heads, nope + 64), dtype=bf))


def test_key_concat_args_accepts_matching_tensors():
    k_pe2, max_position = ops._key_concat_args(**_prefill_tensors())
    assert tuple(k_pe2.shape) == (5, 64) and max_position == 0


@pytest.mark.parametrize("rows", [4, 6, 0])
def test_key_concat_args_rejects_k_out_of_another_token_count(rows):
    args = _prefill_tensors()
    args["k_out"] = torch.zeros((rows, 3, 192), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_out"):
        ops._key_concat_args(**args)


@pytest.mark.parametrize("name,shape", [("q", (4, 3, 192)), ("kv_c_normed", (6, 512)), ("k_pe", (4, 64)),
                                        ("k_out", (5, 3, 190))])
def test_key_concat_args_rejects_other_shapes(name, shape):
    args = _prefill_tensors()
    args[name] = torch.zeros(shape, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ops._key_concat_args(**args)
