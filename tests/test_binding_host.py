"""The Python binding refuses tensors whose shapes do not agree, before the
library is loaded or called.

The C ABI sees pointers and strides only, so a K/V with the wrong batch, head
count or head_dim, or an undersized output, would make a kernel read or
write past an allocation.  These checks run on the CPU: the device check and
the library loader are replaced so that reaching either one fails the test.
"""

import pytest
import torch

from long_context_attention_attn_amd import binding


@pytest.fixture
def no_library(monkeypatch):
    def refuse(*a, **k):
        raise AssertionError("the library was reached with mismatched shapes")

    monkeypatch.setattr(binding, "_require_cuda", lambda *t: None)
    monkeypatch.setattr(binding, "load_library", refuse)
    monkeypatch.setattr(binding, "_stream", refuse)


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


GOOD = dict(q=(2, 8, 100, 128), k=(2, 2, 300, 128), v=(2, 2, 300, 128))

BAD_KV = [
    ("k batch", dict(k=(1, 2, 300, 128), v=(1, 2, 300, 128))),
    ("k heads not dividing", dict(k=(2, 3, 300, 128), v=(2, 3, 300, 128))),
    ("k head_dim", dict(k=(2, 2, 300, 64), v=(2, 2, 300, 64))),
    ("v heads differ from k", dict(v=(2, 1, 300, 128))),
    ("v length differs from k", dict(v=(2, 2, 299, 128))),
    ("v head_dim differs", dict(v=(2, 2, 300, 64))),
    ("k 3-D", dict(k=(2, 300, 128))),
]


def _tensors(over):
    shapes = {**GOOD, **over}
    return _t(*shapes["q"]), _t(*shapes["k"]), _t(*shapes["v"])


@pytest.mark.parametrize("name,over", BAD_KV, ids=[c[0] for c in BAD_KV])
def test_shifted_refuses_mismatched_kv(no_library, name, over):
    q, k, v = _tensors(over)
    with pytest.raises(ValueError):
        binding.attn_shifted_fwd(q, k, v, num_chunks=1, rank=0)


@pytest.mark.parametrize("name,over", BAD_KV, ids=[c[0] for c in BAD_KV])
def test_chunk_refuses_mismatched_kv(no_library, name, over):
    q, k, v = _tensors(over)
    with pytest.raises(ValueError):
        binding.attn_chunk_fwd(q, k, v, kv_pos0=0)


@pytest.mark.parametrize("out_shape,lse_shape", [
    ((2, 8, 99, 128), (2, 8, 100)),     # output one row short
    ((2, 4, 100, 128), (2, 8, 100)),    # output missing heads
    ((2, 8, 100, 64), (2, 8, 100)),     # output head_dim
    ((2, 8, 100, 128), (2, 8, 99)),     # LSE one row short
    ((2, 8, 100, 128), (1, 8, 100)),    # LSE batch
    ((2, 8, 100, 128), (2 * 8 * 100,)),  # LSE flat
])
def test_outputs_must_match_q(no_library, out_shape, lse_shape):
    q, k, v = _tensors({})
    with pytest.raises(ValueError):
        binding.attn_shifted_fwd(q, k, v, num_chunks=1, rank=0, out=_t(*out_shape),
                                 lse=_t(*lse_shape, dtype=torch.float32))
    with pytest.raises(ValueError):
        binding.attn_chunk_fwd(q, k, v, kv_pos0=0, o_part=_t(*out_shape, dtype=torch.float32),
                               lse_part=_t(*lse_shape, dtype=torch.float32))


def test_merge_refuses_mismatched_sides(no_library):
    f = torch.float32
    with pytest.raises(ValueError):
        binding.lse_merge(_t(10, 128, dtype=f), _t(10, dtype=f), _t(9, 128, dtype=f),
                          _t(9, dtype=f))
    with pytest.raises(ValueError):
        binding.lse_merge(_t(10, 128, dtype=f), _t(10, dtype=f), _t(10, 128, dtype=f),
                          _t(11, dtype=f))
    with pytest.raises(ValueError):
        binding.lse_merge(_t(10, 128, dtype=f), _t(12, dtype=f), _t(10, 128, dtype=f),
                          _t(12, dtype=f))


def test_good_shapes_reach_the_library(no_library):
    """The same calls with matching shapes pass every check and stop only at
    the (replaced) library loader."""
    q, k, v = _tensors({})
    with pytest.raises(AssertionError):
        binding.attn_shifted_fwd(q, k, v, num_chunks=3, rank=1)
    with pytest.raises(AssertionError):
        binding.attn_chunk_fwd(q, k, v, kv_pos0=0)
