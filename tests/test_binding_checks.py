"""The Python binding's size checks, on the CPU.  The C ABI takes sizes on
trust, so the binding refuses any tensor smaller than the sizes it passes
(an out-of-bounds access on the GPU otherwise).  These are the helpers the
public functions call before any launch; the GPU test file checks the
public functions themselves."""
import pytest
import torch

import memory_bound_transformer_amd as mbt


def test_rope_tables():
    cs = torch.zeros(64, 32)
    pos = torch.zeros(5, dtype=torch.int64)
    assert mbt._rope_tables(cs, pos, 5, 32, None) == 64
    assert mbt._rope_tables(cs, pos, 5, 32, 10) == 10
    with pytest.raises(ValueError):
        mbt._rope_tables(cs, pos, 5, 32, 65)            # more rows than the cache holds
    with pytest.raises(ValueError):
        mbt._rope_tables(cs, pos, 5, 16, None)          # wrong row width
    with pytest.raises(ValueError):
        mbt._rope_tables(cs, pos, 6, 32, None)          # pos shorter than T
    with pytest.raises(TypeError):
        mbt._rope_tables(cs, pos.int(), 5, 32, None)
    with pytest.raises(TypeError):
        mbt._rope_tables(cs.double(), pos, 5, 32, None)
    with pytest.raises(ValueError):
        mbt._rope_tables(None, pos, 5, 32, 8)
    assert mbt._rope_tables(None, pos, 5, 0, None) == 0


def test_rows_and_norm_args():
    x = torch.zeros(3, 7, 16)
    assert mbt._rows(x) == (21, 16)
    with pytest.raises(ValueError):
        mbt._rows(torch.zeros(4, 0))
    assert mbt._norm_args(x, torch.zeros(3, 7, 16), torch.zeros(16)) == (21, 16)
    with pytest.raises(ValueError):
        mbt._norm_args(x, torch.zeros(3, 7, 15), None)
    with pytest.raises(ValueError):
        mbt._norm_args(x, None, torch.zeros(8))
    with pytest.raises(ValueError):
        mbt._ada_args(x, None, None, torch.zeros(16), torch.zeros(15))


def test_act_rows_and_outputs():
    assert mbt._act_rows(torch.zeros(5, 20)) == (5, 10)
    for bad in (torch.zeros(5, 1), torch.zeros(5, 21), torch.zeros(5, 0)):
        with pytest.raises(ValueError):
            mbt._act_rows(bad)
    mbt._codes(torch.zeros(5, 10, dtype=torch.uint8), (5, 10), "out")
    with pytest.raises(ValueError):
        mbt._codes(torch.zeros(5, 9, dtype=torch.uint8), (5, 10), "out")
    with pytest.raises(TypeError):
        mbt._codes(torch.zeros(5, 10), (5, 10), "out")
    with pytest.raises(TypeError):
        mbt._amax_out(torch.zeros(0))
    with pytest.raises(ValueError):
        mbt._shape(torch.zeros(2, 3), (3, 2), "t")


def test_heads_and_strides():
    qkv = torch.zeros(4, 10, 8)
    q = qkv[:, :6]
    assert mbt._heads3(q, "q") == (4, 6, 8)
    assert mbt._token_stride(q, "q") == 80
    with pytest.raises(ValueError):
        mbt._heads3(torch.zeros(4, 8), "q")
    with pytest.raises(ValueError):
        mbt._token_stride(qkv[:, :, :4], "q")           # heads not contiguous


def test_broadcast_and_overlapping_views_refused():
    """A broadcast (expand()ed) [T, heads, D] view has token stride 0, which
    the C ABI reads as "dense": it would address T rows of an allocation
    holding one.  Overlapping tokens are refused the same way."""
    one = torch.zeros(1, 6, 8)
    wide = one.expand(5, 6, 8)
    assert wide.stride(0) == 0
    with pytest.raises(ValueError, match="token stride"):
        mbt._token_stride(wide, "q_in")
    base = torch.zeros(200)
    overlap = base.as_strided((4, 6, 8), (40, 8, 1))     # tokens 40 apart, rows of 48
    with pytest.raises(ValueError, match="token stride"):
        mbt._token_stride(overlap, "q_out")
    # a single token needs no stride; a padded one keeps its own
    assert mbt._token_stride(one.expand(1, 6, 8), "q") == 48
    assert mbt._token_stride(base.as_strided((3, 6, 8), (50, 8, 1)), "q") == 50
    # no heads: nothing is addressed, so any stride passes
    mbt._token_stride(torch.zeros(4, 0, 8), "k")
    mbt._token_stride(torch.zeros(1, 0, 8).expand(4, 0, 8), "k")


def test_stream_copy_refuses_host_tensors():
    # the calibration copy takes device tensors only; the check comes first
    a = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensors only"):
        mbt.stream_copy(a[:32], a[32:], 1)


class _OnDevice:
    """Stands in for a tensor or stream on a given device (no GPU here)."""
    def __init__(self, index):
        self.is_cuda = True
        self.device = torch.device("cuda", index)
        self.cuda_stream = 1234

    def is_contiguous(self):
        return True


def test_tensors_and_stream_on_the_current_gpu():
    cur = lambda: 0                                     # noqa: E731
    mbt._on_current_gpu([_OnDevice(0), None, _OnDevice(0)], cur)
    with pytest.raises(ValueError):
        mbt._on_current_gpu([_OnDevice(0), _OnDevice(1)], cur)   # two GPUs
    with pytest.raises(ValueError):
        mbt._on_current_gpu([_OnDevice(1)], cur)                 # not the current one
    with pytest.raises(ValueError):
        mbt._on_current_gpu([torch.zeros(2)], cur)               # host memory
    assert mbt._stream(_OnDevice(0), cur) == 1234
    with pytest.raises(ValueError):
        mbt._stream(_OnDevice(1), cur)
