"""The public binding refuses mis-sized GPU tensors before any launch, and
the library keeps working after each refusal."""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mbt():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    import memory_bound_transformer_amd as m
    return m


def z(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype, device=DEV)


def test_prologue_refusals(mbt):
    q, k, w = z(4, 6, 128), z(4, 2, 128), z(128)
    cs = torch.zeros(64, 64, device=DEV)
    pos = torch.zeros(4, dtype=torch.int64, device=DEV)
    for kw in (dict(q_out=z(4, 6, 64)), dict(k_out=z(3, 2, 128)), dict(max_pos=65)):
        with pytest.raises(ValueError):
            mbt.qknorm_rope(q, k, w, w, cs, pos, 64, **kw)
    with pytest.raises(ValueError):
        mbt.qknorm_rope(q, k, w, w, cs, pos[:3], 64)
    with pytest.raises(ValueError):
        mbt.qknorm_rope(q, k, z(64), w, cs, pos, 64)
    with pytest.raises(ValueError):
        mbt.qknorm_rope(q, k, w, w, cs, pos, 32)                     # cos_sin width != rot
    with pytest.raises(ValueError):
        mbt.rope(q, z(4, 2, 64), cs, pos, 64)
    qkv = z(4, 10, 128)
    with pytest.raises(ValueError):
        mbt.qkv_norm_rope_cache(qkv, w, w, cs, pos, pos[:2], z(8, 2, 128), z(8, 2, 128), 6, 64)
    with pytest.raises(ValueError):
        mbt.qkv_norm_rope_cache(qkv, w, w, cs, pos, pos, z(8, 2, 128), z(7, 2, 128), 6, 64)
    # broadcast views: token stride 0 would address T rows of one
    with pytest.raises(ValueError, match="token stride"):
        mbt.qknorm_rope_ex(z(1, 6, 128).expand(4, 6, 128), k, w, w, cs, pos, 64)
    with pytest.raises(ValueError, match="token stride"):
        mbt.qknorm_rope_ex(q, k, w, w, cs, pos, 64, k_out=z(1, 2, 128).expand(4, 2, 128))
    # still healthy
    qo, ko = mbt.qknorm_rope(q, k, w, w, cs, pos, 64)
    torch.cuda.synchronize()
    assert qo.shape == q.shape and ko.shape == k.shape


def test_norm_and_act_refusals(mbt):
    x, r = z(8, 256), z(8, 256)
    with pytest.raises(ValueError):
        mbt.fused_add_rmsnorm(x, z(8, 128), z(256))
    with pytest.raises(ValueError):
        mbt.fused_add_rmsnorm(x, r, z(255))
    with pytest.raises(ValueError):
        mbt.fused_add_rmsnorm_fp8(x, r, z(256), 1.0, y=z(8, 128, dtype=torch.uint8))
    with pytest.raises(TypeError):
        mbt.fused_add_rmsnorm_fp8(x, r, z(256), 1.0, y=z(8, 256))
    with pytest.raises(ValueError):
        mbt.adarms(x, r, z(256), z(256), z(128))
    gu = z(4, 64)
    with pytest.raises(ValueError):
        mbt.gated_act(z(4, 63))
    with pytest.raises(ValueError):
        mbt.gated_act(gu, out=z(4, 31))
    with pytest.raises(ValueError):
        mbt.gated_act_fp8(gu, 1.0, out=z(4, 16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        mbt.quantize_fp8(torch.zeros(16, device=DEV), 1.0, y=z(8, dtype=torch.uint8))
    # still healthy
    y = mbt.fused_add_rmsnorm_fp8(x, r, z(256), 1.0)
    torch.cuda.synchronize()
    assert y.shape == x.shape
