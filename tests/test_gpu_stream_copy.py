"""The calibration copy (mbt_stream_copy) on the GPU: dst equals src byte for
byte at every chunks-per-lane value, on sizes that fill whole blocks and on
ragged tails that end inside a block, inside a wave and at a single 16-byte
chunk; the guard bands on either side of dst keep their fill."""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of sentinel before and after dst
SENTINEL = 0xA5


@pytest.fixture(scope="module")
def mbt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_transformer_amd as m
    return m


def _bytes(n, seed):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda:0", generator=g)


def _check(mbt, nbytes, chunks, seed, src_offset=0, sync=False):
    print(f"stream_copy nbytes={nbytes} chunks={chunks} sync={sync} src_offset={src_offset}",
          flush=True)
    src_buf = _bytes(nbytes + src_offset, seed)
    src = src_buf[src_offset:src_offset + nbytes]
    buf = torch.full((GUARD + nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda:0")
    dst = buf[GUARD:GUARD + nbytes]
    mbt.stream_copy(src, dst, chunks, block_sync=sync)
    torch.cuda.synchronize()
    assert torch.equal(dst, src), f"copy differs at nbytes={nbytes} chunks={chunks}"
    assert bool((buf[:GUARD] == SENTINEL).all()), "bytes before dst written"
    assert bool((buf[GUARD + nbytes:] == SENTINEL).all()), "bytes after dst written"


@pytest.mark.parametrize("sync", [False, True])
@pytest.mark.parametrize("chunks", [1, 2, 4, 8])
@pytest.mark.parametrize("blocks,tail", [(0, 1), (0, 37), (1, 0), (3, 0), (3, 1), (5, 255),
                                         (7, 64 * 3 + 5)])
def test_stream_copy_sizes(mbt, chunks, blocks, tail, sync):
    # a block is 256 lanes x chunks x 16 bytes; `tail` more 16-byte chunks
    nbytes = (blocks * 256 * chunks + tail) * 16
    _check(mbt, nbytes, chunks, seed=1000 * chunks + 10 * blocks + tail, sync=sync)


@pytest.mark.parametrize("chunks,sync", [(1, False), (4, False), (8, True)])
def test_stream_copy_large(mbt, chunks, sync):
    # many blocks, the last one ragged: 64 MiB + 48 bytes
    _check(mbt, (64 << 20) + 48, chunks, seed=77 + chunks, sync=sync)


def test_stream_copy_unaligned_to_blocks(mbt):
    # src 16 bytes past a 256-byte boundary: only 16-byte alignment is needed
    _check(mbt, 1 << 20, 2, seed=5, src_offset=16)


def test_stream_copy_empty_and_rejects(mbt):
    a = torch.zeros(64, dtype=torch.uint8, device="cuda:0")
    mbt.stream_copy(a[:0], a[:0], 4)              # nbytes 0: no-op
    mbt.stream_copy(a[:0], a[:0], 8, block_sync=True)
    with pytest.raises(mbt.MbtError):
        mbt.stream_copy(a[:48], a[16:64], 1)       # overlap
    with pytest.raises(mbt.MbtError):
        mbt.stream_copy(a[8:24], a[32:48], 1)      # src 8 bytes past alignment
    with pytest.raises(ValueError):
        mbt.stream_copy(a[:32], a[32:48], 1)       # byte counts differ
