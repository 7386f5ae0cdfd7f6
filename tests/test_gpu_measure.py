"""The streaming-read reference kernel behind the achievable-bandwidth figure:
it accepts any 16-byte multiple (ragged slices included), rejects the rest on
the host, and leaves the caller's buffer and the device status untouched."""
import pytest
import torch

from attention_perturbation_scoring_amd import dropkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = dropkv.Context(0)
    yield c
    c.close()


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (8 << 20), (8 << 20) + 16 * 777])
def test_stream_read_runs_and_writes_nothing(ctx, nbytes):
    print(f"[case] stream_read {nbytes} bytes", flush=True)
    buf = torch.randint(-2**15, 2**15, (nbytes // 2,), dtype=torch.int16, device="cuda")
    ref = buf.clone()
    ctx.stream_read(buf)
    assert ctx.sync() == dropkv.OK
    assert torch.equal(buf, ref)


def test_stream_read_rejects_bad_sizes(ctx):
    buf = torch.zeros(64, dtype=torch.int16, device="cuda")
    for nbytes in (0, -16, 24):
        with pytest.raises(dropkv.DropKVError) as e:
            ctx.stream_read(buf, nbytes)
        assert e.value.code == dropkv.EINVAL
    with pytest.raises(dropkv.DropKVError):
        ctx.stream_read(buf.data_ptr() + 8, 32)   # misaligned
