"""The streaming-read probe (the read-ceiling kernel of the benchmark) on the
GPU: it runs over sizes with a ragged grid tail and writes nothing for data
whose xor cannot hit its marker (needs an MI355X)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the -m gpu tests need an MI355X")


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 24) + 48])
@pytest.mark.parametrize("nt", [True, False])
def test_read_probe_reads_and_writes_nothing(nbytes, nt):
    import split_kv_decode_amd as mx
    dev = torch.device("cuda:0")
    src = torch.zeros(nbytes, dtype=torch.uint8, device=dev)   # xor of zeros is 0
    sink = torch.full((4,), 7, dtype=torch.int32, device=dev)
    mx.read_probe(src, nt, sink)
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]
