"""GPU: the streaming HBM probe copies bit for bit and reads without writing."""

import pytest

pytestmark = pytest.mark.gpu

tw = pytest.importorskip("activation_sparse_transformer_bf16_amd")


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 << 20, 64 << 20])
def test_stream_probe_copy_and_read(nbytes):
    import torch
    print(f"stream probe {nbytes} bytes", flush=True)
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda:0", generator=g)
    dst = torch.zeros_like(src)
    tw.twell_stream_probe(src, dst, 1)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda:0")
    tw.twell_stream_probe(src, sink, 0)
    torch.cuda.synchronize()
    # the XOR of random bytes equals the sentinel with probability 2^-32
    assert int(sink.item()) in (7, 0x9E3779B9 - (1 << 32))


def test_mfma_probe_runs_and_writes_nothing():
    import torch
    sink = torch.full((1,), 5.0, dtype=torch.float32, device="cuda:0")
    flops = tw.twell_mfma_probe(sink, 10, 8)
    torch.cuda.synchronize()
    assert flops == 2.0 * 32 * 32 * 16 * 8 * 10 * 8 * 8
    assert float(sink.item()) == 5.0
