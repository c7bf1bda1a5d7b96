"""The streaming bandwidth probe (``kda_stream_probe``) that bench.py's
ceilings come from: each mode moves exactly the bytes it says; and the
matrix-core issue probe (``kda_mfma_probe``) beside it."""
import pytest
import torch

from kda_testlib import announce
import linear_attention_prefill_amd as lap

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("n,grid", [(1 << 20, 1024), (4096 + 4 * 37, 3), (4, 1)])
def test_stream_probe_modes(n, grid):
    """n fp32 values (a multiple of 4: 16-byte units), including a tail past
    the unrolled loop and a grid larger than the data."""
    K = lap.kda
    announce("stream probe n=%d grid=%d" % (n, grid))
    g = torch.Generator(device="cpu").manual_seed(n)
    src = torch.randn(n, generator=g).cuda()
    keep = src.clone()
    dst = torch.full((n,), 3.0, device="cuda")
    K.stream_probe(K.KDA_STREAM_COPY, src, dst, grid)
    torch.cuda.synchronize()
    assert torch.equal(dst, src) and torch.equal(src, keep)
    K.stream_probe(K.KDA_STREAM_UPDATE, None, dst, grid)
    torch.cuda.synchronize()
    assert torch.equal(dst, keep * torch.tensor(1.0001, device="cuda"))
    sink = torch.zeros(4 * grid, dtype=torch.uint8, device="cuda")
    K.stream_probe(K.KDA_STREAM_READ, src, sink, grid)
    torch.cuda.synchronize()
    assert torch.equal(src, keep)


def test_mfma_probe_rates():
    """The matrix-core issue probe: eight independent accumulators reach the
    bf16 16x16x32 product's throughput (16 clocks at the published 2.5
    PFLOP/s dense peak, 256 CUs, 2.4 GHz), one accumulator is bound by its
    dependent latency, and the clock ratio gives a plausible core clock."""
    K = lap.kda
    announce("mfma probe chains 1, 2, 4, 8")
    r = {c: K.mfma_probe(c, 2048) for c in (1, 2, 4, 8)}
    for c, x in r.items():
        announce("  chains %d: %.1f core clocks a product at %.0f MHz" % (c, x["clocks_per_product"],
                                                                        x["core_MHz"]))
        assert 500 < x["core_MHz"] < 3500
    assert 15.0 <= r[8]["clocks_per_product"] <= 24.0
    assert r[1]["clocks_per_product"] > r[2]["clocks_per_product"] >= r[8]["clocks_per_product"]
    assert r[4]["clocks_per_product"] <= r[2]["clocks_per_product"]
