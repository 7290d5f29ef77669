"""Measurement probes through the C ABI on the GPU: they run, write only
their sink, and are deterministic.  (Their timings are bench.py's; nothing
here times them.)"""
import pytest
import torch

import diffusion_lm_speculative_amd as sd
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


def test_mfma_probe_runs_and_is_deterministic():
    for wgs, iters in ((1, 1), (256, 8), (300, 3)):
        print(f"mfma probe workgroups={wgs} iters={iters}", flush=True)
        sink = torch.full((wgs * 256 + 64,), -7.0, dtype=torch.float32, device=dev())
        sd.mfma_probe(wgs, iters, sink)
        first = sink.clone()
        sd.mfma_probe(wgs, iters, sink)
        torch.cuda.synchronize()
        assert torch.equal(first, sink)
        assert torch.isfinite(sink).all()
        assert (sink[wgs * 256:] == -7.0).all()  # nothing past the workgroups' lanes
        assert (sink[: wgs * 256] > 0).all()      # every lane stored its (positive) accumulator sum


def test_stream_and_read_probes_touch_nothing_but_run():
    k = torch.randn(2, 8, 256, 128, device=dev()).to(torch.bfloat16)
    v = torch.randn_like(k)
    k0, v0 = k.clone(), v.clone()
    sink = torch.zeros(1, dtype=torch.int32, device=dev())
    sd.stream_probe(k, v, sink)
    sd.read_probe(k, v, sink)
    torch.cuda.synchronize()
    assert torch.equal(k, k0) and torch.equal(v, v0)
