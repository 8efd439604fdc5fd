"""bench.py's timing-only HIP events (TimingEvent): recorded on torch's
current stream, they bracket the work launched between them, on the
default stream and on a side stream, and agree with torch's own events
to within their latency."""
import pytest
import torch

import bench

pytestmark = pytest.mark.gpu

from gpu_helpers import say


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_topk_ids_amd.moe as m
    return m


@pytest.mark.parametrize("side_stream", [False, True])
def test_timing_event_brackets_work(moe, side_stream):
    say(f"[bench timing] side_stream={side_stream}")
    a = torch.ones(64 << 20, dtype=torch.bfloat16, device="cuda")  # 128 MiB
    b = torch.empty_like(a)
    stream = torch.cuda.Stream() if side_stream else torch.cuda.current_stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.neg(a, out=b)  # warm
        t0, t1 = bench.TimingEvent(moe, torch), bench.TimingEvent(moe, torch)
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record()
        t0.record()
        for _ in range(4):
            torch.neg(a, out=b)
        t1.record()
        r1.record()
    torch.cuda.synchronize()
    ms, ref = t0.elapsed_time(t1), r0.elapsed_time(r1)
    say(f"[bench timing] timing-only events {ms * 1e3:.1f} us, torch events {ref * 1e3:.1f} us")
    # 4 x 256 MiB of traffic takes well over 50 us at any HBM rate, and the
    # inner interval cannot be longer than the outer one
    assert 0.05 < ms <= ref + 0.002
    assert torch.equal(b[:1024], -a[:1024])
