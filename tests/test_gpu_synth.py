"""The device filler gives the host filler's bits (so the oracle, fed by the host
filler, sees exactly the inputs the GPU was given)."""
import numpy as np
import pytest

import synth
from moe_testlib import needs_gpu, to_host, torch

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
@pytest.mark.parametrize("first,count,tid,std", [
    (0, 1 << 20, 1, 1.0), (3, 12345, 4, 0.0118), (1 << 24, 99999, 6, 0.0221), (7, 1, 2, 0.5)])
def test_device_fill_matches_host(dtype, first, count, tid, std):
    ref = synth.fill_normal_host(count, first, 0, tid, std, dtype)
    t = torch.empty(count, dtype=torch.float32 if dtype == synth.F32 else torch.bfloat16,
                    device="cuda")
    rc = synth._load_dev().synth_dev_fill_normal(t.data_ptr(), dtype, count, first, 0, tid, std, 0)
    assert rc == 0
    torch.cuda.synchronize()
    got = to_host(t)
    assert np.array_equal(got, ref)


def test_workload_tensors_match_host():
    w = synth.WORKLOADS["dsv3_prefill"]
    for name in ("hidden", "w_router", "bias", "w2"):
        shape = w.shapes()[name]
        dt = torch.float32 if w.dtype_of(name) == synth.F32 else torch.bfloat16
        if name == "w2":
            t = torch.empty(shape[1:], dtype=dt, device="cuda")
            synth.fill_device(w, name, t.data_ptr(), expert=5)
            ref = synth.host_tensor(w, name, expert=5)
        else:
            t = torch.empty(shape, dtype=dt, device="cuda")
            synth.fill_device(w, name, t.data_ptr())
            ref = synth.host_tensor(w, name)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(t), ref), name
