"""The device half of the input generator reproduces the host definition
(same counters, same double-precision formula, same rounding)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

from synth import device, gen  # noqa: E402


@pytest.mark.parametrize("w", [gen.tiny_f32_1k(),
                               gen.scaled(gen.llama8b_128k(needles=16), 8192)],
                         ids=["f32", "bf16"])
def test_device_fill_matches_host(w):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[case] synth {w.name} {w.kv_dtype} L={w.L_cap}", flush=True)
    q, k, v = gen.layer_inputs(w, 0)
    qd, kd, vd = device.layer_to_device(w, 0)
    torch.cuda.synchronize()
    assert np.array_equal(qd.cpu().numpy(), q)
    for host, dev in ((k, kd), (v, vd)):
        if w.kv_dtype == "bf16":
            got = dev.view(torch.int16).cpu().numpy().view(np.uint16)
            a = host.astype(np.int32)
            b = got.astype(np.int32)
        else:
            got = dev.cpu().numpy()
            a = host.view(np.int32).astype(np.int64)
            b = got.view(np.int32).astype(np.int64)
        diff = np.abs(a - b)
        # identical except, at most, a rare last-place difference where the
        # double values straddle a rounding boundary
        assert diff.max() <= 1
        assert (diff > 0).mean() <= 1e-6
