"""Host-side checks of the chained decode step's scheduling
(attention_level_speculation_amd.runtime), with the library calls replaced
by recorders: no GPU work is enqueued.

- The two-stream speculative form refuses to run while either of its
  streams is capturing into a HIP graph, before it enqueues anything (its
  capture crashed the HIP runtime inside hipStreamEndCapture).
- Outside a capture, and in the one-stream form under a capture, it issues
  the calls of its documented order.
"""
import types

import pytest

import attention_level_speculation_amd as al
from attention_level_speculation_amd import _binding as B_
from attention_level_speculation_amd import runtime as rt


class _Tensor:
    """Stands in for the device tensors the runtime only slices and passes
    on."""

    def __init__(self, name):
        self.name = name

    def view(self, *shape):
        return self

    def __getitem__(self, idx):
        return self


@pytest.fixture
def recorder(monkeypatch):
    calls = []

    def rec(name):
        def f(*a, **k):
            calls.append(name)
        return f
    for name in ("spec_decode", "sink_approx", "flash_decode_exact",
                 "lse_combine", "verify", "post_attention"):
        monkeypatch.setattr(B_, name, rec(name))
    return calls


def _step_args(n_layers=2):
    p = al.make_params(1, 8, 2, 64, 100, [100], "bf16", 4, 16, 0.1)
    pp = al.make_post_params(1, 8 * 64, 64, 128, 12 * 64)
    out = {k: _Tensor(k) for k in ("o_approx", "lse_approx", "o_exact",
                                   "lse_exact", "ratio", "commit",
                                   "o_committed")}
    layers = [rt.ModelLayer(_Tensor("k"), _Tensor("v"), None, out,
                            _Tensor("h_in"), _Tensor("h_out"),
                            _Tensor("qkv")) for _ in range(n_layers)]
    ws = (_Tensor("ws"), _Tensor("wa"), _Tensor("wb"))
    sa = types.SimpleNamespace(name="sa", waits=[])
    se = types.SimpleNamespace(name="se", waits=[])
    se.wait_stream = lambda other: se.waits.append(other.name)
    sa.wait_stream = lambda other: sa.waits.append(other.name)
    return p, pp, layers, ws, sa, se


@pytest.mark.parametrize("capturing", ["sa", "se", "both"])
def test_two_stream_step_refused_under_capture(monkeypatch, recorder,
                                               capturing):
    p, pp, layers, ws, sa, se = _step_args()
    monkeypatch.setattr(
        B_, "stream_is_capturing",
        lambda s: capturing == "both" or s.name == capturing)
    monkeypatch.setattr(rt, "q_view", lambda p_, qkv: qkv)
    with pytest.raises(ValueError, match="not captured"):
        rt.model_step(None, p, pp, _Tensor("q0"), layers, *ws, sa, se,
                      speculative=True)
    assert recorder == [] and se.waits == [] and sa.waits == []


def test_two_stream_step_runs_eagerly(monkeypatch, recorder):
    p, pp, layers, ws, sa, se = _step_args()
    monkeypatch.setattr(B_, "stream_is_capturing", lambda s: False)
    monkeypatch.setattr(rt, "q_view", lambda p_, qkv: qkv)
    rt.model_step(None, p, pp, _Tensor("q0"), layers, *ws, sa, se,
                  speculative=True)
    per_layer = ["spec_decode", "post_attention", "post_attention"]
    assert recorder == per_layer * 2
    assert se.waits == ["sa", "sa"]


def test_one_stream_step_allowed_under_capture(monkeypatch, recorder):
    p, pp, layers, ws, sa, se = _step_args()
    monkeypatch.setattr(B_, "stream_is_capturing", lambda s: True)
    monkeypatch.setattr(rt, "q_view", lambda p_, qkv: qkv)
    rt.model_step(None, p, pp, _Tensor("q0"), layers, *ws, sa, se,
                  speculative=True, one_stream=True)
    per_layer = ["sink_approx", "post_attention", "flash_decode_exact",
                 "lse_combine", "verify", "post_attention"]
    assert recorder == per_layer * 2
    assert se.waits == [] and sa.waits == []
