"""GPU parity of the fused gate/up weight layout: the layer reading each
expert's gate and up rows from one fused tensor equals the layer over the
separate tensors bit for bit (same kernels, same arithmetic, other
addresses) and matches the oracle reading the fused tensor itself, for
bf16 (routed + shared, split-K down projection), 4-bit (weight-stream and
tiled kernels) and fp32 weights.
"""
import pytest
import torch

import synth
from tests import gpu_util as gu
from tests.test_gpu_stages import MEDIUM

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["sigmoid-group-shared", "swiglu-bf16-splitk",
                                  "swiglu-bf16-ragged", "u4-decode", "u4-small-k",
                                  "u4-tiled-swiglu-shared", "f32-swiglu-shared"])
def test_fused_gate_up_layer(name):
    cfg = MEDIUM[name]
    fcfg = cfg.replace(layout=synth.FUSED_GATE_UP)
    gu.log(f"[fused gate/up] {name}: T={cfg.T} d={cfg.d} E={cfg.E} F={cfg.F}")
    sep = gu.run_layer(cfg, gu.make_inputs(cfg))
    inp = gu.make_inputs(fcfg)
    assert inp.get("w_up") is None and inp.get("q_up") is None
    fus = gu.run_layer(fcfg, inp)
    for key in ("out", "topk_ids", "topk_w", "slot_row", "offsets"):
        assert torch.equal(sep[key], fus[key]), key
    gu.full_check(fcfg, inp, fus)
