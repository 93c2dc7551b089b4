"""moe_layer_forward_static (the no-allocation entry point, on the library's
static scratch array) against moe_layer_forward on a caller workspace: the
same kernels on the same inputs, so every output is compared bit for bit --
twice in a row on each workload, the second call with fewer tokens, so the
second call runs on the array the first one left behind.  A layer whose
workspace exceeds the array is rejected before any launch."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_group_amd as moe
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
CASES = [
    # the decode-shaped 4-bit layer (the workload such callers serve), then 8 tokens
    (synth.CONFIGS[5], 8),
    # bf16 grouped GEMMs with capacity drops, then a smaller batch
    (C("static-bf16", 140, T=300, d=256, E=8, top_k=2, F=384, capacity_factor=1.25), 77),
    # sigmoid-group routing with a shared expert, then a smaller batch
    (C("static-sigmoid-shared", 141, T=130, d=256, E=16, top_k=4, F=128,
       router=synth.SIGMOID_GROUP, routed_scaling=2.5, n_group=4, topk_group=2,
       shared_experts=1, shared_F=128, router_dtype=synth.BF16, bias_range=0.05), 33),
]


def _outputs(cfg, T):
    dev = "cuda"
    E, k = cfg.E, cfg.top_k
    return {"out": torch.full((T, cfg.d), float("nan"), dtype=torch.float32, device=dev),
            "topk_ids": torch.full((T, k), -7, dtype=torch.int32, device=dev),
            "topk_w": torch.zeros((T, k), dtype=torch.float32, device=dev),
            "offsets": torch.zeros(E + 1, dtype=torch.int32, device=dev),
            "slot_row": torch.full((T, k), -7, dtype=torch.int32, device=dev),
            "errors": torch.zeros(1, dtype=torch.int32, device=dev)}


def _run(cfg, inp, T, static):
    spec = moe.spec_from_config(cfg)
    r = _outputs(cfg, T)
    st = moe.layer_stats(**{n: r[n] for n in ("topk_ids", "topk_w", "offsets", "slot_row",
                                               "errors")})
    x = inp["x"][:T]
    if static:
        moe.moe_layer_forward_static(spec, T, x, inp["w_router"], inp["expert_bias"], inp,
                                     r["out"], stats=st)
    else:
        moe.moe_layer_forward(spec, T, x, inp["w_router"], inp["expert_bias"], inp, r["out"],
                              stats=st, workspace=moe.workspace(spec, T))
    return r


@pytest.mark.parametrize("cfg,T2", CASES, ids=[c.name for c, _ in CASES])
def test_static_entry_matches_workspace_entry(cfg, T2):
    gu.log(f"[no-alloc] {cfg.name}: T={cfg.T} then T={T2}")
    spec = moe.spec_from_config(cfg)
    assert moe.moe_workspace_size(spec, cfg.T) <= moe.STATIC_SCRATCH_BYTES
    inp = gu.make_inputs(cfg)
    inp2 = gu.make_inputs(cfg, base=synth.SEED_BASE + 7)
    runs = []
    for i, (data, T) in enumerate(((inp, cfg.T), (inp2, T2))):
        a = _run(cfg, data, T, static=True)
        b = _run(cfg, data, T, static=False)
        torch.cuda.synchronize()
        for n in a:
            assert torch.equal(a[n], b[n]), f"call {i + 1} (T={T}): {n} differs"
        assert not torch.isnan(a["out"]).any()
        assert int(a["errors"].item()) == 0
        runs.append(a)
    gu.log(f"  both calls bit-identical to moe_layer_forward (kept rows "
           f"{int(runs[0]['offsets'][-1])} then {int(runs[1]['offsets'][-1])})")


def test_static_entry_rejects_layers_beyond_the_array():
    cfg = synth.CONFIGS[2]
    spec = moe.spec_from_config(cfg)
    assert moe.moe_workspace_size(spec, cfg.T) > moe.STATIC_SCRATCH_BYTES
    inp = synth.make_layer_inputs(cfg, "cuda", with_weights=False)
    dummy = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    w = {"w_gate": dummy, "w_up": dummy, "w_down": dummy}
    out = torch.full((cfg.T, cfg.d), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoEError) as e:
        moe.moe_layer_forward_static(spec, cfg.T, inp["x"], inp["w_router"], None, w, out)
    assert e.value.status == 5  # MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)  # nothing was launched
