"""The layer forward captured in a HIP graph (torch.cuda.graph over the
C-ABI call on the capturing stream) and replayed: the layer issues kernels
only -- no memset, no allocation, no host synchronisation -- so a replay
equals an eager call bit for bit.  Each graph is replayed several times,
with eager work and synchronisations in between, and every replay is
checked against the eager result."""
import pytest
import torch

import mixture_experts_layer_group_amd as moe
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

C = synth.LayerConfig
CASES = [synth.CONFIGS[5],
         C("graph-bf16-capacity", 150, T=300, d=256, E=8, top_k=2, F=384, capacity_factor=1.25),
         # enough tiles (256 gate/up, 128 split down units) that the last
         # quarter of every XCD range is claimed at run time: each replay
         # must find the claim counters zeroed by the dispatch it replays
         C("graph-bf16-claims", 152, T=4096, d=512, E=8, top_k=2, F=1024),
         C("graph-sigmoid-shared", 151, T=130, d=256, E=16, top_k=4, F=128,
           router=synth.SIGMOID_GROUP, routed_scaling=2.5, n_group=4, topk_group=2,
           shared_experts=1, shared_F=128, router_dtype=synth.BF16, bias_range=0.05)]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
@pytest.mark.parametrize("static", [False, True], ids=["workspace", "static"])
def test_graph_replay_equals_eager(cfg, static):
    gu.log(f"[graph] {cfg.name} ({'static scratch' if static else 'workspace'})")
    inp = gu.make_inputs(cfg)
    spec = moe.spec_from_config(cfg)
    T, k = cfg.T, cfg.top_k
    ws = moe.workspace(spec, T)
    out = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    st = moe.layer_stats(topk_ids=ids)

    def call():
        if static:
            moe.moe_layer_forward_static(spec, T, inp["x"], inp["w_router"], inp["expert_bias"],
                                         inp, out, stats=st)
        else:
            moe.moe_layer_forward(spec, T, inp["x"], inp["w_router"], inp["expert_bias"], inp,
                                  out, stats=st, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref_out, ref_ids = out.clone(), ids.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        ids.fill_(-1)
        scratch = torch.randn(1 << 20, device="cuda")  # eager work between replays
        scratch.mul_(2.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: output differs"
        assert torch.equal(ids, ref_ids), f"replay {rep}: routing differs"
    gu.log("  3 replays bit-identical to the eager call")
