"""GPU parity at the five workload configurations at full size, in the launch
configuration the benchmark times (one moe_layer_forward call).  Routing and
dispatch are checked in full (logits bound, ids, counts, permutation, drops);
the expert FFN + combine output is checked on a sample of tokens that the
oracle evaluates one by one (their count is printed): the tokens of the last
M tile of every expert's group (the ragged tails), topped up with seeded
random tokens, because the fp64 oracle would take minutes on every token of
the large layers."""
import numpy as np
import pytest

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# output sample size per config (None: every token); tokens of each
# expert's last tile first (per_expert of them), random ones after
SAMPLES = {1: None, 2: (256, 8), 3: (512, 1), 4: (256, 1), 5: None}


def sample_tokens(cfg, n, per_expert):
    def choose(disp):
        toks = set(gu.last_tile_tokens(disp, per_expert))
        rs = np.random.default_rng(cfg.cfg_id)
        for t in rs.permutation(cfg.T):
            if len(toks) >= n:
                break
            toks.add(int(t))
        toks = sorted(toks)
        gu.log(f"  output sample: {len(toks)} tokens ({len(gu.last_tile_tokens(disp, per_expert))} "
               f"from the experts' last M tiles)")
        return toks
    return choose


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_full_size_config(cfg_id):
    cfg = synth.CONFIGS[cfg_id]
    gu.log(f"[full size] config {cfg_id} {cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} "
           f"k={cfg.top_k} F={cfg.F}")
    inp = gu.make_inputs(cfg)
    r = gu.run_layer(cfg, inp)
    choose = None
    if SAMPLES[cfg_id] is not None:
        choose = sample_tokens(cfg, *SAMPLES[cfg_id])
    ids_g, disp = gu.full_check(cfg, inp, r, choose_tokens=choose)
    gu.check_end_to_end_routing(cfg, inp, ids_g, r["logits"].cpu().numpy())
    if cfg.capacity_factor:
        kept = disp["kept"]
        gu.log(f"  load: max count_pre {int(disp['count_pre'].max())}, capacity "
               f"{cfg.T * cfg.top_k // cfg.E}, dropped fraction "
               f"{disp['dropped'] / (cfg.T * cfg.top_k):.3f}, experts at capacity "
               f"{int((kept == kept.max()).sum())}")
