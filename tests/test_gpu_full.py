"""GPU parity at the five workload configurations at full size, in the launch
configuration the benchmark times (one moe_layer_forward call).  Routing and
dispatch are checked in full (logits bound, ids, counts, permutation, drops);
the expert FFN + combine output is checked on seeded samples of tokens that
the oracle evaluates one by one (their count is printed), because the fp64
oracle would take minutes on every token of the large layers."""
import numpy as np
import pytest

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SAMPLES = {1: None, 2: 16, 3: 4, 4: 48, 5: None}


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_full_size_config(cfg_id):
    cfg = synth.CONFIGS[cfg_id]
    gu.log(f"[full size] config {cfg_id} {cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E} "
           f"k={cfg.top_k} F={cfg.F}")
    inp = gu.make_inputs(cfg)
    r = gu.run_layer(cfg, inp)
    n = SAMPLES[cfg_id]
    toks = None
    if n is not None:
        rs = np.random.default_rng(cfg_id)
        toks = sorted(rs.choice(cfg.T, size=n, replace=False).tolist())
    ids_g, disp = gu.full_check(cfg, inp, r, tokens=toks)
    gu.check_end_to_end_routing(cfg, inp, ids_g, r["logits"].cpu().numpy())
    if cfg.capacity_factor:
        kept = disp["kept"]
        gu.log(f"  load: max count_pre {int(disp['count_pre'].max())}, capacity "
               f"{cfg.T * cfg.top_k // cfg.E}, dropped fraction "
               f"{disp['dropped'] / (cfg.T * cfg.top_k):.3f}, experts at capacity "
               f"{int((kept == kept.max()).sum())}")
