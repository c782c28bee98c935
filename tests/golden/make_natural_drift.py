"""Writes tests/golden/natural_drift.json: for the large named workloads, how
far valid fp32 summation orders (tests/_natural.py) drift from the oracle's
free-running chain (1 - cosine of Z), on the rows the full-size parity tests
evaluate.  Uses only the oracle, the seeded input generator and numpy; the
parity tests read the record instead of re-running these chains.

    python tests/golden/make_natural_drift.py [config index ...]   (default 3 4 5)
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from realtime_transformer_amd import datagen  # noqa: E402
from realtime_transformer_amd.configs import CONFIGS  # noqa: E402
import _natural  # noqa: E402
from _samples import rows_for  # noqa: E402

OUT = os.path.join(HERE, "natural_drift.json")


def run(ci):
    cfg = CONFIGS[ci]
    rows, cal_rows = rows_for(ci)
    t0 = time.time()
    r0, y0 = datagen.eval_inputs(cfg)
    cal = datagen.calib_batches(cfg, 4)
    sel = np.arange(cfg.M) if rows is None else np.asarray(rows)
    if cal_rows is not None:
        cr = np.asarray(cal_rows)
        cal = [(r[cr], None if y is None else y[cr]) for r, y in cal]
    nat = _natural.NaturalChains(r0[sel], None if y0 is None else y0[sel])

    def provider(l):
        return lambda: oracle.LayerWeights.quantize(*datagen.layer_weights(cfg, l))

    def post(li, lw, s_x, s_h):
        nat.step(lw, cfg.act, cfg.eps, s_x, s_h)
        print("[%s] layer %d (%.0fs)" % (cfg.name, li, time.time() - t0), flush=True)

    res = oracle.calibrate_and_run((provider(l) for l in range(cfg.L)), cfg.act, cfg.eps, r0[sel],
                                   None if y0 is None else y0[sel], cal, post_layer=post)
    d = nat.distances(oracle.final_hidden(res.r[-1], res.y[-1]))
    return {"shape": [cfg.M, cfg.H, cfg.I, cfg.L], "rows": rows, "cal_rows": cal_rows, "distances": d}


def main():
    which = [int(a) for a in sys.argv[1:]] or [3, 4, 5]
    rec = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for ci in which:
        rec[CONFIGS[ci].name] = run(ci)
        print(CONFIGS[ci].name, rec[CONFIGS[ci].name]["distances"], flush=True)
        with open(OUT, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
