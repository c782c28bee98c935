"""Row samples the full-size parity tests evaluate with the oracle (rows are
independent under static per-tensor scales, so a sample is exact for its
rows).  Shared by the tests and the script that stores the natural drift of
valid summation orders (tests/golden/make_natural_drift.py)."""
import numpy as np


def vlm_prefix_rows():
    """M=788: all 20 text-like rows and 44 image-like rows; 16 calibration rows."""
    rng = np.random.default_rng(31)
    rows = sorted(set(range(768, 788)) | set(rng.choice(768, 44, replace=False).tolist()))
    cal_rows = sorted(set(range(772, 780)) | set(rng.choice(768, 8, replace=False).tolist()))
    return rows, cal_rows


def dit_video_rows():
    """M=4096: 48 evaluated rows and 12 calibration rows."""
    rng = np.random.default_rng(53)
    rows = sorted(rng.choice(4096, 48, replace=False).tolist())
    cal_rows = sorted(rng.choice(4096, 12, replace=False).tolist())
    return rows, cal_rows


# config index -> (rows, cal_rows); None = all rows
SAMPLES = {3: vlm_prefix_rows, 5: dit_video_rows}


def rows_for(index):
    f = SAMPLES.get(index)
    return f() if f else (None, None)
