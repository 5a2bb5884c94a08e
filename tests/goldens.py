"""Reader for the worked-example fixtures under tests/golden/ (plain text, one key per line;
a `rule:` line opens a new expected-output section)."""
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    head, sections, cur = {}, [], None
    with open(os.path.join(GOLDEN_DIR, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split(":", 1))
            if key == "rule":
                cur = {"rule": val}
                sections.append(cur)
            elif cur is None:
                head[key] = val
            else:
                cur[key] = val
    d = int(head["d"])
    out = {
        "d": d,
        "rows_per_group": int(head["rows_per_group"]),
        "x": np.array([int(t, 16) for t in head["x_bf16"].split()], dtype=np.uint16).reshape(-1, d),
        "amax": float(head["amax"]),
        "cases": [],
    }
    for s in sections:
        out["cases"].append({
            "rule": s["rule"],
            "scales": np.array([int(t, 16) for t in s["scales"].split()], dtype=np.uint8),
            "codes": np.array([int(t, 16) for t in s["codes"].split()], dtype=np.uint8),
            "dequant": np.array([int(t, 16) for t in s["dequant_bf16"].split()], dtype=np.uint16),
            # optional: the float32 dequant output as binary32 bit patterns
            "dequant_f32": (np.array([int(t, 16) for t in s["dequant_f32"].split()],
                                     dtype=np.uint32) if "dequant_f32" in s else None),
        })
    return out


ALL = ["w1_grid_roundtrip.txt", "w2_four_over_six.txt", "w3_outlier.txt", "w4_exact_tie.txt",
       "w5_midpoint_ties.txt"]
