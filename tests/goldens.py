"""Reader for the hand-derived fixtures in tests/golden (plain text)."""
import os
from typing import Dict, List, Tuple

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def parse_layout(text: str) -> Tuple[tuple, ...]:
    """'T2 I1x2x2' -> (("T", 2), ("I", 1, 2, 2))."""
    segs = []
    for tok in text.split():
        if tok[0] == "T":
            segs.append(("T", int(tok[1:])))
        elif tok[0] == "I":
            f, h, w = (int(v) for v in tok[1:].split("x"))
            segs.append(("I", f, h, w))
        else:
            raise ValueError(tok)
    return tuple(segs)


def load(name: str) -> Dict[str, object]:
    fields: Dict[str, str] = {}
    with open(os.path.join(GOLDEN_DIR, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    out: Dict[str, object] = {"layout": parse_layout(fields["layout"]), "pos_mode": fields["pos_mode"]}
    for key in ("image_ids", "target_mask", "kv_limit"):
        out[key] = np.asarray([int(v) for v in fields[key].split()], dtype=np.int64)
    out["pos_ids"] = np.asarray([[int(c) for c in t.split(",")] for t in fields["pos_ids"].split()],
                                dtype=np.int64)
    return out


def metadata_fixtures() -> List[str]:
    return sorted(f for f in os.listdir(GOLDEN_DIR) if f.startswith("metadata_") and f.endswith(".txt"))
