"""Record SHA-256 of the generated bf16 tensors (with stored repairs) in synth/hashes.json.

The hashes pin the generator's output across machines with this image: a
regenerated tensor must hash the same.  Large workloads are hashed per head
for heads 0 and H-1 only, to keep the check cheap.

Run:  python -m synth.record_hashes
"""

import hashlib
import json
import os

from .configs import CONFIGS
from .generate import generate, generate_head, load_repairs

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hashes.json")
FULL = ("tiny", "short_video", "wan1p3b")


def digest(arr):
    return hashlib.sha256(arr.tobytes()).hexdigest()


def compute(names=None):
    out = {}
    seen = set()
    for name, spec in CONFIGS.items():
        if names and name not in names:
            continue
        if spec.cfg_id in seen:
            continue
        seen.add(spec.cfg_id)
        if name in FULL:
            data = generate(spec)
            out[name] = {t: digest(a) for t, a in data.items()}
        else:
            rep = load_repairs(spec.cfg_id)
            for h in (0, spec.H - 1):
                part = generate_head(spec, 0, h, repairs=rep)
                out[f"{name}/head{h}"] = {t: digest(a) for t, a in part.items()}
    return out


if __name__ == "__main__":
    with open(PATH, "w") as f:
        json.dump(compute(), f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", PATH)
