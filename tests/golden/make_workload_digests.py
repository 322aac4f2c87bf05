"""Write workload_digests.json: the oracle's container for every named
workload, summarised by its exact escape count, codebook, size and SHA-256
(plus the SHA-256 of the input, to notice generator drift).

Calls only the CPU oracle and the seeded input generators.  Run from the
repository root:  python tests/golden/make_workload_digests.py [names...]
The largest workload needs about 20 GB of host memory and a few minutes.
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import kvgen  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_digests.json")


def sha256(a: np.ndarray) -> str:
    h = hashlib.sha256()
    mv = memoryview(np.ascontiguousarray(a).reshape(-1).view(np.uint8))
    step = 1 << 28
    for i in range(0, len(mv), step):
        h.update(mv[i:i + step])
    return h.hexdigest()


def main(names):
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    for name in names:
        w = kvgen.resolve(name)
        t0 = time.time()
        x = kvgen.generate(w.name)
        c = oracle.encode(x)
        e = int.from_bytes(c[16:24].tobytes(), "little")
        data[w.name] = {
            "n": int(x.size),
            "escapes": e,
            "container_bytes": int(c.size),
            "ratio": round(2 * x.size / c.size, 6),
            "codebook": [int(v) for v in c[160:176]],
            "seg_end": [int.from_bytes(c[32 + 8 * s:40 + 8 * s].tobytes(), "little")
                        for s in range(16)],
            "input_sha256": sha256(x),
            "container_sha256": sha256(c),
        }
        print(name, data[w.name]["escapes"], data[w.name]["ratio"],
              "%.1fs" % (time.time() - t0), flush=True)
        del x, c
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:] or list(kvgen.WORKLOADS))
