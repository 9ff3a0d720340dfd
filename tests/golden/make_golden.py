"""Write oracle_w0_sample.json: a sample of the fp64 oracle's outputs on the
tiny fp32 workload.  Calls only the oracle and the seeded input generator."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import kda_inputs  # noqa: E402
import oracle  # noqa: E402


def main():
    spec, cu, x = kda_inputs.workload(0)
    o, sf = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, eps=1e-6)
    idx = list(range(0, o.size, 997))
    out = {
        "workload": spec["name"],
        "eps": 1e-6,
        "o_flat_index": idx,
        "o_values": [float(o.reshape(-1)[i]) for i in idx],
        "final_state_sum": float(sf.sum()),
        "final_state_abs_sum": float(np.abs(sf).sum()),
        "o_abs_sum": float(np.abs(o).sum()),
    }
    with open(os.path.join(HERE, "oracle_w0_sample.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
