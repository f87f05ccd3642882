"""Write tests/golden/oracle_values.json: oracle results for the inputs that
are too slow to recompute inside every GPU test run.  Calls only the oracle
(and the seeded input generators); run it on the CPU:

    python tests/golden/make_golden.py
"""

import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from workloads import circuits, lattice, trees  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_values.json")


def main():
    vals = json.load(open(OUT)) if os.path.exists(OUT) else {}
    t = time.time()
    c = circuits.brickwork(30, 14, 303)
    net = c.to_network(open_qubits=range(6))
    tree = trees.greedy_tree(net)
    batch = oracle.contract_network(net, tree).reshape(-1)
    vals["brickwork30x14_seed303"] = dict(
        what="<x|U|0> for x = (q0..q5 free, q6..q29 = 0), 30-qubit brickwork depth 14, seed 303, greedy tree",
        batch_sha256=net.digest(), batch_re=batch.real.tolist(), batch_im=batch.imag.tolist(),
        oracle_seconds=time.time() - t)
    print("brickwork30 done", time.time() - t, flush=True)
    t = time.time()
    net = lattice.peps(8, 8, 404)
    z = complex(oracle.contract_network(net, lattice.row_major_tree(8)))
    vals["peps8x8_D8_seed404"] = dict(
        what="Z of the 8x8 D=8 lattice, seed 404, row-major caterpillar tree",
        input_sha256=net.digest(), re=z.real, im=z.imag, oracle_seconds=time.time() - t,
        oracle_threads=oracle.max_threads())
    print("peps done", time.time() - t, z, flush=True)
    json.dump(vals, open(OUT, "w"), indent=1)


if __name__ == "__main__":
    main()
