"""Writes tiny_verify_oracle.txt: the oracle's outputs on the tiny verify workload
(B=2, Hk=1, Hv=2, d=16, T=2, fp32 state, pool of 4, slots [2, 0], seed 0).

It calls only ``oracle`` and the seeded input generator. The file is a regression
fixture of the oracle (its correctness rests on the pins in test_oracle_pins.py);
rerun this script only with a commit that names the reason for the change.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def compute():
    w = workloads.WORKLOADS[0]
    x = workloads.make_inputs(w, seed=0)
    f = {n: x[n].double().numpy() for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "pool")}
    dims = oracle.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, False)
    r = oracle.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"],
                      f["pool"], x["idx"].numpy(), cache_T=w.T, write_final=True, nthreads=1)
    return r


def main():
    r = compute()
    path = os.path.join(HERE, "tiny_verify_oracle.txt")
    with open(path, "w") as fh:
        fh.write("# oracle outputs, tiny verify workload, seed 0 (written by make_golden.py)\n")
        fh.write("# o[b][t][h][j], row-major, then cache[b=0][t=1][h=1][i][j] row-major\n")
        fh.write("o = " + " ".join(repr(float(v)) for v in r["o"].ravel()) + "\n")
        fh.write("cache_0_1_1 = " + " ".join(repr(float(v)) for v in r["cache"][0, 1, 1].ravel()) + "\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
