"""Small text fixtures with the pages' own numbers, each file citing its source."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def accuracy_tables():
    """{(kind, case): [output, state_grad, grad_gate-kernel, grad_wi_0, grad_wi_1, grad_wo]}"""
    out = {}
    with open(os.path.join(HERE, "accuracy_tables_tokamax_gmm_v2.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, case, *vals = line.split()
            out[(kind, case)] = [float(v) for v in vals]
    return out
