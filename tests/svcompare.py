"""Comparison of GPU results with the oracle, decision by decision.

For every sequence the decisions are walked in order: the acceptance tests
0..k, then the final draw.  The first place where the GPU and the oracle part is
allowed only when the oracle's margin for that decision is below TOL (|u - p/q|
for a test, the distance of u*Z to the nearest CDF boundary over Z for the
draw); it is then counted as exempt and the rest of the sequence is skipped.
Any other difference is a hard mismatch.  Greedy sequences (T <= 0 or NaN) get
no exemption.
"""
from __future__ import annotations

import dataclasses

import numpy as np

TOL = 1e-5


@dataclasses.dataclass
class Report:
    sequences: int = 0
    decisions: int = 0
    near_ties: int = 0
    exempt: int = 0
    hard: int = 0
    first_hard: tuple | None = None

    def __str__(self):
        return (f"sequences={self.sequences} decisions={self.decisions} near_ties={self.near_ties} "
                f"exempt={self.exempt} hard={self.hard} first_hard={self.first_hard}")


def compare(gpu_acc, gpu_emi, ora, lens, temps, n, seqs=None, tol=TOL) -> Report:
    gpu_acc = np.asarray(gpu_acc)
    gpu_emi = np.asarray(gpu_emi)
    r = Report()
    B = gpu_acc.shape[0]
    idx = range(B) if seqs is None else seqs
    for oi, b in enumerate(idx):
        r.sequences += 1
        L = int(min(max(int(lens[b]), 0), n))
        T = float(temps[b]) if temps is not None else 0.0
        greedy = not (T > 0)
        ko = int(ora["accepted_len"][oi])
        kg = int(gpu_acc[b])
        am = ora.get("accept_margin")
        dm = ora.get("draw_margin")
        # acceptance decisions that both evaluated
        tests = min(ko, kg) + (1 if min(ko, kg) < L else 0)
        r.decisions += tests + 1
        if not greedy and am is not None:
            r.near_ties += int((am[oi, :min(tests, n)] < tol).sum())
            if dm is not None and dm[oi] < tol:
                r.near_ties += 1

        def hard(what):
            r.hard += 1
            if r.first_hard is None:
                r.first_hard = (b, what, kg, ko, gpu_emi[b].tolist(), ora["emitted"][oi].tolist())

        if kg != ko:
            j = min(kg, ko)
            if not greedy and am is not None and am[oi, j] < tol:
                r.exempt += 1
            else:
                hard(f"accept@{j}")
            continue
        if not np.array_equal(gpu_emi[b, :ko], ora["emitted"][oi, :ko]):
            hard("prefix")
            continue
        if not (gpu_emi[b, ko + 1:] == -1).all():
            hard("tail")
            continue
        if gpu_emi[b, ko] != ora["emitted"][oi, ko]:
            if not greedy and dm is not None and dm[oi] < tol:
                r.exempt += 1
            else:
                hard("draw")
    return r
