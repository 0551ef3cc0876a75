"""Summarise the measured parity errors that the GPU tests append to KDA_PARITY_LOG.

    KDA_PARITY_LOG=/tmp/parity_margins.jsonl python -m pytest tests -m gpu
    python tests/parity_report.py /tmp/parity_margins.jsonl > profiles/parity_margins.md

One row per test: the worst error over its checks of bf16 outputs (rel_bf16) and of fp32
states (rel), each over the whole tensor and per (sequence, head), against the 2e-3 bound.
"""
from __future__ import annotations

import json
import sys


def main(path: str) -> None:
    rows: dict[str, dict] = {}
    for line in open(path):
        r = json.loads(line)
        t = r["test"].split("::", 1)[-1]
        row = rows.setdefault(t, {"bf16": [0.0, 0.0, 0], "fp32": [0.0, 0.0, 0]})
        cell = row[r["kind"]]
        cell[0] = max(cell[0], r["global"])
        cell[1] = max(cell[1], r["per_group"])
        cell[2] += 1
    worst = {k: max(v[k][1] for v in rows.values()) for k in ("bf16", "fp32")}

    def fmt(c):
        return "-" if c[2] == 0 else f"{c[0]:.2e} / {c[1]:.2e}"

    print("# Parity margins of the GPU tests (MI355X against the fp64 CPU oracle)\n")
    print("Bound: 2e-3. Outputs: `rel_bf16` (error beyond the bf16 rounding of the output);")
    print("states: `rel`. Each cell: worst over the test's checks, whole tensor / worst")
    print("(sequence, head) group. A group's output error is taken against the larger of its")
    print("reference and value magnitudes, a state's against its own largest entry.\n")
    print(f"Worst per-group error over all tests: outputs {worst['bf16']:.2e}, states "
          f"{worst['fp32']:.2e}.\n")
    print("| test | outputs (global / group) | states (global / group) |")
    print("|---|---|---|")
    for t, row in rows.items():
        print(f"| `{t}` | {fmt(row['bf16'])} | {fmt(row['fp32'])} |")


if __name__ == "__main__":
    main(sys.argv[1])
