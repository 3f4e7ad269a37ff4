"""Markdown table of the full-size parity runs: per output, the relative
Frobenius error against the fp64 oracle and the worst element's error as a
fraction of its band, for each (workload, rank) case.

    TP_PARITY_REPORT_DIR=<dir> python -m pytest tests/test_gpu_parity.py -m gpu -k full_size
    python tests/parity_report.py <dir> > tests/full_size_parity.md
"""
import glob
import json
import os
import sys

ORDER = ["gpt2_1p2b_tp1_r0", "gpt_8p3b_tp8_r0", "mtnlg_530b_tp8_r0", "bloom_176b_tp8_r0", "bloom_176b_tp8_r7"]


def main(d: str) -> str:
    cases = {os.path.basename(f)[:-5]: json.load(open(f)) for f in glob.glob(os.path.join(d, "*.json"))}
    order = [c for c in ORDER if c in cases] + sorted(c for c in cases if c not in ORDER)
    outs = list(cases[order[0]])
    lines = ["| output | " + " | ".join(order) + " |", "|---" * (len(order) + 1) + "|"]
    for o in outs:
        cells = []
        for c in order:
            r = cases[c].get(o)
            cells.append(f"{r['rel_fro']:.1e} / {r['worst_over_band']:.2f}" if r else "")
        lines.append(f"| `{o}` | " + " | ".join(cells) + " |")
    return "\n".join(lines)


if __name__ == "__main__":
    print(main(sys.argv[1]))
