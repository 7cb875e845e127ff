"""Summarizes rocprofv3 --pmc counter CSVs per kernel (mean over dispatches).

Usage: python profiles/summarize_pmc.py <dir with pN/pN_counter_collection.csv> [kernel-substring ...]
Prints one line per (kernel, counter): mean value per dispatch. FETCH_SIZE and
WRITE_SIZE are in KiB per dispatch as rocprofv3 reports them.
"""
import csv
import glob
import os
import sys
from collections import defaultdict


def load(root):
    acc = defaultdict(list)
    for path in sorted(glob.glob(os.path.join(root, "*", "*counter_collection.csv"))):
        with open(path) as f:
            for row in csv.DictReader(f):
                acc[(row["Kernel_Name"], row["Counter_Name"])].append(float(row["Counter_Value"]))
    return acc


def main():
    root = sys.argv[1]
    keys = sys.argv[2:]
    acc = load(root)
    for (kern, ctr), vals in sorted(acc.items()):
        if keys and not any(k in kern for k in keys):
            continue
        short = kern.split("(")[0]
        print(f"{short:45s} {ctr:28s} {sum(vals) / len(vals):16.1f}  (n={len(vals)})")


if __name__ == "__main__":
    main()
