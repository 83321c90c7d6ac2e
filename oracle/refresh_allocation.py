"""Refresh oracle/kernel_allocation.json -- TEST INFRASTRUCTURE ONLY.

The table records what the compiler allotted to every compiled kernel
instantiation (architectural VGPRs, AGPRs, LDS bytes, scratch bytes per lane
and the waves per SIMD it reports), copied from the resource remarks the
library build collects (tile_shape_autotuning_amd/_lib/kernel_resources.json).
These are facts about the compiled code, not results of the method: the
selection oracle takes them as a fixed input, to count resident workgroups
the way the hardware does and to drop kernels that spill.  A CPU test
compares the committed table with the built library's registry, so a kernel
change that moves an allocation shows up until this script is run again.

Usage: python -m oracle.refresh_allocation
"""
from __future__ import annotations

import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)
SRC = os.path.join(REPO, "tile_shape_autotuning_amd", "_lib", "kernel_resources.json")
OUT = os.path.join(HERE, "kernel_allocation.json")
FIELDS = ("in_bf16", "kind", "bm", "bn", "bk", "wgm", "wgn", "stages", "k_groups", "vgpr", "agpr", "lds", "scratch",
          "occupancy")


def main():
    with open(SRC) as f:
        rows = json.load(f)
    lines = [json.dumps([int(r[k]) for k in FIELDS]) for r in rows]
    with open(OUT, "w") as f:
        f.write('{"fields": ' + json.dumps(list(FIELDS)) + ',\n "kernels": [\n  ' + ",\n  ".join(lines) + "\n]}\n")
    print(f"{OUT}: {len(lines)} kernels")


if __name__ == "__main__":
    main()
