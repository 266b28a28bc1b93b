"""One process of the benchmark's CPU baseline: runs the oracle, as it
stands, over one slice of a sample and reports how long the oracle took.

TEST INFRASTRUCTURE ONLY: started by the CPU-baseline leg of bench.py as a
plain child process (it imports numpy and the oracle, never torch, and
touches no GPU), so that the all-cores baseline splits rows over processes
without changing the oracle.

Usage: python cpu_worker.py <task.json>
  task: {"input": .npy path, "fmt", "flags", "signs", "seed", "offset",
         "axis": 0 (slice rows) or 1 (slice columns, for a transposed
         quantize whose output rows are the source columns),
         "start", "stop"}
Prints one JSON line {"t0", "t1"}: wall-clock seconds (time.time()) around
the oracle call, so the parent can take the span of concurrent workers.
"""
import json
import sys
import time
from pathlib import Path

import numpy as np

sys.path.insert(0, str(Path(__file__).resolve().parent))
import oracle as O  # noqa: E402  (oracle.py beside this file)


def main():
    task = json.loads(Path(sys.argv[1]).read_text())
    x = np.load(task["input"], mmap_mode="r")
    s = slice(task["start"], task["stop"])
    part = np.ascontiguousarray(x[s] if task["axis"] == 0 else x[:, s])
    O.lib()
    t0 = time.time()
    O.quantize(part, task["fmt"], flags=task["flags"], rht_signs=task["signs"], seed=task["seed"],
               offset=task["offset"])
    t1 = time.time()
    print(json.dumps({"t0": t0, "t1": t1}), flush=True)


if __name__ == "__main__":
    main()
