"""HBM calibration on the current GPU (device memory via PyTorch).

1. A device-to-device copy of exactly 256 MiB, repeated: the reference for
   scaling the profiler's HBM byte counters (FETCH_SIZE, WRITE_SIZE) --
   each copy reads and writes 268,435,456 bytes.
2. The read bandwidth of a plain streaming reduction (torch.sum) over 1 GiB,
   the achievable-bandwidth reference beside the published 8 TB/s peak.
"""

import json

import torch


def main(copy_bytes=256 << 20, reps=4, read_bytes=1 << 30):
    src = torch.ones(copy_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    big = torch.ones(read_bytes // 4, dtype=torch.float32, device="cuda")
    for _ in range(3):
        big.sum()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 20
    start.record()
    for _ in range(n):
        big.sum()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / n
    print(json.dumps({"copy_bytes_per_launch": copy_bytes, "copies": reps,
                      "sum_read_bytes": read_bytes, "sum_ms": ms,
                      "sum_read_GBps": read_bytes / (ms * 1e-3) / 1e9}))


if __name__ == "__main__":
    main()
