"""Launch the statistics kernel over one 4096 x 200064 bf16 batch with two block sizes.

A program for hardware-counter runs (rocprofv3 --pmc): 30 warm-up launches with
8192-column blocks, then 10 launches of each shape, alternating, 8192-column
blocks (whole-wavefront groups) and 1024-column blocks (8-lane groups, the
shape of a verification launch).  The vocabulary is split into 8 shards of
25008 columns.  Prints one line per phase so that a long run shows progress.

    python3 -m hbm_probe.block_sizes
"""
import torch

import vocab_argmax_amd as vpa
import workloads

VOCAB, WIDTH, SHARDS, ROWS = 200064, 25008, 8, 4096


def main():
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = workloads.config4(device=dev, seed=1004).logits
    assert tuple(x.shape) == (ROWS, SHARDS * WIDTH), x.shape
    out = {b: torch.empty((SHARDS, ROWS, vpa.stats_slots(WIDTH, SHARDS, b), 2),
                          dtype=torch.int32, device=dev) for b in (8192, 1024)}
    for _ in range(30):
        vpa.block_stats(x, VOCAB, WIDTH, SHARDS, 8192, out=out[8192])
    torch.cuda.synchronize()
    print("warm-up done", flush=True)
    for _ in range(10):
        for b in (8192, 1024):
            vpa.block_stats(x, VOCAB, WIDTH, SHARDS, b, out=out[b])
    torch.cuda.synchronize()
    print("10 launches of each block size done", flush=True)


if __name__ == "__main__":
    main()
