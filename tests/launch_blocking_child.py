"""Child process of the launch-blocking invariance test: runs all-reduces
through the library on inputs from an .npz file and saves the results.
Started with HIP_LAUNCH_BLOCKING=1 in its environment, which HIP reads when
it initialises (marshalling only: no reference arithmetic here)."""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))


def main(src, dst):
    import torch
    import collective_communication_reduce_amd as ccr
    from gpu_helpers import to_dev, to_host

    data = np.load(src)
    xs = [data[f"x{i}"] for i in range(int(data["R"]))]
    out = {}
    modes = {"kernel_s1": dict(), "kernel_overlap_s3": dict(overlap=True, slices=3),
             "sdma_s2": dict(copy_mode="sdma", slices=2)}
    for name, mode in modes.items():
        ts = [to_dev(x) for x in xs]
        with ccr.Context(0, ccr.Config(**mode)) as c:
            ccr.ccr_allreduce(c, ts)
            torch.cuda.synchronize()
        for q, t in enumerate(ts):
            out[f"{name}_{q}"] = to_host(t)
        print(f"child: {name} done", flush=True)
    np.savez(dst, **out)


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
