"""Child process of the environment-invariance tests: runs all-reduces and a
staged send/recv through the library on inputs from an .npz file and saves
the results.  Started with a variable in its environment that is read once
per process (HIP_LAUNCH_BLOCKING=1, read when HIP initialises, a forced
CCR_NONTEMPORAL mode, CCR_RING_HOPS or a CCR_GRID cap), so each setting needs
a process of its own
(marshalling only: no reference arithmetic here)."""
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
    # staged send/recv with kernel copies: 3 rounds of 2 slots, ragged end
    send = [to_dev(x[: x.size // 8 * 8]) for x in xs]  # whole 16-byte vectors
    recv = [torch.zeros_like(t) for t in send]
    with ccr.Context(0, ccr.Config(staging_chunk_bytes=64 << 10, staging_slots=2)) as c:
        ccr.ccr_sendrecv_batch(c, send, recv)
        torch.cuda.synchronize()
    for q, t in enumerate(recv):
        out[f"sendrecv_{q}"] = to_host(t)
    print("child: sendrecv done", flush=True)
    np.savez(dst, **out)


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
