"""Write the oracle outputs the full-size GPU parity tests compare against.

Calls only the oracle (and the seeded input generators): for every
full-size workload, the sampled clips are encoded by oracle.encode_clip in
float64 and stored (as float32) under tests/.oracle_cache/, keyed on the
workload and on the source of the oracle and input generators, so a stale
entry is never read. The tests compute any missing entry themselves.

Usage: python tests/golden/make_oracle_cache.py [workload ...]
"""
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from tests import parity  # noqa: E402


def main(names):
    for name in names or list(parity.FULL_SIZE_SAMPLES):
        w = synth.get_workload(name)
        W = None
        for clip in parity.full_size_clips(w):
            t0 = time.time()
            if W is None:
                W = synth.make_weights(w)
            every = parity.FULL_SIZE_SAMPLES[name]["every"]
            res = parity.oracle_clip(w, clip, W, every=every)
            print(f"{name} clip {clip}: {res['out'].shape} in {time.time() - t0:.1f} s", flush=True)
    for name, clips in parity.EXTRA_CLIPS.items():
        if names and name not in names:
            continue
        w = synth.get_workload(name)
        W = synth.make_weights(w)
        for clip in clips:
            t0 = time.time()
            res = parity.oracle_clip(w, clip, W, every=1)
            print(f"{name} clip {clip}: {res['out'].shape} in {time.time() - t0:.1f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
