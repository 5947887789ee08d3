"""Write the stored plant patches for the large workloads.

Usage: python tests/golden/make_plants.py CONFIG SEED [SEED ...]

Each patch is computed by ``tests/planting.py`` with the CPU oracle only and
saved as ``tests/golden/plants/<config>_s<seed>.json``; the generator replays
it on a fresh draw (``synth.make_inputs(cfg, seed, patch=path)``).
"""
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from tests import planting  # noqa: E402


def path_for(cfg: str, seed: int) -> str:
    return os.path.join(HERE, "plants", f"{cfg}_s{seed}.json")


def main(argv):
    cfg = argv[1]
    for seed in [int(s) for s in argv[2:]]:
        t0 = time.time()
        patch = planting.plant(cfg, seed, verbose=True)
        planting.save_patch(patch, path_for(cfg, seed))
        print(f"{cfg} seed {seed}: attempt {patch['h_attempt']}, {len(patch['ops'])} ops, "
              f"accept {patch['accept_len']}, {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv)
