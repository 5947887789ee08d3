"""Write the stored plant patches for the large workloads.

Usage:
    python tests/golden/make_plants.py CONFIG SEED [SEED ...]
    python tests/golden/make_plants.py CONFIG SEED --accept A [A ...]

Each patch is computed by ``tests/planting.py`` with the CPU oracle only and
saved as ``tests/golden/plants/<config>_s<seed>.json``; the generator replays
it on a fresh draw (``synth.make_inputs(cfg, seed, patch=path)``).

With ``--accept`` the planted ranks are not drawn from the accuracy table but
chosen so that sequence b accepts exactly A_b candidates (one A per sequence):
the path of a depth-A_b node of the tree, then a miss.  Among the tree's
depth-A nodes the one with the largest rank sum is taken (lowest rank tuple
among equals), so the accepted branch is not always the rank-0 one.
"""
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from synth import get_config, make_inputs  # noqa: E402
from tests import planting  # noqa: E402


def path_for(cfg: str, seed: int) -> str:
    return os.path.join(HERE, "plants", f"{cfg}_s{seed}.json")


def ranks_for(cfg_name: str, seed: int, accept):
    """[B, K] planted ranks that make sequence b accept ``accept[b]`` candidates."""
    cfg = get_config(cfg_name)
    if len(accept) != cfg.B:
        raise SystemExit(f"{cfg_name} has {cfg.B} sequences; give one accepted length each")
    inp = make_inputs(cfg, seed)
    plan = planting.plan_for(cfg, inp.acc)
    out = []
    for a in accept:
        at_depth = [t for t in plan.paths if len(t) == a]
        if not at_depth:
            raise SystemExit(f"the tree has no node at depth {a}")
        best = min(at_depth, key=lambda t: (-sum(t), t))
        out.append(list(best) + [-1] * (cfg.K - a))
    return out


def main(argv):
    import faulthandler
    faulthandler.dump_traceback_later(900, repeat=True)   # where a long plant spends its time
    cfg = argv[1]
    if "--accept" in argv:
        i = argv.index("--accept")
        seeds = [int(s) for s in argv[2:i]]
        accept = [int(a) for a in argv[i + 1:]]
        if len(seeds) != 1:
            raise SystemExit("--accept takes exactly one seed")
        ranks = ranks_for(cfg, seeds[0], accept)
    else:
        seeds = [int(s) for s in argv[2:]]
        ranks = None
    for seed in seeds:
        t0 = time.time()
        patch = planting.plant(cfg, seed, verbose=True, ranks=ranks)
        if ranks is not None and patch["accept_len"] != [int(a) for a in accept]:
            raise SystemExit(f"planted accept {patch['accept_len']} != asked {accept}")
        planting.save_patch(patch, path_for(cfg, seed))
        print(f"{cfg} seed {seed}: attempt {patch['h_attempt']}, {len(patch['ops'])} ops, "
              f"accept {patch['accept_len']}, {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main(sys.argv)
