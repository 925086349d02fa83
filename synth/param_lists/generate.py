"""Write the committed parameter-size lists of the seeded flush workloads.

Run once (python -m synth.param_lists.generate); the workloads read the JSON
files it writes, so sizes never depend on the host's libm at run time (the
lognormal draw of the mixed list goes through exp/log).  --check regenerates
the lists and compares them with the committed files.

  owner_flush_w8_402.8M.json  W = 8 bf16 flush of a 402.8M-element
      transformer-shaped gradient (DeepSpeed issue "[REQUEST] DeepCompile
      ZeRO-1: reduce-to-owner instead of AllReduce", Additional context):
      the 151936 x 1024 embedding, then a seeded shuffle of the smallest
      stratified mix of 1024-vectors (78.0%), 1024 x 1024 (15.2%) and
      1024 x 4096 / 4096 x 1024 (6.8%) matrices whose total reaches
      402,800,000 (mean 445,395 elements: about 118 per 52,428,800-element
      bucket).
  mixed_flush_w16_1.2B.json  W = 16 fp32 mixed stress list: lognormal sizes
      around a median of 65536 (sigma of the log 2.0), clipped to
      [1, 2^25], 2% tiny params uniform in [1, 64], drawn until the total is
      exactly 1,200,000,000 (the last draw cut).
"""
import json
import math
import os
import random
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
HIDDEN = 1024
EMBED = 151936 * 1024


def owner_w8_sizes(seed=102, target=402_800_000):
    rng = random.Random(seed)
    N = 0
    while True:
        N += 1
        n_vec = round(0.780 * N)
        n_sq = round(0.152 * N)
        n_wide = N - n_vec - n_sq
        mix = [HIDDEN] * n_vec + [HIDDEN * HIDDEN] * n_sq + [4 * HIDDEN * HIDDEN] * n_wide
        if EMBED + sum(mix) >= target:
            break
    rng.shuffle(mix)
    return [EMBED] + mix


def mixed_w16_sizes(seed=105, target=1_200_000_000):
    rng = random.Random(seed)
    numel = []
    total = 0
    while total < target:
        if rng.random() < 0.02:
            n = rng.randint(1, 64)
        else:
            n = int(round(rng.lognormvariate(math.log(65536.0), 2.0)))
            n = min(max(n, 1), 1 << 25)
        n = min(n, target - total)
        numel.append(n)
        total += n
    return numel


LISTS = {
    "owner_flush_w8_402.8M.json": (owner_w8_sizes, 102),
    "mixed_flush_w16_1.2B.json": (mixed_w16_sizes, 105),
}


def main(check=False):
    ok = True
    for name, (fn, seed) in LISTS.items():
        numel = fn(seed)
        rec = {"name": name[:-5], "seed": seed, "params": len(numel), "total": sum(numel),
               "numel": numel}
        path = os.path.join(HERE, name)
        if check:
            with open(path) as f:
                same = json.load(f) == rec
            print(f"{name}: {'same' if same else 'DIFFERENT'}")
            ok = ok and same
        else:
            with open(path, "w") as f:
                json.dump(rec, f, separators=(",", ":"))
                f.write("\n")
            print(f"wrote {name}: {len(numel)} params, {sum(numel)} elements")
    return ok


if __name__ == "__main__":
    sys.exit(0 if main(check="--check" in sys.argv) else 1)
