"""Offline tile sweep for the MFMA forward kernels, and the static table built
from it.

    python -m scaled_dot_product_fa_amd.tune --sweep [--out PATH]   # needs a GPU
    python -m scaled_dot_product_fa_amd.tune --emit                  # CPU only

``--sweep`` times every MFMA tile the library accepts (forced through the
``FA_TILE`` override) on a grid of shape classes, for both I/O types, both
head dimensions and both masking modes, and writes the timings plus the
winning tile per class to ``tiles.json`` next to this file.  ``--emit`` turns
``tiles.json`` into ``csrc/fa_tiles.inc``, the rule table
``mfma_choose_tile`` compiles in.  The table is keyed by I/O type, head
dimension, causal flag, grid size in 256-row query blocks
(``B*H*ceil(Lq/256)``) and the keys visible to a row (``Lk``, or
``min(Lk, Lq)`` when causal): within one (type, D, causal) triple the first
rule whose minimums the launch reaches applies.  The persistent kernel
(pipe 5) is not in the sweep: it has its own rule ahead of the table and
refuses grids smaller than the part.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
TABLE_JSON = os.path.join(PKG, "tiles.json")
TABLE_INC = os.path.join(PKG, "csrc", "fa_tiles.inc")

# "NWxQBxBNxOCCxPIPE" strings the library accepts (see fa_internal.h)
TILES = {
    64: ["8x1x128x2x3", "8x1x64x2x3", "8x1x64x2x2", "4x1x64x2x2", "4x2x64x1x2",
         "2x1x64x1x2", "1x1x64x1x2",
         "8x1x64x2x0", "4x1x64x2x0", "4x1x64x1x0", "4x2x64x1x0"],
    128: ["8x1x96x2x3", "8x1x64x2x3", "8x1x64x2x2", "4x1x64x2x2", "4x2x64x1x2",
          "2x1x64x1x2", "1x1x64x1x2",
          "8x1x64x2x0", "4x1x64x2x0", "4x1x64x1x0", "4x2x64x1x0"],
}

# (B, H, Lq, Lk): grid sizes from 16 to 2048 blocks of 256 query rows, short
# and long key ranges, and the cross-attention shape
SHAPES = [(1, 4, 1024, 1024), (2, 8, 1024, 1024), (2, 16, 2048, 2048), (16, 16, 512, 512),
          (4, 8, 4096, 4096), (8, 16, 1024, 4096), (4, 16, 4096, 4096), (1, 32, 16384, 16384)]

# classes: (minimum 256-row query blocks, minimum visible keys per row)
CLASSES = [(512, 2048), (128, 0), (0, 0)]

# I/O types swept, with the fa_dtype code the rule table stores
DTYPES = {"bf16": 2, "f16": 1}


def blocks256(B, H, Lq):
    return B * H * ((Lq + 255) // 256)


def sweep(reps: int, out: str) -> dict:
    import torch
    import scaled_dot_product_fa_amd as fa
    from scaled_dot_product_fa_amd import inputs

    dev = torch.device("cuda:0")
    results = []
    for dt in DTYPES:
        for D in (128, 64):
            for (B, H, Lq, Lk) in SHAPES:
                q, k, v = inputs.make_qkv(B, H, Lq, Lk, D, dt, seed=B * 1000 + H + D)
                q, k, v = q.to(dev), k.to(dev), v.to(dev)
                o = torch.empty_like(q)
                lse = torch.empty((B, H, Lq), device=dev, dtype=torch.float32)
                scale = 1.0 / math.sqrt(D)
                for causal in (False, True):
                    # flops of the visible (query, key) pairs (top-left causal)
                    if causal:
                        vis = sum(min(i + 1, Lk) for i in range(Lq))
                    else:
                        vis = Lq * Lk
                    flops = 4.0 * B * H * vis * D
                    tiles = []
                    for tile in TILES[D]:
                        os.environ["FA_TILE"] = tile
                        try:
                            fa.forward(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
                            tiles.append(tile)
                        except fa.FaError:
                            pass
                    torch.cuda.synchronize()
                    # about 10 ms of work per timing; tiles interleaved per repetition
                    est = 4.0 * B * H * Lq * Lk * D / 1e15   # seconds at 1 PFLOP/s
                    n = max(3, min(200, int(0.01 / max(est, 1e-6))))
                    best = {t: math.inf for t in tiles}
                    for _ in range(reps):
                        for tile in tiles:
                            os.environ["FA_TILE"] = tile
                            e0 = torch.cuda.Event(enable_timing=True)
                            e1 = torch.cuda.Event(enable_timing=True)
                            e0.record()
                            for _ in range(n):
                                fa.forward(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
                            e1.record()
                            torch.cuda.synchronize()
                            best[tile] = min(best[tile], e0.elapsed_time(e1) / n)
                    for tile in tiles:
                        rec = dict(dtype=dt, D=D, causal=causal, B=B, H=H, Lq=Lq, Lk=Lk,
                                   blocks256=blocks256(B, H, Lq), kv_visible=min(Lk, Lq) if causal else Lk,
                                   tile=tile, ms=round(best[tile], 5),
                                   tflops=round(flops / (best[tile] * 1e-3) / 1e12, 1))
                        results.append(rec)
                        print(json.dumps(rec), flush=True)
                del q, k, v, o, lse
                torch.cuda.empty_cache()
    os.environ.pop("FA_TILE", None)
    table = dict(device=torch.cuda.get_device_name(0), date=time.strftime("%Y-%m-%d"),
                 dtype=",".join(DTYPES), reps=reps, results=results, rules=choose(results))
    with open(out, "w") as f:
        json.dump(table, f, indent=1)
    return table


def choose(results):
    """Winner per (I/O type, D, causal, class): the tile with the best
    geometric mean throughput over the class's shapes (only tiles timed on
    all of them).  Classes, first match wins: at least 512 query blocks and
    2048 visible keys per row; at least 128 query blocks; the rest."""
    rules = []
    for dt in DTYPES:
        for D in (128, 64):
            for causal in (False, True):
                taken = set()
                for min_blocks, min_kv in CLASSES:
                    sel = [r for r in results if r["dtype"] == dt and r["D"] == D and r["causal"] == causal
                           and r["blocks256"] >= min_blocks and r["kv_visible"] >= min_kv
                           and (r["B"], r["H"], r["Lq"], r["Lk"]) not in taken]
                    shapes = {(r["B"], r["H"], r["Lq"], r["Lk"]) for r in sel}
                    if not shapes:
                        continue
                    taken |= shapes
                    score = {}
                    for tile in {r["tile"] for r in sel}:
                        t = [r["tflops"] for r in sel if r["tile"] == tile]
                        if len(t) == len(shapes):
                            score[tile] = math.exp(sum(math.log(x) for x in t) / len(t))
                    best = max(score, key=score.get)
                    rules.append(dict(dtype=dt, D=D, causal=causal, min_blocks256=min_blocks, min_kv=min_kv,
                                      tile=best, geomean_tflops=round(score[best], 1),
                                      shapes=sorted(shapes)))
    return rules


def emit(table: dict) -> str:
    lines = ["// Tile rules for mfma_choose_tile, generated by",
             "// scaled_dot_product_fa_amd/tune.py --emit from tiles.json (sweep of "
             f"{table['date']},", f"// {table['device']}, {table['dtype']}).  Do not edit by hand.",
             "// { dtype (fa_dtype), D, causal, min 256-row query blocks,",
             "//   min visible keys per row, { nw, qb, bn, occ, pipe } }"]
    for r in table["rules"]:
        nw, qb, bn, occ, pipe = (int(x) for x in r["tile"].split("x"))
        lines.append(f"{{{DTYPES[r['dtype']]}, {r['D']}, {int(r['causal'])}, {r['min_blocks256']}, {r['min_kv']}, "
                     f"{{{nw}, {qb}, {bn}, {occ}, {pipe}}}}},  "
                     f"// {r['geomean_tflops']} TFLOP/s geomean over {len(r['shapes'])} shapes")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--emit", action="store_true")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--out", default=TABLE_JSON)
    args = ap.parse_args(argv)
    if args.sweep:
        sweep(args.reps, args.out)
    if args.emit:
        table = json.load(open(TABLE_JSON))
        with open(TABLE_INC, "w") as f:
            f.write(emit(table))
        print(open(TABLE_INC).read())
    if not (args.sweep or args.emit):
        ap.print_help()
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main())
