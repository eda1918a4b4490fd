"""Offline calibration of the grouped GEMM's schedule cost model.

    python -m moe_expert_load_amd.calibrate          # needs one MI355X

The forward-type GEMM schedules ("Kimi K3 模型结构（8）", rank 内部: the
schedule is picked per step by a time estimate whose key coefficients are
tuned offline; "MoonEP : l'équilibrage parfait", 3. Ordonnancement des GEMM
d'experts) estimate a persistent launch over n tiles of class c (tiles of at
most 64c rows, 2c of 8 MFMA row blocks multiplied) as

    L + ceil(n / G) * (c0 + nk * (c1 + c2 * c))

with nk the tiles' 32-deep k-tiles and G the persistent workgroups.  This
script times the forward grouped GEMM on layouts whose segments all hold the
same row count (64, 128, 256 rows: classes 1, 2, 4) at two k depths (H =
1024 and 7168) and two sizes (4 and 16 rounds of the grid).  The slope
between the sizes gives the time per tile; (c0, c1, c2) are fitted to those
by least squares; L is the mean intercept above an empty call.  The same is
done for the data-gradient GEMM (k depth H').  It prints the constants in
picoseconds, the units of the cost tables in csrc/gemm.hip (forward and
SwiGLU projection: kCostFwd; data gradient: kCostDgrad).
"""
import json
import sys

import numpy as np
import torch

from . import (MODE_INFER, load, make_cfg, moe_gemm_workspace_size, moe_grouped_gemm,
               moe_grouped_gemm_dgrad)


def _time(f, reps=9):
    f()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        f()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts)) * 1e-3


def _grid():
    G = torch.cuda.get_device_properties(0).multi_processor_count
    return G - G % 8


def time_layout(H, Hp, rows, nseg, gen, dgrad=False):
    """Seconds of one grouped GEMM (or data-gradient GEMM) over nseg segments
    of `rows` rows each."""
    S = nseg * rows
    c = make_cfg(1, max(S, 1), max(nseg, 1), 1, H, Hp, 0, MODE_INFER)
    w = torch.randn((max(nseg, 1), H, Hp), device="cuda", generator=gen).to(torch.bfloat16)
    a = torch.randn((max(S, 1), Hp if dgrad else H), device="cuda", generator=gen).to(torch.bfloat16)
    y = torch.empty((max(S, 1), H if dgrad else Hp), dtype=torch.bfloat16, device="cuda")
    cu = torch.arange(0, S + 1, max(rows, 1), dtype=torch.int32, device="cuda")
    if nseg == 0:
        cu = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws = torch.empty(moe_gemm_workspace_size(c), dtype=torch.uint8, device="cuda")
    if dgrad:
        t = _time(lambda: moe_grouped_gemm_dgrad(c, a, w, None, cu, y, 0, 1, ws))
    else:
        t = _time(lambda: moe_grouped_gemm(c, a, w, None, cu, y, 0, 1, ws))
    del w, a, y, cu, ws
    torch.cuda.empty_cache()
    return t


def measure(dgrad=False, width=2048, seed=0):
    """Tile times of the forward (k depth H, output width H') or the data
    gradient (k depth H', output width H) at k depths 1024 and 7168 and an
    output width of `width`."""
    load()
    G = _grid()
    gen = torch.Generator(device="cuda").manual_seed(seed)
    ntn = (width + 255) // 256
    dims = lambda kd: (width, kd) if dgrad else (kd, width)        # (H, H')
    empty = time_layout(*dims(1024), 0, 0, gen, dgrad)
    pts = []
    for kd in (1024, 7168):
        nk = ((kd + 31) // 32 + 3) // 4 * 4
        for rows, cls in ((64, 1), (128, 2), (256, 4)):
            t = {r: time_layout(*dims(kd), rows, r * G // ntn, gen, dgrad) for r in (4, 16)}
            tile = (t[16] - t[4]) / 12
            pts.append({"k_depth": kd, "nk": nk, "rows": rows, "class": cls, "seconds": t,
                        "tile_s": tile, "intercept_s": t[4] - 4 * tile - empty})
    return pts, empty


def fit(points):
    """Least-squares (c0, c1, c2) in picoseconds, and L."""
    A = np.array([[1.0, p["nk"], p["nk"] * p["class"]] for p in points])
    b = np.array([p["tile_s"] for p in points]) * 1e12
    coef, *_ = np.linalg.lstsq(A, b, rcond=None)
    L = float(np.mean([p["intercept_s"] for p in points])) * 1e12
    return [int(round(max(v, 0.0))) for v in coef] + [int(round(max(L, 0.0)))]


def main():
    out = {}
    for name, dg in (("forward", False), ("data_gradient", True)):
        pts, empty = measure(dgrad=dg)
        c0, c1, c2, L = fit(pts)
        for p in pts:
            p["model_tile_s"] = (c0 + p["nk"] * (c1 + c2 * p["class"])) * 1e-12
        out[name] = {"points": pts, "empty_call_s": empty, "tile": c0, "k": c1, "k_block": c2,
                     "launch": L}
    print(json.dumps(out))


if __name__ == "__main__":
    sys.exit(main())
