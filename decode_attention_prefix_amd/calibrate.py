"""Profile-calibrated cost model for the planner (share/fold rule and item
costs), measured on the GPU through the C ABI.

Method, after the CREDIT summary (section III.D "Profitability and Candidate
Selection"; section V.C "Cost-Model Validation"): measure the primitive
rates and a control launch, time the non-cooperating schedule once per
shape (here: every node folded, each request streaming its whole context),
and check the model's profitability decisions against measured crossovers.
This library's model is the planner's share/fold rule: share a node when
(groups below - 1) x its K+V bytes > share_margin x the partial bytes that
sharing adds.  The calibration

  1. times a control step (one request, one token): launch plus one item's
     latency chain, the fixed cost every step pays;
  2. times a grid of one-token items (4096 items): the per-item start cost
     t0 when the GPU is full;
  3. measures the streaming rates of private items (every request its own
     context, 16-row items) and of shared items (128 rows reading one run),
     per page and KV head, from the slope between two sizes;
  4. times a family of two-level trees -- 64 subtrees, each a root of l
     tokens under c single-request leaves of 256 tokens -- with every root
     folded and with every root shared, for several l and c: the measured
     profitable side of each point and the crossover length per c;
  5. asks the planner (host only) what it decides at each point, for the
     default margin and a range of margins, and reports the agreement and
     the margin that agrees best (ties: closest to 1).

Usage: python -m decode_attention_prefix_amd.calibrate [--quick] [--out FILE]
Runs on one GPU; the numbers go to stdout as JSON and, with --out, to a text
summary.
"""
from __future__ import annotations

import argparse
import json
import math
import statistics
import sys
import time

import numpy as np

from . import cap
from . import workloads as wl

HQ, HKV, D = 32, 8, 128
MARGINS = (0.25, 0.5, 1.0, 2.0, 4.0, 8.0, 16.0, 32.0, 64.0)


# ------------------------------------------------------------------ host side

def family_tree(ell: int, c: int, leaf: int = 256, subtrees: int = 64, hq: int = HQ, hkv: int = HKV,
                d: int = D) -> wl.Tree:
    """`subtrees` two-level subtrees under an empty sentinel root: a root of
    `ell` tokens with `c` leaves of `leaf` tokens, one request per leaf."""
    nt, par, paths = [0], [-1], []
    for _ in range(subtrees):
        r = len(nt)
        nt.append(ell)
        par.append(0)
        for _ in range(c):
            paths.append([0, r, len(nt)])
            nt.append(leaf)
            par.append(r)
    return wl.tree_from_lengths(nt, par, paths, hq, hkv, d)


def private_tree(requests: int, tokens: int) -> wl.Tree:
    """Every request a single node of its own: nothing to share."""
    return wl.tree_from_lengths([tokens] * requests, [-1] * requests, [[r] for r in range(requests)],
                                HQ, HKV, D)


def shared_tree(tokens: int, requests: int = 32) -> wl.Tree:
    """One node that `requests` requests all end at: one 128-row group."""
    return wl.tree_from_lengths([tokens], [-1], [[0]] * requests, HQ, HKV, D)


def planner_shares_roots(tree: wl.Tree, subtrees: int, c: int, **opts) -> bool:
    """Whether the planner (auto mode) serves the subtree roots once for all
    their requests: then it makes one group per root and one per leaf."""
    h = cap.cap_tree_upload(tree)
    try:
        p = cap.cap_plan_step(h, **opts)
        try:
            groups = cap.cap_plan_get_stats(p)["num_groups"]
        finally:
            cap.cap_plan_free(p)
    finally:
        cap.cap_tree_free(h)
    if groups == subtrees * (c + 1):
        return True
    assert groups == subtrees * c, groups
    return False


def measured_side(t_share: float, t_fold: float, tie: float = 0.02) -> str:
    """'share', 'fold', or 'tie' when the two are within `tie` of each other."""
    if t_share < t_fold * (1 - tie):
        return "share"
    if t_fold < t_share * (1 - tie):
        return "fold"
    return "tie"


def agrees(model_shares: bool, side: str) -> bool:
    return side == "tie" or (side == "share") == model_shares


def crossover(lengths, sides) -> int | None:
    """Smallest length from which sharing is never measured slower (None if
    folding wins at the largest length)."""
    best = None
    for ell, side in sorted(zip(lengths, sides), reverse=True):
        if side == "fold":
            break
        best = ell
    return best


def fit_margin(points, decide) -> tuple[float, float]:
    """Margin with the highest agreement over `points` [(key, side)], where
    decide(key, margin) -> bool is the model's decision; ties go to the
    margin closest to 1 (in log scale).  Returns (margin, agreement)."""
    scored = []
    for m in MARGINS:
        ok = sum(agrees(decide(k, m), side) for k, side in points)
        scored.append((ok / max(1, len(points)), -abs(math.log(m)), m))
    acc, _, m = max(scored)
    return m, acc


# ------------------------------------------------------------------ GPU side

class StepTimer:
    """Median time of decode + merge on the current stream, caches flushed
    by a 1 GiB read before each step (as in bench.py)."""

    def __init__(self, steps: int = 15, warmup: int = 5):
        import torch
        self.torch = torch
        self.steps, self.warmup = steps, warmup
        self.dev = torch.device("cuda", torch.cuda.current_device())
        self.flush = torch.zeros(1 << 30, dtype=torch.uint8, device=self.dev)
        self.sink = torch.empty(8192, dtype=torch.int32, device=self.dev)

    def stream(self) -> int:
        return self.torch.cuda.current_stream(self.dev).cuda_stream

    def evict(self):
        cap.cap_bench_read(self.flush.data_ptr(), self.flush.numel(), self.sink.data_ptr(), self.stream())

    def pools(self, tree, seed: int = 0):
        torch = self.torch
        g = torch.Generator(device=self.dev)
        g.manual_seed(seed)
        P = int(tree.num_pool_pages)
        k = torch.randn((P, HKV, D // 8, 16, 8), generator=g, device=self.dev).to(torch.bfloat16)
        v = torch.randn((P, HKV, D, 16), generator=g, device=self.dev).to(torch.bfloat16)
        q = torch.randn((tree.num_requests, HQ, D), generator=g, device=self.dev).to(torch.bfloat16)
        return q, k, v

    def time_tree(self, tree, **opts) -> float:
        from .decoder import TreeDecoder
        torch = self.torch
        q, k, v = self.pools(tree)
        dec = TreeDecoder(tree, q, k, v, device=self.dev, **opts)
        try:
            stream = torch.cuda.current_stream(self.dev)
            for _ in range(self.warmup):
                self.evict()
                dec.step(fused=False)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(self.steps)]
            for e in ev:
                self.evict()
                e[0].record(stream)
                dec.step(fused=False)
                e[1].record(stream)
            torch.cuda.synchronize(self.dev)
            return statistics.median(a.elapsed_time(b) for a, b in ev) * 1e3
        finally:
            dec.close()
            del q, k, v

    def read_rate(self) -> float:
        """Achievable streaming read (bytes/s) over 2 GiB."""
        torch = self.torch
        nb = 2 << 30
        buf = torch.empty(nb, dtype=torch.uint8, device=self.dev)
        cap.cap_bench_fill(buf.data_ptr(), nb, 0x3F803F80, self.stream())
        ms = []
        for _ in range(5):
            self.evict()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            cap.cap_bench_read_stream(buf.data_ptr(), nb, self.sink.data_ptr(), self.stream())
            b.record()
            b.synchronize()
            ms.append(a.elapsed_time(b))
        del buf
        return nb / (min(ms) * 1e-3)


def page_head_us(t0: float, t1: float, pages0: int, pages1: int) -> float:
    """Whole-GPU time per page and KV head from the slope between two sizes."""
    return (t1 - t0) / ((pages1 - pages0) * HKV)


def calibrate(quick: bool = False, log=print) -> dict:
    tm = StepTimer(steps=9 if quick else 15, warmup=3 if quick else 5)
    out: dict = {"shape": f"Hq={HQ} Hkv={HKV} D={D}, page 16", "steps_per_timing": tm.steps}
    out["read_rate_gbs"] = round(tm.read_rate() / 1e9, 1)
    log(f"read rate {out['read_rate_gbs']} GB/s")
    out["t_ctrl_us"] = round(tm.time_tree(private_tree(1, 1)), 2)
    t_grid = tm.time_tree(private_tree(512, 1))
    out["t_grid_4096_items_us"] = round(t_grid, 2)
    # 4096 one-page items over 512 workgroup slots: 8 rounds
    out["t0_item_us"] = round((t_grid - out["t_ctrl_us"]) / (4096 / 512), 3)
    log(f"control {out['t_ctrl_us']} us, 4096 one-token items {t_grid:.1f} us, t0 {out['t0_item_us']} us")

    L0, L1 = (1024, 2048) if quick else (1024, 4096)
    tp0 = tm.time_tree(private_tree(256, L0), share_mode=0)
    tp1 = tm.time_tree(private_tree(256, L1), share_mode=0)
    priv = page_head_us(tp0, tp1, 256 * L0 // 16, 256 * L1 // 16)
    S0, S1 = (8192, 16384) if quick else (8192, 32768)
    ts0 = tm.time_tree(shared_tree(S0), share_mode=1)
    ts1 = tm.time_tree(shared_tree(S1), share_mode=1)
    shar = page_head_us(ts0, ts1, S0 // 16, S1 // 16)
    page_bytes = 2 * 16 * D * 2
    out["private"] = {"us_per_page_head_gpu": priv, "gbs": round(page_bytes / (priv * 1e-6) / 1e9, 1),
                      "t_us": [round(tp0, 1), round(tp1, 1)], "tokens_per_request": [L0, L1]}
    out["shared_128_rows"] = {"us_per_page_head_gpu": shar, "gbs": round(page_bytes / (shar * 1e-6) / 1e9, 1),
                              "t_us": [round(ts0, 1), round(ts1, 1)], "root_tokens": [S0, S1]}
    out["shared_cost_measured"] = round(shar / priv, 3)
    log(f"private {out['private']['gbs']} GB/s, shared(128 rows) {out['shared_128_rows']['gbs']} GB/s, "
        f"shared page / private page = {out['shared_cost_measured']}")

    lengths = (16, 64, 256, 1024) if quick else (16, 64, 256, 1024, 4096)
    cs = (2, 8) if quick else (2, 4, 8)
    grid = []
    for c in cs:
        for ell in lengths:
            t = family_tree(ell, c)
            tf = tm.time_tree(t, share_mode=0)
            ts = tm.time_tree(t, share_mode=1)
            side = measured_side(ts, tf)
            model = planner_shares_roots(t, 64, c)
            grid.append({"c": c, "root_tokens": ell, "t_fold_us": round(tf, 2), "t_share_us": round(ts, 2),
                         "measured": side, "model_shares": model, "agrees": agrees(model, side)})
            log(f"c={c} l={ell}: fold {tf:.1f} us, share {ts:.1f} us -> {side}; model "
                f"{'shares' if model else 'folds'}")
    out["grid"] = grid
    out["accuracy_default_margin"] = round(sum(g["agrees"] for g in grid) / len(grid), 3)
    out["crossover_root_tokens"] = {
        str(c): crossover([g["root_tokens"] for g in grid if g["c"] == c],
                          [g["measured"] for g in grid if g["c"] == c]) for c in cs}
    points = [((g["c"], g["root_tokens"]), g["measured"]) for g in grid]
    cache = {}

    def decide(key, m):
        if (key, m) not in cache:
            cache[(key, m)] = planner_shares_roots(family_tree(key[1], key[0]), 64, key[0], share_margin=m)
        return cache[(key, m)]

    m, acc = fit_margin(points, decide)
    out["fitted_margin"] = m
    out["accuracy_fitted_margin"] = round(acc, 3)
    out["model_crossover_root_tokens"] = {}
    for c in cs:
        for name, mm in (("default", 1.0), ("fitted", m)):
            xs = [ell for ell in lengths if decide((c, ell), mm)]
            out["model_crossover_root_tokens"][f"{c}/{name}"] = min(xs) if xs else None
    log(f"agreement {out['accuracy_default_margin']} at the default margin; best margin {m} "
        f"({out['accuracy_fitted_margin']})")
    return out


def summary_text(res: dict, cmd: str) -> str:
    lines = ["Cost-model calibration of the planner (share/fold rule, item costs)",
             f"command: {cmd}", f"shape: {res['shape']}; median of {res['steps_per_timing']} flushed steps",
             "",
             f"achievable read (streaming probe): {res['read_rate_gbs']} GB/s",
             f"control step (1 request, 1 token, decode + merge): {res['t_ctrl_us']} us",
             f"4096 one-token items (8 rounds of 512 workgroups): {res['t_grid_4096_items_us']} us "
             f"-> t0 = {res['t0_item_us']} us per item round",
             f"private items (16 rows): {res['private']['us_per_page_head_gpu']:.5f} us per page-head "
             f"(whole GPU) = {res['private']['gbs']} GB/s",
             f"shared items (128 rows): {res['shared_128_rows']['us_per_page_head_gpu']:.5f} us per page-head "
             f"= {res['shared_128_rows']['gbs']} GB/s",
             f"shared page cost / private page cost: {res['shared_cost_measured']}",
             "",
             "share/fold per subtree root (64 subtrees, c leaves of 256 tokens each):",
             f"{'c':>3s} {'root':>6s} {'fold_us':>9s} {'share_us':>9s} {'measured':>8s} {'model':>7s} {'agrees':>6s}"]
    for g in res["grid"]:
        lines.append(f"{g['c']:3d} {g['root_tokens']:6d} {g['t_fold_us']:9.2f} {g['t_share_us']:9.2f} "
                     f"{g['measured']:>8s} {'share' if g['model_shares'] else 'fold':>7s} "
                     f"{'yes' if g['agrees'] else 'NO':>6s}")
    lines += ["",
              f"measured crossover (root tokens from which sharing is never slower), by c: "
              f"{res['crossover_root_tokens']}",
              f"model crossover by c/margin: {res['model_crossover_root_tokens']}",
              f"agreement at the default margin 1.0: {res['accuracy_default_margin']}",
              f"best margin over {list(MARGINS)}: {res['fitted_margin']} "
              f"(agreement {res['accuracy_fitted_margin']})"]
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true")
    ap.add_argument("--out", default="")
    a = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("calibrate needs a GPU", file=sys.stderr)
        sys.exit(1)
    t0 = time.perf_counter()
    res = calibrate(quick=a.quick, log=lambda s: print(s, file=sys.stderr, flush=True))
    res["wall_s"] = round(time.perf_counter() - t0, 1)
    print(json.dumps(res), flush=True)
    if a.out:
        cmd = "python -m decode_attention_prefix_amd.calibrate" + (" --quick" if a.quick else "")
        with open(a.out, "w") as f:
            f.write(summary_text(res, cmd))


if __name__ == "__main__":
    main()
