"""Benchmark: draft-tree verify rounds/s and committed tokens/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 8b] [--temp 1.0]

A step is one whole round (expand -> mask -> tree attention -> LM head ->
accept, plus the tree q/k/v row gathers) through the C ABI on synthetic
inputs already resident in HBM.  Input sets rotate (8 by default) so that
per-round data (draft rows, prefix KV) is not served from the 256 MB
Infinity Cache; the LM-head weight is one copy.  Prints one JSON line.

The LM-head kernel (one launch per round) is timed with HIP events on the
stream it runs on (every 8th round of the timed loop), giving its achieved HBM
bandwidth against 8 TB/s.  The CPU
oracle is timed on a bounded sample of the same workload as a reference point
(never a target).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_8b_bs1_traffic.txt")
LMHEAD_SRC = os.path.join(ROOT, "eagle_draft_tree_expand_amd", "csrc", "k_lmhead.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def w_bytes(cfg, rows, wts=None):
    """Bytes of W one LM-head launch reads: V x H in its dtype, or, where the
    launch reads the z-packed form (wts.w_z, at most ZPACK_MAX_ROWS rows), one
    header byte per fragment plus 768 bytes per coded and 1024 per raw fragment."""
    if wts is not None and getattr(wts, "w_z", None) is not None and rows <= ZPACK_MAX_ROWS:
        nfrag = (cfg.V + 63) // 64 * (cfg.H // 8)
        return nfrag + (nfrag - wts.z_raw) * 768 + wts.z_raw * 1024
    return cfg.V * cfg.H * (2 if cfg.dtype == "bf16" else 4)


def lmhead_bytes(cfg, rows, wts=None):
    """Algorithmic bytes of one LM-head launch: W once (in the form it is read), X, fp32 logits out."""
    esz = 2 if cfg.dtype == "bf16" else 4
    return w_bytes(cfg, rows, wts) + rows * cfg.H * esz + rows * cfg.V * 4


def round_bytes(cfg, prefix_total, wts=None):
    """Algorithmic bytes of one round: draft rows, prefix KV, tree Q/K/V and O, W, X, logits.
    Without wts, W counts as bf16 (the bytes the round would move from an uncompressed W)."""
    esz = 2 if cfg.dtype == "bf16" else 4
    rows = cfg.B * cfg.N
    draft = cfg.B * cfg.S * cfg.V * 4
    kv = prefix_total * cfg.hkv * cfg.dh * esz * 2
    tree = rows * (cfg.hq + 2 * cfg.hkv) * cfg.dh * esz + rows * cfg.hq * cfg.dh * esz
    return draft + kv + tree + lmhead_bytes(cfg, rows, wts)


ZPACK_MAX_ROWS = 192  # EAGLE_ZPACK_MAX_ROWS
LMHEAD_KERNEL_START = "__global__ __launch_bounds__(kLmThreads) void lmhead_bf16_kernel("


def source_hash(path):
    """Hash of the streaming LM-head kernel's source text (its template line
    through the closing brace), so that edits elsewhere in the file do not
    invalidate counters taken on an unchanged kernel."""
    text = open(path, encoding="utf-8").read()
    a = text.find(LMHEAD_KERNEL_START)
    if a < 0:
        return None
    b = text.find("\n}\n", a)
    return hashlib.sha256(text[a:b + 3].encode()).hexdigest()[:16]


def read_traffic():
    """HBM bytes per LM-head launch from the committed rocprofv3 counter summary,
    only if it was taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    h = source_hash(LMHEAD_SRC)
    if h is None or kv.get("source_sha256_16") != h:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def setup(cfg_name, T, n_sets, device="cuda"):
    import torch

    import synth
    from eagle_draft_tree_expand_amd import round as dround
    cfg = synth.get_config(cfg_name)
    t0 = time.time()
    inps = [synth.make_inputs(cfg, s) for s in range(n_sets)]
    wts = dround.DeviceWeights(inps[0], device)
    sets = []
    prepass = dround.device_static_rows if cfg.static_parent else dround.device_draft_rows
    for inp in inps:
        d = dround.DeviceInputs(inp, device, with_eps=True)
        prepass(cfg, wts, d, T)
        d.eps = None  # only the rows are needed from here on
        sets.append(d)
    torch.cuda.synchronize()
    log(f"[bench] {cfg_name}: inputs + device pre-pass for {n_sets} sets in {time.time() - t0:.1f}s")
    return cfg, inps, wts, sets


LM_EVENT_EVERY = 8  # LM-head launches bracketed by events: every 8th round (a bracketed round idles the GPU ~11 us)


def time_rounds(cfg, wts, sets, T, steps, warmup, device="cuda", warp=None, compact=False, dist=False):
    """Warm up, then time exactly `steps` rounds; within them, the LM-head
    launch of every LM_EVENT_EVERY-th round is timed with events on its stream.
    warp = (top_k, top_p): rounds with both distributions warped (the two row
    warps run inside the timed rounds).  compact: the LM head writes compact
    rows and the walk reads them.  dist: a second pass of as many rounds, each
    bracketed by its own events, gives the spread of the round time (p10, p50,
    p90; the events add their own dispatch to every round of that pass)."""
    import torch

    from eagle_draft_tree_expand_amd import round as dround
    dr = dround.DeviceRound(cfg, device, compact=compact)
    for i in range(warmup):
        dr.step(wts, sets[i % len(sets)], T, round_id=i, warp=warp)
    nev = (steps + LM_EVENT_EVERY - 1) // LM_EVENT_EVERY
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nev)]
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    # one more untimed round between the synchronisation and the start event, so
    # that the GPU is busy when the timed rounds start instead of idling while
    # the host enqueues the first one
    dr.step(wts, sets[warmup % len(sets)], T, round_id=warmup, warp=warp)
    t_start.record()
    for i in range(steps):
        d = sets[i % len(sets)]
        if warp is None and not dr.static:
            dr.expand_masked(d, T, i)
        else:
            dr.expand(d, T, i, warp)
            dr.mask_pos(d)
        dr.gather_qkv(wts)
        dr.attention(d)
        timed = i % LM_EVENT_EVERY == 0
        if timed:
            ev[i // LM_EVENT_EVERY][0].record()
        dr.lmhead(wts, T)
        if timed:
            ev[i // LM_EVENT_EVERY][1].record()
        dr.accept(d, T, i, warp)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    lm_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    spread = None
    if dist:
        pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            pe[i][0].record()
            dr.step(wts, sets[i % len(sets)], T, round_id=i, warp=warp)
            pe[i][1].record()
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) for a, b in pe])
        spread = {q: round(float(np.percentile(per, int(q[1:]))), 4) for q in ("p10", "p50", "p90")}
    # committed tokens: replay the same rounds untimed (results are deterministic)
    committed = 0
    for i in range(steps):
        d = sets[i % len(sets)]
        dr.step(wts, d, T, round_id=i, warp=warp)
        committed += int(dr.acc["n_committed"].sum().item())
    status = int(dr.status.item())
    return dict(total_ms=total_ms, wall_s=wall, lm_ms=lm_ms, committed=committed, status=status, spread=spread)


def time_commit(cfg, wts, inp, rows, T, reps=40, device="cuda"):
    """One round on a cache with room for many commits, then `reps` back-to-back
    commits of its accepted path (each appends after the last) bracketed by
    one pair of events: GPU time per call, gaps between launches included."""
    import torch

    from eagle_draft_tree_expand_amd import round as dround
    room = (reps + 2) * (cfg.D + 1)
    dr = dround.DeviceRound(cfg, device, cap=cfg.Lmax + room)
    data = dround.DeviceInputs(inp, device, room=room)
    data.rows.copy_(rows)
    dr.step(wts, data, T)
    dr.commit(data)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # a spin kernel keeps the GPU busy while the host queues every call, so
    # the calls run back to back and the events time the GPU, not the host
    torch.cuda._sleep(20_000_000)
    e0.record()
    for _ in range(reps):
        dr.commit(data)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    esz = 2 if cfg.dtype == "bf16" else 4
    rows_c = dr.acc["accept_len"].cpu().numpy().astype(np.int64) + 1
    # K and V rows read and written, feature rows read, the whole feature block written
    nbytes = int(rows_c.sum() * (4 * cfg.hkv * cfg.dh + cfg.H) * esz + cfg.B * (cfg.D + 1) * cfg.H * esz)
    return {"us_per_call": round(us, 2), "bytes": nbytes, "committed_rows": int(rows_c.sum()),
            "status": int(dr.status.item())}


def draft_bytes(cfg, inter, prefix_total, wts=None):
    """Algorithmic HBM bytes of one drafting round (D depths): per depth the draft
    layer's weights and the shared LM head once (in the form that depth reads:
    z-packed with wts.w_z at few rows, else bf16), the frontier's embedding rows,
    the draft prefix K/V of every request, and the frontier's rows written by
    the LM head and read back by the expansion."""
    H, Q, KV, V = cfg.H, cfg.hq * cfg.dh, cfg.hkv * cfg.dh, cfg.V
    w = 2 * (2 * H * H + H * (Q + 2 * KV) + Q * H + 3 * inter * H)
    total = 0
    for d in range(cfg.D):
        R = cfg.B * (1 if d == 0 else cfg.k)
        total += w + w_bytes(cfg, R, wts) + R * H * 2 + 2 * prefix_total * KV * 2 + 2 * R * V * 4
    return total


def time_drafting(cfg, wts, inp, T, steps, warmup, device="cuda"):
    """Rounds with the tree drafted depth by depth by a synthetic EAGLE draft head
    (random weights), then the verify pass and acceptance on the drafted rows:
    drafting alone is timed over `steps` rounds, then whole rounds."""
    import torch

    from eagle_draft_tree_expand_amd import draft_head
    from eagle_draft_tree_expand_amd import round as dround
    from synth.draft import make_draft_inputs
    t0 = time.time()
    dinp = make_draft_inputs(cfg, 0)
    head = draft_head.DeviceDraftHead(cfg, dinp, wts, device)
    del dinp
    dr = dround.DeviceRound(cfg, device)
    data = dround.DeviceInputs(inp, device)  # its own row buffer: the drafted rows land there
    torch.cuda.synchronize()
    log(f"[bench] draft head for {cfg.name} ready in {time.time() - t0:.1f}s")
    for i in range(warmup):
        draft_head.draft_tree(head, dr, data, T, i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        draft_head.draft_tree(head, dr, data, T, i)
    b.record()
    torch.cuda.synchronize()
    draft_ms = a.elapsed_time(b) / steps
    a.record()
    for i in range(steps):
        draft_head.draft_tree(head, dr, data, T, i)
        dr.mask_pos(data)
        dr.gather_qkv(wts)
        dr.attention(data)
        dr.lmhead(wts, T)
        dr.accept(data, T, i)
    b.record()
    torch.cuda.synchronize()
    round_ms = a.elapsed_time(b) / steps
    committed = 0
    for i in range(min(steps, 8)):
        draft_head.draft_tree(head, dr, data, T, i)
        dr.mask_pos(data)
        dr.gather_qkv(wts)
        dr.attention(data)
        dr.lmhead(wts, T)
        dr.accept(data, T, i)
        committed += int(dr.acc["n_committed"].sum().item())
    nb = draft_bytes(cfg, head.inter, int(data.prefix_len.sum().item()), wts)
    out = {"workload": f"{cfg.name} shape, tree drafted depth by depth by a synthetic EAGLE draft head "
                       f"(FC 2H->H, one decoder layer with MLP {head.inter}, shared LM head; random weights)",
           "draft_ms_per_round": round(draft_ms, 4), "round_ms": round(round_ms, 4),
           "trees_per_s": round(1000.0 / round_ms * cfg.B, 2),
           "committed_tokens_per_s": round(committed / min(steps, 8) * 1000.0 / round_ms, 1),
           "draft_bytes_per_round": nb,
           "draft_hbm_frac": round(nb / (draft_ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
           "device_status": int(dr.status.item())}
    del head
    return out


# One round's inputs on the device (DeviceInputs attributes), in a dump.
DUMP_INPUTS = ("k_prefix", "v_prefix", "prefix_len", "roots", "uniforms", "rows")


def _to_np(t):
    import torch
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).cpu().numpy()


def dump_round(path, cfg_name, T, round_id=0):
    """Run one round of input set 0 and write its inputs and outputs to an .npz.

    The file holds what the round read (prefix K/V, prefix lengths, roots,
    uniforms, draft rows; bf16 arrays as their 16-bit words), the Gumbel key,
    T and the round id, and every output of the round.  The LM-head weight and
    the per-token q/k/v tables are not stored: the config's seeds rebuild them."""
    from eagle_draft_tree_expand_amd import round as dround
    cfg, _, wts, sets = setup(cfg_name, T, 1)
    d = sets[0]
    dr = dround.DeviceRound(cfg)
    dr.step(wts, d, T, round_id=round_id)
    out = dr.host()
    arrays = {f"in_{k}": _to_np(getattr(d, k)) for k in DUMP_INPUTS}
    arrays.update({f"out_{k}": np.asarray(v) for k, v in out.items() if k != "status"})
    meta = {"config": cfg_name, "T": float(T), "round_id": int(round_id), "seed": int(d.seed),
            "status": int(out["status"])}
    np.savez_compressed(path, meta=np.array(json.dumps(meta)), **arrays)
    return meta


def replay_round(path):
    """Run the round stored by dump_round again and compare every output bit for bit."""
    import torch

    import synth
    from eagle_draft_tree_expand_amd import round as dround
    z = np.load(path)
    meta = json.loads(str(z["meta"]))
    cfg = synth.get_config(meta["config"])
    inp = synth.make_inputs(cfg, 0)
    wts = dround.DeviceWeights(inp)
    d = dround.DeviceInputs(inp)
    for k in DUMP_INPUTS:
        t = getattr(d, k)
        a = torch.from_numpy(z[f"in_{k}"])
        t.copy_((a.view(torch.bfloat16) if t.dtype == torch.bfloat16 else a).to(t.device))
    d.seed = meta["seed"]
    dr = dround.DeviceRound(cfg)
    dr.step(wts, d, meta["T"], round_id=meta["round_id"])
    out = dr.host()
    diff = [k for k, v in out.items()
            if k != "status" and np.asarray(v).tobytes() != z[f"out_{k}"].tobytes()]
    if out["status"] != meta["status"]:
        diff.append("status")
    return {"replay": path, "config": meta["config"], "round_id": meta["round_id"], "outputs": len(out),
            "match": not diff, "mismatched": diff}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg_name, T, inp, budget_s=25.0):
    """The oracle, untuned, on a bounded sample: whole rounds of set 0 (pre-pass excluded),
    with the BLAS threads it starts with, then again with one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import round as oround
    wts = oround._Weights(inp)
    t0 = time.time()
    rows = oround.target_draft_rows(inp, T, wts)
    prep = time.time() - t0

    def rounds(limit_s, max_n):
        n, committed = 0, 0
        t0 = time.time()
        while True:
            r = oround.run_round(inp, T, rows=rows, round_id=n, weights=wts)
            committed += sum(a["n_committed"] for a in r["accept"])
            n += 1
            el = time.time() - t0
            if el > limit_s or n >= max_n:
                return n, committed, el

    n, committed, el = rounds(budget_s * 0.5, 8)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    with threadpool_limits(limits=1):
        n1, c1, el1 = rounds(budget_s * 0.3, 3)
    log(f"[bench] oracle: pre-pass {prep:.1f}s, {n} rounds in {el:.1f}s; one thread: {n1} rounds in {el1:.1f}s")
    return {"value": n * inp.cfg.B / el, "unit": "trees/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} whole rounds of the {cfg_name} workload (input set 0, round ids 0..{n - 1}), "
                      f"draft-row pre-pass excluded; {committed / el:.3f} committed tokens/s",
            "nproc": os.cpu_count(), "cpu_model": _cpu_model(),
            "one_thread": {"value": round(n1 * inp.cfg.B / el1, 4), "unit": "trees/s", "rounds": n1,
                           "committed_tokens_per_s": round(c1 / el1, 3)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="8b")
    ap.add_argument("--temp", type=float, default=1.0)
    ap.add_argument("--sets", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the greedy and batch-64 extra lines")
    ap.add_argument("--only-draft", action="store_true",
                    help="only time the depth-by-depth drafting leg (8b shape) and print its JSON")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (a known-size reference for HBM "
                         "byte counters) and exit")
    ap.add_argument("--dump-round", metavar="PATH",
                    help="run one round of --config (input set 0, round 0) and write its inputs and outputs "
                         "to PATH (.npz), then exit")
    ap.add_argument("--replay", metavar="PATH",
                    help="run the round stored in PATH again, compare every output bit for bit, print JSON")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(each request's round fits one GPU).", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "copies": 3}), flush=True)
        return

    if args.dump_round:
        print(json.dumps({"dumped": args.dump_round, **dump_round(args.dump_round, args.config, args.temp)}),
              flush=True)
        return
    if args.replay:
        r = replay_round(args.replay)
        print(json.dumps(r), flush=True)
        sys.exit(0 if r["match"] else 1)

    if args.only_draft:
        import synth
        from eagle_draft_tree_expand_amd import round as dround
        dcfg = synth.get_config(args.config)
        dinp = synth.make_inputs(dcfg, 0)
        print(json.dumps({"draft": time_drafting(dcfg, dround.DeviceWeights(dinp), dinp, args.temp, args.steps,
                                                 args.warmup)}), flush=True)
        return

    cfg, inps, wts, sets = setup(args.config, args.temp, args.sets)
    r = time_rounds(cfg, wts, sets, args.temp, args.steps, args.warmup, dist=True)
    ms = r["total_ms"] / args.steps
    rounds_s = 1000.0 / ms
    trees_s = rounds_s * cfg.B
    tok_s = r["committed"] / (r["total_ms"] / 1000.0)
    rows = cfg.B * cfg.N
    lm_b = lmhead_bytes(cfg, rows, wts)
    achieved = lm_b / (r["lm_ms"] / 1000.0) / 1e9
    prefix_total = int(sum(int(s.prefix_len.sum().item()) for s in sets) / len(sets))
    rb = round_bytes(cfg, prefix_total, wts)
    rb16 = round_bytes(cfg, prefix_total)
    zp = getattr(wts, "w_z", None) is not None and rows <= ZPACK_MAX_ROWS
    nfrag = (cfg.V + 63) // 64 * (cfg.H // 8)
    traffic = read_traffic() if args.config == "8b" else None
    out = {
        "metric": "draft-tree verify rounds/sec + committed tokens/sec (8B shape, bs=1 and 64)",
        "value": round(trees_s, 2),
        "unit": "trees/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: batch {cfg.B}, hidden {cfg.H}, {cfg.hq}q/{cfg.hkv}kv heads x "
                               f"{cfg.dh}, prefix {cfg.L[0]}-{cfg.L[1]}, vocab {cfg.V}, depth {cfg.D}, "
                               f"top-k {cfg.k}, m {cfg.m}, T={args.temp}",
                   "global_batch": cfg.B, "seq_len": cfg.Lmax, "parallelism": "single GPU",
                   "input_sets": len(sets)},
        "committed_tokens_per_s": round(tok_s, 1),
        "tau_synthetic": round(r["committed"] / (args.steps * cfg.B), 4),
        "round_hbm_fraction": round(rb / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
        "round_bf16_w_fraction": round(rb16 / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
        "w_layout": ({"form": "z-packed (lossless: 12 bits per weight in coded fragments)",
                      "raw_fragments": int(wts.z_raw), "fragments": nfrag,
                      "w_bytes_read": w_bytes(cfg, rows, wts), "w_bytes_bf16": cfg.V * cfg.H * 2}
                     if zp else {"form": "packed bf16"}),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "eagle_lmhead_softmax: lmhead_bf16 + lm_finalize, HIP events on its stream"
                               + (" (z-packed W)" if zp else ""),
                     "bytes_per_launch": lm_b,
                     "avg_launch_ms": round(r["lm_ms"], 5)},
        "device_status": r["status"],
        "per_round_ms": dict(r["spread"], note="each round bracketed by its own events in a second pass"),
    }
    if not args.no_extra:
        # the same rounds with compact target rows (no fp32 logit rows)
        cr = time_rounds(cfg, wts, sets, args.temp, args.steps, args.warmup, compact=True)
        cms = cr["total_ms"] / args.steps
        out["compact"] = {"rows": "fp16 offsets from 128-column block maxima; LM head and walk on them",
                          "trees_per_s": round(1000.0 / cms * cfg.B, 2), "ms_per_step": round(cms, 4),
                          "committed_tokens_per_s": round(cr["committed"] / (cr["total_ms"] / 1000.0), 1),
                          "round_hbm_fraction": round((rb - rows * cfg.V * 2) / (cms / 1000.0) / 1e9 / HBM_PEAK_GBS,
                                                      4),
                          "lmhead_ms": round(cr["lm_ms"], 5), "device_status": cr["status"]}
    if not args.no_extra:
        out["commit"] = time_commit(cfg, wts, inps[0], sets[0].rows, args.temp)
    if not args.no_extra and args.temp > 0:
        wsteps = max(20, args.steps // 4)
        wr = time_rounds(cfg, wts, sets, args.temp, wsteps, 5, warp=(50, 0.9))
        out["warped"] = {"warp": "top_k 50, top_p 0.9 on draft and target rows",
                         "trees_per_s": round(1000.0 * wsteps / wr["total_ms"] * cfg.B, 2),
                         "committed_tokens_per_s": round(wr["committed"] / (wr["total_ms"] / 1000.0), 1),
                         "tau_synthetic": round(wr["committed"] / (wsteps * cfg.B), 4),
                         "device_status": wr["status"]}
        if args.config == "8b":
            # the same warps on draft rows close to the target's, so that warped rounds accept too
            kcfg, _, kwts, ksets = setup("8b_close", args.temp, 4)
            kr = time_rounds(kcfg, kwts, ksets, args.temp, wsteps, 5, warp=(50, 0.9))
            ku = time_rounds(kcfg, kwts, ksets, args.temp, wsteps, 5)
            out["warped_close"] = {"workload": "8b shape, draft rows = target logits + N(0, 0.01^2) noise",
                                   "warp": "top_k 50, top_p 0.9 on draft and target rows",
                                   "trees_per_s": round(1000.0 * wsteps / kr["total_ms"] * kcfg.B, 2),
                                   "committed_tokens_per_s": round(kr["committed"] / (kr["total_ms"] / 1000.0), 1),
                                   "tau_synthetic": round(kr["committed"] / (wsteps * kcfg.B), 4),
                                   "unwarped_tau_synthetic": round(ku["committed"] / (wsteps * kcfg.B), 4),
                                   "device_status": kr["status"] | ku["status"]}
            del kwts, ksets
    if not args.no_extra and args.config == "8b" and args.temp > 0:
        # the same workload drafted as a chain (top-k 1, 8 draft tokens): tree vs chain
        ccfg, _, cwts, csets = setup("8b_chain", args.temp, 4)
        csteps = max(20, args.steps // 4)
        cr = time_rounds(ccfg, cwts, csets, args.temp, csteps, 5)
        out["chain"] = {"workload": "8b shape, chain draft (top-k 1, depth 8, m 8)",
                        "trees_per_s": round(1000.0 * csteps / cr["total_ms"] * ccfg.B, 2),
                        "committed_tokens_per_s": round(cr["committed"] / (cr["total_ms"] / 1000.0), 1),
                        "tau_synthetic": round(cr["committed"] / (csteps * ccfg.B), 4)}
        del csets, cwts
        # EAGLE-1's static tree against a chain with as many draft passes (depth 5 each)
        for key, name, desc in (("static_tree", "8b_static", "8b shape, static EAGLE-1-style tree (root 4 children, "
                                 "depth 5, 22 draft nodes, 14 slots)"),
                                ("chain5", "8b_chain5", "8b shape, chain draft of depth 5 (top-k 1, m 5)")):
            xcfg, _, xwts, xsets = setup(name, args.temp, 4)
            xsteps = max(20, args.steps // 4)
            xr = time_rounds(xcfg, xwts, xsets, args.temp, xsteps, 5)
            out[key] = {"workload": desc, "trees_per_s": round(1000.0 * xsteps / xr["total_ms"] * xcfg.B, 2),
                        "committed_tokens_per_s": round(xr["committed"] / (xr["total_ms"] / 1000.0), 1),
                        "tau_synthetic": round(xr["committed"] / (xsteps * xcfg.B), 4),
                        "device_status": xr["status"]}
            del xsets, xwts
    if not args.no_extra and args.config == "8b" and args.temp > 0:
        out["draft"] = time_drafting(cfg, wts, inps[0], args.temp, max(10, args.steps // 10), 3)
        torch.cuda.empty_cache()
    if not args.no_extra and args.config == "8b":
        # the other single-GPU shapes: 13B (MHA), the 70B layer share (T = 1 and greedy), tiny fp32
        out["configs"] = {}
        for name, T2 in (("13b", 1.0), ("70b", 1.0), ("70b", 0.0), ("tiny", 1.0)):
            ocfg, _, owts, osets = setup(name, T2, 4)
            osteps = max(20, args.steps // 2)
            o = time_rounds(ocfg, owts, osets, T2, osteps, 5)
            oms = o["total_ms"] / osteps
            optot = int(sum(int(x.prefix_len.sum().item()) for x in osets) / len(osets))
            orows = ocfg.B * ocfg.N
            olb = lmhead_bytes(ocfg, orows, owts)
            out["configs"][f"{name}" + ("" if T2 > 0 else "_greedy")] = {
                "workload": f"{ocfg.name}: hidden {ocfg.H}, {ocfg.hq}q/{ocfg.hkv}kv x {ocfg.dh}, prefix {ocfg.Lmax}, "
                            f"vocab {ocfg.V}, depth {ocfg.D}, top-k {ocfg.k}, m {ocfg.m}, T={T2}, {ocfg.dtype}",
                "trees_per_s": round(1000.0 / oms * ocfg.B, 2), "ms_per_step": round(oms, 4),
                "committed_tokens_per_s": round(o["committed"] / (o["total_ms"] / 1000.0), 1),
                "tau_synthetic": round(o["committed"] / (osteps * ocfg.B), 4),
                "round_hbm_fraction": round(round_bytes(ocfg, optot, owts) / (oms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
                "round_bf16_w_fraction": round(round_bytes(ocfg, optot) / (oms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
                "lmhead_ms": round(o["lm_ms"], 5),
                "lmhead_hbm_frac": round(olb / (o["lm_ms"] / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
                "device_status": o["status"]}
            del osets, owts
    if not args.no_extra and args.config == "8b":
        gsteps = max(20, args.steps // 4)
        g = time_rounds(cfg, wts, sets, 0.0, gsteps, 5)
        out["greedy"] = {"trees_per_s": round(1000.0 * gsteps / g["total_ms"] * cfg.B, 2),
                         "committed_tokens_per_s": round(g["committed"] / (g["total_ms"] / 1000.0), 1),
                         "lmhead_ms": round(g["lm_ms"], 5)}
        del sets
        torch.cuda.empty_cache()
        try:
            cfg64, inps64, wts64, sets64 = setup("b64", 1.0, 2)
            b = time_rounds(cfg64, wts64, sets64, 1.0, 10, 2)
            ms64 = b["total_ms"] / 10
            flops = 2.0 * cfg64.B * cfg64.N * cfg64.H * cfg64.V
            bc = time_rounds(cfg64, wts64, sets64, 1.0, 10, 2, compact=True)
            msc = bc["total_ms"] / 10
            b64_compact = {"trees_per_s": round(1000.0 / msc * cfg64.B, 1), "ms_per_round": round(msc, 3),
                           "committed_tokens_per_s": round(bc["committed"] / (bc["total_ms"] / 1000.0), 1),
                           "lmhead_ms": round(bc["lm_ms"], 4),
                           "lmhead_mfma_frac": round(flops / (bc["lm_ms"] / 1000.0) / 1e12 / BF16_PEAK_TFLOPS, 4),
                           "device_status": bc["status"]}
            out["b64"] = {"trees_per_s": round(1000.0 / ms64 * cfg64.B, 1), "ms_per_round": round(ms64, 3),
                          "draft": time_drafting(cfg64, wts64, inps64[0], 1.0, 3, 1),
                          "committed_tokens_per_s": round(b["committed"] / (b["total_ms"] / 1000.0), 1),
                          "lmhead_ms": round(b["lm_ms"], 4),
                          "lmhead_mfma_frac": round(flops / (b["lm_ms"] / 1000.0) / 1e12 / BF16_PEAK_TFLOPS, 4),
                          "commit": time_commit(cfg64, wts64, inps64[0], sets64[0].rows, 1.0),
                          "compact": b64_compact}
            del sets64, wts64
        except Exception as e:  # report, do not hide the main line
            out["b64"] = {"error": repr(e)[:200]}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.config, args.temp, inps[0])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
