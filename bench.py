"""Benchmark of the LCT codec's hot path on one MI355X.

Workload: a Qwen3-4B-shaped parameter set (36 layers, hidden 2560, FFN 9728,
32 q / 8 kv heads of dim 128, vocab 151936, tied embeddings) flattened to
4,022,468,096 BF16 elements, W ~ N(0, 0.02^2) and a momentum buffer
M ~ N(0, 1e-3^2), both resident in HBM; CLEAN layout (65,536-element blocks,
25 words per stream); eta = 1e-3.  Inputs are synthetic and seeded: the pages'
fine-tuning runs used trained weights and data that are not available.

One step = the whole hot path over the set:
    encode  W (dense BF16)          -> compressed W        (lct_encode)
    update  W' = W - eta * M        on compressed W and M  (lct_sgd_step, in place)
    decode  W' (compressed)         -> dense BF16 W        (lct_decode)
The codebooks (lct_codebook_build) are set up once, as the pages prescribe
(no codebook is built during training); their build time is reported apart.

Prints one JSON line.  Per-op times come from HIP events recorded on the
stream the kernels run on; `roofline` is for the op that takes longest, with
its algorithmic bytes (what the format must move: BF16 in/out, the compressed
sides and spilled bytes) over its mean duration.  `cpu_baseline` times the
plain C oracle on a bounded sample of the same blocks (and checks the GPU's
bytes for those blocks against it).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, AMD's published figure
# VALU: 256 CUs x 4 SIMDs x 16 lanes at the 2.4 GHz peak clock (a wave64
# instruction takes four cycles of a 16-lane SIMD)
PEAK_VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
METRIC = "encode/decode GB/s of BF16 input, fused SGD elems/s, % HBM peak, comp. ratio"


def kernel_source_hash() -> str:
    """Hash of the kernels' source with comments and blank space removed, so
    that a change of comments alone keeps recorded counters valid."""
    p = os.path.join(ROOT, "lossless_bf16_tensor_split_amd", "csrc", "kernels.hip")
    src = open(p, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def load_counters(kernel: str, workload: str):
    """Issue counters per launch of a kernel from the committed rocprofv3
    summary, if it exists for this workload and the kernel source is unchanged."""
    path = os.path.join(ROOT, "profiles", "sq_codec_kernels_%s.md" % workload)
    if not os.path.exists(path):
        return None
    m = re.search(r"^counters_json:\s*(\{.*\})\s*$", open(path).read(), re.M)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_source") != kernel_source_hash():
        return None
    return d.get("per_dispatch", {}).get(kernel)


def copy_ceiling(dev, mib=2048, reps=5):
    """What a plain device copy reaches on this HBM (torch's copy of `mib` MiB,
    read plus write bytes over the median time)."""
    import numpy as np
    import torch
    nb = mib << 20
    src = torch.empty(nb, dtype=torch.uint8, device=dev)
    dst = torch.empty(nb, dtype=torch.uint8, device=dev)
    src.fill_(1)
    ms = []
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    t = float(np.median(ms[1:])) / 1e3
    return {"GBps": round(2 * nb / t / 1e9, 1), "bytes": 2 * nb, "kind": "torch device copy, median of %d" % reps}


def load_traffic(kernel: str, workload: str):
    """HBM traffic per launch from a committed rocprofv3 --pmc summary, if one
    exists for this kernel and workload and the kernel source is unchanged."""
    path = os.path.join(ROOT, "profiles", "pmc_%s_%s.md" % (kernel, workload))
    if not os.path.exists(path):
        return None
    m = re.search(r"^traffic_json:\s*(\{.*\})\s*$", open(path).read(), re.M)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_source") != kernel_source_hash():
        return None
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_4b", choices=["qwen3_4b", "gpt162m"])
    ap.add_argument("--cpu-blocks", type=int, default=2048,
                    help="blocks in the oracle's CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-whole-set", action="store_true",
                    help="skip the threaded oracle's check of every block (CPU leg)")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the momentum step timed after the headline step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed steps, copy a buffer of this many MiB once (a plain "
                         "device copy whose HBM bytes are known, to scale rocprofv3 byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the codec would shard by blocks, with one exchange of spilled totals "
              "for the overflow offsets). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import lossless_bf16_tensor_split_amd as L
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()

    if args.workload == "qwen3_4b":
        wspec, mspec, mw, mm, eta = synth.config5()
        wname = "qwen3_4b"
        desc = ("Qwen3-4B-shaped parameter set (tied embeddings), flat, 4,022,468,096 BF16 "
                "elements; W ~ N(0, 0.02^2), M ~ N(0, 1e-3^2); CLEAN 65536/25; eta 1e-3")
    else:
        ws, ms, mw, mm, eta = synth.config3()
        n = sum(s.numel for s in ws)
        wspec = synth.TensorSpec("W.flat", (n,), 3000, "normal", {"sigma": 0.02})
        mspec = synth.TensorSpec("M.flat", (n,), 3001, "normal", {"sigma": 1e-3})
        wname = "gpt162m"
        desc = ("GPT-style 162M parameter set, flat, 162,201,600 BF16 elements; "
                "W ~ N(0, 0.02^2), M ~ N(0, 1e-3^2); CLEAN 65536/25; eta 1e-3")
    n = wspec.numel
    lay = L.lct_layout_init(L.CLEAN)

    # ---------------- set-up (untimed): inputs resident in HBM, codebooks, buffers
    w_dense = synth.draw_device(wspec, dev)
    m_dense = synth.draw_device(mspec, dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cbw = L.lct_codebook_build(L.Model(mw.family, mw.scale, mw.shape), w_dense)
    t_cb = time.perf_counter() - t0
    cbm = L.lct_codebook_build(L.Model(mm.family, mm.scale, mm.shape), m_dense)
    ovf_cap = max(n // 64, 1 << 20)
    scratch = torch.empty(L.lct_sizes(n, lay, ovf_cap).scratch, dtype=torch.uint8, device=dev)
    tw = L.alloc_tensor(n, lay, ovf_cap, dev, scratch)          # encode target
    tm = L.alloc_tensor(n, lay, ovf_cap, dev, scratch)
    L.lct_encode(cbm, m_dense, tm)
    torch.cuda.synchronize()
    assert tm.status_word() == 0, "M overflow capacity exceeded"
    # the update writes W' in place on W's fixed side; its overflow goes to a
    # second region (the overflow side ping-pongs)
    tw2 = L.alloc_tensor(n, lay, ovf_cap, dev, scratch)
    tw2.sf, tw2.pay, tw2.cnt, tw2.obase = tw.sf, tw.pay, tw.cnt, tw.obase
    cpu_in = None
    if not args.no_cpu_baseline:
        # inputs of the CPU leg, taken before anything is overwritten: the
        # sampled blocks of W and M and the shift samples
        blocks = sample_blocks(tw.sizes.nblk, n, lay.block_elems, args.cpu_blocks)
        pos = torch.as_tensor(sample_positions(n), device=dev)
        cpu_in = {"blocks": blocks,
                  "w_blocks": host_blocks_dense(w_dense, blocks, lay.block_elems),
                  "m_blocks": host_blocks_dense(m_dense, blocks, lay.block_elems),
                  "w_sample": w_dense.view(torch.int16)[pos].cpu().numpy().view(np.uint16),
                  "m_sample": m_dense.view(torch.int16)[pos].cpu().numpy().view(np.uint16)}
    whole = None
    if cpu_in is not None and not args.no_whole_set:
        whole = WholeSet(cpu_in, mw, mm, eta, lay, n)
    else:
        del m_dense
        torch.cuda.empty_cache()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
          for _ in range(args.warmup + args.steps)]

    def step(i):
        e = ev[i]
        e[0].record(stream)
        L.lct_encode(cbw, w_dense, tw)
        e[1].record(stream)
        L.lct_sgd_step(cbw, tw, cbm, tm, eta, tw2)
        e[2].record(stream)
        L.lct_decode(cbw, tw2, w_dense)
        e[3].record(stream)

    # the first step runs op by op so that the CPU leg can check each output
    cpu = None
    if cpu_in is not None:
        blocks = cpu_in["blocks"]
        L.lct_encode(cbw, w_dense, tw)
        torch.cuda.synchronize()
        st_enc = tw.status_word()
        g_enc = host_blocks_compressed(tw, blocks)
        g_m = host_blocks_compressed(tm, blocks)
        if whole is not None:
            whole.encode(w_dense, m_dense, tw, tm)
            del m_dense
            torch.cuda.empty_cache()
        L.lct_sgd_step(cbw, tw, cbm, tm, eta, tw2)
        torch.cuda.synchronize()
        st_sgd = tw2.status_word()
        g_sgd = host_blocks_compressed(tw2, blocks)
        if whole is not None:
            whole.sgd(tw2)
        L.lct_decode(cbw, tw2, w_dense)
        torch.cuda.synchronize()
        g_dec = host_blocks_dense(w_dense, blocks, lay.block_elems)
        if whole is not None:
            whole.decode(w_dense)
        cpu = cpu_baseline_leg(cpu_in, (g_enc, g_m, g_sgd, g_dec), cbw, cbm, mw, mm, eta, lay, n)
        if whole is not None:
            cpu["threaded"] = whole.result()
            del whole
    else:
        step(0)
        torch.cuda.synchronize()
        st_enc, st_sgd = tw.status_word(), tw2.status_word()
    ratio_w, ratio_m = tw.ratio(), tm.ratio()
    spill_w, spill_m = tw.spilled(), tm.spilled()

    for i in range(1, args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    assert tw.status_word() == 0 and tw2.status_word() == 0, "overflow capacity exceeded"

    if args.copy_calibration:
        nb = args.copy_calibration << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    copy = copy_ceiling(dev)
    timed = ev[args.warmup:]
    t_enc = float(np.mean([e[0].elapsed_time(e[1]) for e in timed])) / 1e3
    t_sgd = float(np.mean([e[1].elapsed_time(e[2]) for e in timed])) / 1e3
    t_dec = float(np.mean([e[2].elapsed_time(e[3]) for e in timed])) / 1e3
    t_step = float(np.mean([e[0].elapsed_time(e[3]) for e in timed])) / 1e3

    fixed = tw.sizes.fixed
    alg = {
        "encode": 2 * n + fixed + tw.spilled(),
        "decode": fixed + tw2.spilled() + 2 * n,
        "sgd": fixed + tw.spilled() + fixed + tm.spilled() + fixed + tw2.spilled(),
    }
    times = {"encode": t_enc, "decode": t_dec, "sgd": t_sgd}
    # the dominant kernel of each op (the update's full blocks at CLEAN: the
    # ring kernel; its general twin finds no block to do here)
    kname = {"encode": "k_encode", "decode": "k_decode", "sgd": "k_sgd_ring" if lay.cap_words == 25 else "k_sgd"}
    per_op = {}
    for op in ("encode", "decode", "sgd"):
        gbs = alg[op] / times[op] / 1e9
        per_op[op] = {"ms": round(times[op] * 1e3, 4), "alg_bytes": int(alg[op]),
                      "alg_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    for op in per_op:
        per_op[op]["copy_frac"] = round(per_op[op]["alg_GBps"] / copy["GBps"], 4)
    per_op["encode"]["GBps_bf16_input"] = round(2 * n / t_enc / 1e9, 1)
    per_op["decode"]["GBps_bf16_output"] = round(2 * n / t_dec / 1e9, 1)
    per_op["sgd"]["elems_per_s"] = float("%.4g" % (n / t_sgd))
    dom = max(times, key=times.get)
    traffic = load_traffic(kname[dom], wname)
    counters = load_counters(kname[dom], wname)
    achieved = alg[dom] / times[dom] / 1e9
    valu = None
    if counters and "SQ_INSTS_VALU" in counters:
        lane_ops = 64.0 * counters["SQ_INSTS_VALU"] / times[dom]
        valu = {"achieved": float("%.4g" % lane_ops), "peak": PEAK_VALU_LANE_OPS, "unit": "lane-ops/s",
                "frac": round(lane_ops / PEAK_VALU_LANE_OPS, 4),
                "source": "SQ_INSTS_VALU per launch from profiles/sq_codec_kernels_%s.md" % wname}
    # The momentum step (SGD with momentum) on the same workload, timed after
    # the headline step and outside `value`: W (the update's output; the
    # headline step's byte counts are taken above, before these calls rewrite
    # the offsets) and M compressed and resident, a dense BF16 gradient; W' and M' are written in
    # place on the fixed sides while the overflow regions ping-pong between
    # two sets, so every call reads a consistent (W, M) pair.  Each call gets a
    # fresh gradient g ~ N(0, s^2 (1 - mu^2)) with s the spread of M, drawn
    # untimed: then M' = mu*M + g keeps M's distribution (the stationary spread
    # of heavy-ball momentum under independent gradients), as in a run whose
    # momentum has settled.
    next_ops = None
    if not args.no_next:
        mu, reps = 0.9, 6
        g_sigma = mspec.args["sigma"] * math.sqrt(1.0 - mu * mu)
        scratch2 = torch.empty(L.lct_sizes(n, lay, ovf_cap).scratch, dtype=torch.uint8, device=dev)
        tm.scratch = scratch2
        sets = [(tw2, tm)]
        bw = L.alloc_tensor(n, lay, ovf_cap, dev, scratch)
        bm = L.alloc_tensor(n, lay, ovf_cap, dev, scratch2)
        bw.sf, bw.pay, bw.cnt, bw.obase = tw.sf, tw.pay, tw.cnt, tw.obase
        bm.sf, bm.pay, bm.cnt, bm.obase = tm.sf, tm.pay, tm.cnt, tm.obase
        sets.append((bw, bm))
        torch.cuda.empty_cache()
        alg_mom, mom_status = [], 0
        mev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(reps + 1):
            (wi, mi), (wo, mo) = sets[i % 2], sets[(i + 1) % 2]
            spill_in = wi.spilled() + mi.spilled()
            g_dense = synth.draw_device(synth.TensorSpec("g.flat", (n,), wspec.seed + 100 + i, "normal",
                                                         {"sigma": g_sigma}), dev)
            torch.cuda.synchronize()
            if i:
                mev[i - 1][0].record(stream)
            L.lct_momentum_step(cbw, wi, cbm, mi, g_dense, mu, eta, wo, mo)
            if i:
                mev[i - 1][1].record(stream)
            torch.cuda.synchronize()
            mom_status = max(mom_status, wo.status_word(), mo.status_word())
            del g_dense
            if i:
                alg_mom.append(4 * tw.sizes.fixed + 2 * n + spill_in + wo.spilled() + mo.spilled())
        t_mom = float(np.mean([e[0].elapsed_time(e[1]) for e in mev])) / 1e3
        bytes_mom = float(np.mean(alg_mom))
        gbs = bytes_mom / t_mom / 1e9
        mtraffic = load_traffic("k_mom", wname)
        next_ops = {"momentum": {"ms": round(t_mom * 1e3, 4), "alg_bytes": int(bytes_mom),
                                 "alg_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                                 "elems_per_s": float("%.4g" % (n / t_mom)), "mu": mu,
                                 "g_sigma": float("%.4g" % g_sigma),
                                 "status": mom_status,
                                 "traffic": None if mtraffic is None else mtraffic.get("bytes_per_launch")}}
        # shift re-estimation on the momentum step's last W': 4096 elements
        # decoded from the compressed form on the device, the shift search and
        # the new tables on the host (a synchronising call, timed on the host)
        L.lct_codebook_reshift(cbw, wo)
        tr = []
        for _ in range(5):
            t0 = time.perf_counter()
            new = L.lct_codebook_reshift(cbw, wo)
            tr.append(time.perf_counter() - t0)
        next_ops["reshift"] = {"ms": round(1e3 * float(np.median(tr)), 4), "sample": 4096,
                               "shift_before": int(cbw.shift), "shift_after": int(new.shift)}
        del sets, bw, bm, wi, mi, wo, mo
        torch.cuda.empty_cache()
        next_ops["activations"] = activation_leg(L, dev)
        if args.workload == "qwen3_4b":
            next_ops["group"] = group_leg(L, dev, stream, w_dense, mspec, mw, mm, eta, lay)
            del w_dense, tw, tw2, tm, scratch, scratch2
            torch.cuda.empty_cache()
            next_ops["configs"] = configs_leg(L, dev, stream)

    out = {
        "metric": METRIC,
        "value": float("%.5g" % (n / t_step)),
        "unit": "elems/s (encode + fused SGD + decode of every element, one step)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32 codec / f32 update",
        "data": "synthetic (seeded device draws)",
        "config": {"workload": desc, "elements": n, "block_elems": lay.block_elems,
                   "cap_words": lay.cap_words, "eta": eta, "parallelism": "single GPU"},
        "per_op": per_op,
        "compression_ratio": {"W": round(ratio_w, 5), "M": round(ratio_m, 5),
                              "payload_bound": round(16.0 / (8 + 32.0 * lay.cap_words / 256), 5)},
        "spilled_bytes": {"W": spill_w, "M": spill_m},
        "status": {"encode": st_enc, "sgd": st_sgd},
        "codebook_build_ms": round(t_cb * 1e3, 3),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": kname[dom], "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None if traffic is None else traffic.get("bytes_per_launch"),
                     "secondary_valu": valu},
        "hbm_copy": copy,
        "cpu_baseline": cpu,
        "next_ops": next_ops,
    }
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ the other workloads

def configs_leg(L, dev, stream, reps=5):
    """Per-op throughput on the smaller workloads, each op timed alone with
    HIP events (median of `reps`) after a 1 GiB write that evicts the 256 MB
    last-level cache, so that every input comes from HBM:
      - the 2^20-element Gaussian tensor (CLEAN): encode, decode;
      - the three 2^26-element tensors (Laplace, Student-t(3), N(0,1) scaled by
        2^k per 2^20 chunk) in MEDIUM and HIGH, whose streams overflow:
        encode, decode;
      - the flat 162M-parameter GPT-style set (CLEAN): encode W, the fused
        update, decode W';
      - the Qwen3-4B layer's activations (post-SiLU gate, residual with
        outliers, uniform random bits) in CLEAN and MEDIUM: encode, decode.
    Each entry gives GB/s of BF16 input (output for decode), the algorithmic
    bytes (BF16 side, compressed sides, spilled bytes) over the time as a
    fraction of 8 TB/s, the compression ratio, the overflow fraction (spilled
    fields per element), the allocated bits per exponent ((payload +
    overflow bits) / n) and the occupancy the tensor gives the encode and
    decode (their waves, and waves per SIMD of the chip)."""
    import numpy as np
    import torch
    import synth

    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def timed(fn):
        ms = []
        for _ in range(reps):
            flush.fill_(7)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms)) / 1e3

    def entry(t, s, alg, n, inout):
        gbs = alg / s / 1e9
        return {"ms": round(s * 1e3, 4), inout: round(2 * n / s / 1e9, 1),
                "alg_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}

    def codec(x16, model, mode, sgd_with=None):
        n = x16.numel()
        lay = L.lct_layout_init(mode)
        cb = L.lct_codebook_build(L.Model(model.family, model.scale, model.shape), x16)
        t = L.alloc_tensor(n, lay, None, dev)
        y = torch.empty_like(x16)
        t_enc = timed(lambda: L.lct_encode(cb, x16, t))
        st = t.status_word()
        sp = t.spilled()
        t_dec = timed(lambda: L.lct_decode(cb, t, y))
        same = bool(torch.equal(y.view(torch.int16), x16.view(torch.int16)))
        fixed = t.sizes.fixed
        nblk = (n + lay.block_elems - 1) // lay.block_elems
        out = {"n": n, "mode": {0: "CLEAN", 1: "MEDIUM", 2: "HIGH"}[mode],
               "layout": [lay.block_elems, lay.cap_words],
               # one wave per 64 streams of a block, over the chip's 1,024 SIMDs
               "waves": 4 * nblk, "waves_per_simd": round(4 * nblk / 1024.0, 3),
               "encode": entry(t, t_enc, 2 * n + fixed + sp, n, "GBps_bf16_input"),
               "decode": entry(t, t_dec, 2 * n + fixed + sp, n, "GBps_bf16_output"),
               "ratio": round(t.ratio(), 5), "overflow_fraction": round(sp / n, 6),
               "bits_per_exponent": round(8.0 * (t.sizes.pay + sp) / n, 4),
               "status": st, "decoded_identical": same}
        return out, cb, t

    res = {"cache_flush": "1 GiB written before every timed op"}
    x = torch.from_numpy(synth.draw(synth.config1()[0][0]).view(np.int16)).to(dev)
    res["gauss_2^20"], _, _ = codec(x, synth.config1()[0][1], L.CLEAN)
    for spec, model in synth.config2():
        x = torch.from_numpy(synth.draw(spec).view(np.int16)).to(dev)
        for mode in (L.MEDIUM, L.HIGH):
            res["%s_2^26_%s" % (spec.name, {1: "medium", 2: "high"}[mode])], _, t = codec(x, model, mode)
            del t
        del x
        torch.cuda.empty_cache()
    # the 162M-parameter set: the step's three ops
    ws, ms, mw, mm, eta = synth.config3()
    n = sum(s.numel for s in ws)
    w = synth.draw_device(synth.TensorSpec("W.flat", (n,), 3000, "normal", {"sigma": 0.02}), dev)
    m = synth.draw_device(synth.TensorSpec("M.flat", (n,), 3001, "normal", {"sigma": 1e-3}), dev)
    e, cbw, tw = codec(w, mw, L.CLEAN)
    cbm = L.lct_codebook_build(L.Model(mm.family, mm.scale, mm.shape), m)
    tm = L.alloc_tensor(n, tw.layout, n, dev)
    L.lct_encode(cbm, m, tm)
    out = L.alloc_tensor(n, tw.layout, n, dev)
    t_sgd = timed(lambda: L.lct_sgd_step(cbw, tw, cbm, tm, eta, out))
    fixed = tw.sizes.fixed
    alg = 3 * fixed + tw.spilled() + tm.spilled() + out.spilled()
    e["sgd"] = {"ms": round(t_sgd * 1e3, 4), "elems_per_s": float("%.4g" % (n / t_sgd)),
                "alg_GBps": round(alg / t_sgd / 1e9, 1), "hbm_frac": round(alg / t_sgd / 1e9 / PEAK_HBM_GBS, 4),
                "status": out.status_word()}
    res["gpt162m_flat"] = e
    del w, m, tw, tm, out
    torch.cuda.empty_cache()
    for spec, model in synth.config4():
        x = torch.from_numpy(synth.draw(spec).view(np.int16)).to(dev)
        for mode in (L.CLEAN, L.MEDIUM):
            res["act_%s_%s" % (spec.name, {0: "clean", 1: "medium"}[mode])], _, t = codec(x, model, mode)
            del t
        del x
    del flush
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ tensor groups

def group_leg(L, dev, stream, w_dense, mspec, mw, mm, eta, lay, reps=5):
    """The same step on the Qwen3-4B parameter set as its 398 tensors (each
    with its own codebook: the model's base code, the shift from its own
    sample), one group launch per op and one shared overflow region, against
    the same tensors one call each."""
    import numpy as np
    import torch
    import synth

    ns = [int(np.prod(s)) for _, s in synth.qwen3_4b_shapes()]
    offs = np.concatenate([[0], np.cumsum(ns)])
    assert offs[-1] == w_dense.numel() and all(o % 8 == 0 for o in offs)   # 16-byte aligned slices
    m_dense = synth.draw_device(mspec, dev)
    wv = [w_dense[offs[k]:offs[k + 1]] for k in range(len(ns))]
    mv = [m_dense[offs[k]:offs[k + 1]] for k in range(len(ns))]
    basew = L.lct_codebook_build(L.Model(mw.family, mw.scale, mw.shape), None)
    basem = L.lct_codebook_build(L.Model(mm.family, mm.scale, mm.shape), None)
    t0 = time.perf_counter()
    cw = [L.lct_codebook_reshift_dense(basew, v) for v in wv]
    t_cb = time.perf_counter() - t0
    cm = [L.lct_codebook_reshift_dense(basem, v) for v in mv]
    gw = L.LctGroup(ns, lay, cw, wv)
    gm = L.LctGroup(ns, lay, cm, mv)
    cap = sum(ns) // 64
    w_all, m_all = gw.alloc_storage(cap), gm.alloc_storage(cap)
    L.lct_encode_group(gm, m_all)
    w_out = gw.alloc_storage(cap, scratch=w_all.scratch)
    w_out.sf, w_out.pay, w_out.cnt, w_out.obase = w_all.sf, w_all.pay, w_all.cnt, w_all.obase

    def group_step(e):
        e[0].record(stream)
        L.lct_encode_group(gw, w_all)
        e[1].record(stream)
        L.lct_sgd_step_group(gw, w_all, gm, m_all, eta, w_out)
        e[2].record(stream)
        L.lct_decode_group(gw, w_out)
        e[3].record(stream)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps + 2)]
    for e in ev:
        group_step(e)
    torch.cuda.synchronize()
    status = [w_all.status_word(), w_out.status_word(), m_all.status_word()]
    timed = ev[2:]
    ms = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in timed]))
          for i, name in enumerate(["encode", "sgd", "decode"])}
    ms["step"] = float(np.mean([e[0].elapsed_time(e[3]) for e in timed]))
    spilled = [w_all.spilled(), m_all.spilled(), w_out.spilled()]
    # the momentum step on the groups: the gradients bound as a third group's
    # dense buffers, W' and M' in place with overflow regions of their own
    g_dense = synth.draw_device(synth.TensorSpec("g.flat", (sum(ns),), 5300, "normal",
                                                 {"sigma": mspec.args["sigma"] * math.sqrt(1 - 0.81)}), dev)
    gg = L.LctGroup(ns, lay, cm, [g_dense[offs[k]:offs[k + 1]] for k in range(len(ns))])
    m_out = gm.alloc_storage(cap)
    m_out.sf, m_out.pay, m_out.cnt, m_out.obase = m_all.sf, m_all.pay, m_all.cnt, m_all.obase
    mev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(3)]
    L.lct_encode_group(gw, w_all)
    for e in mev:
        # each call reads the previous call's results (W' and M' in place)
        e[0].record(stream)
        L.lct_momentum_step_group(gw, w_all, gm, m_all, gg, 0.9, eta, w_out, m_out)
        e[1].record(stream)
        torch.cuda.synchronize()
        w_all, w_out = w_out, w_all
        m_all, m_out = m_out, m_all
    t_mom = float(np.mean([e[0].elapsed_time(e[1]) for e in mev]))
    mom_status = [w_all.status_word(), m_all.status_word()]
    del g_dense, gg, m_out
    # the same encodes as one call per tensor (each tensor its own storage)
    singles = [L.alloc_tensor(n, lay, max(n // 64, 1024), dev) for n in ns]
    for k in range(len(ns)):
        L.lct_encode(cw[k], wv[k], singles[k])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(len(ns)):
        L.lct_encode(cw[k], wv[k], singles[k])
    e1.record(stream)
    torch.cuda.synchronize()
    t_singles = e0.elapsed_time(e1)
    nblk = int(gw.g.nblk)
    del singles, m_dense, w_all, m_all, w_out, gw, gm
    torch.cuda.empty_cache()
    return {"workload": "Qwen3-4B-shaped parameter set as %d tensors (%d blocks), one group each for W and M"
                        % (len(ns), nblk),
            "ms": {k: round(v, 4) for k, v in ms.items()},
            "elems_per_s": float("%.4g" % (sum(ns) / (ms["step"] / 1e3))),
            "momentum_ms": round(t_mom, 4), "momentum_status": mom_status,
            "encode_one_call_per_tensor_ms": round(t_singles, 4),
            "codebooks_ms": round(1e3 * t_cb, 2), "spilled_bytes": spilled, "status": status}


# ------------------------------------------------------------------ saved activations

def activation_leg(L, dev, seq=3500, hid=2560, ffn=9728, reps=5):
    """One Qwen3-4B-shaped MLP block with its residual at batch 1 and the given
    sequence length, x + down(silu(gate(x)) * up(x)), random weights (std
    0.02) and inputs: forward and backward timed with autograd's saved tensors
    kept as they are, then kept compressed (encoded when saved, decoded when
    backward reads them) by one codec entered each step, as a training loop
    would (its setup, staging pool and pinned words, made once); the time with
    a new codec made inside every step is reported beside it."""
    import numpy as np
    import torch
    from lossless_bf16_tensor_split_amd.activations import ActivationCodec, compressed_activations

    f = torch.nn.functional
    gen = torch.Generator(device=dev)
    gen.manual_seed(9000)

    def randn(*shape, scale=1.0):
        return (torch.randn(*shape, generator=gen, device=dev) * scale).to(torch.bfloat16)

    x = randn(seq, hid).requires_grad_()
    ws = [randn(ffn, hid, scale=0.02).requires_grad_(), randn(ffn, hid, scale=0.02).requires_grad_(),
          randn(hid, ffn, scale=0.02).requires_grad_()]

    def step():
        y = x + f.linear(f.silu(f.linear(x, ws[0])) * f.linear(x, ws[1]), ws[2])
        y.float().square().mean().backward()

    def grads(compress):
        for t in [x] + ws:
            t.grad = None
        if compress:
            with compressed_activations(L.Model(L.POWERLAW, 1.0, 3.0)):
                step()
        else:
            step()
        torch.cuda.synchronize()
        return [t.grad.clone() for t in [x] + ws]

    def timed(compress, fresh=False):
        codec, ms = None, []
        if compress and not fresh:
            codec = ActivationCodec(L.Model(L.POWERLAW, 1.0, 3.0))
        for i in range(reps + 2):
            for t in [x] + ws:
                t.grad = None
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if compress and fresh:
                with compressed_activations(L.Model(L.POWERLAW, 1.0, 3.0)) as codec:
                    step()
            elif compress:
                with codec:
                    step()
            else:
                step()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ms.append(e0.elapsed_time(e1))
        return float(np.median(ms)), codec

    g_plain, g_again, g_lct = grads(False), grads(False), grads(True)
    same = all(torch.equal(a, b) for a, b in zip(g_plain, g_lct))
    repro = all(torch.equal(a, b) for a, b in zip(g_plain, g_again))
    del g_plain, g_again, g_lct
    t_plain, _ = timed(False)
    t_fresh, _ = timed(True, fresh=True)
    t_lct, codec = timed(True)
    steps = reps + 2
    return {"workload": "Qwen3-4B-shaped MLP block, seq %d, hidden %d, FFN %d, BF16" % (seq, hid, ffn),
            "ms_plain": round(t_plain, 3), "ms_compressed": round(t_lct, 3),
            "step_time_increase": round(t_lct / t_plain - 1.0, 4),
            "ms_compressed_new_codec_each_step": round(t_fresh, 3),
            "saved_tensors": codec.saved // steps, "saved_raw_bytes": codec.raw_bytes // steps,
            "saved_stored_bytes": codec.stored_bytes // steps, "ratio": round(codec.ratio(), 5),
            "host_ms_in_save_hooks": round(1e3 * codec.pack_s / steps, 3),
            "host_ms_in_restore_hooks": round(1e3 * codec.unpack_s / steps, 3),
            "grads_identical": same, "plain_grads_reproducible": repro}


# ------------------------------------------------------------------ CPU-baseline leg

class WholeSet:
    """Every block of the step checked against the oracle run over ranges of
    whole blocks on the host's threads (its bytes equal the serial oracle's),
    op by op between the GPU's untimed first step; the oracle's time for the
    same step (encode W, naive SGD round trip, decode W') is the threaded
    baseline.  Works through 4096 blocks at a time."""

    CHUNK = 4096

    def __init__(self, cpu_in, mw, mm, eta, lay, n):
        import oracle
        self.orc = oracle
        self.threads = max(1, min(16, len(os.sched_getaffinity(0))))
        self.ocw = oracle.codebook_from_sample(mw.family, mw.scale, mw.shape, cpu_in["w_sample"])
        self.ocm = oracle.codebook_from_sample(mm.family, mm.scale, mm.shape, cpu_in["m_sample"])
        self.eta, self.lay, self.n = eta, lay, n
        self.B = lay.block_elems
        self.nblk = -(-n // self.B)
        self.ranges = [(b0, min(self.nblk, b0 + self.CHUNK)) for b0 in range(0, self.nblk, self.CHUNK)]
        self.rw, self.rm, self.ro = [], [], []
        self.ok = {"encode_W": True, "encode_M": True, "sgd_W": True, "decode_W": True}
        self.t = {"encode": 0.0, "sgd": 0.0, "decode": 0.0}

    def _chunk(self, t, b0, b1):
        import numpy as np
        B, cw = self.B, self.lay.cap_words
        e0, e1 = b0 * B, min(b1 * B, self.n)
        ob = t.obase[b0:b1 + 1].cpu().numpy().view(np.uint64)
        spill = t.ovf[int(ob[0]):int(ob[-1])].cpu().numpy()
        return self.orc.Compressed(e1 - e0, B, cw, t.sf[e0:e1].cpu().numpy(),
                                   t.pay[b0 * cw * 256:b1 * cw * 256].cpu().numpy().view(np.uint32),
                                   t.cnt[b0 * 256:b1 * 256].cpu().numpy().view(np.uint16),
                                   (ob - ob[0]).astype(np.uint64), spill if spill.size else np.zeros(1, np.uint8))

    @staticmethod
    def _same(a, b):
        import numpy as np
        return (all(np.array_equal(getattr(a, k), getattr(b, k)) for k in ("sf", "pay", "cnt", "obase"))
                and np.array_equal(a.ovf[:a.spilled], b.ovf[:b.spilled]))

    def _dense(self, x, b0, b1):
        import numpy as np
        import torch
        return x.view(torch.int16)[b0 * self.B:min(b1 * self.B, self.n)].cpu().numpy().view(np.uint16)

    def encode(self, w, m, tw, tm):
        cw, th = self.lay.cap_words, self.threads
        for b0, b1 in self.ranges:
            xw, xm = self._dense(w, b0, b1), self._dense(m, b0, b1)
            t0 = time.perf_counter()
            rw = self.orc.encode_threads(self.ocw, xw, self.B, cw, th)
            self.t["encode"] += time.perf_counter() - t0
            rm = self.orc.encode_threads(self.ocm, xm, self.B, cw, th)     # M's set-up: not timed
            self.ok["encode_W"] &= self._same(self._chunk(tw, b0, b1), rw)
            self.ok["encode_M"] &= self._same(self._chunk(tm, b0, b1), rm)
            self.rw.append(rw)
            self.rm.append(rm)

    def sgd(self, out):
        for (b0, b1), rw, rm in zip(self.ranges, self.rw, self.rm):
            t0 = time.perf_counter()
            ro = self.orc.sgd_threads(self.ocw, rw, self.ocm, rm, self.eta, self.threads)
            self.t["sgd"] += time.perf_counter() - t0
            self.ok["sgd_W"] &= self._same(self._chunk(out, b0, b1), ro)
            self.ro.append(ro)
        self.rw, self.rm = [], []

    def decode(self, y):
        import numpy as np
        for (b0, b1), ro in zip(self.ranges, self.ro):
            t0 = time.perf_counter()
            ry = self.orc.decode_threads(self.ocw, ro, self.threads)
            self.t["decode"] += time.perf_counter() - t0
            self.ok["decode_W"] &= bool(np.array_equal(self._dense(y, b0, b1), ry))
        self.ro = []

    def result(self):
        tot = sum(self.t.values())
        return {"value": float("%.4g" % (self.n / tot)), "unit": "elems/s", "cores": self.threads,
                "kind": "oracle",
                "sample": "every block (%d, %d elements): encode W, naive SGD round trip, decode W'; "
                          "the serial C routines over ranges of whole blocks on %d host threads, offsets "
                          "stitched serially; encode %.2f s, sgd %.2f s, decode %.2f s"
                          % (self.nblk, self.n, self.threads, self.t["encode"], self.t["sgd"], self.t["decode"]),
                "parity_whole_set": {k: bool(v) for k, v in self.ok.items()}}


def sample_blocks(nblk: int, n: int, B: int, want: int):
    """Evenly spread full blocks (the last, partial block is left out)."""
    import numpy as np
    full = n // B
    want = min(want, full)
    return np.unique(np.linspace(0, full - 1, want).round().astype(np.int64))


def host_blocks_dense(x, blocks, B):
    import torch
    idx = (torch.as_tensor(blocks, device=x.device)[:, None] * B +
           torch.arange(B, device=x.device)[None, :]).reshape(-1)
    return x.view(torch.int16)[idx].cpu().numpy().view("uint16")


def host_blocks_compressed(t, blocks):
    """The sampled blocks of a device tensor as one oracle tensor (offsets rebased)."""
    import numpy as np
    import torch

    import oracle
    B, cw = t.layout.block_elems, t.layout.cap_words
    dv = t.sf.device
    bt = torch.as_tensor(blocks, device=dv)

    def rows(buf, width):
        idx = (bt[:, None] * width + torch.arange(width, device=dv)[None, :]).reshape(-1)
        return buf[idx].cpu().numpy()

    sf = rows(t.sf, B)
    pay = rows(t.pay, cw * 256).view(np.uint32)
    cnt = rows(t.cnt, 256).view(np.uint16)
    ob = t.obase.cpu().numpy().view(np.uint64)
    spans = [(int(ob[b]), int(ob[b + 1])) for b in blocks]
    ovf_all = t.ovf
    parts = [ovf_all[a:b].cpu().numpy() for a, b in spans]
    ovf = np.concatenate(parts) if parts else np.zeros(0, np.uint8)
    obase = np.zeros(len(blocks) + 1, np.uint64)
    obase[1:] = np.cumsum([b - a for a, b in spans])
    return oracle.Compressed(len(blocks) * B, B, cw, sf, pay, cnt, obase,
                             ovf if ovf.size else np.zeros(1, np.uint8))


def sample_positions(n: int):
    """Positions floor(i * n / m), m = min(n, 4096), of a codebook's shift sample."""
    import numpy as np
    m = min(n, 4096)
    return ((np.arange(m, dtype=np.uint64) * np.uint64(n)) // np.uint64(max(m, 1))).astype(np.int64)


def cpu_baseline_leg(cpu_in, gpu_out, cbw, cbm, mw, mm, eta, lay, n):
    """Time the oracle on the sampled blocks for the same step (encode W,
    naive SGD round trip, decode W') and check the GPU's bytes against it."""
    import numpy as np

    import oracle
    import synth
    B, cw = lay.block_elems, lay.cap_words
    g_enc, g_m, g_sgd, g_dec = gpu_out
    # the oracle's own codebooks, from the model and the shift sample
    ocw = oracle.codebook_from_sample(mw.family, mw.scale, mw.shape, cpu_in["w_sample"])
    ocm = oracle.codebook_from_sample(mm.family, mm.scale, mm.shape, cpu_in["m_sample"])
    same_cb = (np.array_equal(np.frombuffer(bytes(cbw.len), np.uint8), ocw.len)
               and cbw.shift == ocw.shift and cbm.shift == ocm.shift
               and np.array_equal(np.frombuffer(bytes(cbm.len), np.uint8), ocm.len))
    rm = oracle.encode(ocm, cpu_in["m_blocks"], B, cw)     # set-up of M: not timed
    t0 = time.perf_counter()
    rw = oracle.encode(ocw, cpu_in["w_blocks"], B, cw)
    t1 = time.perf_counter()
    ro = oracle.sgd(ocw, rw, ocm, rm, eta)
    t2 = time.perf_counter()
    rd = oracle.decode(ocw, ro)
    t3 = time.perf_counter()
    t_oracle = t3 - t0

    def same(a, b):
        return all(np.array_equal(getattr(a, k), getattr(b, k))
                   for k in ("sf", "pay", "cnt", "obase")) \
            and np.array_equal(a.ovf[:a.spilled], b.ovf[:b.spilled])

    # the momentum step's oracle on the first 512 sampled blocks (naive round
    # trip: decode W and M, dense update, encode W' and M'), with a seeded
    # host gradient of the spread the GPU leg uses
    nm = min(512, len(cpu_in["blocks"])) * B
    gm = synth.to_bf16_bits(np.random.default_rng(5100).normal(0.0, 1e-3 * (1 - 0.81) ** 0.5, nm))
    mw_ = oracle.encode(ocw, cpu_in["w_blocks"][:nm], B, cw)
    mm_ = oracle.encode(ocm, cpu_in["m_blocks"][:nm], B, cw)
    t4 = time.perf_counter()
    oracle.momentum(ocw, mw_, ocm, mm_, gm, 0.9, eta)
    t_mom = time.perf_counter() - t4

    parity = {"codebooks": bool(same_cb), "encode_W": bool(same(g_enc, rw)),
              "encode_M": bool(same(g_m, rm)), "sgd_W": bool(same(g_sgd, ro)),
              "decode_W": bool(np.array_equal(g_dec, rd))}
    ns = len(cpu_in["blocks"]) * B
    return {"value": float("%.4g" % (ns / t_oracle)), "unit": "elems/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d evenly spread full blocks of %d (%d elements): encode W, naive SGD "
                      "round trip, decode W'; serial C; encode %.2f s, sgd %.2f s, decode %.2f s"
                      % (len(cpu_in["blocks"]), n // B, ns, t1 - t0, t2 - t1, t3 - t2),
            "parity_on_sample": parity,
            "next_ops": {"momentum": {"value": float("%.4g" % (nm / t_mom)), "unit": "elems/s",
                                      "sample": "the first %d sampled blocks (%d elements), %.2f s"
                                                % (nm // B, nm, t_mom)}}}


if __name__ == "__main__":
    main()
