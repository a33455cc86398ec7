"""Benchmark of the FP8 fine-grained-scaled NT GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all]

A step is one pass over the workload's GEMMs, each launched once through the
C ABI on the current stream with inputs already resident in HBM.  The default
workload (`all`) is every configuration of the FP8 GEMM family at its real
size: the dense sweep (M in {64,128,4096} x (N,K) in {(2112,7168),
(24576,1536), (32768,512), (7168,16384), (4096,7168), (7168,2048)}), the MoE
contiguous layout (G in {4,8} experts x 8192 rows, (N,K) in {(4096,7168),
(7168,2048)}), the masked decode (G in {1,2,4,16}, M_max=256, same (N,K)) and
the two weight gradients (7168x2048 over 4096 tokens, and over 4 experts of
1024..4096 tokens), A scaled per 1x128, B per 128x128 (or per row along
tokens), bf16 out (fp32 D for the weight gradients).  `value` is the step's
algorithmic FLOPs (2*M_valid*N*K per GEMM) over its measured time, in
TFLOP/s; the timed steps launch the GEMMs back to back.  A separate pass
brackets each GEMM by HIP events on the launch stream (the per-shape table
and the per-workload sub-results under `workloads`); the GEMM with the
largest time is the "dominant kernel", which is also bracketed by events
inside the timed steps, and whose roofline fraction is reported from those
(`roofline.achieved`), next to the median of 50 dispatches each after a
512 MB cache flush (`roofline.cold_median_us`).  The CPU oracle is timed on a
bounded sample of the same workload's outputs (`cpu_baseline`).  The masked
decode GEMMs are also captured into HIP graphs -- the default entry point and
the allocation-free one -- and their replays timed (`masked_graph`); the
contiguous G=8, N=4096, K=7168 GEMM is timed against its form with SwiGLU and
the FP8 re-quantise fused into the epilogue (`fused_swiglu`).

Other workloads (dense, contiguous, masked, wgrad, k_grouped_wgrad, small,
dense_ue8m0, contiguous_ue8m0, masked_ue8m0 -- those sweeps with packed UE8M0
scales --, bf16 -- the
sweep's shapes in BF16 against the bf16 peak --, grouped_bf16 -- contiguous and masked
problems in BF16 --, quantize, the FP8 quantiser
in GB/s, and swiglu_quantize, the SwiGLU + FP8 re-quantise step between an
expert's two GEMMs in GB/s, and contiguous_swiglu, the contiguous sweep with
SwiGLU + re-quantise fused into the GEMM) print a line of the same form.  Exactly one JSON
line goes to stdout.

Before the W warmup steps the step runs untimed for at least half a second so
the GPU clock has settled when timing starts.  `roofline.traffic` is the
dominant GEMM's HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE
counters (each scaled by what the counter reads for a plain device copy of
known size), stored in profiles/; it is reported only while the kernel sources
hash to the version the counters were taken on, else null.

    python bench.py --only NAME[,NAME]   time only the named GEMMs (for counters)
    python bench.py --cold               per-launch table with cold caches (512 MB
                                         flush before each call, outside its events)
    python bench.py --copy-calibration   run a plain 1 GiB device-to-device copy
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOPS (dense/grouped) and % of MI355X FP8 or HBM peak"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "moe_grouped_gemm_x128_amd", "csrc", f)
                  for f in ("dg_kernels.hip", "dg_api.hip", "dg_kernel.h", "dg_quant.hip", "dg_shapes.h",
                            "dg_shapes.hip", "dg_rsrc.h", "dg_fp8_codec.h")]
COLD_DISPATCHES = 50  # cold-cache dispatches of the dominant GEMM (median reported)


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per launch of GEMM `name` from the committed counter summary
    (the json block of profiles/hbm_traffic.md), or None if there is none for
    it or the kernel sources changed since the counters were taken."""
    try:
        text = open(TRAFFIC_FILE).read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(block)
    except (OSError, IndexError, ValueError):
        return None
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    entry = data.get("gemms", {}).get(name)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, three times (its FETCH_SIZE and
    WRITE_SIZE per dispatch calibrate the counters against known bytes)."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


class Call:
    """One GEMM launch of the step plus its algorithmic work.  sample(rng,
    count): the oracle on `count` uniformly drawn outputs of this GEMM,
    returning the FLOPs that took (GEMMs) or (sample, width) for the
    quantisers' row passes."""

    def __init__(self, name, flops, nbytes, fn, sample=None, peak=PEAK_FP8_TFLOPS, group=""):
        self.name, self.flops, self.bytes, self.fn, self.sample = name, flops, nbytes, fn, sample
        self.peak = peak  # dense MFMA peak of the launch's arithmetic type, TFLOP/s
        self.group = group  # workload the GEMM belongs to

    @property
    def bound(self):
        return "mfma" if self.flops / self.bytes >= self.peak * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def _sample_idx(rng, count, *highs):
    return [rng.integers(0, h, count) for h in highs]


# ------------------------------------------------------------- workloads ---

def build_dense(small=False, pow2=False):
    """The dense sweep; pow2: power-of-two scales in the packed UE8M0 format
    (four exponent bytes per int32) through dg_gemm_fp8_nt_ue8m0_packed
    (scales applied by the block-scaled MFMA)."""
    import torch
    import moe_grouped_gemm_x128_amd as dg
    from harness import inputs, workloads

    shapes = [workloads.DENSE_SMALL] if small else workloads.dense_sweep()
    seed = shapes[0]["seed"]
    a_by_k, b_by_nk, calls = {}, {}, []
    for s in shapes:
        m, n, k = s["m"], s["n"], s["k"]
        mmax = max(x["m"] for x in shapes if x["k"] == k)
        pack = inputs.pack_ue8m0 if pow2 else (lambda s: s)
        if k not in a_by_k:
            a, sa = inputs.quantize_1x128(inputs._normal(inputs._rng(seed + k, 0), (mmax, k)), pow2)
            a_by_k[k] = (a, sa, _dev(a), _dev(pack(sa)))
        if (n, k) not in b_by_nk:
            b, sb = inputs.quantize_128x128(inputs._normal(inputs._rng(seed + n * 7 + k, 1), (n, k)), pow2)
            b_by_nk[(n, k)] = (b, sb, _dev(b), _dev(pack(sb)))
        a, sa, da, dsa = a_by_k[k]
        b, sb, db, dsb = b_by_nk[(n, k)]
        da_m, dsa_m = da[:m], dsa[:m]
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        gemm = dg.dg_gemm_fp8_nt_ue8m0_packed if pow2 else dg.dg_gemm_fp8_nt
        fn = (lambda da_m=da_m, dsa_m=dsa_m, db=db, dsb=dsb, out=out, gemm=gemm:
              gemm(da_m, dsa_m, db, dsb, out))
        swords = (k // 128 + 3) // 4 if pow2 else k // 128  # 4-byte scale words per row
        nbytes = m * k + m * swords * 4 + n * k + ((n + 127) // 128) * swords * 4 + m * n * 2

        def sample(rng, count, a=a[:m], sa=sa[:m], b=b, sb=sb, m=m, n=n, k=k):
            import oracle
            r, c = _sample_idx(rng, count, m, n)
            oracle.gemm_fp8_nt_at(a, sa, b, sb, r, c)
            return 2.0 * k * count

        calls.append(Call(s["name"] + ("_ue8m0" if pow2 else ""), 2.0 * m * n * k, nbytes, fn, sample,
                          group="dense"))
    desc = ("dense FP8 NT GEMM sweep: M in {64,128,4096} x (N,K) in {(2112,7168),(24576,1536),"
            "(32768,512),(7168,16384),(4096,7168),(7168,2048)}" if not small else "dense M=128 N=256 K=512")
    name = "dense_small" if small else ("dense_sweep_ue8m0" if pow2 else "dense_sweep")
    scales = "A 1x128, B 128x128, " + ("packed UE8M0 (four exponent bytes per int32)" if pow2 else "fp32")
    return calls, {"workload": name, "description": desc, "shapes": len(calls), "scales": scales, "out": "bf16"}


def build_contiguous(pow2=False):
    """MoE contiguous layout at 8192 rows per expert.  The G=4 problems are the
    first four experts of the G=8 ones: the same seeded streams give the same
    rows, weights and padding counts (make_contiguous draws them in order), so
    each (N,K) is generated once and G=4 uses views of it.  pow2: power-of-two
    scales in the packed UE8M0 format (dg_grouped_fp8_contiguous_ue8m0_packed)."""
    import torch
    import moe_grouped_gemm_x128_amd as dg
    from harness import inputs, workloads

    pack = inputs.pack_ue8m0 if pow2 else (lambda s: s)
    gemm = dg.dg_grouped_fp8_contiguous_ue8m0_packed if pow2 else dg.dg_grouped_fp8_contiguous
    calls = []
    by_nk = {}
    for s in sorted(workloads.contiguous_sweep(), key=lambda s: -s["g"]):
        g, rpe, n, k = s["g"], s["rows_per_expert"], s["n"], s["k"]
        if (n, k) not in by_nk:
            c = inputs.make_contiguous(g, rpe, n, k, s["seed"], pow2=pow2)
            by_nk[(n, k)] = (c, _dev(c.a), _dev(pack(c.sa)), _dev(c.b), _dev(pack(c.sb)), _dev(c.m_indices))
        c, da, dsa, db, dsb, dids = by_nk[(n, k)]
        assert g <= c.g
        mt = g * rpe
        a, sa, b, sb, ids = c.a[:mt], c.sa[:mt], c.b[:g], c.sb[:g], c.m_indices[:mt]
        da_g, dsa_g, db_g, dsb_g, ids_g = da[:mt], dsa[:mt], db[:g], dsb[:g], dids[:mt]
        out = torch.empty((mt, n), dtype=torch.bfloat16, device="cuda")
        fn = (lambda da=da_g, dsa=dsa_g, db=db_g, dsb=dsb_g, out=out, ids=ids_g, gemm=gemm:
              gemm(da, dsa, db, dsb, out, ids))
        valid_rows = np.flatnonzero(ids >= 0)
        mv = valid_rows.size
        kb, nb = (k // 128 + 3) // 4 if pow2 else k // 128, (n + 127) // 128  # 4-byte scale words per row
        nbytes = mv * k + mv * kb * 4 + g * n * k + g * nb * kb * 4 + mt * 4 + mv * n * 2

        def sample(rng, count, a=a, sa=sa, b=b, sb=sb, ids=ids, rows=valid_rows, n=n, k=k):
            import oracle
            r = rows[rng.integers(0, rows.size, count)]
            cl = rng.integers(0, n, count)
            oracle.grouped_contiguous_at(a, sa, b, sb, ids, r, cl)
            return 2.0 * k * count

        call = Call(s["name"] + ("_ue8m0" if pow2 else ""), 2.0 * mv * n * k, nbytes, fn, sample,
                    group="contiguous_ue8m0" if pow2 else "contiguous")
        call.operands = (da_g, dsa_g, db_g, dsb_g, ids_g, out)
        calls.append(call)
    order = [s["name"] + ("_ue8m0" if pow2 else "") for s in workloads.contiguous_sweep()]
    calls.sort(key=lambda c: order.index(c.name))
    return calls, {"workload": "contiguous_sweep_ue8m0" if pow2 else "contiguous_sweep", "description":
                   "MoE contiguous: G in {4,8}, 8192 rows per expert minus U{0..127} padding rows, "
                   "(N,K) in {(4096,7168),(7168,2048)}"
                   + ("; packed UE8M0 scales (four exponent bytes per int32)" if pow2 else "")}


def build_contiguous_swiglu():
    """The contiguous sweep's problems as an expert's first linear layer with
    SwiGLU and the 1x128 FP8 re-quantise fused into the GEMM epilogue
    (dg_grouped_fp8_contiguous_swiglu): B [G, N, K] holds the gate rows
    [0, N/2) and the up rows [N/2, N); out fp8 [M_total, N/2] + fp32 scales.
    Algorithmic FLOPs as the GEMM's; bytes = operands + codes + scales."""
    import torch
    import moe_grouped_gemm_x128_amd as dg

    base, _ = build_contiguous()
    calls = []
    for c in base:
        da, dsa, db, dsb, ids, _ = c.operands
        mt, k = da.shape
        g, n, _ = db.shape
        i = n // 2
        q = torch.empty((mt, i), dtype=torch.uint8, device="cuda")
        sc = torch.empty((mt, i // 128), dtype=torch.float32, device="cuda")
        fn = (lambda da=da, dsa=dsa, db=db, dsb=dsb, q=q, sc=sc, ids=ids:
              dg.dg_grouped_fp8_contiguous_swiglu(da, dsa, db, dsb, q, sc, ids))
        ids_h = ids.cpu().numpy()
        valid_rows = np.flatnonzero(ids_h >= 0)
        mv = valid_rows.size
        nbytes = c.bytes - mv * n * 2 + mv * i + mv * (i // 128) * 4
        a_h, sa_h = da.cpu().numpy(), dsa.cpu().numpy()
        b_h, sb_h = db.cpu().numpy(), dsb.cpu().numpy()

        def sample(rng, count, a=a_h, sa=sa_h, b=b_h, sb=sb_h, ids=ids_h, rows=valid_rows, i=i, k=k):
            """The oracle's composition on whole 1x128 output groups: the
            gate and up GEMM outputs of each, rounded to bf16, then its SwiGLU
            + quantiser; returns the GEMM FLOPs that took."""
            import oracle
            groups = max(1, count // 256)
            r = rows[rng.integers(0, rows.size, groups)]
            gi = rng.integers(0, i // 128, groups)
            cols = (gi[:, None] * 128 + np.arange(128)[None, :])
            cols = np.concatenate([cols, cols + i], axis=1)           # gate | up
            x, _ = oracle.grouped_contiguous_at(a, sa, b, sb, ids, np.repeat(r, 256), cols.ravel())
            oracle.swiglu_quantize_1x128(oracle.round_bf16(x).reshape(groups, 256))
            return 2.0 * k * 256 * groups

        name = c.name.replace("contig_", "contig_swiglu_")
        calls.append(Call(name, c.flops, nbytes, fn, sample, group="contiguous_swiglu"))
    return calls, {"workload": "contiguous_swiglu_sweep", "description":
                   "MoE contiguous first linear layer with SwiGLU + FP8 1x128 re-quantise fused: G in {4,8}, "
                   "8192 rows per expert minus U{0..127} padding rows, (N=2I,K) in {(4096,7168),(7168,2048)}",
                   "out": "e4m3 [M_total, N/2] + fp32 1x128 scales"}


def fused_swiglu_compare(calls, per_ms, reps=20):
    """The contiguous G=8, N=4096, K=7168 GEMM of the step against its fused
    form: the unfused path is the GEMM (its per-call time from the step's
    table) plus the stand-alone SwiGLU quantiser on its bf16 output; the fused
    path is one call.  Medians of `reps` event-bracketed launches."""
    import torch
    import moe_grouped_gemm_x128_amd as dg
    idx = [j for j, c in enumerate(calls) if c.name == "contig_g8_n4096_k7168" and hasattr(c, "operands")]
    if not idx:
        return None
    c = calls[idx[0]]
    da, dsa, db, dsb, ids, out = c.operands
    mt, i = da.shape[0], db.shape[1] // 2
    q = torch.empty((mt, i), dtype=torch.uint8, device="cuda")
    sc = torch.empty((mt, i // 128), dtype=torch.float32, device="cuda")

    def med(fn):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    swiglu = med(lambda: dg.dg_swiglu_quantize_fp8_1x128(out, q, sc))
    fused = med(lambda: dg.dg_grouped_fp8_contiguous_swiglu(da, dsa, db, dsb, q, sc, ids))
    gemm = float(per_ms[idx[0]])
    return {"problem": "contig_g8_n4096_k7168 as gate|up, I=2048", "gemm_us": round(gemm * 1e3, 1),
            "swiglu_quantize_us": round(swiglu * 1e3, 1), "unfused_us": round((gemm + swiglu) * 1e3, 1),
            "fused_us": round(fused * 1e3, 1), "fused_tflops": round(c.flops / (fused * 1e-3) / 1e12, 1),
            "speedup": round((gemm + swiglu) / fused, 3)}


def build_masked(pow2=False):
    """MoE masked decode; pow2: power-of-two scales in the packed UE8M0 format
    (dg_grouped_fp8_masked_ue8m0_packed)."""
    import torch
    import moe_grouped_gemm_x128_amd as dg
    from harness import inputs, workloads

    pack = inputs.pack_ue8m0 if pow2 else (lambda s: s)
    gemm = dg.dg_grouped_fp8_masked_ue8m0_packed if pow2 else dg.dg_grouped_fp8_masked
    calls = []
    for s in workloads.masked_sweep():
        x = inputs.make_masked(s["g"], s["m_max"], s["n"], s["k"], s["seed"], pow2=pow2)
        da, dsa, db, dsb, mm = _dev(x.a), _dev(pack(x.sa)), _dev(x.b), _dev(pack(x.sb)), _dev(x.masked_m)
        out = torch.empty((x.g, x.m_max, x.n), dtype=torch.bfloat16, device="cuda")
        fn = (lambda da=da, dsa=dsa, db=db, dsb=dsb, out=out, mm=mm, gemm=gemm:
              gemm(da, dsa, db, dsb, out, mm))
        fn_na = (lambda da=da, dsa=dsa, db=db, dsb=dsb, out=out, mm=mm:
                 dg.dg_grouped_fp8_masked_noalloc(da, dsa, db, dsb, out, mm))
        valid = np.clip(x.masked_m, 0, x.m_max)
        mv = int(valid.sum())
        kb, nb = (x.k // 128 + 3) // 4 if pow2 else x.k // 128, (x.n + 127) // 128  # scale words per row
        nbytes = mv * x.k + mv * kb * 4 + x.g * x.n * x.k + x.g * nb * kb * 4 + x.g * 4 + mv * x.n * 2

        def sample(rng, count, x=x, valid=valid):
            import oracle
            gs = rng.choice(np.flatnonzero(valid > 0), count)
            rows = (rng.random(count) * valid[gs]).astype(np.int64)
            cols = rng.integers(0, x.n, count)
            oracle.grouped_masked_at(x.a, x.sa, x.b, x.sb, x.masked_m, gs, rows, cols)
            return 2.0 * x.k * count

        c = Call(s["name"] + ("_ue8m0" if pow2 else ""), 2.0 * mv * x.n * x.k, nbytes, fn, sample,
                 group="masked_ue8m0" if pow2 else "masked")
        if not pow2:
            c.fn_noalloc = fn_na
        calls.append(c)
    return calls, {"workload": "masked_sweep_ue8m0" if pow2 else "masked_sweep", "description":
                   "MoE masked decode: G in {1,2,4,16}, M_max=256, masked_m ~ U{64..192}, "
                   "(N,K) in {(4096,7168),(7168,2048)}"
                   + ("; packed UE8M0 scales (four exponent bytes per int32)" if pow2 else "")}


def build_wgrad(kgrouped=False):
    import moe_grouped_gemm_x128_amd as dg
    from harness import inputs, workloads

    s = workloads.K_GROUPED_WGRAD if kgrouped else workloads.WGRAD
    w = inputs.make_wgrad(s["m"], s["n"], s["ks"], s["seed"])
    da, dsa, db, dsb = _dev(w.a), _dev(w.sa), _dev(w.b), _dev(w.sb)
    d = _dev(w.d0 if kgrouped else w.d0[0])
    t = sum(w.ks)
    g = len(w.ks)
    if kgrouped:
        fn = lambda: dg.dg_k_grouped_wgrad_fp8_nt(da, dsa, db, dsb, d, w.ks)
    else:
        fn = lambda: dg.dg_wgrad_fp8_nt(da, dsa, db, dsb, d)
    nbytes = (w.m + w.n) * t + (w.m + w.n) * (t // 128) * 4 + g * 2 * 4 * w.m * w.n
    ks = np.array(w.ks, np.int64)

    def sample(rng, count):
        import oracle
        rows, cols = _sample_idx(rng, count, w.m, w.n)
        if kgrouped:
            gs = rng.integers(0, g, count)
            oracle.k_grouped_wgrad_at(w.a, w.sa, w.b, w.sb, ks, w.d0, gs, rows, cols)
            return 2.0 * float(ks[gs].sum())
        oracle.wgrad_at(w.a, w.sa, w.b, w.sb, w.d0[0], rows, cols)
        return 2.0 * t * count

    calls = [Call(s["name"], 2.0 * w.m * w.n * t, nbytes, fn, sample, group="wgrad")]
    return calls, {"workload": s["name"], "description":
                   f"weight gradient D[{w.m},{w.n}] += over tokens {w.ks}, 1x128 scales on both operands, fp32 D"}


def build_all():
    """Every configuration of the GEMM family in one step: the dense sweep,
    the contiguous and masked MoE layouts and both weight gradients."""
    calls = []
    for b in (build_dense, build_contiguous, build_masked, build_wgrad, lambda: build_wgrad(kgrouped=True)):
        calls += b()[0]
    return calls, {"workload": "fp8_gemm_all",
                   "description": "dense sweep (18 GEMMs) + MoE contiguous (G 4/8 x 8192 rows, 4 GEMMs) + MoE "
                                  "masked decode (G 1/2/4/16, 8 GEMMs) + weight gradient and K-grouped weight "
                                  "gradient, one step",
                   "gemms": len(calls), "scales": "A 1x128, B 128x128 (weight gradients: 1x128 on both)",
                   "out": "bf16 (weight gradients: fp32 D)"}


def build_bf16():
    """The dense sweep's shapes in BF16 (dg_gemm_bf16_nt): N(0,1) operands
    rounded to bf16, no scales; roofline against the bf16 dense peak."""
    import torch
    import moe_grouped_gemm_x128_amd as dg
    from harness import inputs, workloads

    shapes = workloads.dense_sweep()
    seed = shapes[0]["seed"]
    a_by_k, b_by_nk, calls = {}, {}, []
    to_dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    for s in shapes:
        m, n, k = s["m"], s["n"], s["k"]
        mmax = max(x["m"] for x in shapes if x["k"] == k)
        if k not in a_by_k:
            a = inputs._to_bf16_bits(inputs._normal(inputs._rng(seed + k, 0), (mmax, k)))
            a_by_k[k] = (a, to_dev(a))
        if (n, k) not in b_by_nk:
            b = inputs._to_bf16_bits(inputs._normal(inputs._rng(seed + n * 7 + k, 1), (n, k)))
            b_by_nk[(n, k)] = (b, to_dev(b))
        a, da = a_by_k[k]
        b, db = b_by_nk[(n, k)]
        da_m = da[:m]
        out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        fn = lambda da_m=da_m, db=db, out=out: dg.dg_gemm_bf16_nt(da_m, db, out)
        nbytes = 2 * (m * k + n * k + m * n)

        def sample(rng, count, a=a[:m], b=b, m=m, n=n, k=k):
            import oracle
            r, c = _sample_idx(rng, count, m, n)
            oracle.gemm_bf16_nt_at(a, b, r, c)
            return 2.0 * k * count

        calls.append(Call(s["name"] + "_bf16", 2.0 * m * n * k, nbytes, fn, sample, peak=PEAK_BF16_TFLOPS,
                          group="bf16"))
    return calls, {"workload": "dense_sweep_bf16", "description": "the dense sweep's 18 shapes in BF16",
                   "shapes": len(calls), "scales": "none", "out": "bf16"}


def build_grouped_bf16():
    """The grouped layouts in BF16 (dg_grouped_bf16_contiguous and
    dg_grouped_bf16_masked): the contiguous sweep's G=4 problems and the masked
    decode's G=4 and G=16 problems at N=4096, K=7168, with N(0,1) operands
    rounded to bf16 and no scales; rooflines against the bf16 dense peak and HBM."""
    import torch
    import moe_grouped_gemm_x128_amd as dg
    from harness import inputs, workloads

    to_dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    calls = []
    for s in workloads.contiguous_sweep():
        if s["g"] != 4:
            continue
        g, rpe, n, k = s["g"], s["rows_per_expert"], s["n"], s["k"]
        x = inputs.make_contiguous_bf16(g, rpe, n, k, s["seed"])
        da, db, ids = to_dev(x.a), to_dev(x.b), _dev(x.ctrl)
        out = torch.empty((g * rpe, n), dtype=torch.bfloat16, device="cuda")
        fn = lambda da=da, db=db, out=out, ids=ids: dg.dg_grouped_bf16_contiguous(da, db, out, ids)
        rows = np.flatnonzero(x.ctrl >= 0)
        mv = rows.size
        nbytes = 2 * (mv * k + g * n * k + mv * n) + g * rpe * 4

        def sample(rng, count, x=x, rows=rows, n=n, k=k, g=g):
            import oracle
            r = rows[rng.integers(0, rows.size, count)]
            c = rng.integers(0, n, count)
            for e in range(g):
                sel = np.flatnonzero(x.ctrl[r] == e)
                oracle.gemm_bf16_nt_at(x.a, x.b[e], r[sel], c[sel])
            return 2.0 * k * count

        calls.append(Call(s["name"] + "_bf16", 2.0 * mv * n * k, nbytes, fn, sample, peak=PEAK_BF16_TFLOPS,
                          group="grouped_bf16"))
    for s in workloads.masked_sweep():
        if s["g"] not in (4, 16) or s["n"] != 4096:
            continue
        g, m_max, n, k = s["g"], s["m_max"], s["n"], s["k"]
        mm = inputs._rng(s["seed"], 4).integers(64, 193, size=g).astype(np.int32)
        x = inputs.make_masked_bf16(g, m_max, n, k, s["seed"], masked_m=mm)
        da, db, dmm = to_dev(x.a), to_dev(x.b), _dev(mm)
        out = torch.empty((g, m_max, n), dtype=torch.bfloat16, device="cuda")
        fn = lambda da=da, db=db, out=out, dmm=dmm: dg.dg_grouped_bf16_masked(da, db, out, dmm)
        mv = int(mm.sum())
        nbytes = 2 * (mv * k + g * n * k + mv * n) + g * 4

        def sample(rng, count, x=x, mm=mm, n=n, k=k, g=g):
            import oracle
            gs = rng.integers(0, g, count)
            r = (rng.random(count) * mm[gs]).astype(np.int64)
            c = rng.integers(0, n, count)
            for e in range(g):
                sel = np.flatnonzero(gs == e)
                oracle.gemm_bf16_nt_at(x.a[e], x.b[e], r[sel], c[sel])
            return 2.0 * k * count

        calls.append(Call(s["name"] + "_bf16", 2.0 * mv * n * k, nbytes, fn, sample, peak=PEAK_BF16_TFLOPS,
                          group="grouped_bf16"))
    return calls, {"workload": "grouped_bf16", "description":
                   "MoE contiguous G=4 x 8192 rows (ragged padding), (N,K) in {(4096,7168),(7168,2048)}, and masked "
                   "decode G in {4,16}, M_max=256, masked_m ~ U{64..192}, N=4096, K=7168, in BF16",
                   "scales": "none", "out": "bf16"}


QUANT_METRIC = "FP8 quantiser GB/s (absmax/448 fp32 scales) and % of MI355X HBM peak"


def build_quantize():
    """The quantiser on the GEMM workloads' fp32 operands: the MoE contiguous
    activations (G=8 x 8192 rows), the dense activations and the largest dense
    weight, and the two token-contiguous weight-gradient operands (X and dY of
    4096 tokens, transposed).  Inputs are seeded N(0,1) fp32 drawn on the
    device; algorithmic bytes = 4 read + 1 written per element + the scales."""
    import torch
    import moe_grouped_gemm_x128_amd as dg
    from harness import inputs

    gen = torch.Generator(device="cuda")
    gen.manual_seed(inputs.SEED_BASE + 5)
    specs = [("quant_1x128_m65536_k7168", 0, 65536, 7168), ("quant_1x128_m4096_k7168", 0, 4096, 7168),
             ("quant_128x128_n7168_k16384", 1, 7168, 16384), ("quant_1x128T_t4096_f7168", 2, 4096, 7168),
             ("quant_1x128T_t4096_f2048", 2, 4096, 2048), ("quant_1x128_ue8m0_m65536_k7168", 3, 65536, 7168),
             ("quant_128x128_ue8m0_n7168_k16384", 4, 7168, 16384)]
    calls = []
    for name, mode, r, c in specs:
        x = torch.randn((r, c), generator=gen, device="cuda", dtype=torch.float32)
        if mode == 0:
            q = torch.empty((r, c), dtype=torch.uint8, device="cuda")
            sc = torch.empty((r, c // 128), dtype=torch.float32, device="cuda")
            fn = lambda x=x, q=q, sc=sc: dg.dg_quantize_fp8_1x128(x, q, sc)
        elif mode == 1:
            q = torch.empty((r, c), dtype=torch.uint8, device="cuda")
            sc = torch.empty(((r + 127) // 128, c // 128), dtype=torch.float32, device="cuda")
            fn = lambda x=x, q=q, sc=sc: dg.dg_quantize_fp8_128x128(x, q, sc)
        elif mode == 2:
            q = torch.empty((c, r), dtype=torch.uint8, device="cuda")
            sc = torch.empty((c, r // 128), dtype=torch.float32, device="cuda")
            fn = lambda x=x, q=q, sc=sc: dg.dg_quantize_fp8_1x128_transposed(x, q, sc)
        elif mode == 3:  # power-of-two scales, packed UE8M0 words
            q = torch.empty((r, c), dtype=torch.uint8, device="cuda")
            sc = torch.empty((r, (c // 128 + 3) // 4), dtype=torch.int32, device="cuda")
            fn = lambda x=x, q=q, sc=sc: dg.dg_quantize_fp8_1x128_ue8m0(x, q, sc)
        else:
            q = torch.empty((r, c), dtype=torch.uint8, device="cuda")
            sc = torch.empty(((r + 127) // 128, (c // 128 + 3) // 4), dtype=torch.int32, device="cuda")
            fn = lambda x=x, q=q, sc=sc: dg.dg_quantize_fp8_128x128_ue8m0(x, q, sc)
        nbytes = r * c * 5 + sc.numel() * 4

        def sample(rng, rows, x=x, mode=mode, c=c):
            """The oracle on the first `rows` rows (a multiple of 128, at most
            the input's own); returns the algorithmic bytes covered."""
            import oracle
            rows = min(rows, x.shape[0])
            h = x[:rows].cpu().numpy()
            f = (oracle.quantize_1x128, oracle.quantize_128x128, oracle.quantize_1x128_transposed,
                 oracle.quantize_1x128_ue8m0, oracle.quantize_128x128_ue8m0)[mode]
            f(h)
            return rows * c * 5

        calls.append(Call(name, 0.0, nbytes, fn, (sample, c), group="quantize"))
    return calls, {"workload": "quantize", "description":
                   "FP8 quantiser: 1x128 activations [65536,7168] and [4096,7168], 128x128 weights "
                   "[7168,16384], token-contiguous 1x128 transposed [4096,7168] and [4096,2048]; "
                   "the first and third with power-of-two scales in packed UE8M0 words",
                   "scales": "absmax/448 fp32 (packed UE8M0: the next power of two)", "in": "fp32", "out": "e4m3"}


SWIGLU_METRIC = "SwiGLU + FP8 1x128 re-quantise GB/s (bf16 in, e4m3 + fp32 scales out) and % of MI355X HBM peak"


def build_swiglu():
    """SwiGLU + 1x128 quantise of the first linear's bf16 output [M, 2I] for
    the MoE workloads: the contiguous layout's G=8 x 8192 rows with N = 2I of
    4096 and of 7168, and a masked decode batch of 16 groups x 256 rows
    (N = 4096).  Inputs are seeded N(0,1) bf16 drawn on the device;
    algorithmic bytes = 4 read + 1 written per output element + the scales."""
    import torch
    import moe_grouped_gemm_x128_amd as dg
    from harness import inputs

    gen = torch.Generator(device="cuda")
    gen.manual_seed(inputs.SEED_BASE + 6)
    specs = [("swiglu_quant_m65536_n4096", 65536, 2048), ("swiglu_quant_m65536_n7168", 65536, 3584),
             ("swiglu_quant_m4096_n4096", 4096, 2048)]
    calls = []
    for name, m, i in specs:
        c = torch.randn((m, 2 * i), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        q = torch.empty((m, i), dtype=torch.uint8, device="cuda")
        sc = torch.empty((m, i // 128), dtype=torch.float32, device="cuda")
        fn = lambda c=c, q=q, sc=sc: dg.dg_swiglu_quantize_fp8_1x128(c, q, sc)
        nbytes = m * i * 5 + sc.numel() * 4

        def sample(rng, rows, c=c, i=i):
            """The oracle on the first `rows` rows; returns the algorithmic
            bytes covered."""
            import oracle
            rows = min(rows, c.shape[0])
            bits = c[:rows].view(torch.int16).cpu().numpy().view(np.uint16)
            oracle.swiglu_quantize_1x128(bits)
            return rows * i * 5 + rows * (i // 128) * 4

        calls.append(Call(name, 0.0, nbytes, fn, (sample, i), group="swiglu_quantize"))
    return calls, {"workload": "swiglu_quantize", "description":
                   "SwiGLU (gate | up halves) + FP8 1x128 quantise of the first linear's bf16 output: "
                   "[65536, 4096], [65536, 7168] (G=8 x 8192 rows) and [4096, 4096] (16 x 256 decode rows)",
                   "scales": "absmax/448 fp32", "in": "bf16", "out": "e4m3"}


def cpu_baseline_quantize(calls, seconds):
    """Time the oracle quantiser on the first rows of each input (GB/s of
    algorithmic traffic), sized to about `seconds` of CPU work."""
    import oracle
    rng = np.random.default_rng(12345)
    rows = 128
    while True:
        t = time.perf_counter()
        for c in calls:
            c.sample[0](rng, rows)
        dt = time.perf_counter() - t
        if dt >= 0.1 * seconds or rows >= 65536:
            break
        rows *= 2
    rows = int(rows * seconds / max(dt, 1e-9)) // 128 * 128
    rows = min(65536, max(128, rows))
    # whole passes over that sample until the budget is spent
    t = time.perf_counter()
    nbytes, passes = 0, 0
    while passes == 0 or time.perf_counter() - t < seconds:
        nbytes += sum(c.sample[0](rng, rows) for c in calls)
        passes += 1
    dt = time.perf_counter() - t
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{passes} pass(es) over the first {rows} rows of each of the {len(calls)} inputs "
                      f"({nbytes / 1e9:.2f} GB of algorithmic traffic, {dt:.1f} s, C oracle with OpenMP, "
                      f"host copy included)"}


# --------------------------------------------------------------- timing ---

SPIN_CYCLES = 4_000_000  # ~2 ms of GPU clock: covers the host's enqueue of one pass


def per_call_times(calls, steps, cold=False):
    """Mean duration (ms) of each GEMM: HIP events around every call on the
    launch stream, over `steps` passes.  Used for the per-shape table and to
    find the dominant GEMM; not the timed steps (each event record takes GPU
    time between kernels that a real caller would not spend).  Each pass
    starts with a short spin kernel (torch.cuda._sleep) so the host enqueues
    the pass while the GPU spins: the event pairs then time the GPU's
    execution of each call, as the profiler's kernel durations do, rather
    than the host's launch cost, which a call shorter than ~10 us would
    otherwise show.  cold: a 512 MB buffer (more than the 256 MB MALL plus
    the L2s) is overwritten before each call, outside its event pair, so
    every call starts with cold caches."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if cold else None
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(steps)]
    spin = getattr(torch.cuda, "_sleep", None)
    torch.cuda.synchronize()
    for s in range(steps):
        if spin is not None:
            spin(SPIN_CYCLES)
        for i, c in enumerate(calls):
            if cold:
                flush.fill_(s & 0xff)
            ev[s][i][0].record()
            c.fn()
            ev[s][i][1].record()
    torch.cuda.synchronize()
    per = np.array([[ev[s][i][0].elapsed_time(ev[s][i][1]) for i in range(len(calls))] for s in range(steps)])
    return per.mean(axis=0)


def time_steps(calls, steps, warmup, settle_s=0.5, cold=False):
    """Returns (total ms of the K timed steps, per-call mean ms, index of the
    dominant call, its mean ms inside the timed steps).

    A first pass with events around every call gives the per-call times and
    picks the dominant call (largest time).  Then W untimed warmup steps and
    the K timed steps, launched back to back as a caller would, between a
    synchronisation and an event pair on both sides; inside them only the
    dominant call is bracketed by HIP events (on the launch stream), for the
    live roofline figure."""
    import torch
    t = time.perf_counter()
    while time.perf_counter() - t < settle_s:  # let the clock settle (untimed)
        for c in calls:
            c.fn()
        torch.cuda.synchronize()
    per_ms = per_call_times(calls, steps, cold)
    dom = int(np.argmax(per_ms))
    for _ in range(warmup):
        for c in calls:
            c.fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        for i, c in enumerate(calls):
            if i == dom:
                ev[s][0].record()
                c.fn()
                ev[s][1].record()
            else:
                c.fn()
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    return total_ms, per_ms, dom, dom_ms


def cpu_baseline(calls, seconds):
    """Time the CPU oracle on a bounded sample of the workload's outputs: the
    same number of uniformly drawn outputs of every GEMM, sized so the timed
    pass takes about `seconds`."""
    import oracle
    usable = [c for c in calls if c.sample is not None]
    if not usable:
        return None
    rng = np.random.default_rng(12345)
    # calibrate: grow the sample until one pass takes a measurable share of
    # the budget, then size the timed sample to the whole budget
    per_shape = 16
    while True:
        t = time.perf_counter()
        for c in usable:
            c.sample(rng, per_shape)
        dt = time.perf_counter() - t
        if dt >= 0.1 * seconds or per_shape >= 1 << 22:
            break
        per_shape *= 4
    per_shape = int(max(16, per_shape * seconds / max(dt, 1e-9)))
    t = time.perf_counter()
    flops = sum(c.sample(rng, per_shape) for c in usable)
    dt = time.perf_counter() - t
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{per_shape} uniformly drawn outputs of each of the {len(usable)} GEMMs "
                      f"({flops / 1e9:.1f} GFLOP, {dt:.1f} s, fp64 C oracle with OpenMP)"}


def cold_median(call, dispatches=COLD_DISPATCHES):
    """Median duration (ms) of `dispatches` launches of one GEMM, each after a
    512 MB buffer (more than the MALL plus the L2s) is overwritten, each
    bracketed by HIP events on the launch stream."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(dispatches)]
    call.fn()
    torch.cuda.synchronize()
    for i in range(dispatches):
        flush.fill_(i & 0xff)
        ev[i][0].record()
        call.fn()
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def graph_replay_ms(fns, reps=20):
    """Capture `fns` (called in order) into one HIP graph on a side stream and
    return the median replay time (ms), events around each replay."""
    import torch
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for f in fns:
            f()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for f in fns:
                f()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def masked_graph(calls, per_ms):
    """The masked decode GEMMs of the step: eager (sum of the per-call times),
    captured with the default entry point (which does not split K under
    capture) and captured with the allocation-free one (which keeps the split
    in its fixed scratch)."""
    idx = [i for i, c in enumerate(calls) if c.group == "masked"]
    if not idx:
        return None
    ms = [calls[i] for i in idx]
    eager = float(sum(per_ms[i] for i in idx))
    default = graph_replay_ms([c.fn for c in ms])
    noalloc = graph_replay_ms([c.fn_noalloc for c in ms])
    flops = sum(c.flops for c in ms)
    return {"gemms": len(ms), "eager_us": round(eager * 1e3, 1), "graph_us": round(default * 1e3, 1),
            "graph_noalloc_us": round(noalloc * 1e3, 1),
            "eager_tflops": round(flops / (eager * 1e-3) / 1e12, 1),
            "graph_tflops": round(flops / (default * 1e-3) / 1e12, 1),
            "graph_noalloc_tflops": round(flops / (noalloc * 1e-3) / 1e12, 1)}


def workload_summary(calls, per_ms):
    """Per workload of the step: its GEMMs' summed per-call time, TFLOP/s and
    its dominant GEMM with that GEMM's fraction of its own bound."""
    out = {}
    for grp in dict.fromkeys(c.group for c in calls):
        idx = [i for i, c in enumerate(calls) if c.group == grp]
        ms = float(sum(per_ms[i] for i in idx))
        flops = sum(calls[i].flops for i in idx)
        nbytes = sum(calls[i].bytes for i in idx)
        d = max(idx, key=lambda i: per_ms[i])
        c = calls[d]
        tf = c.flops / (per_ms[d] * 1e-3) / 1e12
        gbs = c.bytes / (per_ms[d] * 1e-3) / 1e9
        out[grp] = {"gemms": len(idx), "us": round(ms * 1e3, 1), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "dominant": c.name, "dominant_bound": c.bound,
                    "dominant_frac": round(tf / c.peak if c.bound == "mfma" else gbs / PEAK_HBM_GBS, 4)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="all",
                    choices=["all", "dense", "small", "contiguous", "masked", "wgrad", "k_grouped_wgrad", "quantize",
                             "dense_ue8m0", "bf16", "swiglu_quantize", "contiguous_swiglu", "contiguous_ue8m0",
                             "masked_ue8m0", "grouped_bf16"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold-median", action="store_true", help="skip the cold-cache median of the dominant GEMM")
    ap.add_argument("--settle-seconds", type=float, default=0.5, help="untimed run before the warmup steps")
    ap.add_argument("--only", default="", help="comma-separated GEMM names to time (others skipped)")
    ap.add_argument("--copy-calibration", action="store_true", help="run the counter-calibration copy and exit")
    ap.add_argument("--cold", action="store_true",
                    help="per-launch table with a 512 MB cache flush before each call (the timed steps are unchanged)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (the kernel runs on one "
              "GPU's share of the work); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log(f"device {torch.cuda.get_device_name(0)}, building workload {args.workload}")
    builders = {"all": build_all, "dense": build_dense, "small": lambda: build_dense(small=True),
                "contiguous": build_contiguous, "masked": build_masked,
                "wgrad": build_wgrad, "k_grouped_wgrad": lambda: build_wgrad(kgrouped=True),
                "quantize": build_quantize, "dense_ue8m0": lambda: build_dense(pow2=True), "bf16": build_bf16,
                "swiglu_quantize": build_swiglu, "contiguous_swiglu": build_contiguous_swiglu,
                "contiguous_ue8m0": lambda: build_contiguous(pow2=True),
                "masked_ue8m0": lambda: build_masked(pow2=True), "grouped_bf16": build_grouped_bf16}
    if args.copy_calibration:
        copy_calibration()
        return
    calls, config = builders[args.workload]()
    if args.only:
        keep = set(args.only.split(","))
        calls = [c for c in calls if c.name in keep]
        assert calls, f"--only matched none of the workload's GEMMs"
        config = dict(config, only=sorted(keep))
    log(f"{len(calls)} GEMMs per step; timing {args.steps} steps after {args.warmup} warmup")
    total_ms, per_ms, dom, dms = time_steps(calls, args.steps, args.warmup, args.settle_seconds, args.cold)
    if args.cold:
        config = dict(config, per_launch="cold caches (512 MB flush before each call)")
    ms_per_step = total_ms / args.steps
    step_flops = sum(c.flops for c in calls)

    shapes = []
    for c, ms in zip(calls, per_ms):
        tf = c.flops / (ms * 1e-3) / 1e12
        gbs = c.bytes / (ms * 1e-3) / 1e9
        frac = tf / c.peak if c.bound == "mfma" else gbs / PEAK_HBM_GBS
        shapes.append({"name": c.name, "us": round(ms * 1e3, 2), "tflops": round(tf, 1),
                       "gbs": round(gbs, 1), "bound": c.bound, "frac": round(frac, 4)})
        log(f"{c.name:52s} {ms * 1e3:9.1f} us {tf:8.1f} TFLOP/s {gbs:8.1f} GB/s {c.bound} {frac:.3f}")
    dc = calls[dom]
    if dc.bound == "mfma":
        achieved, peak, unit = dc.flops / (dms * 1e-3) / 1e12, dc.peak, "TFLOP/s"
    else:
        achieved, peak, unit = dc.bytes / (dms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    roofline = {"bound": dc.bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(dc.name), "kernel": dc.name,
                "flops_per_launch": dc.flops, "bytes_per_launch": dc.bytes, "avg_us": round(dms * 1e3, 2)}
    if not args.no_cold_median:
        log(f"cold median of {COLD_DISPATCHES} dispatches of {dc.name}")
        cms = cold_median(dc)
        cold = dc.flops / (cms * 1e-3) / 1e12 if dc.bound == "mfma" else dc.bytes / (cms * 1e-3) / 1e9
        roofline.update({"cold_median_us": round(cms * 1e3, 2), "cold_achieved": round(cold, 2),
                         "cold_frac": round(cold / peak, 4), "cold_dispatches": COLD_DISPATCHES})
    extra = {}
    if len({c.group for c in calls}) > 1 or args.workload == "all":
        extra["workloads"] = workload_summary(calls, per_ms)
    if any(c.group == "masked" for c in calls) and not args.only:
        log("masked decode GEMMs captured into HIP graphs")
        extra["masked_graph"] = masked_graph(calls, per_ms)
    if any(c.group == "contiguous" for c in calls) and not args.only:
        log("contiguous GEMM against its fused SwiGLU + re-quantise form")
        extra["fused_swiglu"] = fused_swiglu_compare(calls, per_ms)

    quant = args.workload in ("quantize", "swiglu_quantize")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline_quantize(calls, args.cpu_seconds) if quant else cpu_baseline(calls, args.cpu_seconds)

    if quant:  # a stream, not a contraction: whole-step algorithmic bytes per second
        swiglu = args.workload == "swiglu_quantize"
        value, unit, metric, dtype = sum(c.bytes for c in calls) / (ms_per_step * 1e-3) / 1e9, "GB/s", \
            SWIGLU_METRIC if swiglu else QUANT_METRIC, "f32"
        data = "synthetic (seeded N(0,1) bf16)" if swiglu else "synthetic (seeded N(0,1) fp32)"
    else:
        bf16 = args.workload in ("bf16", "grouped_bf16")
        value, unit, metric, dtype = step_flops / (ms_per_step * 1e-3) / 1e12, "TFLOP/s", METRIC, \
            "bf16" if bf16 else "fp8"
        data = "synthetic (seeded N(0,1), bf16)" if bf16 else "synthetic (seeded N(0,1), e4m3-quantised)"
    line = {"metric": metric, "value": round(value, 2),
            "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": data,
            "config": config, "roofline": roofline, "cpu_baseline": cpu, **extra, "per_shape": shapes}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
