"""Benchmark: block-scaled INT8 GEMM throughput of one hidden-4096 transformer
block's linears (fwd + dgrad + wgrad) in the INT8 data flow, on one MI355X.

A step is one pass of the whole hot path over one batch of 8192 tokens:
  quantize X and the four weights (fp32 -> INT8 + 32x32 scales),
  QKV / out-proj / FC1 forward GEMMs with on-chip requantization,
  requantization of the (fp32) attention output before the out-projection,
  INT8 GELU between FC1 and FC2, FC2 forward,
  quantize the fp32 gradients entering the block (dY of FC2, dO of the
  out-projection, dQKV of the attention), the eight dgrad/wgrad GEMMs, and
  the INT8 GELU backward between FC2's dgrad output and FC1's backward GEMMs.
Every GEMM emits INT8 codes + per-block scales.

value = (sum of 2*M*N*K over the 12 GEMMs) / (wall time of one step); the
memory-bound kernels' time is inside the step, so this is a lower bound on
GEMM-only TOPS (also reported).  Inputs are seeded synthetic data already
resident in HBM.  Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0          # MI355X dense INT8 MFMA, published
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_hidden4096.md")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle baseline sample (0 disables it)")
    p.add_argument("--extras", type=int, default=1,
                   help="1: after the timed step also measure the quantization-error harness, residual add, "
                        "LayerNorm and the hidden-1024 MLP; 0: the step only")
    p.add_argument("--bf16-steps", type=int, default=5,
                   help="steps of the bf16 reference (the same 12 GEMMs with torch.mm in bfloat16; 0 skips it)")
    p.add_argument("--cpu-full", type=int, default=1,
                   help="1: also time the oracle on the tiny, GPT2-base, GPT2-medium MLP and memory-bound "
                        "workloads in full (about 1-2 minutes of CPU); 0: skip")
    p.add_argument("--ceilings", type=int, default=1,
                   help="1: measure the ceilings (register-only MFMA and MFMA + rescale loops, streaming "
                        "copies) the kernels are reported against; 0: skip")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain elementwise copy (dst = src * 1) of MIB mebibytes 5 times (the "
                        "known-size reference for the FETCH_SIZE/WRITE_SIZE counters) and exit")
    return p.parse_args()


class Step:
    """Preallocated buffers and the ordered kernel list of one step."""

    def __init__(self, dev):
        import numpy as np
        import torch

        from int8_block_quantized_amd import inputs
        from int8_block_quantized_amd import jetfire as jf

        self.jf = jf
        self.wl = inputs.hidden4096_block()
        T = 8192
        t0 = time.time()
        self.host = {}
        self.fp = {}
        for name in ("X", "A", "Wqkv", "Wo", "W1", "W2", "dY", "dO", "dQKV"):
            arr = self.wl.make(name)
            self.host[name] = arr
            self.fp[name] = torch.from_numpy(arr).to(dev)
        log(f"inputs generated and uploaded in {time.time() - t0:.1f} s")

        def i8(r, c):
            return (torch.empty((r, c), dtype=torch.int8, device=dev),
                    torch.empty((r // 32, c // 32), dtype=torch.float32, device=dev))

        q = {}
        for name, t in self.fp.items():
            q[name] = i8(*t.shape)
        for name, (r, c) in {"QKV": (T, 12288), "O": (T, 4096), "H": (T, 16384), "G": (T, 16384),
                             "Y": (T, 4096), "dG": (T, 16384), "dW2": (16384, 4096), "dX1": (T, 4096),
                             "dH": (T, 16384), "dW1": (4096, 16384), "dA": (T, 4096), "dWo": (4096, 4096),
                             "dX": (T, 4096), "dWqkv": (4096, 12288)}.items():
            q[name] = i8(r, c)
        self.q = q
        Q = lambda n: q[n]

        # (kind, label, args)   kinds: quant, requant, gemm, gelu, gelu_bwd
        self.ops = [
            ("quant", "quantize X", ("X",)),
            ("quant", "quantize Wqkv", ("Wqkv",)),
            ("quant", "quantize Wo", ("Wo",)),
            ("quant", "quantize W1", ("W1",)),
            ("quant", "quantize W2", ("W2",)),
            ("gemm", "qkv.fwd", ("X", "Wqkv", 0, 0, "QKV")),
            ("requant", "requant A", ("A",)),
            ("gemm", "out.fwd", ("A", "Wo", 0, 0, "O")),
            ("gemm", "fc1.fwd", ("X", "W1", 0, 0, "H")),
            ("gelu", "gelu H", ("H", "G")),
            ("gemm", "fc2.fwd", ("G", "W2", 0, 0, "Y")),
            ("quant", "quantize dY", ("dY",)),
            ("gemm", "fc2.dgrad", ("dY", "W2", 0, 1, "dG")),
            ("gemm", "fc2.wgrad", ("G", "dY", 1, 0, "dW2")),
            ("gelu_bwd", "gelu_bwd dG", ("dG", "H", "dH")),
            ("gemm", "fc1.dgrad", ("dH", "W1", 0, 1, "dX1")),
            ("gemm", "fc1.wgrad", ("X", "dH", 1, 0, "dW1")),
            ("quant", "quantize dO", ("dO",)),
            ("gemm", "out.dgrad", ("dO", "Wo", 0, 1, "dA")),
            ("gemm", "out.wgrad", ("A", "dO", 1, 0, "dWo")),
            ("quant", "quantize dQKV", ("dQKV",)),
            ("gemm", "qkv.dgrad", ("dQKV", "Wqkv", 0, 1, "dX")),
            ("gemm", "qkv.wgrad", ("X", "dQKV", 1, 0, "dWqkv")),
        ]
        self.meta = {}
        for kind, label, a in self.ops:
            if kind == "gemm":
                an, bn, ta, tb, cn = a
                qa, qb = Q(an)[0], Q(bn)[0]
                M = qa.shape[1] if ta else qa.shape[0]
                K = qa.shape[0] if ta else qa.shape[1]
                N = qb.shape[0] if tb else qb.shape[1]
                self.meta[label] = {"kind": kind, "M": M, "N": N, "K": K, "tA": ta, "tB": tb,
                                    "ops": 2 * M * N * K}
            elif kind in ("quant", "requant"):
                r, c = self.fp[a[0]].shape
                self.meta[label] = {"kind": kind, "bytes": r * c * 4 + r * c + (r * c // 1024) * 4}
            elif kind == "gelu":
                r, c = Q(a[0])[0].shape
                self.meta[label] = {"kind": kind, "bytes": 2 * r * c + 2 * (r * c // 1024) * 4}
            else:
                r, c = Q(a[0])[0].shape
                self.meta[label] = {"kind": kind, "bytes": 3 * r * c + 3 * (r * c // 1024) * 4}
        self.gemm_ops = sum(m["ops"] for m in self.meta.values() if m["kind"] == "gemm")
        assert self.gemm_ops == self.wl.gemm_ops()

    def run_op(self, kind, a):
        jf, q = self.jf, self.q
        if kind == "quant":
            jf.quantize_block(self.fp[a[0]], q=q[a[0]][0], s=q[a[0]][1])
        elif kind == "requant":
            jf.requant_block(self.fp[a[0]], q=q[a[0]][0], s=q[a[0]][1])
        elif kind == "gemm":
            an, bn, ta, tb, cn = a
            jf.gemm_i8_blockscaled(q[an][0], q[an][1], q[bn][0], q[bn][1], ta, tb, out="i8",
                                   c=q[cn][0], sc=q[cn][1])
        elif kind == "gelu":
            jf.gelu_i8(q[a[0]][0], q[a[0]][1], qo=q[a[1]][0], so=q[a[1]][1])
        elif kind == "gelu_bwd":
            jf.gelu_bwd_i8(q[a[0]][0], q[a[0]][1], q[a[1]][0], q[a[1]][1], qo=q[a[2]][0], so=q[a[2]][1])

    def run(self, events=None):
        for i, (kind, label, a) in enumerate(self.ops):
            if events is not None:
                events[i][0].record()
            self.run_op(kind, a)
            if events is not None:
                events[i][1].record()


def kernel_name(meta):
    """Kernel family of a step entry (one HIP kernel instantiation each)."""
    if meta["kind"] == "gemm":
        return f"gemm_i8bs tA={meta['tA']} tB={meta['tB']} i8-out"
    return {"quant": "quantize_block f32", "requant": "quantize_block f32", "gelu": "gelu_i8",
            "gelu_bwd": "gelu_bwd_i8"}[meta["kind"]]


def read_traffic():
    """key: value lines of the traffic summary (rocprofv3 FETCH_SIZE + WRITE_SIZE per
    launch of each GEMM kernel family, scaled by the plain-copy calibration)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    out = {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            out[k.strip()] = v.strip().strip("`")
    return out


def profile_traffic(family: str):
    """HBM bytes per launch of a GEMM kernel family from the committed counter
    summary, or None when that summary was taken on other GEMM sources (its
    source_digest differs) or does not list the family."""
    tr = read_traffic()
    if tr and tr.get("source_digest") == source_digest() and f"traffic[{family}]" in tr:
        return int(tr[f"traffic[{family}]"])
    return None


def source_digest() -> str:
    h = hashlib.sha256()
    for f in ("csrc/gemm.hip", "csrc/jf_tile_order.h", "csrc/jf_device.h", "_build.py"):   # the kernel, how it is compiled
        h.update(open(os.path.join(ROOT, "int8_block_quantized_amd", f), "rb").read())
    return h.hexdigest()[:16]


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count()}


def cpu_full_configs():
    """The oracle timed in full on the tiny forward, GPT2-base linear,
    GPT2-medium MLP and memory-bound workloads (every GEMM output block, the
    whole GELU / GELU backward / quantize) with the threads it uses."""
    import numpy as np

    import oracle
    from int8_block_quantized_amd import inputs

    out = {"threads": oracle.get_threads(), **cpu_info()}

    def gemm_set(wl, cache, keep=()):
        t_all, ops, kept = 0.0, 0, {}
        for (label, ta, tb, M, N, K, an, bn) in wl.gemms():
            for n in (an, bn):
                if n not in cache:
                    cache[n] = oracle.quantize(wl.make(n))
            t = time.perf_counter()
            r = oracle.gemm_i8(*cache[an], *cache[bn], ta=ta, tb=tb)
            t_all += time.perf_counter() - t
            ops += 2 * M * N * K
            if label in keep:
                kept[label] = r
        return t_all, ops, kept

    wl = inputs.tiny_forward()
    t0 = time.perf_counter()
    qx, sx = oracle.quantize(wl.make("X"))
    qw, sw = oracle.quantize(wl.make("W"))
    oracle.gemm_i8(qx, sx, qw, sw)
    out["tiny_forward"] = {"seconds": round(time.perf_counter() - t0, 4),
                           "what": "quantize X and W (256x256), block-scaled GEMM 256^3 with INT8 output"}
    for key, wl in (("gpt2_base_linear", inputs.gpt2_base_linear()), ("gpt2_medium_mlp", inputs.gpt2_medium_mlp())):
        cache = {}
        secs, ops, kept = gemm_set(wl, cache, keep=("fc1.fwd",))
        e = {"gemm_seconds": round(secs, 2), "gemm_ops": ops, "tops": round(ops / secs / 1e12, 5)}
        if key == "gpt2_medium_mlp":
            t = time.perf_counter()
            oracle.gelu(*kept["fc1.fwd"])
            e["gelu_seconds"] = round(time.perf_counter() - t, 2)
            e["gelu_what"] = "INT8 GELU of FC1's forward output, 8192x4096"
        e["what"] = f"{wl.name}: every GEMM (fwd, dgrad, wgrad) in full, INT8 output"
        out[key] = e
        log(f"cpu full: {key} {e}")
    x = inputs.memory_bound().make("X")
    t = time.perf_counter()
    q, sc = oracle.quantize(x)
    tq = time.perf_counter() - t
    t = time.perf_counter()
    oracle.gelu(q, sc)
    tg = time.perf_counter() - t
    n = x.size
    out["memory_bound"] = {"quantize_seconds": round(tq, 2), "quantize_gbs": round(n * (5 + 4 / 1024) / tq / 1e9, 2),
                           "gelu_seconds": round(tg, 2), "gelu_gbs": round(n * (2 + 8 / 1024) / tg / 1e9, 2),
                           "what": "16384x16384: quantize fp32 -> INT8, then INT8 GELU, in full"}
    out["kind"] = "oracle"
    return out


def cpu_baseline(step, target_s):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np

    import oracle

    threads = oracle.get_threads()
    wl = step.wl
    t0 = time.time()
    cq = {}

    def codes(name):
        # the GELU output G is a pipeline intermediate; for timing, the
        # workload's synthetic H stands in (and its synthetic dH for the
        # GELU-backward output)
        if name not in cq:
            src = {"G": "H"}.get(name, name)
            cq[name] = oracle.quantize(step.host[src] if src in step.host else wl.make(src))
        return cq[name]

    gemms = [(label, m, a) for (kind, label, a), m in
             ((op, step.meta[op[1]]) for op in step.ops) if kind == "gemm"]
    for label, m, a in gemms:
        codes(a[0]), codes(a[1])
    log(f"cpu baseline: oracle quantized operands in {time.time() - t0:.1f} s")

    def sample(frac, seed=0):
        g = np.random.default_rng(seed)
        ops, secs = 0, 0.0
        for label, m, a in gemms:
            nbM, nbN = m["M"] // 32, m["N"] // 32
            n = max(1, int(round(frac * nbM * nbN)))
            blks = np.stack([g.integers(nbM, size=n), g.integers(nbN, size=n)], 1)
            (qa, sa), (qb, sb) = codes(a[0]), codes(a[1])
            t = time.perf_counter()
            oracle.gemm_i8_blocks(qa, sa, qb, sb, blks, ta=m["tA"], tb=m["tB"])
            secs += time.perf_counter() - t
            ops += n * 2 * 32 * 32 * m["K"]
        return ops, secs

    ops0, s0 = sample(2e-4, seed=1)
    frac = 2e-4 * max(1.0, target_s / max(s0, 1e-3))
    frac = min(frac, 0.05)
    ops, secs = sample(frac, seed=2)
    return {"value": ops / secs / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle", **cpu_info(),
            "extrapolated": True,
            "sample": (f"{frac * 100:.3f}% of the output 32x32 blocks of each of the 12 GEMMs "
                       f"(random, seeded), INT8 output, {ops / 1e9:.1f} G ops in {secs:.1f} s; "
                       "synthetic H/dH stand in for the GELU output and the GELU-backward output")}


def bf16_reference(step, steps):
    """The same 12 GEMM shapes as plain bfloat16 GEMMs (torch.mm, i.e. the
    vendor BLAS), for the INT8-vs-bf16 comparison of the linear layers.
    Operands are laid out beforehand (no transposed views), outputs are bf16,
    inputs random N(0,1).  Returns (GEMMs only, GEMMs + the bf16 GELU of the
    FC1 output and its backward): the second is the bf16 counterpart of the
    INT8 step, which also runs its GELU, GELU backward and quantizations."""
    import torch

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    mats = []
    for kind, label, a in step.ops:
        if kind != "gemm":
            continue
        m = step.meta[label]
        A = torch.randn((m["M"], m["K"]), device=dev, generator=g).to(torch.bfloat16)
        B = torch.randn((m["K"], m["N"]), device=dev, generator=g).to(torch.bfloat16)
        C = torch.empty((m["M"], m["N"]), device=dev, dtype=torch.bfloat16)
        mats.append((A, B, C))

    fc1 = step.meta["fc1.fwd"]
    h = torch.randn((fc1["M"], fc1["N"]), device=dev, generator=g).to(torch.bfloat16)
    dh = torch.randn((fc1["M"], fc1["N"]), device=dev, generator=g).to(torch.bfloat16)

    def run():
        for A, B, C in mats:
            torch.mm(A, B, out=C)

    def run_layer():
        run()
        torch.nn.functional.gelu(h)                    # erf form
        torch.ops.aten.gelu_backward(dh, h)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    ms, layer_ms = timed(run), timed(run_layer)
    del mats, h, dh
    torch.cuda.empty_cache()
    return ms, layer_ms


def int8_library_reference(step, steps):
    """The same 12 GEMM shapes as plain INT8 GEMMs with int32 output
    (torch._int_mm, i.e. the vendor BLAS): the contraction alone, with no
    per-block scales, no rescale and no requantization -- the rate the INT8
    matrix cores reach through the library, for context.  Random int8
    operands, A row-major, B column-major (the library's preferred layout)."""
    import torch

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    mats = []
    for kind, label, a in step.ops:
        if kind != "gemm":
            continue
        m = step.meta[label]
        A = torch.randint(-127, 128, (m["M"], m["K"]), device=dev, generator=g, dtype=torch.int8)
        B = torch.randint(-127, 128, (m["N"], m["K"]), device=dev, generator=g, dtype=torch.int8).t()
        mats.append((A, B))

    def run():
        for A, B in mats:
            torch._int_mm(A, B)

    run()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        run()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del mats
    torch.cuda.empty_cache()
    return ms


def quant_error_section(step, reps=10):
    """jf_quant_error on the step's input activations X (8192 x 4096, outlier
    columns): per scale granularity the mean squared quantization error and
    the kernels' time.  Block scales take one pass over X; rows, columns and
    the tensor take two (maxima, then errors)."""
    import torch

    jf = step.jf
    x = step.fp["X"]
    n = x.numel()
    res = {}
    for gran in ("block", "token", "channel", "tensor"):
        s, e = jf.quant_error(x, gran)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            jf.quant_error(x, gran, s, e)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / reps * 1e3
        passes = 1 if gran == "block" else 2
        res[gran] = {"mse": float(e.item()) / n, "us": round(us, 1),
                     "read_gbs": round(passes * 4 * n / (us * 1e-6) / 1e9, 1), "passes": passes}
    res["block_vs_token_mse"] = round(res["block"]["mse"] / res["token"]["mse"], 4)
    res["what"] = "X 8192x4096 (N(0,1), 0.5% of columns x100): sum (x - s q)^2 / n per scale granularity"
    return res


def _time_us(fn, reps):
    import torch

    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e3


def data_flow_ops_section(step, reps=20):
    """The residual add and LayerNorm (INT8 in and out) on the step's shapes:
    R = X + A (8192 x 4096), then LayerNorm of R over the hidden dimension."""
    import numpy as np
    import torch

    jf = step.jf
    qx, sx = step.q["X"]
    qa, sa = step.q["A"]
    dev = qx.device
    jf.quantize_block(step.fp["X"], q=qx, s=sx)
    jf.requant_block(step.fp["A"], q=qa, s=sa)
    qr, sr = torch.empty_like(qx), torch.empty_like(sx)
    ql, sl = torch.empty_like(qx), torch.empty_like(sx)
    g = np.random.default_rng(11)
    C = qx.shape[1]
    gamma = torch.from_numpy(g.normal(1.0, 0.1, C).astype(np.float32)).to(dev)
    beta = torch.from_numpy(g.normal(0.0, 0.1, C).astype(np.float32)).to(dev)
    n = qx.numel()
    add_us = _time_us(lambda: jf.add_i8(qx, sx, qa, sa, qr, sr), reps)
    ln_us = _time_us(lambda: jf.layernorm_i8(qr, sr, gamma, beta, 1e-5, ql, sl), reps)
    nblk = n // 1024
    return {"residual_add": {"us": round(add_us, 1), "gbs": round((3 * n + 12 * nblk) / (add_us * 1e-6) / 1e9, 1),
                             "bytes_per_element": 3.0117},
            "layernorm": {"us": round(ln_us, 1), "gbs": round((2 * n + 8 * nblk) / (ln_us * 1e-6) / 1e9, 1),
                          "bytes_per_element": 2.0078},
            "what": "R = X + A and LayerNorm(R) on 8192x4096 per-block INT8 tensors (INT8 in and out); GB/s of "
                    "algorithmic bytes (inputs and outputs once)"}


def mlp1024_section(reps=10):
    """The GPT2-medium-like MLP (8192 tokens, 1024 -> 4096 -> 1024) in the
    INT8 data flow (quantize X, W1, W2, dY; FC1 -> GELU -> FC2; FC2 dgrad and
    wgrad; GELU backward; FC1 dgrad and wgrad: 13 kernels) against its six
    GEMM shapes as bfloat16 torch.mm."""
    import torch

    from int8_block_quantized_amd import inputs
    from int8_block_quantized_amd import jetfire as jf

    dev = torch.device("cuda:0")
    wl = inputs.gpt2_medium_mlp()
    fp = {n: torch.from_numpy(wl.make(n)).to(dev) for n in ("X", "W1", "W2", "dY2")}
    T = 8192

    def buf(r, c):
        return (torch.empty((r, c), dtype=torch.int8, device=dev),
                torch.empty((r // 32, c // 32), dtype=torch.float32, device=dev))

    q = {n: buf(*t.shape) for n, t in fp.items()}
    for n, (r, c) in {"H": (T, 4096), "G": (T, 4096), "Y": (T, 1024), "dG": (T, 4096), "dW2": (4096, 1024),
                      "dH": (T, 4096), "dX": (T, 1024), "dW1": (1024, 4096)}.items():
        q[n] = buf(r, c)

    def gemm(a, b, ta, tb, c):
        jf.gemm_i8_blockscaled(q[a][0], q[a][1], q[b][0], q[b][1], ta, tb, out="i8", c=q[c][0], sc=q[c][1])

    gemms = [("X", "W1", 0, 0, "H"), ("G", "W2", 0, 0, "Y"), ("dY2", "W2", 0, 1, "dG"), ("G", "dY2", 1, 0, "dW2"),
             ("dH", "W1", 0, 1, "dX"), ("X", "dH", 1, 0, "dW1")]

    def step():
        for n in ("X", "W1", "W2"):
            jf.quantize_block(fp[n], q=q[n][0], s=q[n][1])
        gemm(*gemms[0])
        jf.gelu_i8(q["H"][0], q["H"][1], qo=q["G"][0], so=q["G"][1])
        gemm(*gemms[1])
        jf.quantize_block(fp["dY2"], q=q["dY2"][0], s=q["dY2"][1])
        gemm(*gemms[2])
        gemm(*gemms[3])
        jf.gelu_bwd_i8(q["dG"][0], q["dG"][1], q["H"][0], q["H"][1], qo=q["dH"][0], so=q["dH"][1])
        gemm(*gemms[4])
        gemm(*gemms[5])

    def gemms_only():
        for gm in gemms:
            gemm(*gm)

    ops = wl.gemm_ops()
    step_us = _time_us(step, reps)
    gemm_us = _time_us(gemms_only, reps)
    g = torch.Generator(device=dev)
    g.manual_seed(8)
    mats = []
    for a, b, ta, tb, c in gemms:
        M, N = q[c][0].shape
        K = q[a][0].shape[0] if ta else q[a][0].shape[1]
        mats.append((torch.randn((M, K), device=dev, generator=g).to(torch.bfloat16),
                     torch.randn((K, N), device=dev, generator=g).to(torch.bfloat16),
                     torch.empty((M, N), device=dev, dtype=torch.bfloat16)))

    def bf16():
        for A, B, C in mats:
            torch.mm(A, B, out=C)

    h = torch.randn((8192, 4096), device=dev, generator=g).to(torch.bfloat16)
    dh = torch.randn((8192, 4096), device=dev, generator=g).to(torch.bfloat16)

    def bf16_layer():
        bf16()
        torch.nn.functional.gelu(h)
        torch.ops.aten.gelu_backward(dh, h)

    bf_us = _time_us(bf16, reps)
    bfl_us = _time_us(bf16_layer, reps)
    del mats, q, fp, h, dh
    torch.cuda.empty_cache()
    return {"int8_step_ms": round(step_us / 1e3, 4), "int8_step_tops": round(ops / (step_us * 1e-6) / 1e12, 1),
            "int8_gemm_ms": round(gemm_us / 1e3, 4), "int8_gemm_tops": round(ops / (gemm_us * 1e-6) / 1e12, 1),
            "bf16_gemm_ms": round(bf_us / 1e3, 4), "bf16_tflops": round(ops / (bf_us * 1e-6) / 1e12, 1),
            "int8_gemm_speedup": round(bf_us / gemm_us, 3), "gemm_ops": ops,
            "bf16_layer_ms": round(bfl_us / 1e3, 4), "int8_step_speedup": round(bfl_us / step_us, 3),
            "what": "GPT2-medium-like MLP, 8192 tokens, 1024->4096->1024: INT8 data flow (13 kernels) and its "
                    "6 INT8 GEMMs vs the same 6 GEMM shapes as torch.mm in bfloat16; bf16 layer: those GEMMs "
                    "plus the bf16 GELU of the 8192x4096 FC1 output and its backward, against the INT8 data flow"}


CEIL = {"mfma_only": 0, "mfma_rescale": 1, "mfma_bias_rescale": 2, "copy_i8": 3, "copy_f32_to_i8": 4,
        "copy_2i8_to_i8": 5}


def ceilings_section():
    """Measured ceilings (libjfceil.so): the INT8 matrix-core rate with no
    other work, the GEMM's per-(block, k-block) arithmetic (MFMA, convert,
    fma) with no memory traffic, the same with the partial converted through
    the MFMA's C operand, and streaming copies with the memory-bound kernels'
    byte patterns on 16384^2 elements (two input sets in turn)."""
    import ctypes

    from int8_block_quantized_amd import _build

    if not os.path.exists(_build.CEIL_PATH):
        _build.build_ceilings()
    lib = ctypes.CDLL(_build.CEIL_PATH)
    lib.jfc_measure.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_double)]
    lib.jfc_measure.restype = ctypes.c_int
    n = 16384 * 16384
    plan = {"mfma_only": (20000, 10), "mfma_rescale": (5000, 10), "mfma_bias_rescale": (5000, 10),
            "copy_i8": (n, 20), "copy_f32_to_i8": (4 * n, 10), "copy_2i8_to_i8": (n, 20)}
    out = {}
    for name, (size, reps) in plan.items():
        rate, us = ctypes.c_double(), ctypes.c_double()
        rc = lib.jfc_measure(CEIL[name], size, reps, ctypes.byref(rate), ctypes.byref(us))
        if rc != 0:
            raise RuntimeError(f"jfc_measure({name}) failed: hip error {rc}")
        unit = "TOPS" if name.startswith("mfma") else "GB/s"
        out[name] = {"rate": round(rate.value, 1), "unit": unit, "us": round(us.value, 1)}
    out["what"] = ("register-only loops on 256 CUs x 4 wavefronts per SIMD (2x2 output blocks per wavefront): "
                   "v_mfma_i32_32x32x32_i8 alone; each MFMA followed by the GEMM's rescale (cvt + fma per "
                   "result); the same with the bias conversion (sub + fma); streaming copies 16384^2 "
                   "int8->int8, fp32->int8, two int8 -> int8")
    return out


def small_configs_section(reps=50):
    """GPU times of the tiny forward (256^3) and the GPT2-base linear
    (4096 tokens, 768 -> 3072) workloads."""
    import torch

    from int8_block_quantized_amd import inputs
    from int8_block_quantized_amd import jetfire as jf

    dev = torch.device("cuda:0")
    out = {}
    wl = inputs.tiny_forward()
    x, w = (torch.from_numpy(wl.make(n)).to(dev) for n in ("X", "W"))
    qx, sx = jf.quantize_block(x)
    qw, sw = jf.quantize_block(w)
    qy, sy = jf.gemm_i8_blockscaled(qx, sx, qw, sw)
    cy = jf.gemm_i8_blockscaled(qx, sx, qw, sw, out="f32")

    def tiny_i8():
        jf.quantize_block(x, q=qx, s=sx)
        jf.quantize_block(w, q=qw, s=sw)
        jf.gemm_i8_blockscaled(qx, sx, qw, sw, c=qy, sc=sy)

    def tiny_f32():
        jf.quantize_block(x, q=qx, s=sx)
        jf.quantize_block(w, q=qw, s=sw)
        jf.gemm_i8_blockscaled(qx, sx, qw, sw, out="f32", c=cy)
        jf.requant_block(cy, q=qy, s=sy)

    ops = 2 * 256 ** 3
    for key, fn in (("tiny_i8_out_us", tiny_i8), ("tiny_f32_out_requant_us", tiny_f32)):
        out[key] = round(_time_us(fn, reps), 2)
    # the same three calls captured once in a HIP graph and replayed (no host work per kernel)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tiny_i8()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        tiny_i8()
    out["tiny_i8_out_graph_us"] = round(_time_us(graph.replay, reps), 2)
    out["tiny_gemm_i8_us"] = round(_time_us(lambda: jf.gemm_i8_blockscaled(qx, sx, qw, sw, c=qy, sc=sy), reps), 2)
    # the same calls straight through the C ABI with prepared arguments: no per-call Python argument checks,
    # so the time is the kernels' own (the binding's checks cost several microseconds per call)
    import ctypes

    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a_qx = (jf.JF_F32, p(x), 256, 256, 256, p(qx), 256, p(sx), st)
    a_qw = (jf.JF_F32, p(w), 256, 256, 256, p(qw), 256, p(sw), st)
    a_mm = (0, 0, 256, 256, 256, p(qx), 256, p(sx), p(qw), 256, p(sw), jf.JF_OUT_I8, p(qy), 256, p(sy), st)

    def tiny_abi():
        jf.lib.jf_quantize_block(*a_qx)
        jf.lib.jf_quantize_block(*a_qw)
        jf.lib.jf_gemm_i8_blockscaled(*a_mm)

    for fn, args in ((jf.lib.jf_quantize_block, a_qx), (jf.lib.jf_quantize_block, a_qw),
                     (jf.lib.jf_gemm_i8_blockscaled, a_mm)):
        if fn(*args) != jf.JF_OK:
            raise RuntimeError(f"{fn.__name__}: {jf.status_str(fn(*args))}")
    out["tiny_i8_out_abi_us"] = round(_time_us(tiny_abi, reps), 2)
    out["tiny_gemm_i8_abi_us"] = round(_time_us(lambda: jf.lib.jf_gemm_i8_blockscaled(*a_mm), reps), 2)
    out["tiny_gemm_tops"] = round(ops / (out["tiny_gemm_i8_abi_us"] * 1e-6) / 1e12, 2)
    out["tiny_what"] = ("tiny forward 256x256x256: quantize X and W, GEMM with INT8 output (i8_out; i8_out_graph: "
                        "the three calls replayed from a captured HIP graph); or binary32 output then "
                        "jf_requant_block (f32_out_requant); the GEMM alone (gemm_i8); *_abi: the same calls made "
                        "directly through the C ABI with prepared arguments (no Python argument checks)")
    wl = inputs.gpt2_base_linear()
    fp = {n: torch.from_numpy(wl.make(n)).to(dev) for n in ("X", "W", "dY")}
    q = {n: jf.quantize_block(t) for n, t in fp.items()}
    res = {}
    tot_us, tot_ops = 0.0, 0
    for (label, ta, tb, M, N, K, an, bn) in wl.gemms():
        c, sc = jf.gemm_i8_blockscaled(q[an][0], q[an][1], q[bn][0], q[bn][1], ta, tb)
        us = _time_us(lambda: jf.gemm_i8_blockscaled(q[an][0], q[an][1], q[bn][0], q[bn][1], ta, tb, c=c, sc=sc),
                      reps)
        res[label] = {"us": round(us, 1), "tops": round(2 * M * N * K / (us * 1e-6) / 1e12, 1)}
        tot_us += us
        tot_ops += 2 * M * N * K
    out["gpt2_base_linear"] = {**res, "total_us": round(tot_us, 1), "tops": round(tot_ops / (tot_us * 1e-6) / 1e12, 1),
                               "what": "4096 tokens, 768 -> 3072: fwd, dgrad, wgrad with INT8 output"}
    torch.cuda.empty_cache()
    return out


def memory_bound_section(reps=20):
    """The memory-bound workload: a 16384 x 16384 fp32 activation (N(0,1),
    1% of columns x100) through jf_quantize_block, then jf_gelu_i8 on its codes.
    Two copies of every input are used in turn so no call finds its input in
    the 256 MB Infinity Cache.  Algorithmic bytes per element: quantize 4 + 1
    + 4/1024, GELU 1 + 1 + 8/1024."""
    import torch

    from int8_block_quantized_amd import inputs
    from int8_block_quantized_amd import jetfire as jf

    dev = torch.device("cuda:0")
    x = torch.from_numpy(inputs.memory_bound().make("X")).to(dev)
    xs = [x, x.clone()]
    R, C = x.shape
    n = R * C
    qs = [jf.quantize_block(t) for t in xs]
    q, s = torch.empty_like(qs[0][0]), torch.empty_like(qs[0][1])
    qo, so = torch.empty_like(q), torch.empty_like(s)
    i = [0]

    def quant():
        i[0] ^= 1
        jf.quantize_block(xs[i[0]], q=q, s=s)

    def gelu():
        i[0] ^= 1
        jf.gelu_i8(qs[i[0]][0], qs[i[0]][1], qo=qo, so=so)

    y = torch.empty((R, C), dtype=torch.bfloat16, device=dev)

    def dequant():
        i[0] ^= 1
        jf.dequantize_block(qs[i[0]][0], qs[i[0]][1], dtype=torch.bfloat16, y=y)

    q_us = _time_us(quant, reps)
    g_us = _time_us(gelu, reps)
    d_us = _time_us(dequant, reps)
    qb, gb, db = n * (5 + 4 / 1024), n * (2 + 8 / 1024), n * (3 + 4 / 1024)
    check = gelu_copy_check(x, qs[0][1], *jf.gelu_i8(qs[0][0], qs[0][1]), y)
    del xs, x, qs, y
    torch.cuda.empty_cache()
    out = {}
    for name, us, nb in (("quantize", q_us, qb), ("gelu", g_us, gb), ("dequantize_bf16", d_us, db)):
        gbs = nb / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 1), "gbs": round(gbs, 1), "frac_of_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    out["gelu_bf16_copy_check"] = check
    out["what"] = ("16384x16384 fp32 N(0,1) with 1% of columns x100: jf_quantize_block (fp32 -> INT8 + 32x32 "
                   "scales), then jf_gelu_i8 on the codes, and jf_dequantize_block of codes to bfloat16 "
                   "(3 + 4/1024 B per element); two input copies used in turn")
    return out


def gelu_copy_check(x, s1, qg, sg, y):
    """The bfloat16 dequantized copy of the INT8 GELU output against the
    binary64 GELU of the original fp32 activation (outside any timed region).
    Per element the data flow's error is bounded by the input quantization
    (|x - s1 q1| <= s1 (1/2 + 2e-5) with the quotient's rounding, times
    max |GELU'| < 1.13), the output code rounding (s2 (1/2 + 2e-5)) and the
    bfloat16 rounding (half an ulp of 8 significant bits: 2^-8 (1 + 2^-7)
    relative to the rounded value);
    reported: the largest error over that bound, the largest error in output
    code units (err / s2) and the normwise relative error."""
    import torch

    from int8_block_quantized_amd import jetfire as jf

    jf.dequantize_block(qg, sg, dtype=torch.bfloat16, y=y)
    R, C = x.shape
    worst_bound = worst_lsb = num = den = 0.0
    for r0 in range(0, R, 2048):
        xs = x[r0:r0 + 2048].double()
        g = 0.5 * xs * torch.special.erfc(-xs / math.sqrt(2.0))
        yb = y[r0:r0 + 2048].double()
        e = (yb - g).abs()
        e1 = s1[r0 // 32:(r0 + 2048) // 32].double().repeat_interleave(32, 0).repeat_interleave(32, 1)
        e2 = sg[r0 // 32:(r0 + 2048) // 32].double().repeat_interleave(32, 0).repeat_interleave(32, 1)
        bound = 1.13 * e1 * (0.5 + 2e-5) + e2 * (0.5 + 2e-5) + 2.0 ** -8 * (1 + 2.0 ** -7) * yb.abs() + 1e-30
        worst_bound = max(worst_bound, float((e / bound).max()))
        worst_lsb = max(worst_lsb, float((e / torch.where(e2 > 0, e2, torch.ones_like(e2))).max()))
        num += float((e * e).sum())
        den += float((g * g).sum())
        del xs, g, yb, e, e1, e2, bound
    return {"max_err_over_bound": round(worst_bound, 4), "max_err_output_lsb": round(worst_lsb, 4),
            "rel_fro": float(f"{math.sqrt(num / den):.4e}"),
            "what": "bf16(fl(s2 q2)) of jf_gelu_i8's output vs binary64 GELU(x) of the fp32 input"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path has no multi-GPU part)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        dev = torch.device("cuda:0")
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            # a plain streaming kernel: reads and writes MIB each (copy_ of a
            # contiguous tensor goes to the runtime's blit path instead)
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(f"copied {args.copy_calibration} MiB x 5", file=sys.stderr)
        return

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)
    from int8_block_quantized_amd import _build

    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    dev = torch.device("cuda:0")
    step = Step(dev)

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    n_ops = len(step.ops)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_ops)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for k in range(args.steps):
        step.run(ev[k])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps

    # per-kernel durations (ms) over the timed steps: the mean (what the
    # rocprofv3 kernel statistics average, used for the roofline) and the median
    per, per_med = {}, {}
    for i, (kind, label, a) in enumerate(step.ops):
        d = sorted(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps))
        per[label] = sum(d) / len(d)
        per_med[label] = d[len(d) // 2]
    step_spans = sorted(ev[k][0][0].elapsed_time(ev[k][n_ops - 1][1]) for k in range(args.steps))
    ms_step_median = step_spans[len(step_spans) // 2]

    families = {}
    for label, m in step.meta.items():
        f = families.setdefault(kernel_name(m), {"ms": 0.0, "launches": 0, "ops": 0, "bytes": 0})
        f["ms"] += per[label]
        f["launches"] += 1
        f["ops"] += m.get("ops", 0)
        f["bytes"] += m.get("bytes", 0)
    dom_name, dom = max(families.items(), key=lambda kv: kv[1]["ms"])
    if "gemm" in dom_name:
        achieved = dom["ops"] / (dom["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "unit": "TOPS", "peak": INT8_PEAK_TOPS}
    else:
        achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "unit": "GB/s", "peak": HBM_PEAK_GBS}
    roof.update({"kernel": dom_name, "achieved": round(achieved, 2),
                 "frac": round(achieved / roof["peak"], 4),
                 "avg_launch_us": round(dom["ms"] / dom["launches"] * 1e3, 2),
                 "launches_per_step": dom["launches"], "traffic": profile_traffic(dom_name)})

    gemm_ms = sum(per[l] for l, m in step.meta.items() if m["kind"] == "gemm")
    value = step.gemm_ops / (ms_step * 1e-3) / 1e12
    kernels = {}
    for label, m in step.meta.items():
        e = {"us_median": round(per_med[label] * 1e3, 1), "us_mean": round(per[label] * 1e3, 1)}
        if m["kind"] == "gemm":
            e["tops"] = round(m["ops"] / (per_med[label] * 1e-3) / 1e12, 1)
        else:
            e["gbs"] = round(m["bytes"] / (per_med[label] * 1e-3) / 1e9, 1)
        kernels[label] = e

    bf16 = None
    if args.bf16_steps > 0:
        bms, blms = bf16_reference(step, args.bf16_steps)
        bf16 = {"ms_per_step": round(bms, 4), "tflops": round(step.gemm_ops / (bms * 1e-3) / 1e12, 2),
                "int8_gemm_speedup": round(bms / gemm_ms, 3),
                "layer_ms_per_step": round(blms, 4), "int8_step_speedup": round(blms / ms_step, 3),
                "what": "the 12 GEMM shapes as torch.mm in bfloat16 (vendor BLAS), operands pre-laid-out, "
                        "bf16 outputs; compared with the INT8 GEMMs' time in the step. layer: the same GEMMs "
                        "plus the bf16 GELU of the 8192x16384 FC1 output and its backward, against the whole "
                        "INT8 step (its GEMMs, quantizations, GELU and GELU backward)"}
    i8lib = None
    if args.bf16_steps > 0:
        try:
            lms = int8_library_reference(step, args.bf16_steps)
            i8lib = {"ms_per_step": round(lms, 4), "tops": round(step.gemm_ops / (lms * 1e-3) / 1e12, 2),
                     "frac_of_int8_peak": round(step.gemm_ops / (lms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                     "block_scaled_over_plain_time": round(gemm_ms / lms, 3),
                     "what": "the 12 GEMM shapes as plain INT8 GEMMs with int32 output (torch._int_mm, vendor "
                             "BLAS): no block scales, rescale or requantization; the matrix cores' rate for "
                             "the contraction alone"}
        except Exception as exc:  # context only, never gating
            log(f"int8 library reference failed: {exc!r}")

    qerr = quant_error_section(step) if args.extras else None
    dfo = data_flow_ops_section(step) if args.extras else None

    mlp1024 = mlp1024_section() if args.extras else None
    membound = memory_bound_section() if args.extras else None
    small = small_configs_section() if args.extras else None
    ceil = None
    if args.ceilings:
        try:
            ceil = ceilings_section()
        except Exception as exc:  # context only, never gating
            log(f"ceilings failed: {exc!r}")
    if ceil:
        if roof["bound"] == "mfma":
            roof["ceiling"] = ceil["mfma_rescale"]["rate"]
            roof["ceiling_what"] = "measured register-only MFMA + rescale (cvt + fma) loop: this numerics' bound"
            roof["frac_of_ceiling"] = round(roof["achieved"] / ceil["mfma_rescale"]["rate"], 4)
            roof["mfma_only_measured"] = ceil["mfma_only"]["rate"]
        if membound:
            for name, cp in (("quantize", "copy_f32_to_i8"), ("gelu", "copy_i8")):
                membound[name]["copy_bound_gbs"] = ceil[cp]["rate"]
                membound[name]["frac_of_copy"] = round(membound[name]["gbs"] / ceil[cp]["rate"], 4)
    cpu_full = None
    if args.cpu_full:
        try:
            cpu_full = cpu_full_configs()
        except Exception as exc:  # reported, never gating
            log(f"cpu full configs failed: {exc!r}")

    cpu = None
    if args.cpu_seconds > 0:
        try:
            cpu = cpu_baseline(step, args.cpu_seconds)
        except Exception as exc:  # the baseline is reported, never gating
            log(f"cpu baseline failed: {exc!r}")

    out = {
        "metric": "block-scaled INT8 GEMM TOPS (fwd+dgrad+wgrad), hidden 4096; % of INT8 MFMA peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(ms_step_median, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "hidden-4096 transformer-block linears, 8192 tokens (8x1024): "
                               "QKV 4096->12288, out-proj 4096->4096, FC1 4096->16384, FC2 16384->4096; "
                               "fwd+dgrad+wgrad in the INT8 data flow with quantize/requant/GELU/GELU backward",
                   "tokens": 8192, "hidden": 4096, "gemms": 12, "gemm_ops_per_step": step.gemm_ops,
                   "block": 32},
        "frac_of_int8_peak": round(value / INT8_PEAK_TOPS, 4),
        "gemm_only_tops": round(step.gemm_ops / (gemm_ms * 1e-3) / 1e12, 2),
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_full_configs": cpu_full,
        "ceilings": ceil,
        "small_configs": small,
        "bf16_reference": bf16,
        "int8_library_reference": i8lib,
        "quant_error": qerr,
        "data_flow_ops": dfo,
        "mlp_hidden1024": mlp1024,
        "memory_bound": membound,
        "kernels": kernels,
        "host_wall_s": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
