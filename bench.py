"""Benchmark of the blockwise-FP8 linear layer hot path on one MI355X.

One step = one decoder layer's linear work at M tokens (default 4096, hidden
2048, intermediate 6144), everything the path computes:
  for each linear (qkv, o, gate_up, down):
    quantise X (1x128 row-wise and token-dimension, both from one read), W
    (128x128 with the transposed copy) and dY (both orientations, one read), then
    forward Y = X W^T (BF16 out), dgrad dX = dY W (BF16 out),
    wgrad dW = dY^T X (FP32 out).
Inputs are seeded synthetic BF16 tensors (X ~ N(0,1), W ~ N(0,0.02),
dY ~ N(0,1e-3)) already resident in HBM; outputs are preallocated, so the
timed region holds only kernel launches of libfp8blk.

Prints one JSON line.  `value` is GEMM TFLOP/s of the whole step (the 12 GEMMs'
2*M*N*K divided by the step time, quantisers included), from K steps between
two HIP events with no event inside a step (each event record costs the stream
about 5 us).  `roofline` covers the dominant kernel (the block GEMM), timed in a
second pass of K steps with one event bracket around each linear's three GEMMs
on the stream the kernels run on; its `frac` is taken against the FP8 dense
MFMA peak, the metric's own.  Per-GEMM figures come from K back-to-back
launches of each GEMM.  Before the W warm-up steps, untimed steps run for
--clock-warmup-s seconds (default 0.5): the GPU idles during the host-side
setup, and a timed region that starts before its clock has settled reads about
3% slow.  `cpu_baseline` times the numpy oracle on a bounded token
sample of the same layer with all host threads, and on the same sample with
one thread (`single_thread`), quantisers (GB/s) and GEMMs (TFLOP/s) apart.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"f16": 2500.0, "fp8": 5000.0}
PEAK_HBM_GBS = 8000.0
# HBM bytes per block-GEMM launch from FETCH_SIZE/WRITE_SIZE counters of this
# workload (used only while the summary's kernel-source digest still matches).
TRAFFIC_SUMMARY = "block_gemm_traffic_layer_m4096.txt"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--cpu-single-thread-tokens", type=int, default=4096)
    ap.add_argument("--no-fp8-path", action="store_true", help="skip timing the FP8 matrix-core GEMM path")
    ap.add_argument("--no-bf16-baseline", action="store_true", help="skip timing the BF16 GEMMs of the same shapes")
    ap.add_argument("--no-fusion", action="store_true", help="skip timing the fused producers")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 28-layer M=8192 sweep")
    ap.add_argument("--no-layer", action="store_true", help="skip the whole decoder layer fwd+bwd")
    ap.add_argument("--no-small-configs", action="store_true", help="skip the kernel-by-kernel timing of configurations 1 and 5")
    ap.add_argument("--clock-warmup-s", type=float, default=0.5,
                    help="untimed steps for this many seconds before the warm-up steps, so that the timed "
                         "region starts at the GPU's steady-state clock")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="launch one plain device copy of this size first (counter calibration)")
    return ap.parse_args()


class LayerBuffers:
    """Device inputs and preallocated outputs for one linear of the layer."""

    def __init__(self, torch, B, W, name, k, n, M, dev, cfg=2, layer=0, outliers=False):
        import numpy as np
        self.name, self.k, self.n, self.M = name, k, n, M
        # outliers (the 8192-token sweep): round(1% of K) input channels scaled by 32
        self.xb, self.wb, self.dyb = W.layer_tensors(cfg, layer, name, M, outliers=outliers)
        to = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        self.x, self.w, self.dy = to(self.xb), to(self.wb), to(self.dyb)
        # Outputs (allocated once, reused every step).
        self.xq, self.sx = B.fp8_quant_1x128(self.x)
        self.xqT, self.sxT = B.fp8_quant_1x128(self.x, transpose_out=True)
        self.wq, self.sw, self.wqT, self.swT = B.fp8_quant_128x128(self.w, with_transpose=True)
        self.dyq, self.sdy = B.fp8_quant_1x128(self.dy)
        self.dyqT, self.sdyT = B.fp8_quant_1x128(self.dy, transpose_out=True)
        self.y = torch.empty((M, n), dtype=torch.bfloat16, device=dev)
        self.dx = torch.empty((M, k), dtype=torch.bfloat16, device=dev)
        self.dw = torch.empty((n, k), dtype=torch.float32, device=dev)

    def flops(self):
        return 3 * 2 * self.M * self.n * self.k

    def gemm_flops(self):
        """2*M*N*K of the fwd, dgrad and wgrad GEMMs (all three equal)."""
        return [2 * self.M * self.n * self.k] * 3

    def gemm_bytes(self):
        """Algorithmic bytes of the fwd, dgrad and wgrad GEMMs: operands once, scales, output."""
        M, n, k = self.M, self.n, self.k
        mp = -(-M // 128) * 128
        fwd = M * k + n * k + 4 * M * (k // 128) + 4 * (n // 128) * (k // 128) + 2 * M * n
        dgrad = M * n + k * n + 4 * M * (n // 128) + 4 * (k // 128) * (n // 128) + 2 * M * k
        wgrad = n * mp + k * mp + 4 * (n + k) * (mp // 128) + 4 * n * k
        return [fwd, dgrad, wgrad]

    def quant_bytes(self, dual=True, M=None):
        """Algorithmic HBM bytes of the step's quantisers (inputs read once per kernel),
        at M tokens (default: the buffers' token count)."""
        M, n, k = (self.M if M is None else M), self.n, self.k
        row = lambda r, c: r * c * 3 + r * (-(-c // 128)) * 4          # 2 B in, 1 B out, scales
        tok = lambda r, c: r * c * 2 + c * (-(-r // 128) * 128) + c * (-(-r // 128)) * 4
        blk = n * k * 2 + 2 * n * k + 2 * 4 * (-(-n // 128)) * (-(-k // 128))
        both = row(M, k) + tok(M, k) + row(M, n) + tok(M, n)
        return blk + (both - 2 * M * k - 2 * M * n if dual else both)

    def quantise(self, B, dual=True):
        """All quantisers of the step; `dual` makes both 1x128 orientations of X and dY from one read."""
        if dual:
            B.fp8_quant_1x128_dual(self.x, self.xq, self.sx, self.xqT, self.sxT)
        else:
            B.fp8_quant_1x128(self.x, q=self.xq, scales=self.sx)
            B.fp8_quant_1x128(self.x, transpose_out=True, q=self.xqT, scales=self.sxT)
        B.fp8_quant_128x128(self.w, True, self.wq, self.sw, self.wqT, self.swT)
        if dual:
            B.fp8_quant_1x128_dual(self.dy, self.dyq, self.sdy, self.dyqT, self.sdyT)
        else:
            B.fp8_quant_1x128(self.dy, q=self.dyq, scales=self.sdy)
            B.fp8_quant_1x128(self.dy, transpose_out=True, q=self.dyqT, scales=self.sdyT)

    def gemm_calls(self, B, fp8_mc=False):
        """The forward, data-gradient and weight-gradient GEMM launches, as callables."""
        return [lambda: B.fp8_block_gemm_fwd(self.xq, self.sx, self.wq, self.sw, y=self.y, fp8_matrix_core=fp8_mc),
                lambda: B.fp8_block_gemm_dgrad(self.dyq, self.sdy, self.wqT, self.swT, dx=self.dx,
                                               fp8_matrix_core=fp8_mc),
                lambda: B.fp8_block_gemm_wgrad(self.dyqT, self.sdyT, self.xqT, self.sxT, M=self.M, dw=self.dw,
                                               fp8_matrix_core=fp8_mc)]

    def gemms(self, B, fp8_mc=False):
        """The three GEMMs of this linear."""
        for f in self.gemm_calls(B, fp8_mc):
            f()


def cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(W, layers, sample_tokens, single_thread_tokens):
    """The numpy oracle on the first `sample_tokens` tokens of every linear of the
    layer with all host threads, then on the first `single_thread_tokens` with
    one BLAS thread (the oracle itself is the same code either way).

    Quantisers and GEMMs are timed apart: the GEMMs as TFLOP/s (2*M*N*K), the
    quantisers as GB/s of the GPU step's algorithmic quantiser bytes at the
    sample's token count (the oracle reads its inputs once per orientation)."""
    import numpy as np
    from oracle import gemm, quant

    def run(tokens):
        flops = qbytes = 0
        tq = tg = 0.0
        for L in layers:
            xs, dys = L.xb[:tokens], L.dyb[:tokens]
            t0 = time.perf_counter()
            xq, sx = quant.quant_1x128_rows(xs)
            xqT, sxT = quant.quant_1x128_tokens(xs)
            wq, sw = quant.quant_128x128(L.wb)
            wqT, swT = quant.quant_128x128(np.ascontiguousarray(L.wb.T))
            dyq, sdy = quant.quant_1x128_rows(dys)
            dyqT, sdyT = quant.quant_1x128_tokens(dys)
            t1 = time.perf_counter()
            gemm.fwd(xq, sx, wq, sw, budget=False)
            gemm.dgrad(dyq, sdy, wqT, swT, budget=False)
            gemm.wgrad(dyqT, sdyT, xqT, sxT, budget=False)
            t2 = time.perf_counter()
            tq, tg = tq + (t1 - t0), tg + (t2 - t1)
            flops += 3 * 2 * tokens * L.n * L.k
            qbytes += L.quant_bytes(True, tokens)
        return flops, qbytes, tq, tg

    def report(tokens, threads):
        flops, qbytes, tq, tg = run(tokens)
        dt = tq + tg
        return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
                "gemm_tflops": round(flops / tg / 1e12, 6),
                "quantiser_gbps": round(qbytes / tq / 1e9, 3),
                "seconds": {"quantisers": round(tq, 2), "gemms": round(tg, 2)},
                "sample": (f"one layer's 4 linears (quantisers + fwd/dgrad/wgrad) on the first {tokens} tokens, "
                           f"numpy float64 oracle, {threads} BLAS thread(s), {dt:.1f} s")}

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    out = report(sample_tokens, threads)
    out["kind"] = "oracle"
    out["cpu_model"] = cpu_model()
    if threadpool_limits is not None and single_thread_tokens > 0:
        with threadpool_limits(limits=1):
            out["single_thread"] = report(single_thread_tokens, 1)
    return out


def bf16_baseline(torch, B, layers, steps, warmup, fp8_gemm_ms, fp8_step_ms, fp8_mc_gemm_ms):
    """The same 12 GEMM shapes in plain BF16: this library's BF16 kernel and hipBLASLt (torch.mm).

    For every linear: forward [M, k] x [n, k]^T, dgrad [M, n] x [k, n]^T and
    wgrad [n, M] x [k, M]^T, each as C = A . B^T with BF16 operands resident
    in HBM.  hipBLASLt gets the second operand pre-transposed ([L, J]
    row-major, prepared outside the timed region).  Ratios > 1 mean the FP8
    path is faster.
    """
    ops = []
    for L in layers:
        dyT = L.dy.t().contiguous()
        xT = L.x.t().contiguous()
        wT = L.w.t().contiguous()
        for a, b in ((L.x, L.w), (L.dy, wT), (dyT, xT)):
            ops.append((a, b, b.t().contiguous(), torch.empty((a.shape[0], b.shape[0]), dtype=torch.bfloat16,
                                                              device=a.device)))
    flops = sum(2 * a.shape[0] * b.shape[0] * a.shape[1] for a, b, _, _ in ops)
    mk = lambda: torch.cuda.Event(enable_timing=True)

    def run(fn):
        """GEMM ms per step, one event bracket around each linear's three GEMMs (as
        the FP8 step's GEMM time is taken)."""
        for _ in range(warmup):
            for op in ops:
                fn(*op)
        torch.cuda.synchronize()
        groups = [ops[i:i + 3] for i in range(0, len(ops), 3)]
        evs = [[(mk(), mk()) for _ in groups] for _ in range(steps)]
        for s in range(steps):
            for (e0, e1), grp in zip(evs[s], groups):
                e0.record()
                for op in grp:
                    fn(*op)
                e1.record()
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for row in evs for e0, e1 in row) / steps

    own_ms = run(lambda a, b, bt, c: B.bf16_gemm_nt(a, b, c=c))
    blas_ms = run(lambda a, b, bt, c: torch.mm(a, bt, out=c))
    out = {"gemm_gflop_per_step": round(flops / 1e9, 3),
           "own_kernel": {"gemm_ms_per_step": round(own_ms, 4), "tflops": round(flops / (own_ms * 1e-3) / 1e12, 1)},
           "hipblaslt": {"gemm_ms_per_step": round(blas_ms, 4), "tflops": round(flops / (blas_ms * 1e-3) / 1e12, 1)},
           "speedup_fp8_exact_gemms_vs_own_bf16": round(own_ms / fp8_gemm_ms, 3),
           "speedup_fp8_exact_gemms_vs_hipblaslt": round(blas_ms / fp8_gemm_ms, 3),
           "speedup_fp8_exact_step_vs_hipblaslt_gemms": round(blas_ms / fp8_step_ms, 3),
           "note": "BF16 GEMMs of the same 12 shapes; the FP8 step includes its quantisers"}
    if fp8_mc_gemm_ms is not None:
        out["speedup_fp8_matrix_core_gemms_vs_hipblaslt"] = round(blas_ms / fp8_mc_gemm_ms, 3)
    return out


def layer_sweep(torch, B, W, dev, n_layers=28, M=8192, sweeps=3):
    """Configuration 4: the whole hot path of 28 decoder layers at 8192 tokens.

    Each layer quantises X (both orientations), W (with its transposed copy) and
    dY (both orientations) of its four linears and runs their forward, dgrad and
    wgrad GEMMs.  Inputs have 1% outlier channels.  Two seeded layer sets
    (layers 0 and 1) are generated and alternate over the 28 layers, which keeps
    the input generation to seconds; the kernels' work does not depend on which
    set a layer reads.
    """
    sets = [[LayerBuffers(torch, B, W, n, k, nout, M, dev, cfg=4, layer=l, outliers=True) for n, k, nout in W.LINEARS]
            for l in (0, 1)]

    def sweep():
        for layer in range(n_layers):
            for L in sets[layer % 2]:
                L.quantise(B)
                L.gemms(B)

    sweep()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(sweeps):
        sweep()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / sweeps
    flops = n_layers * sum(L.flops() for L in sets[0])
    out = {"layers": n_layers, "tokens": M, "ms_per_sweep": round(ms, 3), "gemm_tflop_per_sweep": round(flops / 1e12, 3),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "inputs": "two seeded layer sets (1% outlier channels x32) alternating over the layers"}
    del sets
    torch.cuda.empty_cache()
    return out


def producer_fusion(torch, B, layers, steps, warmup):
    """Fused producers against their unfused form (PyTorch BF16 op, then the dual quantiser).

    SwiGLU: the down projection's input from the gate and up halves of the
    gate_up forward output [M, 12288]; RMSNorm: the qkv input [M, 2048] with a
    BF16 gain.  The two forms round differently: the fused SwiGLU rounds
    silu(g) * u once to BF16, PyTorch's F.silu(g) * u rounds silu(g) first and
    the product again, so a few codes can differ; the timing compares the
    same amount of work.
    """
    import torch.nn.functional as F
    gu = [L for L in layers if L.name == "gate_up"][0]
    qkv = [L for L in layers if L.name == "qkv"][0]
    B.fp8_block_gemm_fwd(gu.xq, gu.sx, gu.wq, gu.sw, y=gu.y)
    half = gu.n // 2
    g, u = gu.y[:, :half], gu.y[:, half:]
    M = g.shape[0]
    x = qkv.x
    gamma = (1.0 + 0.1 * torch.randn(x.shape[1], device=x.device)).to(torch.bfloat16)
    outs_s = B.fp8_quant_1x128_dual(g.contiguous())
    outs_r = B.fp8_quant_1x128_dual(x)
    rstd = torch.empty(M, dtype=torch.float32, device=x.device)
    mk = lambda: torch.cuda.Event(enable_timing=True)

    def t(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = mk(), mk()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e3

    fused_s = t(lambda: B.fp8_swiglu_quant_1x128_dual(g, u, None, *outs_s))
    unfused_s = t(lambda: B.fp8_quant_1x128_dual(F.silu(g) * u, *outs_s))
    fused_r = t(lambda: B.fp8_rmsnorm_quant_1x128_dual(x, gamma, 1e-6, None, rstd, *outs_r))
    unfused_r = t(lambda: B.fp8_quant_1x128_dual(F.rms_norm(x, (x.shape[1],), gamma, 1e-6), *outs_r))
    sw_bytes = M * half * (2 + 2 + 1 + 1) + 8 * M * half // 128
    rn_bytes = M * x.shape[1] * (2 + 2 + 1 + 1) + 8 * M * x.shape[1] // 128 + 4 * M
    return {"swiglu_to_fp8": {"shape": [M, half], "fused_us": round(fused_s, 2), "unfused_us": round(unfused_s, 2),
                              "speedup": round(unfused_s / fused_s, 3),
                              "fused_gbps": round(sw_bytes / (fused_s * 1e-6) / 1e9, 1)},
            "rmsnorm_to_fp8": {"shape": [M, x.shape[1]], "fused_us": round(fused_r, 2),
                               "unfused_us": round(unfused_r, 2), "speedup": round(unfused_r / fused_r, 3),
                               "fused_gbps": round(rn_bytes / (fused_r * 1e-6) / 1e9, 1)},
            "note": "unfused = PyTorch BF16 op (F.silu(g) * u, F.rms_norm) then fp8_quant_1x128_dual; "
                    "fused RMSNorm reads x twice (row statistics, then the fused pass)"}


def decoder_layer(torch, steps, warmup, batch=2, seq=4096):
    """Forward + backward of one whole decoder layer (hidden 2048, 16 query and 8
    key/value heads of 128, intermediate 6144) at 2 x 4096 tokens, with the four
    linears as Fp8Linear (exact block products, and the FP8 matrix
    instructions) and, for comparison, as BF16 nn.Linear (hipBLASLt).

    A second, hooked pass of each layer brackets each linear's forward and
    backward (for FP8: quantisers, GEMMs, main_grad accumulation) with events on
    the current stream, which gives the linears' share of the layer's time.
    """
    from blockwise_fp8_linear_quant_amd.layer import DecoderLayer
    g = torch.Generator().manual_seed(17)
    x0 = (torch.randn((batch, seq, 2048), generator=g) * 0.5).to(torch.bfloat16).cuda()
    dy = (torch.randn((batch, seq, 2048), generator=g) * 1e-3).to(torch.bfloat16).cuda()
    mk = lambda: torch.cuda.Event(enable_timing=True)

    def run(lay, n):
        for _ in range(n):
            x = x0.detach().requires_grad_(True)
            lay.zero_grad(set_to_none=True)
            lay(x).backward(dy)

    def t(lay):
        run(lay, warmup)
        torch.cuda.synchronize()
        e0, e1 = mk(), mk()
        e0.record()
        run(lay, steps)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def linear_share(lay):
        spans = []

        def pre(mod, *a):
            e = mk()
            e.record()
            spans.append([e, None])

        def post(mod, *a):
            e = mk()
            e.record()
            spans[-1][1] = e
        hooks = []
        for lin in lay.linears():
            hooks += [lin.register_forward_pre_hook(pre), lin.register_forward_hook(post),
                      lin.register_full_backward_pre_hook(pre), lin.register_full_backward_hook(post)]
        run(lay, warmup)
        torch.cuda.synchronize()
        spans.clear()
        e0, e1 = mk(), mk()
        e0.record()
        run(lay, steps)
        e1.record()
        torch.cuda.synchronize()
        total = e0.elapsed_time(e1) / steps
        lin_ms = sum(a.elapsed_time(b) for a, b in spans) / steps
        for h in hooks:
            h.remove()
        return lin_ms, lin_ms / total

    tokens = batch * seq
    lin_flops = 3 * 2 * tokens * (2048 * (4096 + 2048 + 12288) + 6144 * 2048)
    attn_flops = 3.5 * 4 * batch * seq * seq * 16 * 128 / 2
    out = {"tokens": tokens, "batch": batch, "seq": seq}
    for kind in ("fp8", "fp8_unfused", "fp8_matrix_core", "bf16"):
        if kind == "fp8_unfused":
            lay = DecoderLayer(linears="fp8", seed=5, fused=False)
        else:
            lay = DecoderLayer(linears=kind, seed=5)
        ms = t(lay)
        lin_ms, share = linear_share(lay)
        out[kind] = {"layer_ms": round(ms, 3), "linears_ms": round(lin_ms, 3),
                     "linears_tflops": round(lin_flops / (lin_ms * 1e-3) / 1e12, 1),
                     "linears_share_of_layer_time": round(share, 3)}
        del lay
        torch.cuda.empty_cache()
    for kind in ("fp8", "fp8_unfused", "fp8_matrix_core"):
        out[kind]["layer_speedup_vs_bf16"] = round(out["bf16"]["layer_ms"] / out[kind]["layer_ms"], 3)
        out[kind]["linears_speedup_vs_bf16"] = round(out["bf16"]["linears_ms"] / out[kind]["linears_ms"], 3)
    out["linears_share_of_layer_flops"] = round(lin_flops / (lin_flops + attn_flops), 3)
    out["note"] = ("fwd+bwd; attention is PyTorch SDPA (causal, GQA) in BF16, RoPE and head norms PyTorch BF16; "
                   "fp8 and fp8_matrix_core fuse the two RMSNorms and the SwiGLU into the next linear's quantiser "
                   "(their backward by PyTorch kernels on a recomputed forward), fp8_unfused and bf16 run them as PyTorch "
                   "BF16 ops; "
                   "linears' time from events around each linear's forward and backward (hooked pass; for the "
                   "fused kinds it includes the fused producers); FP8 linears include their quantisers and FP32 "
                   "main_grad accumulation")
    return out


def quantisers_cold(torch, B, layers, steps, warmup, qbytes, copies=3):
    """The step's quantisers with their inputs read from HBM: X, W and dY of the
    four linears are cloned `copies` times (about 1.1 GB for three, over four
    times the 256 MB last-level cache) and each step-equivalent takes the next
    copy, so no call finds its input cached from an earlier one."""
    sets = [[(L.x.clone(), L.w.clone(), L.dy.clone()) for L in layers] for _ in range(copies)]
    orig = [(L.x, L.w, L.dy) for L in layers]

    def one(c):
        for L, (x, w, dy) in zip(layers, sets[c]):
            L.x, L.w, L.dy = x, w, dy
            L.quantise(B, dual=True)

    for i in range(warmup):
        one(i % copies)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    n = max(steps, copies)
    for i in range(n):
        one(i % copies)
    e1.record()
    torch.cuda.synchronize()
    for L, (x, w, dy) in zip(layers, orig):
        L.x, L.w, L.dy = x, w, dy
    ms = e0.elapsed_time(e1) / n
    footprint = sum(t.numel() * t.element_size() for st in sets for trio in st for t in trio)
    del sets
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "gbps": round(qbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(qbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "input_copies": copies, "input_footprint_gb": round(footprint / 1e9, 2)}


def small_configs(torch, B, W, dev, reps=20):
    """Configurations 1 and 5, kernel by kernel.

    1: X [256, 2048] ~ N(0,1), W [2048, 2048] ~ N(0,0.02): row-wise 1x128
       quantiser for X, 128x128 for W, forward GEMM with FP32 output.
    5: the ragged stress case, down projection at 3000 tokens: X [3000, 6144]
       Student-t with zero groups and spikes, W [2048, 6144], dY [3000, 2048]:
       dual quantiser for X, 128x128 for W, token-dimension quantiser for dY,
       forward GEMM (BF16 out) and weight gradient (FP32 out).
    These launches are shorter than Python takes to issue them, so each rep first
    queues a spin kernel (torch.cuda._sleep) that keeps the GPU busy while the
    rep's launches and their events are enqueued; every event pair then brackets
    one kernel.  Medians over the reps.
    """
    import numpy as np
    to = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    out = {}

    def run(name, kernels, flops, qbytes):
        for fn, _ in kernels:          # warm-up (and allocation of every output)
            fn()
        torch.cuda.synchronize()
        times = [[] for _ in kernels]
        s0, s1 = mk(), mk()
        for _ in range(reps):
            evs = [(mk(), mk()) for _ in kernels]
            s0.record()
            torch.cuda._sleep(2_000_000)
            s1.record()
            for (fn, _), (a, b) in zip(kernels, evs):
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            for t, (a, b) in zip(times, evs):
                t.append(a.elapsed_time(b) * 1e3)
        med = [float(np.median(t)) for t in times]
        per = {label: round(us, 2) for (_, label), us in zip(kernels, med)}
        nq = len(qbytes)
        q_us, g_us = sum(med[:nq]), sum(med[nq:])
        out[name] = {"kernel_us": per, "total_us": round(sum(med), 2),
                     "gemm_tflops": round(flops / (g_us * 1e-6) / 1e12, 1),
                     "quantiser_gbps": round(sum(qbytes) / (q_us * 1e-6) / 1e9, 1),
                     "spin_ms": round(s0.elapsed_time(s1), 3)}

    # Configuration 1.
    x = to(W.normal_bf16((256, 2048), 1.0, W.seed_for(1, 0, "o", "x")))
    w = to(W.normal_bf16((2048, 2048), 0.02, W.seed_for(1, 0, "o", "w")))
    xq, sx = B.fp8_quant_1x128(x)
    wq, sw, _, _ = B.fp8_quant_128x128(w)
    y = torch.empty((256, 2048), dtype=torch.float32, device=dev)
    run("config1", [(lambda: B.fp8_quant_1x128(x, q=xq, scales=sx), "quant_1x128 X [256, 2048]"),
                    (lambda: B.fp8_quant_128x128(w, False, wq, sw), "quant_128x128 W [2048, 2048]"),
                    (lambda: B.fp8_block_gemm_fwd(xq, sx, wq, sw, y=y), "fwd 256x2048x2048 FP32")],
        2 * 256 * 2048 * 2048, [256 * 2048 * 3 + 256 * 16 * 4, 2048 * 2048 * 3 + 256 * 4])

    # Configuration 5.
    M, K, N = 3000, 6144, 2048
    Mp = -(-M // 128) * 128
    x = to(W.student_t_stress((M, K), W.seed_for(5, 0, "down", "x")))
    w = to(W.normal_bf16((N, K), 0.02, W.seed_for(5, 0, "down", "w")))
    dy = to(W.normal_bf16((M, N), 1e-3, W.seed_for(5, 0, "down", "dy")))
    xq, sx, xqT, sxT = B.fp8_quant_1x128_dual(x)
    wq, sw, _, _ = B.fp8_quant_128x128(w)
    dyqT, sdyT = B.fp8_quant_1x128(dy, transpose_out=True)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((N, K), dtype=torch.float32, device=dev)
    run("config5", [(lambda: B.fp8_quant_1x128_dual(x, xq, sx, xqT, sxT), "dual 1x128 X [3000, 6144]"),
                    (lambda: B.fp8_quant_128x128(w, False, wq, sw), "quant_128x128 W [2048, 6144]"),
                    (lambda: B.fp8_quant_1x128(dy, transpose_out=True, q=dyqT, scales=sdyT),
                     "token-dim 1x128 dY [3000, 2048]"),
                    (lambda: B.fp8_block_gemm_fwd(xq, sx, wq, sw, y=y), "fwd 3000x2048x6144 BF16"),
                    (lambda: B.fp8_block_gemm_wgrad(dyqT, sdyT, xqT, sxT, M=M, dw=dw), "wgrad 2048x6144 over 3000")],
        2 * 2 * M * N * K,
        [M * K * 2 + M * K + K * Mp + 4 * (M * (K // 128) + K * (Mp // 128)),
         N * K * 3 + 4 * (N // 128) * (K // 128),
         M * N * 2 + N * Mp + 4 * N * (Mp // 128)])
    out["note"] = ("each kernel bracketed by its own events behind a queued spin kernel; quantiser_gbps uses "
                   "algorithmic bytes (BF16 read once, codes and scales written once)")
    return out


def copy_probe(torch, dev, mib):
    """A plain device copy of known size (float32 multiply by one), launched once.

    Under ``rocprofv3 --pmc FETCH_SIZE`` / ``WRITE_SIZE`` its counters give the
    bytes-per-unit factor that turns the GEMM's counters into HBM bytes."""
    n = mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    return n * 4


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU path is not built.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from blockwise_fp8_linear_quant_amd import binding as B
    from blockwise_fp8_linear_quant_amd import profiling
    from blockwise_fp8_linear_quant_amd import workloads as W

    dev = torch.device("cuda:0")
    M = args.tokens
    layers = [LayerBuffers(torch, B, W, n, k, nout, M, dev) for n, k, nout in W.LINEARS]
    torch.cuda.synchronize()
    if args.copy_probe_mib:
        copy_probe(torch, dev, args.copy_probe_mib)

    def step(fp8_mc=False, marks=None):
        """One pass over the four linears.  marks[i] (three events) brackets linear
        i's quantisers and then its three GEMMs when given."""
        for i, L in enumerate(layers):
            if marks is not None:
                marks[i][0].record()
            L.quantise(B, dual=True)
            if marks is not None:
                marks[i][1].record()
            L.gemms(B, fp8_mc)
            if marks is not None:
                marks[i][2].record()

    def timed(fp8_mc):
        """Three timed passes of K steps each (after W warm-up steps):
        1. ms per step, from two events around the K steps only (no event inside a
           step: each event record costs the stream about 5 us);
        2. GEMM and quantiser ms per step, from one event bracket around each
           linear's quantisers and one around its three GEMMs, with the p10/p50/p90
           of the GEMM time over the steps;
        3. ms of each GEMM [linear][op], from K launches of it back to back
           between two events (back_to_back).
        Returns (ms/step, GEMM ms/step, per-GEMM ms, quantiser ms/step, wall s of
        pass 1, GEMM spread)."""
        mk = lambda: torch.cuda.Event(enable_timing=True)
        t_end = time.perf_counter() + args.clock_warmup_s
        while time.perf_counter() < t_end:
            step(fp8_mc)
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            step(fp8_mc)
        torch.cuda.synchronize()
        start, end = mk(), mk()
        t_wall = time.perf_counter()
        start.record()
        for _ in range(args.steps):
            step(fp8_mc)
        end.record()
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
        ms_step = start.elapsed_time(end) / args.steps

        marks = [[[mk() for _ in range(3)] for _ in layers] for _ in range(args.steps)]
        for s in range(args.steps):
            step(fp8_mc, marks[s])
        torch.cuda.synchronize()
        gemm_steps = sorted(sum(marks[s][i][1].elapsed_time(marks[s][i][2]) for i in range(len(layers)))
                            for s in range(args.steps))
        gemm_ms = sum(gemm_steps) / args.steps
        quant_ms = sum(marks[s][i][0].elapsed_time(marks[s][i][1])
                       for s in range(args.steps) for i in range(len(layers))) / args.steps
        pct = lambda q: gemm_steps[min(len(gemm_steps) - 1, int(q * (len(gemm_steps) - 1) + 0.5))]

        per_gemm = [[back_to_back(f) for f in L.gemm_calls(B, fp8_mc)] for L in layers]
        return ms_step, gemm_ms, per_gemm, quant_ms, t_wall, [pct(0.1), pct(0.5), pct(0.9)]

    def back_to_back(f):
        """ms of one launch of f: K launches between two events, queued behind a spin
        kernel so that the GPU never waits for Python to issue the next launch."""
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(4_000_000)
        e0.record()
        for _ in range(args.steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # Timed region (default path: exact block products on the F16 matrix path).
    ms_step, gemm_ms, per_gemm, quant_ms, t_wall, gemm_spread = timed(False)
    flops = sum(L.flops() for L in layers)
    gemm_b2b_ms = sum(sum(r) for r in per_gemm)
    value = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["fp8"]        # the metric's own peak: FP8 dense MFMA
    n_launch = 3 * len(layers)
    alg_bytes = sum(sum(L.gemm_bytes()) for L in layers) / n_launch
    gemms = {}
    for L, row in zip(layers, per_gemm):
        for op, ms, fl in zip(("fwd", "dgrad", "wgrad"), row, L.gemm_flops()):
            gemms[f"{op}_{L.name}"] = {"us": round(ms * 1e3, 2), "tflops": round(fl / (ms * 1e-3) / 1e12, 1)}
    qbytes = sum(L.quant_bytes() for L in layers)
    quant_kernels = {}
    for L in layers:
        calls = {"dual_x": lambda: B.fp8_quant_1x128_dual(L.x, L.xq, L.sx, L.xqT, L.sxT),
                 "blocks_w": lambda: B.fp8_quant_128x128(L.w, True, L.wq, L.sw, L.wqT, L.swT),
                 "dual_dy": lambda: B.fp8_quant_1x128_dual(L.dy, L.dyq, L.sdy, L.dyqT, L.sdyT)}
        for name, f in calls.items():
            quant_kernels[f"{name}_{L.name}"] = back_to_back(f)
    quant_b2b_ms = sum(quant_kernels.values())

    # The same quantiser outputs from the separate row-wise and token-dimension
    # kernels (two reads of X and dY), for comparison with the single-read path.
    def quant_only(dual):
        for _ in range(args.warmup):
            for L in layers:
                L.quantise(B, dual)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            for L in layers:
                L.quantise(B, dual)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps
    sep_ms = quant_only(False)
    sep_bytes = sum(L.quant_bytes(False) for L in layers)

    cold = quantisers_cold(torch, B, layers, args.steps, args.warmup, qbytes)

    traffic = None
    tr = profiling.read_traffic(os.path.join(ROOT, "profiles", TRAFFIC_SUMMARY))
    if tr is not None and args.tokens == 4096:
        traffic = float(tr["gemm_hbm_bytes_per_launch"])

    fast = None
    f_gemm_ms = None
    if not args.no_fp8_path:
        f_ms, f_gemm_ms, _, _, _, _ = timed(True)
        fast = {"ms_per_step": round(f_ms, 4), "value": round(flops / (f_ms * 1e-3) / 1e12, 3),
                "gemm_tflops": round(flops / (f_gemm_ms * 1e-3) / 1e12, 3),
                "gemm_frac_of_fp8_peak": round(flops / (f_gemm_ms * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4),
                "gemm_ms_per_step": round(f_gemm_ms, 4), "launches_per_step": n_launch,
                "avg_launch_us": round(f_gemm_ms / n_launch * 1e3, 2),
                "note": "fp8_block_gemm with FP8BLK_GEMM_FP8_MATRIX_CORE: v_mfma_f32_32x32x64_f8f6f4 block "
                        "products, hardware-truncated inside groups of 8 (not the default path)"}

    out = {
        "metric": "Blockwise-FP8 GEMM TFLOP/s + % FP8 MFMA peak, 2B-layer shapes, M=4096",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": f"one Puro-2B decoder layer's linears (qkv 2048->4096, o 2048->2048, "
                               f"gate_up 2048->12288, down 6144->2048), quantise + fwd + dgrad + wgrad",
                   "tokens": M, "hidden": 2048, "intermediate": 6144, "gemm_gflop_per_step": round(flops / 1e9, 3)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / peak, 4),
                     "frac_of_issued_f16_peak": round(gemm_tflops / PEAK_TFLOPS["f16"], 4),
                     "traffic": round(traffic) if traffic is not None else None,
                     "algorithmic_bytes_per_launch": round(alg_bytes),
                     "kernel": "block_gemm_f16_kernel / block_gemm_f16_kgroups_kernel (E4M3 codes -> exact F16 MFMA, "
                               "FP32 block rescale)",
                     "launches_per_step": n_launch,
                     "avg_launch_us": round(gemm_ms / n_launch * 1e3, 2),
                     "gemm_ms_per_step": round(gemm_ms, 4),
                     "gemm_ms_per_step_p10_p50_p90": [round(v, 4) for v in gemm_spread],
                     "gemm_ms_back_to_back": round(gemm_b2b_ms, 4),
                     "note": "peak = FP8 dense MFMA (the metric's); the exact path issues F16 matrix "
                             "instructions, whose dense peak is half of it (frac_of_issued_f16_peak); "
                             "GEMM time per step from one event bracket around each linear's three GEMMs "
                             "inside the step (ms_per_step itself has no event inside a step); "
                             "gemm_ms_back_to_back sums the per-GEMM figures of `gemms`"},
        "gemms": gemms,
        "quantisers": {"ms_per_step": round(quant_ms, 4), "algorithmic_gb": round(qbytes / 1e9, 4),
                       "gbps": round(qbytes / (quant_ms * 1e-3) / 1e9, 1) if quant_ms > 0 else None,
                       "frac_hbm_peak": round(qbytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                       if quant_ms > 0 else None,
                       "path": "single-read dual 1x128 quantiser for X and dY + 128x128 for W",
                       "timing": "ms_per_step: one event bracket around each linear's three quantisers inside "
                                 "the step (each bracket adds about 5 us); back_to_back: each quantiser launched "
                                 "K times in a row behind a queued spin kernel (GPU time only)",
                       "back_to_back": {"ms_per_step": round(quant_b2b_ms, 4),
                                        "gbps": round(qbytes / (quant_b2b_ms * 1e-3) / 1e9, 1),
                                        "frac_hbm_peak": round(qbytes / (quant_b2b_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                        "kernel_us": {k: round(v * 1e3, 2) for k, v in quant_kernels.items()}},
                       "separate_kernels": {"ms_per_step": round(sep_ms, 4), "algorithmic_gb": round(sep_bytes / 1e9, 4),
                                            "gbps": round(sep_bytes / (sep_ms * 1e-3) / 1e9, 1)},
                       "cold_inputs": cold},
        "wall_s_timed": round(t_wall, 3),
        "clock_warmup_s": args.clock_warmup_s,
        "fp8_matrix_core_path": fast,
    }
    if not args.no_sweep:
        out["cfg4_sweep"] = layer_sweep(torch, B, W, dev)
    if not args.no_small_configs:
        out["small_configs"] = small_configs(torch, B, W, dev)
    if not args.no_fusion:
        out["producer_fusion"] = producer_fusion(torch, B, layers, args.steps, args.warmup)
    if not args.no_layer:
        out["decoder_layer"] = decoder_layer(torch, args.steps, args.warmup)
    if not args.no_bf16_baseline:
        out["bf16_baseline"] = bf16_baseline(torch, B, layers, args.steps, args.warmup, gemm_ms, ms_step, f_gemm_ms)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W, layers, args.cpu_sample_tokens, args.cpu_single_thread_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
