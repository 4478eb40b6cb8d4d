#!/usr/bin/env python3
"""Throughput of the NVFP4 MoE hot path on one MI355X.

One step = the whole path over one batch of synthetic decode input:
  1. moe_fp4_quantize: the step's BF16 token activations -> NVFP4 (dynamic
     tensor scale), one row per token;
  2. moe_grouped_gemm_fp4: every expert's GEMM over the tokens routed to it
     (rows gathered through a row index), FP32 accumulation, BF16 output.
Both run in the HIP library; inputs are resident in HBM before timing starts.
The expert weights are constant, so they are rearranged once at set-up into the
packed layout the GEMM loads fastest (moe_fp4_pack_weights, untimed; its own
duration is reported); --layout rowmajor times the GEMM on row-major weights.

Weights are rotated over several device copies so that each step streams
weights that neither the L2 nor the 256 MB Infinity Cache holds (the decode
case, where every layer's experts differ from the previous one's).

Prints ONE JSON line (the value is whole-step TFLOP/s; the GEMM kernel's HBM
roofline and the CPU oracle's throughput on the same workload ride along).
Kernel durations come from HIP events around back-to-back launches of that
kernel alone on the launch stream (rocprofv3's per-kernel average measures
the same thing).

  python bench.py [--steps K] [--warmup W] [--workload c3] [--secondary c4]
  python bench.py --swiglu     # + gate+up GEMM with the SwiGLU + NVFP4 epilogue vs unfused
  python bench.py --finalize   # + finalize: fused atomics vs plain GEMM + token-order combine
  python bench.py --layer      # + a whole MoE FFN layer (eager and from a HIP graph)
  python bench.py --copy-calibration   # a plain copy of known size, for counter scaling
  python bench.py --ceilings           # torch's read / write / copy rates on 1 GiB, and the
                                       # decode weight-stream pattern with no arithmetic
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "grouped FP4 GEMM TFLOPS & HBM GB/s (% roofline) at 16/32 tokens/expert"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, AMD published
FP4_PEAK_TFLOPS = 10066.0       # dense MXFP4 MFMA, AMD published
F16_PEAK_TFLOPS = 2516.6        # dense FP16 MFMA, AMD published
ROTATE_BYTES = 1.0e9            # weight bytes cycled through between reuses
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_grouped_gemm.txt")
GEMM_SOURCES = [os.path.join(ROOT, "block_scaled_fp4_05_amd", "csrc", f)
                for f in ("grouped_gemm_kernel.h", "grouped_gemm.hip", "gemm_common.h", "fp4_device.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3", help="c1, c2, c3, c4, c5 or c5b (default c3)")
    ap.add_argument("--secondary", default="c4",
                    help="second workload reported in the same line ('none' to skip)")
    ap.add_argument("--layout", default="packed", choices=("packed", "rowmajor"),
                    help="weight-code layout the GEMM reads (default packed)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--swiglu", action="store_true",
                    help="also time the gate+up GEMM with the SwiGLU + NVFP4 epilogue against "
                         "the unfused GEMM, activation and quantiser")
    ap.add_argument("--finalize", action="store_true",
                    help="also time the finalize GEMM (routing-weighted sum into token order) "
                         "against the plain GEMM plus a separate weighted combine")
    ap.add_argument("--layer", action="store_true",
                    help="also time a whole MoE FFN layer on this shard: quantise, gate+up GEMM "
                         "with the SwiGLU + NVFP4 epilogue, down-projection GEMM, token-order "
                         "combine (the workload's weights are the gate+up projection)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only print streaming rates: torch's read, write and copy on 1 GiB and the decode weight-stream pattern with no arithmetic")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a device copy of known size (counter scale factor)")
    return ap.parse_args()


# ------------------------------------------------------------------ inputs --

def alg_bytes(w, offsets, tokens_used):
    """Algorithmic HBM bytes of one grouped-GEMM launch: every non-empty expert's
    packed weights and scales once, every distinct token row once, the row index,
    the BF16 output, the offsets and the scales."""
    import numpy as np
    nz = int(np.count_nonzero(np.diff(offsets)))
    m = int(offsets[-1])
    per_elem = 0.5 + 1.0 / 16.0
    wb = nz * w.n * w.k * per_elem
    ab = tokens_used * w.k * per_elem
    ob = 2.0 * m * w.n
    misc = 4.0 * m + 4.0 * (w.experts + 1) + 4.0 * w.experts + 4.0
    return wb + ab + ob + misc, dict(weights=wb, activations=ab, output=ob, index_offsets=misc,
                                     nonempty_experts=nz)


def quant_alg_bytes(tokens, k):
    """Algorithmic bytes of the activation quantiser: BF16 in once, codes + scales out."""
    return tokens * k * 2.0 + tokens * k * (0.5 + 1.0 / 16.0) + 4.0


class Problem:
    """Device-resident inputs of one workload (weights quantised on the GPU by
    moe_fp4_quantize from the seeded FP32 weights)."""

    def __init__(self, name, keep_host_weights=False, layout="packed"):
        import numpy as np
        import torch
        from block_scaled_fp4_05_amd import moe_fp4
        from workloads import configs

        w = configs.WORKLOADS[name]
        self.w = w
        dev = torch.device("cuda")
        row_token, offsets = configs.routing(w)
        self.row_token, self.offsets = row_token, offsets
        self.m_total = int(offsets[-1])
        x = configs.activations(w)
        self.x_host = x
        self.x = torch.from_numpy(x).to(dev).to(torch.bfloat16)
        self.idx = torch.from_numpy(row_token).to(dev)
        self.off = torch.from_numpy(offsets).to(dev)
        E, n, k = w.experts, w.n, w.k
        w_q = torch.empty((E, n, k // 2), dtype=torch.uint8, device=dev)
        w_sf = torch.empty((E, n, k // 16), dtype=torch.uint8, device=dev)
        w_scale = torch.empty(E, dtype=torch.float32, device=dev)
        self.host_weights = [] if keep_host_weights else None
        t0 = time.time()
        for e in range(E):
            we = configs.expert_weight(w, e)
            if keep_host_weights:
                self.host_weights.append(we)
            wt = torch.from_numpy(we).to(dev)
            moe_fp4.quantize(wt, tensor_scale=w_scale[e:e + 1], q=w_q[e], sf=w_sf[e], dynamic=True)
        torch.cuda.synchronize()
        log(f"{name}: weights quantised on the GPU in {time.time() - t0:.1f}s")
        self.packed = layout == "packed"
        self.pack_us = None
        if self.packed:
            w_pk = torch.empty_like(w_q)
            moe_fp4.pack_weights(w_q, out=w_pk)  # first call loads the kernel
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            moe_fp4.pack_weights(w_q, out=w_pk)
            e1.record()
            torch.cuda.synchronize()
            self.pack_us = round(e0.elapsed_time(e1) * 1e3, 1)
            del w_q
            w_q = w_pk
        wbytes = E * n * k * (0.5 + 1.0 / 16.0)
        copies = max(1, min(8, math.ceil(ROTATE_BYTES / wbytes)))
        self.weights = [(w_q, w_sf, w_scale)]
        for _ in range(copies - 1):
            self.weights.append((w_q.clone(), w_sf.clone(), w_scale.clone()))
        self.q = torch.empty((w.tokens, k // 2), dtype=torch.uint8, device=dev)
        self.sf = torch.empty((w.tokens, k // 16), dtype=torch.uint8, device=dev)
        self.g = torch.empty(1, dtype=torch.float32, device=dev)
        self.out = torch.empty((self.m_total, n), dtype=torch.bfloat16, device=dev)
        self.flops = 2.0 * self.m_total * n * k
        self.gemm_bytes, self.gemm_bytes_parts = alg_bytes(w, offsets, len(np.unique(row_token)))
        self.quant_bytes = quant_alg_bytes(w.tokens, k)
        torch.cuda.synchronize()

        self._prepare_raw()

    def _prepare_raw(self):
        """The timed loops call the C entry points directly with pointers prepared
        here, once: the checked wrappers validate every tensor on every call, which
        costs host time comparable to the ~8 us quantiser.  One call through each
        checked wrapper first validates exactly these arguments."""
        import ctypes
        import torch
        from block_scaled_fp4_05_amd import moe_fp4
        w = self.w
        k, n = w.k, w.n
        moe_fp4.quantize(self.x, tensor_scale=self.g, q=self.q, sf=self.sf, dynamic=True)
        for w_q, w_sf, w_scale in self.weights:
            moe_fp4.grouped_gemm(self.q, self.sf, self.g, w_q, w_sf, w_scale, self.off,
                                 a_row_index=self.idx, out=self.out, m_total=self.m_total,
                                 packed=self.packed)
        torch.cuda.synchronize()
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        self._stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self._quant_args = (ptr(self.x), moe_fp4.IN_BF16, w.tokens, k, self.x.stride(0),
                            ptr(self.q), ptr(self.sf), ptr(self.g), moe_fp4.SCALE_DYNAMIC,
                            self._stream)
        fn = moe_fp4.lib().moe_grouped_gemm_fp4_packed if self.packed else moe_fp4.lib().moe_grouped_gemm_fp4
        self._gemm_fn = fn
        self._gemm_args = [(ptr(self.q), ptr(self.sf), ptr(self.g), w.tokens, ptr(self.idx),
                            ptr(w_q), ptr(w_sf), ptr(w_scale), ptr(self.off), w.experts,
                            self.m_total, n, k, ptr(self.out), self.out.stride(0), self._stream)
                           for w_q, w_sf, w_scale in self.weights]

    def quantize(self, i=0):
        from block_scaled_fp4_05_amd import moe_fp4
        st = moe_fp4.lib().moe_fp4_quantize(*self._quant_args)
        if st != moe_fp4.OK:
            raise moe_fp4.MoeFp4Error(st, "moe_fp4_quantize")

    def gemm(self, i):
        from block_scaled_fp4_05_amd import moe_fp4
        st = self._gemm_fn(*self._gemm_args[i % len(self._gemm_args)])
        if st != moe_fp4.OK:
            raise moe_fp4.MoeFp4Error(st, "grouped GEMM")

    def step(self, i):
        """One pass of the hot path: quantise the step's activations, then the
        grouped GEMM over every expert (weights rotated by step)."""
        self.quantize(i)
        self.gemm(i)


def warm(fn, seconds=0.25, min_calls=3):
    """Run fn back to back for about `seconds` (at least min_calls), then synchronise:
    long enough for the GPU's clocks to settle under the kernel's own load, which a
    few calls after an idle set-up phase are not for millisecond-scale kernels."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < min_calls or time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def measure(prob, steps, warmup):
    """Time `steps` whole steps after `warmup` untimed ones, then the two kernels
    of the path on their own (each launched `steps` times back to back between
    two HIP events on the launch stream, so per-launch event overhead does not
    inflate a kernel's duration).  Returns wall time per step and per-kernel
    averages."""
    import torch
    from block_scaled_fp4_05_amd import moe_fp4
    warm(prob.step)
    for i in range(warmup):
        prob.step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        prob.step(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    region_ms = e0.elapsed_time(e1)
    step_dist = grouped(prob.step, steps, warmup)

    def back_to_back(fn):
        warm(fn)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps, grouped(fn, steps)

    quant_ms, quant_dist = back_to_back(prob.quantize)
    gemm_ms, gemm_dist = back_to_back(prob.gemm)
    return dict(wall_ms_per_step=(t1 - t0) * 1e3 / steps, gpu_ms_per_step=region_ms / steps,
                quant_ms=quant_ms, gemm_ms=gemm_ms, step_dist=step_dist, quant_dist=quant_dist,
                gemm_dist=gemm_dist)


def grouped(fn, calls, first=0, groups=10):
    """Spread of per-call durations: `calls` back-to-back calls in `groups` equal
    groups with one HIP event between groups (an event between every two calls
    adds a few microseconds to each on this part), each group giving its mean per
    call.  A separate pass from the timed one."""
    import torch
    per = max(1, calls // groups)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
    ev[0].record()
    i = first
    for gi in range(groups):
        for _ in range(per):
            fn(i)
            i += 1
        ev[gi + 1].record()
    torch.cuda.synchronize()
    r = spread([ev[gi].elapsed_time(ev[gi + 1]) / per for gi in range(groups)])
    r["calls_per_group"] = per
    return r


def spread(ms):
    """Median, 10th and 90th percentile of durations given in ms, in us."""
    import numpy as np
    a = np.asarray(ms, np.float64) * 1e3
    return {"median_us": round(float(np.median(a)), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def finalize_report(prob, steps):
    """The MoE finalize step on this workload (each routed row, times a seeded routing
    weight, summed into its token's row), three ways:
      fused    moe_grouped_gemm_fp4_finalize (FP32 atomic adds in the GEMM's epilogue)
               plus zeroing the caller's FP32 token buffer;
      two-pass the plain GEMM (BF16 rows) followed by moe_fp4_combine (token order, FP32
               sums, BF16 out);
      torch    the plain GEMM followed by a weighted index_add (for reference)."""
    import numpy as np
    import torch
    from block_scaled_fp4_05_amd import moe_fp4
    w = prob.w
    dev = torch.device("cuda")
    weight = torch.from_numpy(np.random.default_rng(700).uniform(0.0, 1.0, prob.m_total)
                              .astype(np.float32)).to(dev)
    tokens = torch.empty((w.tokens, w.n), dtype=torch.float32, device=dev)

    def timed(fn):
        warm(fn)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3

    def fused(i):
        w_q, w_sf, w_scale = prob.weights[i % len(prob.weights)]
        moe_fp4.grouped_gemm_finalize(prob.q, prob.sf, prob.g, w_q, w_sf, w_scale, prob.off,
                                      prob.idx, weight, tokens, a_row_index=prob.idx,
                                      m_total=prob.m_total, packed=prob.packed)

    def zero(i):
        tokens.zero_()

    def plain(i):
        w_q, w_sf, w_scale = prob.weights[i % len(prob.weights)]
        moe_fp4.grouped_gemm(prob.q, prob.sf, prob.g, w_q, w_sf, w_scale, prob.off,
                             a_row_index=prob.idx, out=prob.out, m_total=prob.m_total,
                             packed=prob.packed)

    idx64 = prob.idx.to(torch.int64)

    def combine(i):
        tokens.index_add_(0, idx64, prob.out.float() * weight[:, None])

    # Token -> routed rows map (rows are sorted by expert; a token's rows in row order).
    row_token = prob.row_token.astype(np.int64)
    order = np.argsort(row_token, kind="stable")
    topk = w.topk
    tr_host = np.full((w.tokens, topk), -1, np.int32)
    counts = np.bincount(row_token, minlength=w.tokens)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    slot = np.arange(len(order)) - np.repeat(starts, counts)
    tr_host[row_token[order], slot] = order.astype(np.int32)
    token_rows = torch.from_numpy(tr_host).to(dev)
    wt_host = np.where(tr_host >= 0, weight.cpu().numpy()[np.maximum(tr_host, 0)], 0.0)
    token_weights = torch.from_numpy(wt_host.astype(np.float32)).to(dev)
    combined = torch.empty((w.tokens, w.n), dtype=torch.bfloat16, device=dev)

    def lib_combine(i):
        moe_fp4.combine(prob.out, token_rows, token_weights, out=combined)

    # The device's FP32 atomic-add rate on the most favourable pattern: every
    # wavefront adds into 256 contiguous bytes (torch's index_add_ over a flat
    # buffer, each element hit twice), as many adds as the fused epilogue makes.
    n_adds = prob.m_total * w.n
    flat = torch.zeros((n_adds + 1) // 2, dtype=torch.float32, device=dev)
    flat_idx = torch.arange(n_adds, device=dev, dtype=torch.int64) % flat.numel()
    flat_src = torch.ones(n_adds, dtype=torch.float32, device=dev)

    def atomics(i):
        flat.index_add_(0, flat_idx, flat_src)

    res = dict(fused_us=round(timed(fused), 2), zero_us=round(timed(zero), 2),
               plain_gemm_us=round(timed(plain), 2), combine_us=round(timed(lib_combine), 2),
               torch_index_add_us=round(timed(combine), 2))
    res["atomic_adds"] = n_adds
    res["coalesced_atomic_adds_us"] = round(timed(atomics), 2)
    res["coalesced_atomic_gadds_per_s"] = round(n_adds / (res["coalesced_atomic_adds_us"] * 1e-6) / 1e9, 1)
    del flat, flat_idx, flat_src
    comb_bytes = prob.m_total * w.n * 2 + w.tokens * w.n * 2 + w.tokens * topk * 8
    res["combine_gbps"] = round(comb_bytes / (res["combine_us"] * 1e-6) / 1e9, 1)
    # Parity of one fused call against the unfused pipeline on the same inputs (the
    # oracle comparison is in the tests): both accumulate into zeroed buffers.
    tokens.zero_()
    fused(0)
    got = tokens.clone()
    tokens.zero_()
    plain(0)
    combine(0)
    torch.cuda.synchronize()
    err = ((got - tokens).norm(dim=1) / tokens.norm(dim=1).clamp_min(1e-30)).max().item()
    res["max_token_rel_diff_fused_vs_torch"] = round(err, 6)
    plain(0)
    lib_combine(0)
    torch.cuda.synchronize()
    err2 = ((combined.float() - tokens).norm(dim=1) / tokens.norm(dim=1).clamp_min(1e-30)).max().item()
    res["max_token_rel_diff_combine_vs_torch"] = round(err2, 6)
    res["note"] = ("the two-pass and torch paths round rows to BF16 before summing, the fused "
                   "path does not; the combine also rounds its output to BF16")
    return res


def swiglu_report(prob, steps):
    """The gate+up projection with the SwiGLU + NVFP4 epilogue on this workload (the
    first half of the N weight rows is the gate, the second half the up projection;
    weights N(0, 1/K), i.e. the workload's N(0,1) weights with their tensor scales
    divided by sqrt(K), so the pre-activations are O(1) as in a trained layer), two ways:
      fused    moe_grouped_gemm_fp4_swiglu: the NVFP4 intermediate straight from the GEMM;
      unfused  the plain GEMM (BF16 rows), torch's silu(gate) * up in FP32, then
               moe_fp4_quantize with the same static scale on the FP32 activation.
    The static scale is the intermediate's amax / 2688 from one unfused pass (set-up)."""
    import torch
    from block_scaled_fp4_05_amd import moe_fp4
    w = prob.w
    if w.n % 32:
        raise SystemExit("--swiglu needs N a multiple of 32 (N = 2I)")
    inter = w.n // 2
    dev = torch.device("cuda")
    scaled = [(q, sf, (s / w.k ** 0.5).contiguous()) for q, sf, s in prob.weights]
    h_scale = torch.empty(1, dtype=torch.float32, device=dev)
    h_q = torch.empty((prob.m_total, inter // 2), dtype=torch.uint8, device=dev)
    h_sf = torch.empty((prob.m_total, inter // 16), dtype=torch.uint8, device=dev)
    u_q, u_sf = torch.empty_like(h_q), torch.empty_like(h_sf)

    def timed(fn):
        warm(fn)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3

    def fused(i):
        w_q, w_sf, w_scale = scaled[i % len(scaled)]
        moe_fp4.grouped_gemm_swiglu(prob.q, prob.sf, prob.g, w_q, w_sf, w_scale, prob.off, h_scale,
                                    a_row_index=prob.idx, h_q=h_q, h_sf=h_sf,
                                    m_total=prob.m_total, packed=prob.packed)

    def plain(i):
        w_q, w_sf, w_scale = scaled[i % len(scaled)]
        moe_fp4.grouped_gemm(prob.q, prob.sf, prob.g, w_q, w_sf, w_scale, prob.off,
                             a_row_index=prob.idx, out=prob.out, m_total=prob.m_total,
                             packed=prob.packed)

    def act():
        y = prob.out.float()
        return torch.nn.functional.silu(y[:, :inter]) * y[:, inter:]

    def unfused(i):
        plain(i)
        moe_fp4.quantize(act(), tensor_scale=h_scale, q=u_q, sf=u_sf, dynamic=False)

    plain(0)
    h_scale.copy_(act().abs().max().reshape(1) / 2688.0)
    res = dict(inter=inter, h_scale=round(h_scale.item(), 6), fused_us=round(timed(fused), 2),
               unfused_us=round(timed(unfused), 2), plain_gemm_us=round(timed(plain), 2))
    fused_bytes = (prob.gemm_bytes - prob.gemm_bytes_parts["output"]
                   + prob.m_total * inter * (0.5 + 1.0 / 16.0) + 4.0)
    res["fused_bytes"] = int(fused_bytes)
    res["fused_gbps"] = round(fused_bytes / (res["fused_us"] * 1e-6) / 1e9, 1)
    res["fused_hbm_frac"] = round(res["fused_gbps"] / HBM_PEAK_GBS, 4)
    # Agreement of one fused call with the unfused pipeline (which rounds the GEMM
    # output to BF16 before the activation); the oracle comparison is in the tests.
    fused(0)
    unfused(0)
    torch.cuda.synchronize()
    res["scale_mismatch_frac_vs_unfused"] = round((h_sf != u_sf).float().mean().item(), 5)
    res["byte_mismatch_frac_vs_unfused"] = round((h_q != u_q).float().mean().item(), 5)
    return res


def layer_report(prob, steps):
    """One whole Mixture-of-Experts FFN layer on this shard, from the library's entry
    points (the chain the layer test checks against the oracle):
      1. moe_fp4_quantize       the step's BF16 tokens -> NVFP4 (dynamic scale);
      2. moe_grouped_gemm_fp4_swiglu  gate+up (this workload's weights, the first N/2
                                rows the gate; tensor scales divided by sqrt(K) so the
                                pre-activations are O(1)) -> the NVFP4 intermediate
                                h [m_total][N/2] at a static scale calibrated once;
      3. moe_grouped_gemm_fp4   down projection: h (routed rows, in order) times seeded
                                N(0,1) weights [E][K][N/2] -> BF16 rows [m_total][K];
      4. moe_fp4_combine        routing-weighted sum of each token's rows -> BF16 tokens.
    Both weight sets are packed and rotated over device copies like the workload's."""
    import numpy as np
    import torch
    from block_scaled_fp4_05_amd import moe_fp4
    from workloads import gen
    w = prob.w
    if w.n % 64:
        raise SystemExit("--layer needs N a multiple of 64 (N = 2I, I a multiple of 32)")
    inter, hidden, E = w.n // 2, w.k, w.experts
    dev = torch.device("cuda")
    scaled = [(q, sf, (sc / w.k ** 0.5).contiguous()) for q, sf, sc in prob.weights]
    # Down-projection weights [E][hidden][inter], seeded N(0,1), quantised on the GPU.
    w2_q = torch.empty((E, hidden, inter // 2), dtype=torch.uint8, device=dev)
    w2_sf = torch.empty((E, hidden, inter // 16), dtype=torch.uint8, device=dev)
    w2_scale = torch.empty(E, dtype=torch.float32, device=dev)
    for e in range(E):
        we = torch.from_numpy(gen.expert_weight(e, hidden, inter, 400 + w.index)).to(dev)
        moe_fp4.quantize(we, tensor_scale=w2_scale[e:e + 1], q=w2_q[e], sf=w2_sf[e], dynamic=True)
    w2_scale /= inter ** 0.5
    if prob.packed:
        w2_q = moe_fp4.pack_weights(w2_q)
    down = [(w2_q, w2_sf, w2_scale)] + [(w2_q.clone(), w2_sf.clone(), w2_scale.clone())
                                        for _ in range(len(prob.weights) - 1)]
    h_scale = torch.empty(1, dtype=torch.float32, device=dev)
    h_q = torch.empty((prob.m_total, inter // 2), dtype=torch.uint8, device=dev)
    h_sf = torch.empty((prob.m_total, inter // 16), dtype=torch.uint8, device=dev)
    rows = torch.empty((prob.m_total, hidden), dtype=torch.bfloat16, device=dev)
    # Token -> routed rows (a token's rows in row order) and seeded routing weights.
    row_token = prob.row_token.astype(np.int64)
    order = np.argsort(row_token, kind="stable")
    counts = np.bincount(row_token, minlength=w.tokens)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    tr_host = np.full((w.tokens, w.topk), -1, np.int32)
    tr_host[row_token[order], np.arange(len(order)) - np.repeat(starts, counts)] = order
    weight = np.random.default_rng(800 + w.index).uniform(0.0, 1.0, prob.m_total)
    wt_host = np.where(tr_host >= 0, weight[np.maximum(tr_host, 0)], 0.0).astype(np.float32)
    token_rows = torch.from_numpy(tr_host).to(dev)
    token_weights = torch.from_numpy(wt_host).to(dev)
    out = torch.empty((w.tokens, hidden), dtype=torch.bfloat16, device=dev)

    def quant(i):
        moe_fp4.quantize(prob.x, tensor_scale=prob.g, q=prob.q, sf=prob.sf, dynamic=True)

    def gate_up(i):
        q13, sf13, s13 = scaled[i % len(scaled)]
        moe_fp4.grouped_gemm_swiglu(prob.q, prob.sf, prob.g, q13, sf13, s13, prob.off, h_scale,
                                    a_row_index=prob.idx, h_q=h_q, h_sf=h_sf,
                                    m_total=prob.m_total, packed=prob.packed)

    def down_proj(i):
        q2, sf2, s2 = down[i % len(down)]
        moe_fp4.grouped_gemm(h_q, h_sf, h_scale, q2, sf2, s2, prob.off, out=rows,
                             m_total=prob.m_total, packed=prob.packed)

    def comb(i):
        moe_fp4.combine(rows, token_rows, token_weights, out=out)

    def layer(i):
        quant(i)
        gate_up(i)
        down_proj(i)
        comb(i)

    # Static intermediate scale: amax of one unfused gate+up activation / 2688.
    quant(0)
    q13, sf13, s13 = scaled[0]
    moe_fp4.grouped_gemm(prob.q, prob.sf, prob.g, q13, sf13, s13, prob.off, a_row_index=prob.idx,
                         out=prob.out, m_total=prob.m_total, packed=prob.packed)
    y = prob.out.float()
    h_scale.copy_((torch.nn.functional.silu(y[:, :inter]) * y[:, inter:]).abs().max().reshape(1)
                  / 2688.0)

    def timed(fn):
        warm(fn)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps * 1e3

    # The quantiser alone through the prepared direct call (the checked wrapper's
    # host time is comparable to the kernel's); the layer and its graph use the
    # wrappers, which launch on the current (capturing) stream.
    res = dict(tokens=w.tokens, experts=E, topk=w.topk, hidden=hidden, inter=inter,
               layer_us=round(timed(layer), 2), quantize_us=round(timed(prob.quantize), 2),
               gate_up_swiglu_us=round(timed(gate_up), 2), down_us=round(timed(down_proj), 2),
               combine_us=round(timed(comb), 2))
    # The same chain replayed from a HIP graph (one layer per weight copy in one
    # capture), which leaves only the GPU's own gaps between the launches.  Every
    # replay is checked against the eager result, bit for bit, with eager work and
    # synchronisations in between.
    ncopy = len(scaled)
    layer(ncopy - 1)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(ncopy):
            layer(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(ncopy):
            layer(i)
    replays_ok = True
    for _ in range(3):
        out.zero_()
        layer(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replays_ok = replays_ok and bool(torch.equal(out, eager))
    if not replays_ok:
        raise SystemExit("layer graph replay differs from the eager layer")
    reps = max(1, steps // ncopy)
    warm(lambda i: graph.replay())
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    res["layer_graph_us"] = round(a.elapsed_time(b) / (reps * ncopy) * 1e3, 2)
    res["graph_replays_match_eager"] = replays_ok
    flops = 2.0 * prob.m_total * (w.n * hidden + hidden * inter)
    res["layer_tflops"] = round(flops / (res["layer_us"] * 1e-6) / 1e12, 2)
    res["tokens_per_s"] = round(w.tokens / (res["layer_us"] * 1e-6), 1)
    nz = int(np.count_nonzero(np.diff(prob.offsets)))
    wbytes = nz * (w.n * hidden + hidden * inter) * (0.5 + 1.0 / 16.0)
    res["weight_bytes"] = int(wbytes)
    res["weight_stream_gbps"] = round(wbytes / (res["layer_us"] * 1e-6) / 1e9, 1)
    return res


def plan_of(prob):
    from block_scaled_fp4_05_amd import moe_fp4
    w = prob.w
    return moe_fp4.plan(w.experts, prob.m_total, w.n, w.k)


def summary(prob, r):
    ms = r["wall_ms_per_step"]
    gemm_s = r["gemm_ms"] * 1e-3
    return dict(
        workload=prob.w.name,
        ms_per_step=round(ms, 4),
        tflops_step=round(prob.flops / (ms * 1e-3) / 1e12, 2),
        gbps_step=round((prob.gemm_bytes + prob.quant_bytes) / (ms * 1e-3) / 1e9, 1),
        gemm_us=round(r["gemm_ms"] * 1e3, 2),
        quantize_us=round(r["quant_ms"] * 1e3, 2),
        # Per launch (per step): median, p10, p90 over 10 groups of back-to-back calls.
        gemm_us_dist=r["gemm_dist"],
        quantize_us_dist=r["quant_dist"],
        step_us_dist=r["step_dist"],
        gemm_tflops=round(prob.flops / gemm_s / 1e12, 2),
        gemm_gbps=round(prob.gemm_bytes / gemm_s / 1e9, 1),
        gemm_hbm_frac=round(prob.gemm_bytes / gemm_s / 1e9 / HBM_PEAK_GBS, 4),
        gemm_fp4_peak_frac=round(prob.flops / gemm_s / 1e12 / FP4_PEAK_TFLOPS, 5),
        gemm_f16_mfma_peak_frac=round(prob.flops / gemm_s / 1e12 / F16_PEAK_TFLOPS, 5),
        tile=plan_of(prob),
        weight_layout="packed" if prob.packed else "rowmajor",
        weight_pack_us=prob.pack_us,
        weight_copies_rotated=len(prob.weights),
    )


# --------------------------------------------------------------- counters --

def sources_digest():
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, layout):
    """HBM bytes per grouped-GEMM launch from the committed counter summary, or None
    when it is missing, for another workload or weight layout, or taken on other
    kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith("#"):
                key, v = line.split(":", 1)
                vals[key.strip()] = v.strip()
    try:
        if (vals.get("workload") != workload or vals.get("layout", "rowmajor") != layout
                or vals.get("sources_sha256_16") != sources_digest()):
            return None
        return float(vals["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------- CPU baseline --

def cpu_baseline(prob):
    """The oracle (plain C + OpenMP) on the same workload: quantise the step's
    activations and run the whole grouped GEMM, timed on the host cores.  Its
    weights come from the oracle's own quantiser on the same seeded FP32 weights."""
    import numpy as np
    from oracle import oracle as orc
    w = prob.w
    E, n, k = w.experts, w.n, w.k
    w_q = np.empty((E, n, k // 2), np.uint8)
    w_sf = np.empty((E, n, k // 16), np.uint8)
    w_scale = np.empty(E, np.float32)
    for e in range(E):
        w_q[e], w_sf[e], w_scale[e] = orc.quantize(prob.host_weights[e])
    # Whole steps, repeated until about 10 s of host time (at most 30 steps);
    # the figures are means per step.
    q_s = g_s = 0.0
    passes = 0
    while passes == 0 or (q_s + g_s < 10.0 and passes < 30):
        t0 = time.perf_counter()
        a_q, a_sf, a_scale = orc.quantize(prob.x_host)
        t1 = time.perf_counter()
        R, ref = orc.grouped_gemm(a_q, a_sf, a_scale, w_q, w_sf, w_scale, prob.offsets,
                                  a_row_index=prob.row_token)
        t2 = time.perf_counter()
        q_s += t1 - t0
        g_s += t2 - t1
        passes += 1
    secs = (q_s + g_s) / passes
    base = dict(value=round(prob.flops / secs / 1e12, 6), unit="TFLOPS", cores=orc.num_threads(),
                kind="oracle",
                sample=f"whole {w.name} step: quantise {w.tokens}x{k} activations + grouped GEMM "
                       f"over all {prob.m_total} routed rows ({E} experts, N={n}, K={k}), "
                       f"{passes} steps, mean per step",
                seconds=round(secs, 3), quantize_s=round(q_s / passes, 3),
                gemm_s=round(g_s / passes, 3), steps=passes)
    return base, R, ref


def parity(got, R, ref):
    """Row errors of the GPU output (last timed step, BF16 bits) against the oracle's."""
    import numpy as np
    from oracle import oracle as orc
    err, _ = orc.row_error(got, ref, R)
    return dict(rows=int(err.size), max_row_err=float(err.max()), tol=2e-3,
                ok=bool(np.all(err <= 2e-3)))


# -------------------------------------------------------------------- main --

def ceilings():
    """Streaming rates of this GPU with torch's own kernels, as context for the roofline
    fractions: a read of 1 GiB (a sum), a write of 1 GiB (a fill) and a copy of 1 GiB
    (1 GiB read + 1 GiB written), each the mean of back-to-back calls after a 0.25 s warm-up."""
    import torch
    nbytes = 1 << 30
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    out = {}

    def rate(fn, traffic):
        warm(lambda i: fn())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 20 * 1e3
        return {"us": round(us, 1), "gbps": round(traffic / (us * 1e-6) / 1e9, 1)}

    out["read_1GiB_sum"] = rate(lambda: a.sum(), nbytes)
    out["write_1GiB_fill"] = rate(lambda: b.fill_(2.0), nbytes)
    out["copy_1GiB"] = rate(lambda: b.copy_(a), 2 * nbytes)
    del a, b
    out["stream_probe"] = stream_probe_rates()
    out["peak_gbps"] = HBM_PEAK_GBS
    print(json.dumps({"ceilings": out}), flush=True)


def stream_probe_rates():
    """Read rates of the decode GEMM's weight-stream pattern with no arithmetic
    (libmoe_fp4_probe.so, built by build()): 2,048 wavefronts, each reading one
    decode N-tile's weights (64 rows x 6,144 K x 0.5625 bytes = 221,184 bytes) in
    16 KB stages of 1 KB loads, two stages in flight; in its own region per
    wavefront (the GEMM's layout) or with the wavefronts sweeping the buffer
    together; with and without the non-temporal hint.  Three copies of the
    buffer (1.36 GB, more than the caches hold) are read in turn."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "block_scaled_fp4_05_amd", "libmoe_fp4_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
    L = ctypes.CDLL(path)
    fn = L.moe_fp4_stream_probe
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    waves, per_wave = 2048, 64 * 6144 * 9 // 16
    stages = per_wave // 16384
    nbytes = waves * per_wave
    read = waves * stages * 16384
    g = torch.Generator(device="cuda").manual_seed(5)
    bufs = [torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
            for _ in range(3)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {"waves": waves, "bytes_read_per_launch": read}
    for layout, lname in ((0, "regions"), (1, "interleaved")):
        for nt in (0, 1):
            def run(i):
                rc = fn(bufs[i % 3].data_ptr(), nbytes, per_wave, stages, waves, layout, nt,
                        sink.data_ptr(), stream)
                if rc != 0:
                    raise RuntimeError(f"moe_fp4_stream_probe returned {rc}")
            warm(run)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(30):
                run(i)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / 30 * 1e3
            res[f"{lname}_{'nt' if nt else 'plain'}"] = {
                "us": round(us, 1), "gbps": round(read / (us * 1e-6) / 1e9, 1)}
    return res


def copy_calibration():
    import torch
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": nbytes, "bytes_written": nbytes,
                      "dispatches": 3}), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (each GPU would run "
              "its own expert shard independently); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from block_scaled_fp4_05_amd import moe_fp4
    moe_fp4.lib()  # the HIP library must be built: there is no fallback
    if args.copy_calibration:
        copy_calibration()
        return
    if args.ceilings:
        ceilings()
        return

    want_cpu = not args.no_cpu_baseline
    prob = Problem(args.workload, keep_host_weights=want_cpu, layout=args.layout)
    log(f"{args.workload}: {args.warmup} warmup + {args.steps} timed steps")
    r = measure(prob, args.steps, args.warmup)
    main_s = summary(prob, r)
    log(json.dumps(main_s))
    # The last timed step's output, taken now: the optional reports below reuse
    # prob.out for other projections.
    head_out = prob.out.view(torch.int16).cpu().numpy().view(np.uint16)

    gemm_s = r["gemm_ms"] * 1e-3
    achieved = prob.gemm_bytes / gemm_s / 1e9
    traffic = measured_traffic(args.workload, args.layout)
    roof = {"bound": "hbm", "kernel": "k_grouped_gemm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic, "algorithmic_bytes": int(prob.gemm_bytes),
            "avg_launch_us": round(r["gemm_ms"] * 1e3, 2),
            "median_launch_us": r["gemm_dist"]["median_us"]}

    fin = None
    if args.finalize:
        fin = finalize_report(prob, args.steps)
        log("finalize " + json.dumps(fin))
    if args.swiglu:
        swi = swiglu_report(prob, args.steps)
        log("swiglu " + json.dumps(swi))
    if args.layer:
        lay = layer_report(prob, args.steps)
        log("layer " + json.dumps(lay))

    secondary = None
    if args.secondary and args.secondary != "none" and args.secondary != args.workload:
        p2 = Problem(args.secondary, layout=args.layout)
        r2 = measure(p2, args.steps, args.warmup)
        secondary = summary(p2, r2)
        log(json.dumps(secondary))
        del p2
        torch.cuda.empty_cache()

    base = None
    par = None
    if want_cpu:
        log("timing the CPU oracle on the same workload")
        base, R, ref = cpu_baseline(prob)
        par = parity(head_out, R, ref)

    w = prob.w
    line = {
        "metric": METRIC,
        "value": main_s["tflops_step"],
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_s["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 x e4m3/16) -> exact f16 mfma, f32 acc, bf16 out",
        "data": "synthetic (seeded N(0,1) activations and weights, seeded routing)",
        "config": {"workload": f"{w.name}: {w.experts} experts, {w.tokens} tokens top-{w.topk} "
                               f"({w.routing} routing), K={w.k}, N={w.n}",
                   "experts": w.experts, "tokens": w.tokens, "topk": w.topk,
                   "m_total": prob.m_total, "n": w.n, "k": w.k},
        "hbm_gbps": main_s["gbps_step"],
        "gemm": main_s,
        "roofline": roof,
        "cpu_baseline": base,
        "parity_vs_oracle": par,
        "secondary": secondary,
    }
    if fin is not None:
        line["finalize"] = fin
    if args.swiglu:
        line["swiglu"] = swi
    if args.layer:
        line["layer"] = lay
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
