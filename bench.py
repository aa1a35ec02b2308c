#!/usr/bin/env python3
"""Benchmark of the dequant-in-kernel GEMM hot path on one MI355X.

Default workload (the headline): decode-shaped W4A16 GEMM, N = K = 4096,
group_size 128, M in {1, 4, 16}. One step = one qgemm_w4 call per M (three
launches). Weights, scales, activations and outputs are rotated over enough
device copies (>= 1 GiB) that every launch reads its operands from HBM, not
from the 256 MB Infinity Cache or the L2s. The default line also carries the
other half of the metric, the M = 2048, N = K = 4096 W4A16 GEMM, timed the same
way over its own K steps (object `prefill_square`, TFLOP/s and its own
roofline).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--config decode|prefill|square|decode_bf16|prefill_bf16|decode_gate|prefill_gate|
                              decode_nk|prefill_nk|grouped|grouped_kn|grouped_w4|grouped_w4_bf16|kproj|kvproj|
                              kvproj_e4m3|kproj_e4m3h]

Prints one JSON line. `value` is algorithmic HBM bytes per second over the timed
steps (the decode shapes are bound by HBM); TFLOP/s is reported beside it. The
`roofline` object uses the kernel's average launch duration measured with HIP
events on the launch stream; `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload. `roofline.attainable` is min(peak, arithmetic
intensity x bandwidth) for the bound that applies. `context` (skip with
--no-context) frames the result: the same launches on one cache-resident input
set; for the HBM-bound configs the library's read-only streaming kernels over
rotated buffers of the same byte count (one contiguous chunk per workgroup: a
practical HBM ceiling; for the decode also the column-strip pattern that any
full-K kernel must use on a [K/8, N] weight), with the GEMM's launch time as a
fraction of theirs; and, for the MFMA-bound configs, torch.matmul on dense
operands of the same GEMM shape (a practical MFMA figure).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2516.6
FP8_MFMA_PEAK_TFLOPS = 5033.2
ROTATE_BYTES = 1 << 30

# HBM traffic per launch of each workload's kernel, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, each scaled by what the same counter reads for a
# 256 MiB device copy); the summaries and commands are in profiles/. A figure is
# reported only while the kernel sources still hash to the value it was taken at.
KERNEL_SOURCES = {
    "decode": ["capi.cpp", "device_common.h", "launch.h", "w4_decode.hip"],
    "prefill": ["capi.cpp", "device_common.h", "launch.h", "w4_prefill.hip"],
    "square": ["capi.cpp", "device_common.h", "launch.h", "w4_prefill.hip"],
    "decode_bf16": ["capi.cpp", "device_common.h", "launch.h", "w4_decode.hip"],
    "prefill_bf16": ["capi.cpp", "device_common.h", "launch.h", "w4_prefill.hip"],
    "prefill_gate": ["capi.cpp", "device_common.h", "launch.h", "w4_prefill.hip"],
    "decode_gate": ["capi.cpp", "device_common.h", "launch.h", "w4_decode.hip"],
    "decode_nk": ["capi.cpp", "device_common.h", "launch.h", "w4_decode.hip"],
    "prefill_nk": ["capi.cpp", "device_common.h", "launch.h", "w4_prefill.hip"],
    "grouped": ["capi.cpp", "device_common.h", "launch.h", "grouped_bf16.hip"],
    "grouped_kn": ["capi.cpp", "device_common.h", "launch.h", "grouped_bf16.hip"],
    "grouped_w4": ["capi.cpp", "device_common.h", "launch.h", "w4_prefill.hip"],
    "grouped_w4_bf16": ["capi.cpp", "device_common.h", "launch.h", "w4_prefill.hip"],
    "kproj": ["capi.cpp", "device_common.h", "launch.h", "kproj_fp8.hip"],
    "kvproj": ["capi.cpp", "device_common.h", "launch.h", "kproj_fp8.hip"],
    "kvproj_e4m3": ["capi.cpp", "device_common.h", "launch.h", "kproj_fp8.hip"],
    "kproj_e4m3h": ["capi.cpp", "device_common.h", "launch.h", "kproj_fp8.hip"],
}
MEASURED_TRAFFIC = {
    # workload: (bytes per launch, source hash the counters were taken at)
    "decode": (9240453, "76549ddc9471fadf"),
    "prefill": (224980633, "46aa373959a6e520"),
    "square": (85233930, "46aa373959a6e520"),
    "grouped": (367974254, "f021ee2cd95f4c65"),
    "grouped_kn": (365920284, "f021ee2cd95f4c65"),
    "grouped_w4": (113938561, "46aa373959a6e520"),
    "kproj": (85680489, "5ee8476366591581"),
    "decode_gate": (9252737, "76549ddc9471fadf"),
    "prefill_gate": (245829817, "46aa373959a6e520"),
    "decode_bf16": (9230896, "76549ddc9471fadf"),
    "prefill_bf16": (245911596, "46aa373959a6e520"),
    "decode_nk": (9234587, "76549ddc9471fadf"),
    "prefill_nk": (222580139, "46aa373959a6e520"),
    "kvproj": (202264507, "5ee8476366591581"),
    "kvproj_e4m3": (193908141, "5ee8476366591581"),
    "grouped_w4_bf16": (113988733, "46aa373959a6e520"),
    "kproj_e4m3h": (64451824, "5ee8476366591581"),
}


def kernel_source_hash(cfg):
    """Hash of the kernel sources with comments and blank space removed, so that a
    change of wording leaves the figure valid and any change of code voids it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[cfg]:
        with open(os.path.join(ROOT, "grouped_gemm_qgemm_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(cfg):
    t = MEASURED_TRAFFIC.get(cfg)
    if t is None or t[1] != kernel_source_hash(cfg):
        return None
    return t[0]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="decode", choices=["decode", "prefill", "square", "decode_bf16", "prefill_bf16",
                                                           "decode_gate", "prefill_gate", "decode_nk", "prefill_nk",
                                                           "kvproj", "kvproj_e4m3",
                                                           "kproj_e4m3h",
                                                           "grouped", "grouped_kn", "grouped_w4", "grouped_w4_bf16",
                                                           "kproj"])
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-context", action="store_true", help="skip the hot / read / dense-GEMM context numbers")
    p.add_argument("--no-square", action="store_true",
                   help="decode config: skip the M = 2048, N = K = 4096 half of the metric")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--source-hash", action="store_true", help="print the kernel source hash of --config and exit")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="before warmup, run 5 device-to-device copies of this many MiB (a plain copy kernel "
                        "of known size whose HBM counters calibrate FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


def event_time_ms(torch, fn_launches, stream):
    """Total ms of a sequence of launches, bracketed by events on `stream`."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    fn_launches()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e)


def cpu_cores():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def w4_bytes(M, N, K, gs):
    return M * K * 2 + K * N // 2 + (K // gs) * N * 2 + M * N * 2


def epi_extra_bytes(M, N, epi):
    """Bias read, residual read, and the output shrinking to N / 2 under the gate."""
    n_out = N // 2 if epi & 4 else N
    return (N * 2 if epi & 1 else 0) + (M * n_out * 2 if epi & 2 else 0) - (M * (N - n_out) * 2)


class DecodeW4:
    name = "w4a16_decode_N4096_K4096_gs128_M1_4_16"
    kernel = "w4_decode_lds_kernel"
    bound = "hbm"
    dtype = "f16"
    launch_shape = (256, 512)   # the decode kernel's grid: N / 16 workgroups of eight waves
    epi = 0   # qgemm_w4_epilogue flags (0: plain qgemm_w4)
    nk = False   # weights and scales stored [N, K/8] / [N, K/gs] (qgemm_w4_nk)

    def __init__(self, torch, q, synth):
        self.torch, self.q = torch, q
        cfgs = synth.W4_DECODE
        N, K = cfgs[0]["N"], cfgs[0]["K"]
        self.N, self.K, self.gs = N, K, 128
        self.Ms = [c["M"] for c in cfgs]
        self.inputs = [synth.w4_inputs(**c, dtype=self.dtype) for c in cfgs]
        foot = sum(w4_bytes(M, N, K, 128) for M in self.Ms)
        self.R = max(1, math.ceil(ROTATE_BYTES / foot))
        dev = torch.device("cuda")
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float16
        bh, sh = self.inputs[0].b, self.inputs[0].scales
        if self.nk:
            bh, sh = np.ascontiguousarray(bh.T), np.ascontiguousarray(sh.T)
        b = torch.from_numpy(bh.view(np.int32)).to(dev)
        s = torch.from_numpy(sh.view(np.int16)).to(dev).view(tdt)
        n_out = N // 2 if self.epi & 4 else N
        self.epi_ops = [synth.w4_epilogue_operands(7 + i, M, n_out, N, self.dtype) for i, M in enumerate(self.Ms)]
        dev16 = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(tdt)
        bias = dev16(self.epi_ops[0][0]) if self.epi & 1 else None
        self.slots = []
        for r in range(self.R):
            slot = []
            for i, M in enumerate(self.Ms):
                a = torch.from_numpy(self.inputs[i].a.view(np.int16)).to(dev).view(tdt)
                res = dev16(self.epi_ops[i][1]) if self.epi & 2 else None
                slot.append((torch.empty(M, n_out, dtype=tdt, device=dev), a, b.clone(), s.clone(), bias, res))
            self.slots.append(slot)
        self.bytes_per_step = sum(w4_bytes(M, N, K, 128) + epi_extra_bytes(M, N, self.epi) for M in self.Ms)
        self.flops_per_step = sum(2 * M * N * K for M in self.Ms)

    def launches(self, step):
        slot = self.slots[step % self.R]
        if self.epi:
            return [lambda c=c, a=a, b=b, s=s, bi=bi, r=r: self.q.qgemm_w4_epilogue(c, a, b, s, self.epi, bi, r, 128)
                    for (c, a, b, s, bi, r) in slot]
        fn = self.q.qgemm_w4_nk if self.nk else self.q.qgemm_w4
        return [lambda c=c, a=a, b=b, s=s: fn(c, a, b, s, 128) for (c, a, b, s, _, _) in slot]

    def unit_bytes(self):
        return self.bytes_per_step / len(self.Ms)

    def unit_flops(self):
        return self.flops_per_step / len(self.Ms)

    @property
    def read_strip_shape(self):
        # packed B [K/8, N] words, one 16-column strip (64 bytes) per workgroup
        return None if self.nk else (self.K // 8, self.N, 64)

    def cpu_sample(self):
        import oracle
        for i, w in enumerate(self.inputs):
            if self.epi:
                oracle.qgemm_w4_epilogue(w.a, w.b, w.scales, w.group_size, self.epi, self.epi_ops[0][0],
                                         self.epi_ops[i][1], dtype=self.dtype)
            else:
                oracle.qgemm_w4(w.a, w.b, w.scales, w.group_size, dtype=self.dtype)
        return self.flops_per_step, self.bytes_per_step, "full steps (M = 1, 4, 16)"

    def describe(self):
        d = {"workload": self.name, "M": self.Ms, "N": self.N, "K": self.K, "group_size": self.gs,
             "pack_factor": 8, "rotating_copies": self.R}
        if self.epi:
            d["epilogue"] = "bias + silu_gate + residual" if self.epi == 7 else self.epi
        if self.nk:
            d["layout"] = "b_packed [N, K/8], scales [N, K/128]"
        return d

    def dense_equivalent(self):
        return None   # a dense GEMV here measures launch overhead, not the GEMM


class PrefillW4:
    """Prefill-shaped W4A16: M=2048, K=4096, N=11008 (or N=4096 for the square shape)."""
    kernel = "w4_prefill_dma_kernel"
    bound = "mfma"
    dtype = "f16"
    mfma_kind = 0   # the MFMA issue loop of the same kind (qg_mfma_loop): fp16
    epi = 0   # qgemm_w4_epilogue flags (0: plain qgemm_w4)
    nk = False   # weights and scales stored [N, K/8] / [N, K/gs] (qgemm_w4_nk)

    def __init__(self, torch, q, synth, square=False):
        self.torch, self.q = torch, q
        cfg = synth.W4_SQUARE_PREFILL if square else synth.W4_PREFILL
        self.w = synth.w4_inputs(**cfg, dtype=self.dtype)
        M, N, K = self.w.shape
        self.M, self.N, self.K = M, N, K
        self.name = f"w4a16_prefill_M{M}_N{N}_K{K}_gs128" + ("_bf16" if self.dtype == "bf16" else "")
        if self.epi:
            self.name += "_bias_silugate_residual" if self.epi == 7 else f"_epi{self.epi}"
        foot = w4_bytes(M, N, K, 128) + epi_extra_bytes(M, N, self.epi)
        self.R = max(1, math.ceil(ROTATE_BYTES / foot))
        dev = torch.device("cuda")
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float16
        a = torch.from_numpy(self.w.a.view(np.int16)).to(dev).view(tdt)
        bh, sh = self.w.b, self.w.scales
        if self.nk:
            bh, sh = np.ascontiguousarray(bh.T), np.ascontiguousarray(sh.T)
            self.name += "_nk"
        b = torch.from_numpy(bh.view(np.int32)).to(dev)
        sc = torch.from_numpy(sh.view(np.int16)).to(dev).view(tdt)
        n_out = N // 2 if self.epi & 4 else N
        self.bias_bits, self.res_bits = synth.w4_epilogue_operands(7, M, n_out, N, self.dtype)
        dev16 = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(tdt)
        bias = dev16(self.bias_bits) if self.epi & 1 else None
        res = dev16(self.res_bits) if self.epi & 2 else None
        self.slots = [(torch.empty(M, n_out, dtype=tdt, device=dev), a.clone(), b.clone(), sc.clone(), bias,
                       None if res is None else res.clone()) for _ in range(self.R)]
        self.bytes_per_step = foot
        self.flops_per_step = 2 * M * N * K

    def launches(self, step):
        c, a, b, s, bi, r = self.slots[step % self.R]
        if self.epi:
            return [lambda: self.q.qgemm_w4_epilogue(c, a, b, s, self.epi, bi, r, 128)]
        if self.nk:
            return [lambda: self.q.qgemm_w4_nk(c, a, b, s, 128)]
        return [lambda: self.q.qgemm_w4(c, a, b, s, 128)]

    def unit_bytes(self):
        return self.bytes_per_step

    def unit_flops(self):
        return self.flops_per_step

    def cpu_sample(self):
        import oracle
        rows = 256
        if self.epi:
            oracle.qgemm_w4_epilogue(self.w.a[:rows], self.w.b, self.w.scales, 128, self.epi, self.bias_bits,
                                     self.res_bits[:rows], dtype=self.dtype)
        else:
            oracle.qgemm_w4(self.w.a[:rows], self.w.b, self.w.scales, 128, dtype=self.dtype)
        return (2 * rows * self.N * self.K, w4_bytes(rows, self.N, self.K, 128) + epi_extra_bytes(rows, self.N, self.epi),
                f"{rows} of {self.M} rows")

    def describe(self):
        d = {"workload": self.name, "M": self.M, "N": self.N, "K": self.K, "group_size": 128,
             "pack_factor": 8, "rotating_copies": self.R}
        if self.epi:
            d["epilogue"] = "bias + silu_gate + residual" if self.epi == 7 else self.epi
        if self.nk:
            d["layout"] = "b_packed [N, K/8], scales [N, K/128]"
        return d

    def dense_equivalent(self):
        return (self.M, self.K, self.N, self.torch.bfloat16 if self.dtype == "bf16" else self.torch.float16)


class PrefillW4Gate(PrefillW4):
    """The 2048 x 11008 x 4096 prefill as a gated MLP up-projection: bias, SiLU-gated
    column pairs (output 2048 x 5504) and a residual add, fused into the GEMM."""
    epi = 7


class DecodeW4Gate(DecodeW4):
    """The decode workload with bias, SiLU-gated column pairs (output M x 2048) and residual."""
    name = "w4a16_decode_N4096_K4096_gs128_M1_4_16_bias_silugate_residual"
    kernel = "w4_decode_lds_epi_kernel"
    epi = 7


class DecodeW4NK(DecodeW4):
    """The decode workload with weights and scales stored [N, K/8] / [N, K/128]."""
    name = "w4a16_decode_N4096_K4096_gs128_M1_4_16_nk"
    kernel = "w4_decode_lds_nk_kernel"
    nk = True


class PrefillW4NK(PrefillW4):
    """The 2048 x 11008 x 4096 prefill with weights and scales stored [N, K/8] / [N, K/128]."""
    nk = True


class DecodeW4BF16(DecodeW4):
    """The decode workload with bf16 activations, scales and output."""
    name = "w4a16_decode_N4096_K4096_gs128_M1_4_16_bf16"
    dtype = "bf16"


class PrefillW4BF16(PrefillW4):
    """The 2048 x 11008 x 4096 prefill with bf16 activations, scales and output."""
    dtype = "bf16"
    mfma_kind = 1


class GroupedBF16:
    """64 experts, 4096 routed rows, K=2048, N=1408, 10% of groups skipped (seed 4), experts stored [E, N, K]."""
    kernel = "grouped_bf16_wl_kernel"
    bound = "hbm"
    dtype = "bf16"
    transpose_b = True

    def __init__(self, torch, q, synth):
        self.torch, self.q = torch, q
        d = synth.grouped_inputs()
        self.d = d
        T, K = d.a.shape
        E, N, _ = d.b.shape
        self.T, self.K, self.N, self.E = T, K, N, E
        off = d.a_offsets.astype(np.int64)
        rows = off[1:] - off[:-1]
        act = (d.expert_ids >= 0) & (rows > 0)
        self.active_rows = int(rows[act].sum())
        self.active_experts = len(set(d.expert_ids[act].tolist()))
        self.bytes_per_step = (self.active_rows * K * 2 + self.active_experts * N * K * 2
                               + self.active_rows * N * 2 + (E + 1) * 4 + E * 4)
        self.flops_per_step = 2 * self.active_rows * N * K
        self.R = max(1, math.ceil(ROTATE_BYTES / (d.b.nbytes + d.a.nbytes + T * N * 2)))
        dev = torch.device("cuda")
        a = torch.from_numpy(d.a.view(np.int16)).to(dev).view(torch.bfloat16)
        bh = d.b if self.transpose_b else np.ascontiguousarray(d.b.transpose(0, 2, 1))
        b = torch.from_numpy(bh.view(np.int16)).to(dev).view(torch.bfloat16)
        off_t = torch.from_numpy(d.a_offsets.view(np.int32)).to(dev)
        ids = torch.from_numpy(d.expert_ids).to(dev)
        self.slots = [(torch.empty(T, N, dtype=torch.bfloat16, device=dev), a.clone(), off_t, b.clone() if r else b, ids)
                      for r in range(self.R)]
        self.usage = [int(v) for v in d.usage]
        self.name = f"grouped_bf16_E{E}_T{T}_K{K}_N{N}_skip10pct" + ("" if self.transpose_b else "_b_KxN")

    def launches(self, step):
        c, a, off, b, ids = self.slots[step % self.R]
        return [lambda: self.q.grouped_gemm(c, a, off, b, ids, self.usage, self.transpose_b)]

    def unit_bytes(self):
        return self.bytes_per_step

    def unit_flops(self):
        return self.flops_per_step

    def cpu_sample(self):
        import oracle
        d = self.d
        G = 8
        usage = np.array([d.usage[0], G], np.uint32)
        c0 = np.zeros((self.T, self.N), np.uint16)
        if self.transpose_b:
            oracle.grouped_gemm(c0, d.a, d.a_offsets, d.b, d.expert_ids, usage)
        else:
            oracle.grouped_gemm(c0, d.a, d.a_offsets, np.ascontiguousarray(d.b.transpose(0, 2, 1)), d.expert_ids,
                                usage, transpose_b=False)
        off = d.a_offsets.astype(np.int64)
        rows = sum(int(off[g + 1] - off[g]) for g in range(G) if d.expert_ids[g] >= 0)
        ne = sum(1 for g in range(G) if d.expert_ids[g] >= 0)
        byt = rows * self.K * 2 + ne * self.N * self.K * 2 + rows * self.N * 2
        return 2 * rows * self.N * self.K, byt, f"first {G} of {self.E} groups"

    def describe(self):
        return {"workload": self.name, "experts": self.E, "routed_rows": self.T, "K": self.K, "N": self.N,
                "active_rows": self.active_rows, "active_experts": self.active_experts,
                "transpose_b": self.transpose_b,
                "rotating_copies": self.R}

    def dense_equivalent(self):
        return None   # HBM-bound: the copy of the same byte count is the context number


class GroupedBF16KN(GroupedBF16):
    """The same grouped workload with the experts stored [E, K, N] (transpose_b = False)."""
    kernel = "grouped_bf16_kernel"
    transpose_b = False


class GroupedW4:
    """64 int4 experts (group 128), 4096 routed rows, K=2048, N=1408, 10% of groups skipped (seed 6)."""
    kernel = "w4_grouped_kernel"
    bound = "hbm"
    dtype = "f16"
    mfma_kind = 0

    def __init__(self, torch, q, synth):
        self.torch, self.q = torch, q
        d = synth.grouped_w4_inputs(dtype=self.dtype)
        self.d = d
        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float16
        T, K = d.a.shape
        E, _, N = d.b.shape
        self.T, self.K, self.N, self.E = T, K, N, E
        off = d.a_offsets.astype(np.int64)
        rows = off[1:] - off[:-1]
        act = (d.expert_ids >= 0) & (rows > 0)
        self.active_rows = int(rows[act].sum())
        self.active_experts = len(set(d.expert_ids[act].tolist()))
        gs = d.group_size
        self.bytes_per_step = (self.active_rows * K * 2 + self.active_experts * (K * N // 2 + (K // gs) * N * 2)
                               + self.active_rows * N * 2 + (E + 1) * 4 + E * 4)
        self.flops_per_step = 2 * self.active_rows * N * K
        self.R = max(1, math.ceil(ROTATE_BYTES / (d.b.nbytes + d.scales.nbytes + d.a.nbytes + T * N * 2)))
        dev = torch.device("cuda")
        a = torch.from_numpy(d.a.view(np.int16)).to(dev).view(tdt)
        b = torch.from_numpy(d.b.view(np.int32)).to(dev)
        s = torch.from_numpy(d.scales.view(np.int16)).to(dev).view(tdt)
        off_t = torch.from_numpy(d.a_offsets.view(np.int32)).to(dev)
        ids = torch.from_numpy(d.expert_ids).to(dev)
        self.slots = [(torch.empty(T, N, dtype=tdt, device=dev), a.clone(), off_t, b.clone(), s.clone(),
                       ids) for _ in range(self.R)]
        self.usage = [int(v) for v in d.usage]
        self.name = (f"grouped_w4a16_E{E}_T{T}_K{K}_N{N}_gs{gs}_skip10pct"
                     + ("_bf16" if self.dtype == "bf16" else ""))

    def launches(self, step):
        c, a, off, b, s, ids = self.slots[step % self.R]
        return [lambda: self.q.grouped_gemm_w4(c, a, off, b, s, ids, self.usage, self.d.group_size)]

    def unit_bytes(self):
        return self.bytes_per_step

    def unit_flops(self):
        return self.flops_per_step

    def cpu_sample(self):
        import oracle
        d = self.d
        G = 8
        usage = np.array([d.usage[0], G], np.uint32)
        c0 = np.zeros((self.T, self.N), np.uint16)
        oracle.grouped_gemm_w4(c0, d.a, d.a_offsets, d.b, d.scales, d.expert_ids, usage, d.group_size,
                               dtype=self.dtype)
        off = d.a_offsets.astype(np.int64)
        rows = sum(int(off[g + 1] - off[g]) for g in range(G) if d.expert_ids[g] >= 0)
        ne = sum(1 for g in range(G) if d.expert_ids[g] >= 0)
        byt = rows * self.K * 2 + ne * (self.N * self.K // 2 + (self.K // d.group_size) * self.N * 2) + rows * self.N * 2
        return 2 * rows * self.N * self.K, byt, f"first {G} of {self.E} groups"

    def describe(self):
        return {"workload": self.name, "experts": self.E, "routed_rows": self.T, "K": self.K, "N": self.N,
                "group_size": self.d.group_size, "pack_factor": 8, "active_rows": self.active_rows,
                "active_experts": self.active_experts, "rotating_copies": self.R}

    def dense_equivalent(self):
        return None


class GroupedW4BF16(GroupedW4):
    """The grouped W4 workload with bf16 activations, scales and output."""
    dtype = "bf16"
    mfma_kind = 1


class KProjFP8:
    """8 sequences (lengths U[1,1024], seed 5: T=4312), hidden 4096 bf16, W [4096,1024] e4m3 with 1x128x128
    block scales, bf16 keys written into a paged cache (page 128, 2 layers, layer 1)."""
    kernel = "kproj_bf16_dma_kernel"
    bound = "mfma"
    dtype = "bf16"
    mfma_kind = 1   # bf16 MFMAs on weights converted from e4m3
    planes = 1          # 2: keys and values ([W_k | W_v]) in one call
    cache = "bf16"      # or "fp8": e4m3 cache with one f32 scale per head row (G = 128)
    hidden = "bf16"     # or "fp8": e4m3 hidden rows, one f32 scale per token per 128 columns

    def __init__(self, torch, q, synth):
        self.torch, self.q = torch, q
        k = synth.kproj_inputs(planes=self.planes, cache=self.cache, qgran=128, hidden=self.hidden)
        self.k = k
        T, Kh = k.hidden.shape
        N = k.weight.shape[1]
        self.T, self.Kh, self.N = T, Kh, N
        self.flops_per_step = 2 * T * Kh * N
        out_bytes = T * N * (1 + 4 / 128) if self.cache == "fp8" else T * N * 2   # codes + scales, or bf16
        self.bytes_per_step = (k.hidden.nbytes + Kh * N + k.input_scale.nbytes + k.weight_scale.nbytes + out_bytes
                               + k.row_offsets.nbytes + k.cache_lengths.nbytes + k.page_table.nbytes)
        foot = k.hidden.nbytes + k.weight.nbytes + k.blocks.nbytes + k.input_scale.nbytes
        self.R = max(1, math.ceil(ROTATE_BYTES / foot))
        dev = torch.device("cuda")
        if self.hidden == "fp8":
            h = torch.from_numpy(k.hidden).to(dev).view(torch.float8_e4m3fn)
        else:
            h = torch.from_numpy(k.hidden.view(np.int16)).to(dev).view(torch.bfloat16)
        w = torch.from_numpy(k.weight).to(dev).view(torch.float8_e4m3fn)
        isc = torch.from_numpy(k.input_scale).to(dev)
        wsc = torch.from_numpy(k.weight_scale).to(dev)
        if self.cache == "fp8":
            blocks = torch.from_numpy(k.blocks).to(dev)
            kvs = torch.from_numpy(k.scales).to(dev)
        else:
            blocks = torch.from_numpy(k.blocks.view(np.int16)).to(dev).view(torch.bfloat16)
            kvs = None
        self.offs = torch.from_numpy(k.row_offsets.view(np.int32)).to(dev)
        self.cl = torch.from_numpy(k.cache_lengths.view(np.int32)).to(dev)
        self.pt = torch.from_numpy(k.page_table.view(np.int32)).to(dev)
        self.slots = [(h.clone(), w.clone(), isc.clone(), wsc.clone(), blocks.clone(),
                       None if kvs is None else kvs.clone()) for _ in range(self.R)]
        self.name = (f"{'kvproj' if self.planes == 2 else 'kproj'}_fp8_paged_T{T}_K{Kh}_N{N}_page128"
                     + ("_e4m3cache_g128" if self.cache == "fp8" else "")
                     + ("_e4m3hidden" if self.hidden == "fp8" else ""))

    def launches(self, step):
        h, w, isc, wsc, blocks, kvs = self.slots[step % self.R]
        k = self.k
        fn = self.q.kv_matmul_ragged_paged_scale if self.planes == 2 else self.q.k_matmul_ragged_paged_scale
        return [lambda: fn(h, self.offs, w, isc, wsc, blocks, self.cl, self.pt, k.layer_idx, kv_scales=kvs,
                           quantization_granularity=k.qgran)]

    def unit_bytes(self):
        return self.bytes_per_step

    def unit_flops(self):
        return self.flops_per_step

    def cpu_sample(self):
        import oracle
        k = self.k
        rows = 512
        if self.cache == "fp8":
            y = oracle.kproj_exact(k.hidden[:rows], k.weight, k.input_scale[:rows], k.weight_scale)
            oracle.quantize_runs(y, 128)
        else:
            oracle.kproj_rows(k.hidden[:rows], k.weight, k.input_scale[:rows], k.weight_scale)
        return 2 * rows * self.Kh * self.N, rows * self.Kh * k.hidden.itemsize + self.Kh * self.N + rows * self.N * 2, \
            f"{rows} of {self.T} token rows (matmul + rounding or quantization; placement excluded)"

    def describe(self):
        k = self.k
        return {"workload": self.name, "tokens": self.T, "batch": len(k.row_offsets) - 1, "hidden": self.Kh,
                "N": self.N, "page_size": int(k.blocks.shape[3]), "layers": int(k.blocks.shape[0]),
                "layer_idx": k.layer_idx, "granularity_mnk": [1, 128, 128], "rotating_copies": self.R,
                "planes": self.planes, "cache": "e4m3, one f32 scale per 128" if self.cache == "fp8" else "bf16",
                "hidden": "e4m3, one f32 scale per 1x128" if self.hidden == "fp8" else "bf16"}

    def dense_equivalent(self):
        return (self.T, self.Kh, self.N, self.torch.bfloat16)


class KProjE4M3Hidden(KProjFP8):
    """The K-projection workload with e4m3 hidden rows: both MFMA operands are e4m3."""
    kernel = "kproj_f8f8_dma_kernel"
    dtype = "e4m3"
    mfma_kind = 2
    hidden = "fp8"
    mfma_peak = FP8_MFMA_PEAK_TFLOPS

    def dense_equivalent(self):
        return None


class KVProjFP8(KProjFP8):
    """Keys and values in one call: [W_k | W_v] [4096, 2048], planes 0 and 1 of the bf16 cache."""
    planes = 2


class KVProjFP8Cache(KProjFP8):
    """Keys and values in one call into an e4m3 cache with one f32 scale per head row."""
    planes = 2
    cache = "fp8"


def graph_time_ms(torch, launch_lists, reps=3):
    """Best-of-`reps` ms per launch of a HIP graph holding every launch in `launch_lists`."""
    fns = [f for fl in launch_lists for f in fl]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        best = min(best, event_time_ms(torch, g.replay, torch.cuda.current_stream()))
    del g
    return best / len(fns)


def context_numbers(torch, q, wl, steps, avg_launch_ms):
    """Numbers that frame the result (outside the timed region):
    * hot: the same launches on one input set, so the inputs stay in cache;
    * read_contiguous: the library's read-only streaming kernel over the workload's
      algorithmic byte count per launch, one contiguous chunk per workgroup, rotated
      over >= 1 GiB like the workload: a practical HBM ceiling for that many bytes;
    * read_strips (decode): the same kernel reading the packed weight matrix one
      16-column strip per workgroup, every packed row: the pattern of a kernel that
      gives each workgroup a column strip and all of K;
    * torch_dense: torch.matmul (hipBLASLt) on dense operands of the same GEMM shape,
      timed eagerly: a practical MFMA figure for the MFMA-bound workloads;
    * mfma_loop (MFMA-bound and grouped W4 workloads): the library's MFMA issue loop
      of the workload's MFMA kind on every CU (two waves per SIMD, nothing but
      MFMAs), its FLOP rate and the shader clock it held: what the matrix cores
      sustain on this chip, against the published peak;
    * empty_launch (decode): a kernel that does nothing, in the GEMM's launch shape:
      the floor under one launch of that shape."""
    out = {}
    n_launch = len(wl.launches(0))
    hot_ms = graph_time_ms(torch, [wl.launches(0) for _ in range(max(steps // 2, 10))])
    out["hot_avg_launch_us"] = round(hot_ms * 1e3, 3)
    if wl.bound == "hbm":
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        nbytes = int(wl.unit_bytes()) // 16 * 16
        R = max(2, math.ceil(ROTATE_BYTES / nbytes))
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(R)]
        rd_ms = graph_time_ms(torch, [[lambda b=b: q.read_contiguous(b, sink, 2 * 256)] for b in bufs] * 3)
        out["read_contiguous_us"] = round(rd_ms * 1e3, 3)
        out["read_contiguous_GBs"] = round(nbytes / (rd_ms * 1e-3) / 1e9, 1)
        out["gemm_frac_of_read_contiguous"] = round(rd_ms / avg_launch_ms, 4)
        del bufs
        strip = getattr(wl, "read_strip_shape", None)
        if strip is not None:
            rows, cols, strip_bytes = strip
            R = max(2, math.ceil(ROTATE_BYTES / (rows * cols * 4)))
            bufs = [torch.ones(rows, cols, dtype=torch.int32, device="cuda") for _ in range(R)]
            st_ms = graph_time_ms(torch, [[lambda b=b: q.read_strips(b, strip_bytes, sink)] for b in bufs] * 3)
            out["read_strips_us"] = round(st_ms * 1e3, 3)
            out["read_strips_shape"] = {"rows": rows, "row_bytes": cols * 4, "strip_bytes": strip_bytes}
            out["gemm_frac_of_read_strips"] = round(st_ms / avg_launch_ms, 4)
            del bufs
    dense = wl.dense_equivalent()
    if dense is not None:
        M, K, N, dt = dense
        a = torch.randn(M, K, device="cuda").to(dt)
        b = torch.randn(K, N, device="cuda").to(dt)
        c = torch.empty(M, N, device="cuda", dtype=dt)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        reps = 20
        ms = event_time_ms(torch, lambda: [torch.matmul(a, b, out=c) for _ in range(reps)],
                           torch.cuda.current_stream()) / reps
        out["torch_dense_us"] = round(ms * 1e3, 3)
        out["torch_dense_TFLOPs"] = round(2 * M * N * K / (ms * 1e-3) / 1e12, 1)
        del a, b, c
    kind = getattr(wl, "mfma_kind", None)
    if kind is not None:
        out["mfma_loop"] = mfma_loop_numbers(torch, q, kind)
        out["gemm_frac_of_mfma_loop"] = round(wl.unit_flops() / (avg_launch_ms * 1e-3) / 1e12
                                              / out["mfma_loop"]["TFLOPs"], 4)
    shape = getattr(wl, "launch_shape", None)
    if shape is not None:
        e_ms = graph_time_ms(torch, [[lambda: q.empty_launch(*shape)] for _ in range(200)])
        out["empty_launch_us"] = round(e_ms * 1e3, 3)
        out["empty_launch_shape"] = {"workgroups": shape[0], "threads": shape[1]}
    out["launches_per_step"] = n_launch
    return out


def mfma_loop_numbers(torch, q, kind, workgroups=256, iters=512, launches=20):
    """FLOP rate of the MFMA issue loop (graph-timed, best of three) and the mean
    shader clock its workgroups measured (s_memtime against the 100 MHz counter)."""
    clocks = torch.zeros(2 * workgroups, dtype=torch.int64, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    ms = graph_time_ms(torch, [[lambda: q.mfma_loop(kind, iters, workgroups, clocks, sink)]
                               for _ in range(launches)])
    c = clocks.view(workgroups, 2).double()
    mhz = float((c[:, 0] / c[:, 1]).mean()) * 100.0
    flops = workgroups * 8 * iters * 8 * q.MFMA_LOOP_FLOPS[kind]
    name = {v: k for k, v in q.MFMA_LOOP_KINDS.items()}[kind]
    return {"kind": name, "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1), "clock_MHz": round(mhz),
            "us_per_launch": round(ms * 1e3, 3), "workgroups": workgroups, "iters": iters}


WORKLOADS = {"decode": DecodeW4, "prefill": PrefillW4,
             "square": lambda t, q, sy: PrefillW4(t, q, sy, square=True),
             "decode_bf16": DecodeW4BF16, "prefill_bf16": PrefillW4BF16,
             "decode_gate": DecodeW4Gate, "prefill_gate": PrefillW4Gate,
             "decode_nk": DecodeW4NK, "prefill_nk": PrefillW4NK,
             "kvproj": KVProjFP8, "kvproj_e4m3": KVProjFP8Cache, "kproj_e4m3h": KProjE4M3Hidden,
             "grouped": GroupedBF16, "grouped_kn": GroupedBF16KN, "grouped_w4": GroupedW4,
             "grouped_w4_bf16": GroupedW4BF16, "kproj": KProjFP8}


def time_workload(torch, wl, steps, warmup):
    """Warm up, capture `steps` steps in one HIP graph and time one replay with events
    on the stream it runs on (synchronised on both sides). Returns (ms, wall_s)."""
    for i in range(warmup):
        for f in wl.launches(i):
            f()
    torch.cuda.synchronize()
    # The K steps are captured once into a HIP graph so the GPU runs the kernels
    # back to back; from Python each launch costs more than the kernel itself.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            for f in wl.launches(i):
                f()
    torch.cuda.synchronize()
    graph.replay()                      # warm replay
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = event_time_ms(torch, graph.replay, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del graph
    return ms, wall


def roofline_of(wl, ms, steps, traffic):
    """The value, its unit and the roofline object of the dominant kernel."""
    ms_per_step = ms / steps
    n_launch = len(wl.launches(0))
    avg_launch_ms = ms / (steps * n_launch)
    gbs = wl.bytes_per_step / (ms_per_step * 1e-3) / 1e9
    tflops = wl.flops_per_step / (ms_per_step * 1e-3) / 1e12
    ai = wl.unit_flops() / wl.unit_bytes()        # FLOP per algorithmic byte
    mfma_peak = getattr(wl, "mfma_peak", F16_MFMA_PEAK_TFLOPS)   # the contraction's own dtype
    if wl.bound == "hbm":
        value, unit = gbs, "GB/s"
        achieved, peak, runit = wl.unit_bytes() / (avg_launch_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
        attainable = min(HBM_PEAK_GBS, mfma_peak * 1e3 / ai)
    else:
        value, unit = tflops, "TFLOP/s"
        achieved, peak, runit = wl.unit_flops() / (avg_launch_ms * 1e-3) / 1e12, mfma_peak, "TFLOP/s"
        attainable = min(mfma_peak, ai * HBM_PEAK_GBS / 1e3)
    roof = {"bound": wl.bound, "achieved": round(achieved, 3), "peak": peak,
            "unit": runit, "frac": round(achieved / peak, 4), "traffic": traffic,
            "kernel": wl.kernel, "avg_launch_us": round(avg_launch_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": wl.unit_bytes(),
            "algorithmic_flops_per_launch": wl.unit_flops(),
            "attainable": round(attainable, 1), "frac_attainable": round(achieved / attainable, 4),
            "frac_hbm": round(wl.unit_bytes() / (avg_launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "frac_mfma": round(wl.unit_flops() / (avg_launch_ms * 1e-3) / 1e12 / mfma_peak, 4)}
    return value, unit, gbs, tflops, ms_per_step, avg_launch_ms, roof


def cpu_baseline(wl, seconds, unit):
    t0 = time.perf_counter()
    n = 0
    fl = by = 0
    while True:
        f, b, what = wl.cpu_sample()
        fl += f
        by += b
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    cv = by / dt / 1e9 if wl.bound == "hbm" else fl / dt / 1e12
    return {"value": round(cv, 6), "unit": unit, "cores": cpu_cores(), "kind": "oracle",
            "sample": f"{n} x ({what}) of the same workload, fp64 numpy oracle, {dt:.1f} s"}


def main():
    args = parse()
    if args.source_hash:
        print(kernel_source_hash(args.config))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        print("bench.py: only --gpus 1 is supported (single-GPU build)", file=sys.stderr)
        sys.exit(2)
    import torch
    import grouped_gemm_qgemm_amd as q
    import synth
    q.load()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    wl = WORKLOADS[args.config](torch, q, synth)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 18          # int32 elements
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # timed region: exactly K steps
    ms, wall = time_workload(torch, wl, args.steps, args.warmup)
    value, unit, gbs, tflops, ms_per_step, avg_launch_ms, roof = roofline_of(wl, ms, args.steps,
                                                                             measured_traffic(args.config))
    out = {
        "metric": "W4A16 GEMM TFLOP/s + HBM GB/s (% roofline) at M=1..16 and M=2048, N=K=4096",
        "value": round(value, 3), "unit": unit,
        "gbs": round(gbs, 2), "tflops": round(tflops, 3),
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": wl.describe(),
        "roofline": roof,
        "wall_s": round(wall, 3),
    }
    if not args.no_context:
        out["context"] = context_numbers(torch, q, wl, args.steps, avg_launch_ms)
    if args.config == "decode" and not args.no_square:
        # the metric's other half: M = 2048, N = K = 4096, its own K timed steps
        sq = PrefillW4(torch, q, synth, square=True)
        sq_ms, sq_wall = time_workload(torch, sq, args.steps, args.warmup)
        sv, su, _, _, sq_ms_step, sq_avg, sq_roof = roofline_of(sq, sq_ms, args.steps, measured_traffic("square"))
        out["prefill_square"] = {"workload": sq.describe(), "value": round(sv, 3), "unit": su,
                                 "ms_per_step": round(sq_ms_step, 6), "steps": args.steps, "wall_s": round(sq_wall, 3),
                                 "roofline": sq_roof}
        if not args.no_context:
            out["prefill_square"]["context"] = context_numbers(torch, q, sq, args.steps, sq_avg)
        if not args.no_cpu:
            out["prefill_square"]["cpu_baseline"] = cpu_baseline(sq, args.cpu_seconds / 2, su)
        del sq
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, unit)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
