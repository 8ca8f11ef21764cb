"""Benchmark of the 4-bit weight-quantized matmul hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-clock-probe]

One step runs every row of the hot path once, each on inputs already resident
in HBM:
  decode    affine GEMV, T=1, D=5120, N=13824 (the headline), then its
            deferred-dequantisation variant (int8 activations) and batches of
            8 and 32 rows (qmm_gemm: the multi-row kernel, its rows held in
            LDS, then streamed) on the same weights
  qkv       a Q/K/V triple (5120, 1024, 1024 rows of D=5120) sharing one x: one
            GEMV over the matrices packed as one, then the three separately
  prefill   affine GEMM, T=2048, D=5120, N=13824 (bf16 MFMA)
  moe_dec   MXFP4 grouped GEMV, 16 of 896 experts: gate_up 6144x3584, then
            down 3584x3072 (a fresh expert draw every step)
  moe_pre   routing of 512 tokens, top-16 over 896 experts, on the GPU
            (qmm_route), then the MXFP4 grouped GEMM (gate_up) on its tables
  moe_ffn   the rest of the expert FFN on the same routed rows: gate_up with
            the SwiGLU activation fused, down on the activated rows, and the
            renormalised weighted combine back to the 512 tokens
Weights of the decode and prefill rows rotate over enough packed copies (> 2x
the 256 MB Infinity Cache) that every launch reads HBM, not the cache.  After the timed
steps, a plain streaming read of the decode row's byte count (qmm_stream_read,
rotated the same way, timed the same way) is reported as the achievable read
ceiling at that size (`stream_ceiling`), and when the prefill row runs, a
dense bf16 GEMM of its shape through the vendor library (torch.matmul, no
dequantisation) is timed beside it (`prefill_gemm.bf16_library_gemm`).

After the GPU measurements an oracle phase checks the outputs of the last
timed step of every workload against the CPU oracle (max |err|/tol, on a
stated sample for the large ones: `accuracy`) and times the oracle on the
same samples on this host, extrapolated to one whole workload
(`cpu_baseline`, with the CPU model, its logical CPUs and the BLAS threads
the oracle used; the decode GEMV also on one thread).

Each kernel launch gets HIP start/stop events stamped by its own dispatch
(qmm_profile_next -> hipExtLaunchKernel, on the stream it runs on); their
average interval, the kernel's execution time, gives achieved GB/s (bytes the algorithm must move: packed
weights + activations + outputs) or TFLOP/s against the chip's peaks.  The
headline is the decode GEMV's GB/s.  rank 0 prints one JSON line.
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
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0         # MI355X dense bf16 MFMA
METRIC = "decode GEMV HBM GB/s (% of peak) + prefill GEMM TFLOP/s (% MFMA peak)"


class HipEvents:
    """Raw hipEvent_t handles (libamdhip64 through ctypes), so a launch can have
    its start/stop stamped by the dispatch itself (qmm_profile_next)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.events = []

    def new(self) -> int:
        h = self.ct.c_void_p()
        err = self.hip.hipEventCreate(self.ct.byref(h))
        if err:
            raise RuntimeError(f"hipEventCreate: {err}")
        self.events.append(h.value)
        return h.value

    def record(self, ev: int, stream: int) -> None:
        err = self.hip.hipEventRecord(self.ct.c_void_p(ev), self.ct.c_void_p(stream))
        if err:
            raise RuntimeError(f"hipEventRecord: {err}")

    def ms(self, a: int, b: int) -> float:
        out = self.ct.c_float()
        err = self.hip.hipEventElapsedTime(self.ct.byref(out), self.ct.c_void_p(a), self.ct.c_void_p(b))
        if err:
            raise RuntimeError(f"hipEventElapsedTime: {err}")
        return out.value

    def close(self):
        for h in self.events:
            self.hip.hipEventDestroy(self.ct.c_void_p(h))
        self.events = []


def kernel_sources_hash(files) -> str:
    """Hash of the sources' code with comments and blank space taken out, so a
    comment edit does not retire counters taken on the same code."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)    # block comments
        text = re.sub(r"//[^\n]*", " ", text)                  # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


GEMV_SOURCES = ["bit_weight_quantized_amd/csrc/qmm_gemv.hip", "bit_weight_quantized_amd/csrc/qmm_device.h",
                "bit_weight_quantized_amd/csrc/qmm_internal.h", "bit_weight_quantized_amd/csrc/qmm_launch.h"]


def recorded_traffic(kernel_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the kernel as it is now."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    r = rec.get("decode_gemv")
    if not r or r.get("kernel_sources_hash") != kernel_hash:
        return None
    return r.get("hbm_bytes_per_launch")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=24, help="packed copies of the decode weights")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock-probe", action="store_true",
                    help="skip the back-to-back runs that sample the engine clock and board power")
    ap.add_argument("--rows", default="decode,qkv,prefill,moe_dec,moe_pre,moe_ffn",
                    help="comma list of decode, qkv, prefill, moe_dec, moe_pre, moe_ffn (needs moe_pre); "
                         "'copy' adds a plain 256 MiB device copy used to calibrate HBM byte counters")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(its kernels run on one GPU's share at the real shapes); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import bit_weight_quantized_amd as qmm
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    qmm.load()
    dev = "cuda"
    A, M = qmm.QMM_AFFINE4_G64, qmm.QMM_MXFP4_G32
    rows = [r for r in args.rows.split(",") if r]
    props = torch.cuda.get_device_properties(0)

    def T(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        elif a.dtype == np.uint32:
            a = a.view(np.int32)
        return torch.from_numpy(a).to(dev)

    def log(*a):
        print("[bench]", *a, file=sys.stderr, flush=True)

    work = {}     # row -> list of (launch fn(step), name, bytes, flops)
    ctx = {}      # workload -> host inputs and GPU outputs for the oracle phase
    t_setup = time.time()

    # ---- decode: affine GEMV 13824 x 5120 -------------------------------------------------
    c1 = synth.CONFIGS[1]
    n1, d1 = c1["n"], c1["d"]
    if "decode" in rows:
        w1 = synth.affine_weights(synth.seed_of(1), n1, d1)
        p = torch.empty(qmm.qmm_packed_bytes(A, n1, d1), dtype=torch.uint8, device=dev)
        qmm.qmm_pack(A, n1, d1, T(w1.codes), T(w1.scale), T(w1.bias), p)
        copies = [p] + [p.clone() for _ in range(args.rotate - 1)]
        x1 = T(synth.activations(synth.seed_of(1), synth.S_X, 1, d1))
        y1 = torch.empty(n1, dtype=torch.int16, device=dev)
        b1 = n1 * d1 * 36 // 64 + 2 * d1 + 2 * n1
        y1i = torch.empty(n1, dtype=torch.int16, device=dev)
        work["decode"] = [(lambda s: qmm.qmm_gemv(A, copies[s % len(copies)], n1, d1, x1, y1),
                           "gemv", b1, 2.0 * n1 * d1),
                          # the deferred-dequantisation variant (int8 activations) on the same weights
                          (lambda s: qmm.qmm_gemv_int8(A, copies[(s + 12) % len(copies)], n1, d1, x1, y1i),
                           "gemv_int8", b1, 2.0 * n1 * d1)]
        # a batch of 8 decode rows on the same weights: qmm_gemm as chosen by
        # the library (the multi-row kernel here; under a forced kernel, with
        # the workspace that kernel asks for, every kernel of the call inside
        # the stamped interval)
        x8h = synth.activations(synth.seed_of(1), synth.S_X, 8, d1, sub=3)
        x8 = T(x8h)
        y8 = torch.empty(8, n1, dtype=torch.int16, device=dev)
        ctx["batch8"] = dict(w=w1, x=x8h, y=y8)
        ws8b = qmm.qmm_workspace_bytes(A, 8, n1, d1)
        ws8 = torch.empty(ws8b // 4, dtype=torch.float32, device=dev) if ws8b else None
        b8 = n1 * d1 * 36 // 64 + 2 * 8 * d1 + 2 * 8 * n1
        work["decode"].append((lambda s: qmm.qmm_gemm(A, copies[(s + 6) % len(copies)], 8, n1, d1, x8, y8, ws8),
                               "gemm_t8", b8, 2.0 * 8 * n1 * d1))
        # and a batch of 32 rows (the multi-row kernel with its rows streamed)
        x32h = synth.activations(synth.seed_of(1), synth.S_X, 32, d1, sub=4)
        x32 = T(x32h)
        y32 = torch.empty(32, n1, dtype=torch.int16, device=dev)
        ctx["batch32"] = dict(w=w1, x=x32h, y=y32)
        ws32b = qmm.qmm_workspace_bytes(A, 32, n1, d1)
        ws32 = torch.empty(ws32b // 4, dtype=torch.float32, device=dev) if ws32b else None
        b32 = n1 * d1 * 36 // 64 + 2 * 32 * d1 + 2 * 32 * n1
        work["decode"].append((lambda s: qmm.qmm_gemm(A, copies[(s + 18) % len(copies)], 32, n1, d1, x32, y32, ws32),
                               "gemm_t32", b32, 2.0 * 32 * n1 * d1))
        # the small GEMV workload (T=1, D=256, N=512): 73.7 KB of weights, held
        # in cache after the first launch -- latency, not bandwidth, is its measure
        c0 = synth.CONFIGS[0]
        n0, d0 = c0["n"], c0["d"]
        w0 = synth.affine_weights(synth.seed_of(0), n0, d0)
        p0 = torch.empty(qmm.qmm_packed_bytes(A, n0, d0), dtype=torch.uint8, device=dev)
        qmm.qmm_pack(A, n0, d0, T(w0.codes), T(w0.scale), T(w0.bias), p0)
        x0h = synth.activations(synth.seed_of(0), synth.S_X, 1, d0)
        x0, y0 = T(x0h), torch.empty(n0, dtype=torch.int16, device=dev)
        b0 = n0 * d0 * 36 // 64 + 2 * d0 + 2 * n0
        work["decode"].append((lambda s: qmm.qmm_gemv(A, p0, n0, d0, x0, y0), "gemv_cfg0_512x256", b0, 2.0 * n0 * d0))
        ctx["cfg0"] = dict(name=c0["name"], w=w0, x=x0h, y=y0, bytes=b0, budget=1.0)
        ctx["cfg1"] = dict(name=c1["name"], w=w1, x=synth.activations(synth.seed_of(1), synth.S_X, 1, d1), y=y1,
                           bytes=b1, budget=3.0)
        log("decode ready", len(copies), "copies")

    # ---- fused projections: a Q/K/V triple sharing x as one GEMV, against three ----------
    if "qkv" in rows:
        dq = 5120
        shapes = (5120, 1024, 1024)   # a GQA split of the 5120 hidden size
        qw = [synth.affine_weights(synth.seed_of(1) + 100 + i, nq, dq) for i, nq in enumerate(shapes)]
        fw = synth.Affine(np.concatenate([w.codes for w in qw]), np.concatenate([w.scale for w in qw]),
                          np.concatenate([w.bias for w in qw]))

        def packed_copies(w, count=16):
            pk = torch.empty(qmm.qmm_packed_bytes(A, w.n, w.d), dtype=torch.uint8, device=dev)
            qmm.qmm_pack(A, w.n, w.d, T(w.codes), T(w.scale), T(w.bias), pk)
            return [pk] + [pk.clone() for _ in range(count - 1)]

        fcopies = packed_copies(fw)
        scopies = [packed_copies(w) for w in qw]
        xq = T(synth.activations(synth.seed_of(1) + 100, synth.S_X, 1, dq))
        yq = torch.empty(fw.n, dtype=torch.int16, device=dev)
        ys = [torch.empty(w.n, dtype=torch.int16, device=dev) for w in qw]
        nb = lambda nn: nn * dq * 36 // 64 + 2 * dq + 2 * nn
        work["qkv"] = [(lambda s: qmm.qmm_gemv(A, fcopies[s % 16], fw.n, dq, xq, yq), "gemv_qkv_fused",
                        nb(fw.n), 2.0 * fw.n * dq)]
        for i, (w, nm) in enumerate(zip(qw, ("q", "k", "v"))):
            work["qkv"].append(((lambda i, w: lambda s: qmm.qmm_gemv(A, scopies[i][s % 16], w.n, dq, xq, ys[i]))(i, w),
                                f"gemv_{nm}", nb(w.n), 2.0 * w.n * dq))
        log("qkv ready")

    # ---- prefill: affine GEMM 2048 x 5120 x 13824 ------------------------------------------
    if "prefill" in rows:
        c2 = synth.CONFIGS[2]
        t2, n2, d2 = c2["t"], c2["n"], c2["d"]
        w2 = synth.affine_weights(synth.seed_of(2), n2, d2)
        p2 = torch.empty(qmm.qmm_packed_bytes(A, n2, d2), dtype=torch.uint8, device=dev)
        qmm.qmm_pack(A, n2, d2, T(w2.codes), T(w2.scale), T(w2.bias), p2)
        # sixteen packed copies (637 MB, more than twice the 256 MB Infinity
        # Cache): each call reads weights that the calls before it evicted
        p2s = [p2] + [p2.clone() for _ in range(15)]
        x2 = T(synth.activations(synth.seed_of(2), synth.S_X, t2, d2))
        y2 = torch.empty(t2, n2, dtype=torch.int16, device=dev)
        # affine weights: the activations go to fp16 in the workspace first (the
        # pre-pass kernel is inside the stamped interval)
        ws2 = torch.empty(qmm.qmm_workspace_bytes(A, t2, n2, d2) // 4, dtype=torch.float32, device=dev)
        b2 = n2 * d2 * 36 // 64 + 2 * t2 * d2 + 2 * t2 * n2
        work["prefill"] = [(lambda s: qmm.qmm_gemm(A, p2s[s % len(p2s)], t2, n2, d2, x2, y2, ws2),
                            "gemm", b2, 2.0 * t2 * n2 * d2)]
        ctx["cfg2"] = dict(name=c2["name"], w=w2, x=synth.activations(synth.seed_of(2), synth.S_X, t2, d2), y=y2,
                           t=t2, flops=2.0 * t2 * n2 * d2)
        log("prefill ready")

    # ---- MoE: 896-expert MXFP4 stacks built on the device ----------------------------------
    if "moe_dec" in rows or "moe_pre" in rows:
        import synth.gpu as sg
        gu_n, gu_d, dn_n, dn_d = 6144, 3584, 3584, 3072
        gsz = qmm.qmm_packed_bytes(M, gu_n, gu_d)
        gu = torch.empty(gsz * 896, dtype=torch.uint8, device=dev)
        sg.expert_stack(synth.seed_of(3), "gate_up", 896,
                        lambda c, e, ptr: qmm.qmm_pack(M, gu_n, gu_d, c, e, None, ptr), gsz, gsz, gu)
        log("gate_up stack ready", gu.numel() / 1e9, "GB")
    if "moe_ffn" in rows and "moe_pre" not in rows:
        raise SystemExit("the moe_ffn rows run on moe_pre's routing tables: ask for moe_pre too")
    if "moe_dec" in rows or "moe_ffn" in rows:
        dsz = qmm.qmm_packed_bytes(M, dn_n, dn_d)
        dn = torch.empty(dsz * 896, dtype=torch.uint8, device=dev)
        sg.expert_stack(synth.seed_of(3), "down", 896,
                        lambda c, e, ptr: qmm.qmm_pack(M, dn_n, dn_d, c, e, None, ptr), dsz, dsz, dn)
        log("down stack ready")
    if "moe_dec" in rows:
        seed3 = synth.seed_of(3)
        x3 = T(synth.activations(seed3, synth.S_X, 1, gu_d))
        z3 = T(synth.activations(seed3, synth.S_Z, 16, dn_d))
        nsteps = args.steps + args.warmup
        draws = T(np.stack([synth.draw_experts(seed3, 16, 896, s) for s in range(nsteps)]).astype(np.int32))
        offs = T(np.arange(17, dtype=np.int32))
        zero_idx = T(np.zeros(16, np.int32))
        iden_idx = T(np.arange(16, dtype=np.int32))
        h3 = torch.empty(16, gu_n, dtype=torch.int16, device=dev)
        o3 = torch.empty(16, dn_n, dtype=torch.int16, device=dev)
        bg = 16 * (gsz - 256) + 2 * gu_d + 2 * 16 * gu_n
        bd = 16 * (dsz - 256) + 2 * 16 * dn_d + 2 * 16 * dn_n
        ctx["cfg3"] = dict(name=synth.CONFIGS[3]["name"], experts=synth.draw_experts(seed3, 16, 896, args.steps - 1),
                           x=synth.activations(seed3, synth.S_X, 1, gu_d), z=synth.activations(seed3, synth.S_Z, 16, dn_d),
                           h=h3, o=o3, bytes=None,
                           gate_up=lambda e: synth.expert_gate_up(seed3, e), down=lambda e: synth.expert_down(seed3, e))
        work["moe_dec"] = [
            (lambda s: qmm.qmm_grouped_gemm(M, gu, gsz, 896, gu_n, gu_d, x3, 1, zero_idx, draws[s],
                                            offs, 16, 16, 1, h3), "grouped_gemv_gate_up", bg,
             2.0 * 16 * gu_n * gu_d),
            (lambda s: qmm.qmm_grouped_gemm(M, dn, dsz, 896, dn_n, dn_d, z3, 16, iden_idx, draws[s],
                                            offs, 16, 16, 1, o3), "grouped_gemv_down", bd,
             2.0 * 16 * dn_n * dn_d),
        ]
        ctx["cfg3"]["bytes"] = bg + bd
    if "moe_pre" in rows:
        # routed on the GPU every step (qmm_route), its tables driving the grouped
        # matmul directly: segments dense over all 896 experts, empty ones included
        seed4 = synth.seed_of(4)
        xb, rb, bias = synth.router_inputs(seed4)
        t4, ne, k4 = xb.shape[0], rb.shape[0], 16
        x4, r4, bias4 = T(xb), T(rb), torch.from_numpy(bias).to(dev)
        scores4 = torch.empty(t4, ne, dtype=torch.float32, device=dev)
        topk4 = torch.empty(t4, k4, dtype=torch.int32, device=dev)
        se = torch.empty(ne, dtype=torch.int32, device=dev)
        so = torch.empty(ne + 1, dtype=torch.int32, device=dev)
        ri = torch.empty(t4 * k4, dtype=torch.int32, device=dev)
        route = lambda s: qmm.qmm_route(x4, t4, gu_d, r4, ne, bias4, k4, scores4, topk4, se, so, ri)
        route(0)
        sizes = np.diff(so.cpu().numpy())        # setup only: the byte count needs the active experts
        n_active = int(np.count_nonzero(sizes))
        y4 = torch.empty(t4 * k4, gu_n, dtype=torch.int16, device=dev)
        b4 = n_active * (gsz - 256) + 2 * xb.size + 2 * t4 * k4 * gu_n
        br = 2 * xb.size + 2 * rb.size + 4 * ne + 4 * t4 * ne + 4 * t4 * k4 + 8 * t4 * k4 + 8 * ne
        moe_pre_info = dict(active_experts=n_active, routed_rows=t4 * k4, max_seg_rows=int(sizes.max()))
        work["moe_pre"] = [
            (route, "route", br, 2.0 * t4 * ne * gu_d),
            (lambda s: qmm.qmm_grouped_gemm(M, gu, gsz, 896, gu_n, gu_d, x4, t4, ri, se, so, ne, t4 * k4,
                                            t4, y4), "grouped_gemm", b4, 2.0 * t4 * k4 * gu_n * gu_d)]
        ctx["cfg4"] = dict(name=synth.CONFIGS[4]["name"], x=xb, y=y4, flops=2.0 * t4 * k4 * gu_n * gu_d,
                           gate_up=lambda e: synth.expert_gate_up(synth.seed_of(3), e),
                           seg_offsets=None, row_index=None, tables=(so, ri))
        log("moe_pre ready", moe_pre_info)
    if "moe_ffn" in rows:
        # the rest of the expert FFN on the same routed rows: gate_up with the
        # SwiGLU activation fused, down on the activated rows (already in grouped
        # order), the renormalised weighted combine back to the 512 tokens
        m4 = t4 * k4
        h4 = torch.empty(m4, gu_n // 2, dtype=torch.int16, device=dev)
        o4 = torch.empty(m4, dn_n, dtype=torch.int16, device=dev)
        out4 = torch.empty(t4, dn_n, dtype=torch.int16, device=dev)
        bsw = n_active * (gsz - 256) + 2 * xb.size + 2 * m4 * (gu_n // 2)
        bdn = n_active * (dsz - 256) + 2 * m4 * dn_d + 2 * m4 * dn_n
        bcb = 2 * m4 * dn_n + 2 * t4 * dn_n + 4 * t4 * k4 * 2 + 4 * m4 + 4 * (ne + 1)
        work["moe_ffn"] = [
            (lambda s: qmm.qmm_grouped_gemm_swiglu(M, gu, gsz, 896, gu_n, gu_d, x4, t4, ri, se, so, ne, m4,
                                                   t4, h4), "grouped_gemm_swiglu", bsw,
             2.0 * m4 * gu_n * gu_d),
            (lambda s: qmm.qmm_grouped_gemm(M, dn, dsz, 896, dn_n, dn_d, h4, m4, None, se, so, ne, m4, t4, o4),
             "grouped_gemm_down", bdn, 2.0 * m4 * dn_n * dn_d),
            (lambda s: qmm.qmm_moe_combine(o4, m4, dn_n, t4, k4, topk4, scores4, ne, so, ri, out4),
             "moe_combine", bcb, 2.0 * m4 * dn_n),
        ]
        log("moe_ffn ready")
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    if "copy" in rows:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        work["copy"] = [(lambda s: dst.copy_(src), "copy_256MiB", 2 * src.numel(), 0.0)]

    launches = [(row, fn, name, nb, fl) for row in rows for (fn, name, nb, fl) in work[row]]
    stream = torch.cuda.current_stream()
    hev = HipEvents()
    ev = [[(hev.new(), hev.new()) for _ in launches] for _ in range(args.steps)]

    for s in range(args.warmup):
        for (_, fn, _, _, _) in launches:
            fn(s + args.steps)
    torch.cuda.synchronize()

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for s in range(args.steps):
        for i, (row, fn, _, _, _) in enumerate(launches):
            if row == "copy":            # not a libqmm launch: plain stream events
                hev.record(ev[s][i][0], stream.cuda_stream)
                fn(s)
                hev.record(ev[s][i][1], stream.cuda_stream)
            else:
                qmm.qmm_profile_next(ev[s][i][0], ev[s][i][1])   # stamped by the kernel's dispatch
                fn(s)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps

    results = {}
    for i, (row, fn, name, nb, fl) in enumerate(launches):
        us = np.array([hev.ms(ev[s][i][0], ev[s][i][1]) * 1e3 for s in range(args.steps)])
        mean = float(us.mean())
        results[name] = dict(row=row, us_mean=round(mean, 3), us_median=round(float(np.median(us)), 3),
                             us_p10=round(float(np.percentile(us, 10)), 3),
                             us_p90=round(float(np.percentile(us, 90)), 3),
                             bytes=int(nb), flops=fl,
                             GBps=round(nb / mean / 1e3, 1), TFLOPs=round(fl / mean / 1e6, 2),
                             hbm_frac=round(nb / mean / 1e3 / HBM_PEAK_GBPS, 4),
                             mfma_frac=round(fl / mean / 1e6 / BF16_PEAK_TFLOPS, 4))

    # read ceiling at the decode size: a plain streaming read of the same number
    # of bytes, rotated over as many buffers, timed the same way (not part of a step)
    stream_ceiling = None
    if "decode" in rows:
        sbytes = b1 // 16 * 16
        sbufs = [torch.empty(sbytes, dtype=torch.uint8, device=dev).fill_(1) for _ in range(args.rotate)]
        sink = torch.empty(2048, dtype=torch.int32, device=dev)
        for i in range(10):
            qmm.qmm_stream_read(sbufs[i % len(sbufs)], sbytes, sink)
        sev = [(hev.new(), hev.new()) for _ in range(max(args.steps, 100))]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(sev):
            qmm.qmm_profile_next(a, b)
            qmm.qmm_stream_read(sbufs[i % len(sbufs)], sbytes, sink)
        torch.cuda.synchronize()
        sus = np.array([hev.ms(a, b) * 1e3 for a, b in sev])
        stream_ceiling = {"kernel": "stream_read_kernel", "bytes": int(sbytes), "launches": len(sev),
                          "us_mean": round(float(sus.mean()), 3), "us_median": round(float(np.median(sus)), 3),
                          "GBps": round(sbytes / float(sus.mean()) / 1e3, 1),
                          "frac": round(sbytes / float(sus.mean()) / 1e3 / HBM_PEAK_GBPS, 4)}
        del sbufs

    # dense bf16 GEMM of the prefill shape through the vendor library (torch.matmul,
    # hipBLASLt), no dequantisation: what the matrix cores sustain on this machine for
    # this shape with full-entropy operands; context beside the prefill row, not
    # part of a step
    library_gemm = None
    if "prefill" in rows:
        xb = x2.view(torch.bfloat16)
        wt = torch.randn(d2, n2, device=dev, dtype=torch.float32).to(torch.bfloat16)   # [D, N] contiguous
        for _ in range(3):
            torch.matmul(xb, wt)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            torch.matmul(xb, wt)
        e1.record()
        torch.cuda.synchronize()
        lus = e0.elapsed_time(e1) * 1e3 / 20
        library_gemm = {"what": "torch.matmul bf16 [2048,5120]x[5120,13824] (hipBLASLt), no dequantisation",
                        "us_mean": round(lus, 2), "TFLOPs": round(2.0 * t2 * n2 * d2 / lus / 1e6, 1),
                        "frac": round(2.0 * t2 * n2 * d2 / lus / 1e6 / BF16_PEAK_TFLOPS, 4)}
        del wt

    # the engine clock and board power while one kernel runs back to back for
    # ~0.2 s (sysfs, sampled on a host thread): the clock the chip holds under
    # that load, against its peak
    under_load = {}
    hw = None if args.no_clock_probe else gpu_sysfs_dir()
    if hw:
        # (launch name in the step, label, calls: ~0.2 s each); the calls rerun
        # the step's own launches, whose outputs they rewrite with the same values
        by_name = {name: fn for (_, fn, name, _, _) in launches}
        probes = [("gemv", "decode_gemv", 20000), ("gemm", "prefill_gemm", 700),
                  ("grouped_gemm", "moe_prefill_grouped_gemm", 140)]
        nsteps = args.steps + args.warmup
        for key, label, count in probes:
            if key not in by_name:
                continue
            fn = by_name[key]
            torch.cuda.synchronize()
            with ClockSampler(hw) as cs:
                for i in range(count):
                    fn(i % nsteps)
                torch.cuda.synchronize()
            under_load[label] = cs.summary()

    hev.close()
    out = {
        "metric": METRIC,
        "value": None, "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded counter-based generator; no weights or datasets)",
        "config": {"workload": synth.CONFIGS[1]["name"], "t": 1, "d": d1, "n": n1,
                   "format": "affine4_g64", "rotation_copies": args.rotate,
                   "step": "decode GEMV (+ int8 variant, + 8- and 32-row batches) + fused Q/K/V GEMV (and the three separately) + prefill GEMM"
                           " + MoE decode grouped GEMV x2 + MoE prefill route + grouped GEMM"
                           " + expert FFN (gate_up with SwiGLU, down, combine)"
                   if rows == ["decode", "qkv", "prefill", "moe_dec", "moe_pre", "moe_ffn"] else ",".join(rows)},
    }
    if "gemv" in results:
        g = results["gemv"]
        out["value"] = g["GBps"]
        kh = kernel_sources_hash(GEMV_SOURCES)
        traffic = recorded_traffic(kh)
        out["roofline"] = {"bound": "hbm", "achieved": g["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": g["hbm_frac"], "traffic": traffic, "kernel": "gemv_kernel<affine>",
                           "algorithmic_bytes_per_launch": g["bytes"], "kernel_sources_hash": kh}
    if stream_ceiling is not None:
        out["stream_ceiling"] = stream_ceiling
        if "roofline" in out:
            out["roofline"]["achievable_stream_GBps"] = stream_ceiling["GBps"]
    if "gemm" in results:
        g = results["gemm"]
        out["prefill_gemm"] = {"value": g["TFLOPs"], "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS,
                               "frac": g["mfma_frac"], "us_mean": g["us_mean"],
                               "workload": synth.CONFIGS[2]["name"]}
        if library_gemm is not None:
            out["prefill_gemm"]["bf16_library_gemm"] = library_gemm
            out["prefill_gemm"]["vs_bf16_library"] = round(library_gemm["us_mean"] / g["us_mean"], 3)
    out["rows"] = results
    if "moe_pre" in rows:
        out["rows"]["grouped_gemm"].update(moe_pre_info)
    out["gpu"] = {"name": props.name, "cus": props.multi_processor_count,
                  "hip": torch.version.hip, "torch": torch.__version__}
    # a kernel forced through QMM_FORCE_KERNEL (A/B runs) is named in the line
    ks = qmm.qmm_get_kernel()
    out["kernel_setting"] = {0: "auto", 1: "tile", 2: "tile_unsplit", 3: "few_row",
                             4: "grouped_matmul", 5: "multi_row"}.get(ks, f"invalid ({ks})")
    out["setup_s"] = round(t_setup, 1)
    out["wall_s_timed"] = round(wall, 3)

    out["gpu"].update(hip_runtime())
    out["gpu"]["under_load"] = under_load or None
    if not args.no_cpu_baseline and ctx:
        # GPU outputs of the last timed step to the host, then the oracle
        for c in ctx.values():
            for k in ("y", "h", "o"):
                if k in c and hasattr(c[k], "cpu"):
                    c[k] = c[k].cpu().numpy().view(np.uint16)
            if "tables" in c:
                c["seg_offsets"], c["row_index"] = (t_.cpu().numpy() for t_ in c.pop("tables"))
        log("oracle phase")
        t_or = time.time()
        acc, base, info = oracle_phase(ctx)
        out["accuracy"] = acc
        if "cfg1" in base:
            b = base["cfg1"]
            out["cpu_baseline"] = {"value": b["GBps"], "unit": "GB/s", "cores": info["blas_threads"], "kind": "oracle",
                                   "sample": f"{b['sample']} of the decode workload {b['workload']} (fp64 dequantisation "
                                             f"in numpy, one thread; fp64 matvec in the numpy BLAS, "
                                             f"{info['blas_threads']} threads)",
                                   "value_single_thread": b["GBps_single_thread"], **info, "configs": base}
        else:
            out["cpu_baseline"] = {"kind": "oracle", **info, "configs": base}
        log("oracle phase", round(time.time() - t_or, 1), "s")
    print(json.dumps(out), flush=True)
    return 0


def hip_runtime():
    """The HIP runtime the kernels ran on: the libamdhip64 this process mapped
    (libqmm binds to the copy torch loaded first) and the ROCm release of the
    machine."""
    lib = None
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    lib = line.split()[-1]
                    break
    except OSError:
        pass
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    out = {"hip_runtime_library": lib, "rocm_release": rocm}
    # peak engine and memory clocks as the runtime reports them (kHz;
    # hipDeviceAttributeClockRate = 5, hipDeviceAttributeMemoryClockRate = 60)
    try:
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        dev, v = ctypes.c_int(), ctypes.c_int()
        if hip.hipGetDevice(ctypes.byref(dev)) == 0:
            for key, attr in (("peak_sclk_MHz", 5), ("peak_mclk_MHz", 60)):
                if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev) == 0:
                    out[key] = round(v.value / 1000)
    except OSError:
        pass
    return out


def gpu_sysfs_dir():
    """The sysfs directory of the GPU this process runs on (found by the PCI
    bus id HIP reports), or None where its clock table is not readable."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        dev = ctypes.c_int()
        buf = ctypes.create_string_buffer(64)
        if hip.hipGetDevice(ctypes.byref(dev)) or hip.hipDeviceGetPCIBusId(buf, 64, dev):
            return None
        d = "/sys/bus/pci/devices/" + buf.value.decode().strip().lower()
    except (OSError, UnicodeDecodeError):
        return None
    return d if os.access(os.path.join(d, "pp_dpm_sclk"), os.R_OK) else None


class ClockSampler:
    """Samples the GPU's current engine clock (the "S:" line of the driver's
    pp_dpm_sclk table, or its starred level) and board power (hwmon
    power1_input or power1_average) every ~2 ms on a host thread while a
    workload runs; reads sysfs only, never the GPU."""

    def __init__(self, d):
        import glob
        import threading
        self.sclk_path = os.path.join(d, "pp_dpm_sclk")
        self.power_path = None
        for name in ("power1_input", "power1_average"):
            hits = sorted(glob.glob(os.path.join(d, "hwmon", "hwmon*", name)))
            if hits:
                self.power_path = hits[0]
                break
        self.sclk, self.power = [], []
        self.stop_flag = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _sclk(self):
        try:
            with open(self.sclk_path) as f:
                lines = f.read().splitlines()
        except OSError:
            return None
        pick = [ln for ln in lines if ln.strip().startswith("S:")] or [ln for ln in lines if ln.rstrip().endswith("*")]
        for ln in pick:
            for tok in ln.replace(":", " ").split():
                if tok.lower().endswith("mhz") and tok[:-3].isdigit():
                    return float(tok[:-3])
        return None

    def _run(self):
        while not self.stop_flag.is_set():
            v = self._sclk()
            if v:
                self.sclk.append(v)
            if self.power_path:
                try:
                    with open(self.power_path) as f:
                        self.power.append(float(f.read().strip()) / 1e6)
                except (OSError, ValueError):
                    pass
            time.sleep(0.002)

    def __enter__(self):
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop_flag.set()
        self.thread.join()

    def summary(self):
        if not self.sclk:
            return None
        return {"sclk_MHz_median": round(float(np.median(self.sclk))), "sclk_MHz_min": round(float(np.min(self.sclk))),
                "power_W_median": round(float(np.median(self.power)), 1) if self.power else None,
                "samples": len(self.sclk)}


def host_info():
    """The host the oracle runs on: CPU model, logical CPUs, and the BLAS
    threads numpy's matmul uses (the oracle's only multithreaded step)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "blas_threads": int(blas)}


def timed(fn, *a):
    t0 = time.perf_counter()
    r = fn(*a)
    return r, time.perf_counter() - t0


def oracle_phase(ctx, single_thread=True):
    """After the timed steps: the GPU outputs of every workload against the
    oracle (max |err|/tol per workload, on the stated sample), and the oracle's
    own time on the same sample, extrapolated to one whole workload -- the CPU
    baseline.  Runs on the host, after every GPU measurement."""
    import oracle
    acc, base = {}, {}
    info = host_info()

    def rec(name, r, n, sample):
        acc[name] = {"max_err_over_tol": round(r["max_ratio"], 4), "ok": bool(r["ok"]), "outputs_checked": int(n),
                     "sample": sample}

    def single(fn, *a):
        if not single_thread:
            return None
        try:
            from threadpoolctl import threadpool_limits
        except Exception:
            return None
        with threadpool_limits(1):
            return timed(fn, *a)[1]

    # configs 0 and 1: whole GEMVs, all threads and one thread
    for key in ("cfg0", "cfg1"):
        if key not in ctx:
            continue
        c = ctx[key]
        (yr, ar), dt = timed(oracle.gemm_affine, c["x"], c["w"].codes, c["w"].scale, c["w"].bias)
        reps, tot = 1, dt
        while tot < c.get("budget", 0.0) and reps < 50:
            tot += timed(oracle.gemm_affine, c["x"], c["w"].codes, c["w"].scale, c["w"].bias)[1]
            reps += 1
        st = single(oracle.gemm_affine, c["x"], c["w"].codes, c["w"].scale, c["w"].bias)
        rec(key, oracle.check(c["y"], yr[0], ar[0]), yr.size, "every output")
        base[key] = {"workload": c["name"], "seconds": round(tot / reps, 4), "GBps": round(c["bytes"] / (tot / reps) / 1e9, 4),
                     "seconds_single_thread": None if st is None else round(st, 4),
                     "GBps_single_thread": None if st is None else round(c["bytes"] / st / 1e9, 4),
                     "sample": f"{reps} whole GEMVs"}
    # the 8-row decode batch on config 1's weights: every output
    if "batch8" in ctx:
        c = ctx["batch8"]
        yr, ar = oracle.gemm_affine(c["x"], c["w"].codes, c["w"].scale, c["w"].bias)
        rec("decode_batch8", oracle.check(c["y"], yr, ar), yr.size, "every output of the 8-row batch")
    if "batch32" in ctx:
        c = ctx["batch32"]
        yr, ar = oracle.gemm_affine(c["x"], c["w"].codes, c["w"].scale, c["w"].bias)
        rec("decode_batch32", oracle.check(c["y"], yr, ar), yr.size, "every output of the 32-row batch")
    # config 2: the weights dequantised once, then 64 of the 2048 rows
    if "cfg2" in ctx:
        c = ctx["cfg2"]
        w_hat, t_deq = timed(oracle.dequant_affine, c["w"].codes, c["w"].scale, c["w"].bias)
        rows = np.linspace(0, c["t"] - 1, 64).astype(int)
        (yr, ar), t_mm = timed(oracle.matmul, c["x"][rows], w_hat)
        rec("cfg2", oracle.check(c["y"][rows], yr, ar), yr.size, "64 of the 2048 rows (evenly spaced), every column")
        full = t_deq + t_mm * c["t"] / len(rows)
        base["cfg2"] = {"workload": c["name"], "seconds": round(full, 3), "GFLOPs": round(c["flops"] / full / 1e9, 3),
                        "sample": "dequantisation of all weights + 64 of 2048 rows, extrapolated to 2048 rows"}
    # config 3: two of the 16 routed experts, gate_up and down
    if "cfg3" in ctx:
        c = ctx["cfg3"]
        worst, n_out, t_or = 0.0, 0, 0.0
        ok = True
        for i in (0, len(c["experts"]) - 1):
            e = int(c["experts"][i])
            t0 = time.perf_counter()
            g = c["gate_up"](e)
            yr, ar = oracle.gemm_mxfp4(c["x"], g.codes, g.e8m0)
            dw = c["down"](e)
            yr2, ar2 = oracle.gemm_mxfp4(c["z"][i:i + 1], dw.codes, dw.e8m0)
            t_or += time.perf_counter() - t0
            for r in (oracle.check(c["h"][i], yr[0], ar[0]), oracle.check(c["o"][i], yr2[0], ar2[0])):
                worst, ok = max(worst, r["max_ratio"]), ok and r["ok"]
            n_out += yr.size + yr2.size
        acc["cfg3"] = {"max_err_over_tol": round(worst, 4), "ok": ok, "outputs_checked": n_out,
                       "sample": "2 of the 16 routed experts (the last step's draw), gate_up and down, every output"}
        full = t_or * len(c["experts"]) / 2
        base["cfg3"] = {"workload": c["name"], "seconds": round(full, 3), "GBps": round(c["bytes"] / full / 1e9, 4),
                        "sample": "2 of 16 experts (weights generated, dequantised, multiplied), extrapolated to 16"}
    # config 4: six routed segments on the GPU router's own tables
    if "cfg4" in ctx:
        c = ctx["cfg4"]
        sizes = np.diff(c["seg_offsets"])
        active = np.nonzero(sizes)[0]
        rng = np.random.default_rng(4)
        pick = sorted({int(active[np.argmax(sizes[active])]), *rng.choice(active, 5, replace=False).tolist()})
        worst, n_out, t_or, ok = 0.0, 0, 0.0, True
        for e in pick:
            r0, r1 = int(c["seg_offsets"][e]), int(c["seg_offsets"][e + 1])
            t0 = time.perf_counter()
            g = c["gate_up"](e)
            yr, ar = oracle.gemm_mxfp4(c["x"][c["row_index"][r0:r1]], g.codes, g.e8m0)
            t_or += time.perf_counter() - t0
            r = oracle.check(c["y"][r0:r1], yr, ar)
            worst, ok, n_out = max(worst, r["max_ratio"]), ok and r["ok"], n_out + yr.size
        acc["cfg4"] = {"max_err_over_tol": round(worst, 4), "ok": ok, "outputs_checked": n_out,
                       "sample": f"{len(pick)} of {len(active)} routed segments (the largest and 5 at random), "
                                 "every row and column, on the GPU router's tables"}
        full = t_or * len(active) / len(pick)
        base["cfg4"] = {"workload": c["name"], "seconds": round(full, 3), "GFLOPs": round(c["flops"] / full / 1e9, 3),
                        "sample": f"{len(pick)} of {len(active)} active experts, extrapolated by expert count"}
    return acc, base, info


if __name__ == "__main__":
    sys.exit(main())
