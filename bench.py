#!/usr/bin/env python3
"""Benchmark of the NVFP4 hot path on one MI355X.

One step = one pass over every row of the path, each on its own seeded
synthetic workload:
  decode_b1   the 27B-class dense layer at batch 1: five GEMVs (gate, up 5120->17408,
              down 17408->5120, QKV 5120->7168, O 5120->5120), fp32 outputs
  decode_b32  the same layer's weights at 32 decode tokens: five skinny GEMMs, bf16 outputs
  moe         32 tokens through a 512-expert, top-10 MoE layer (hidden 2048, expert
              width 512): route; gate/up + SwiGLU, each workgroup grouping the
              routed rows first; down; scatter
  prefill     a 512-token prompt through gate, up (5120->17408) and down (17408->5120)
  gemv_1k     one 1024 x 1024 GEMV at batch 1 (latency-bound: reported in us and GB/s)
The headline `value` is the batch-1 layer's weight-stream rate in GB/s
(algorithmic bytes: NVFP4 weights + x + y).  Weights are rotated over several
device copies so that no copy is re-read before > 1 GiB of other traffic:
the 256 MB Infinity Cache cannot serve repeats.  After the timed steps the
ceiling probes (libnvfp4_probes.so) measure what this machine sustains for a
streaming read in the weights' tile unit and for the bf16 and FP4 matrix
instructions with random operands; every row's fraction of nominal peak is
reported next to its fraction of that measured ceiling.

Prints ONE JSON line on stdout; details go to stderr.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
MODEL_27B_BYTES_PER_TOKEN = 27e9 * 0.5625  # weights-only stream of a 27B NVFP4 model


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipTimingEvents:
    """HIP events for the per-row intervals, recorded on the stream the rows
    launch on.  They are created with hipEventDisableSystemFence: recording
    one then does not write back and invalidate the caches, a cost that would
    otherwise land inside the interval it closes (several microseconds, more
    after a row that writes tens of megabytes).  Elapsed times are read only
    after a device synchronisation."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        # The HIP runtime that torch has loaded (same soname), not a second copy.
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def new(self):
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.events.append(ev)
        return ev

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ev, self.ct.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target length of the oracle sample")
    p.add_argument("--no-probes", action="store_true", help="skip the ceiling probes after the timed steps")
    p.add_argument("--rows", default="decode_b1,decode_b32,moe,prefill,gemv_1k",
                   help="rows to run; optional, not default: quantize (the NVFP4 quantiser over the layer), "
                        "decode_m2 .. decode_m8 (the layer at decode widths 2..8), head_b1 (the output head, batch 1), "
                        "moe_stream (the MoE layer with experts streamed from host memory), prefill_w4a4 (the prefill "
                        "products as W4A4 on the FP4 matrix cores)")
    p.add_argument("--order", default="prefill,moe,decode_b32,gemv_1k,decode_b1",
                   help="row order within a step (the batch-1 GEMV last: see the note at the plan)")
    p.add_argument("--graphs", action="store_true", help="replay per-row HIP graphs instead of direct launches")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path runs on a single "
              f"MI355X; see the multi-GPU design notes)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from bit_quantized_decode_amd import binding as B
    from bit_quantized_decode_amd import inputs as I

    dev = torch.device("cuda:0")
    B.lib()
    rows = set(args.rows.split(","))
    t_setup = time.time()

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---- the dense layer (batch 1 and batch 32 share weights) ----------------
    layer = I.DENSE_LAYER
    dense_copies = 4
    packed = [[None] * len(layer) for _ in range(dense_copies)]
    b1_inputs = hashlib.sha256()   # the batch-1 layer's codes, scales and x, as the oracle baseline also hashes them
    for j, mat in enumerate(layer):
        c, s = I.nvfp4_matrix(I.DECODE_B1, mat.matrix_id, mat.n, mat.k)
        for a_ in (c, s, I.activations(I.DECODE_B1, mat.matrix_id, 1, mat.k)):
            b1_inputs.update(np.ascontiguousarray(a_).tobytes())
        p0 = B.pack(u8(c), u8(s))
        for cp in range(dense_copies):
            packed[cp][j] = p0 if cp == 0 else p0.clone()
    x1 = [bf16(I.activations(I.DECODE_B1, m.matrix_id, 1, m.k)[0]) for m in layer]
    y1 = [torch.empty(m.n, dtype=torch.float32, device=dev) for m in layer]
    x32 = [bf16(I.activations(I.DECODE_B32, m.matrix_id, 32, m.k)) for m in layer]
    y32 = [torch.empty((32, m.n), dtype=torch.bfloat16, device=dev) for m in layer]
    ws_split = B.workspace(64 << 20, dev)   # counters + split-K partials of the batched layer calls
    b1_bytes = sum(B.packed_bytes(m.n, m.k) + 2 * m.k + 4 * m.n for m in layer)
    b1_weight_bytes = sum(B.packed_bytes(m.n, m.k) for m in layer)
    b32_bytes = sum(B.packed_bytes(m.n, m.k) + 2 * 32 * m.k + 2 * 32 * m.n for m in layer)
    b32_flops = sum(2 * 32 * m.n * m.k for m in layer)

    # ---- MoE --------------------------------------------------------------
    shape = I.MoeShape()
    moe_pools = []
    if "moe" in rows or "moe_stream" in rows:
        w = I.moe_weights(I.MOE_32T, shape)
        stride_gu = B.packed_bytes(shape.inter, shape.hidden)
        stride_d = B.packed_bytes(shape.hidden, shape.inter)

        def pool(codes, scales, stride):
            out = torch.empty(shape.experts * stride, dtype=torch.uint8, device=dev)
            for e in range(shape.experts):
                out[e * stride:(e + 1) * stride].copy_(B.pack(u8(codes[e]), u8(scales[e])))
            return out

        pg, pu, pd = (pool(w.gate_codes, w.gate_scales, stride_gu), pool(w.up_codes, w.up_scales, stride_gu),
                      pool(w.down_codes, w.down_scales, stride_d))
        moe_pools = [(pg, pu, pd), (pg.clone(), pu.clone(), pd.clone())]
        moe_x = bf16(I.activations(I.MOE_32T, 0, shape.tokens, shape.hidden))
        moe_logits = torch.from_numpy(I.router_logits(I.MOE_32T, shape.tokens, shape.experts, shape.zipf_s)).to(dev)
        sts = [torch.from_numpy(a).to(dev) for a in (w.gate_st, w.up_st, w.down_st)]
        moe_out = {}
        moe_ws = B.workspace(B.moe_workspace_bytes(shape.tokens, shape.experts, shape.top_k, shape.hidden,
                                                   shape.inter), dev, kind="moe")
        del w

    # The row routes a different batch of 32 tokens each step: 16 seeded
    # routings (other tokens and router noise, the same Zipf expert
    # popularity) over the two weight pools, 32 prepared calls in turn.
    moe_routings = 16
    moe_calls, moe_call_bytes, moe_call_active = [], [], []
    if "moe" in rows:
        per_expert = 3 * B.packed_bytes(shape.inter, shape.hidden)
        fixed = (2 * shape.tokens * shape.hidden + 4 * shape.tokens * shape.experts + 4 * shape.tokens * shape.hidden
                 + 8 * shape.tokens * shape.top_k)
        for r in range(moe_routings):
            xr = moe_x if r == 0 else bf16(I.activations(I.MOE_32T, r, shape.tokens, shape.hidden))
            lr = moe_logits if r == 0 else torch.from_numpy(
                I.router_logits(I.MOE_32T, shape.tokens, shape.experts, shape.zipf_s, batch=r)).to(dev)
            for cp in range(2):
                pg_, pu_, pd_ = moe_pools[cp]
                call, o_ = B.moe_grouped_prepared(xr, lr, shape.top_k, pg_, pu_, pd_, stride_gu, stride_gu, stride_d,
                                                  sts[0], sts[1], sts[2], shape.inter, y_dtype=torch.float32,
                                                  ws=moe_ws, outputs=moe_out)
                moe_calls.append(call)
            torch.cuda.synchronize()
            active = int((moe_out["expert_counts"].cpu() > 0).sum())
            moe_call_active += [active, active]
            moe_call_bytes += [active * per_expert + fixed] * 2

    def run_moe(cp):
        moe_calls[cp]()

    # ---- optional: the same layer with the experts streamed from pinned host
    # memory through a device cache of 64 expert slots (1/8 of the experts);
    # each step routes a new batch of 32 tokens (other tokens, the same expert
    # popularity), 64 batches in turn -------------------------------------
    stream_state = {}
    if "moe_stream" in rows:
        es = B.ExpertStream(*moe_pools[0], stride_gu, stride_gu, stride_d, shape.experts, 64, dev)
        batches = 64
        sx = [bf16(I.activations(I.MOE_32T, 100 + r, shape.tokens, shape.hidden)) for r in range(batches)]
        slg = [torch.from_numpy(I.router_logits(I.MOE_32T, shape.tokens, shape.experts, shape.zipf_s, batch=r)).to(dev)
               for r in range(batches)]
        s_out = {}
        stream_state.update(es=es, stats=[], out=s_out)

    def run_moe_stream(cp):
        es = stream_state["es"]
        B.moe_grouped(sx[cp], slg[cp], shape.top_k, es, None, None, None, None, None, sts[0], sts[1], sts[2],
                      shape.inter, y_dtype=torch.float32, ws=moe_ws, outputs=stream_state["out"])
        stream_state["stats"].append(es.stats())

    # ---- prefill ----------------------------------------------------------
    pre = I.PREFILL_MATRICES
    pre_copies = 2
    pre_packed = [[None] * len(pre) for _ in range(pre_copies)]
    pre_x, pre_y = [], []
    if "prefill" in rows:
        for j, mat in enumerate(pre):
            c, s = I.nvfp4_matrix(I.PREFILL_512, mat.matrix_id, mat.n, mat.k)
            p0 = B.pack(u8(c), u8(s))
            for cp in range(pre_copies):
                pre_packed[cp][j] = p0 if cp == 0 else p0.clone()
            pre_x.append(bf16(I.activations(I.PREFILL_512, mat.matrix_id, 512, mat.k)))
            pre_y.append(torch.empty((512, mat.n), dtype=torch.bfloat16, device=dev))
    pre_flops = sum(2 * 512 * m.n * m.k for m in pre)
    pre_bytes = sum(B.packed_bytes(m.n, m.k) + 2 * 512 * m.k + 2 * 512 * m.n for m in pre)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s")

    # ---- one step: each row's launches, made directly with their arguments
    # marshalled once per weight copy (prepared library calls), so that the
    # events around a row, on the kernels' own stream, bracket its kernels.
    # (--graphs replays per-row HIP graphs instead; on ROCm a graph launch
    # adds more GPU-side time than direct launches: 5-7 us per row.)
    # The layer's five products go out as one batched launch (per row).
    b1_calls = [B.gemv_batched_prepared([(packed[cp][j], m.n, m.k, I.TENSOR_SCALE, x1[j], y1[j])
                                         for j, m in enumerate(layer)], ws=ws_split)
                for cp in range(dense_copies)] if "decode_b1" in rows else []

    def row_b1(cp):
        b1_calls[cp]()

    b32_calls = [B.gemm_batched_prepared([(packed[cp][j], m.n, m.k, I.TENSOR_SCALE, x32[j], y32[j])
                                          for j, m in enumerate(layer)], ws=ws_split)
                 for cp in range(dense_copies)] if "decode_b32" in rows else []

    def row_b32(cp):
        b32_calls[cp]()

    # ---- optional rows: decode widths 2..8 (the layer's five products in one
    # batched launch, bf16 out) and the output head at batch 1 ----------------
    extra_rows = {}
    for r in sorted(rows):
        if r.startswith("decode_m") and r[len("decode_m"):].isdigit():
            mw = int(r[len("decode_m"):])
            if not 2 <= mw <= 8:
                raise SystemExit(f"{r}: decode widths 2..8 only (1 is decode_b1, 32 is decode_b32)")
            xw = [bf16(I.activations(I.DECODE_WIDTHS, m.matrix_id, mw, m.k)) for m in layer]
            yw = [torch.empty((mw, m.n), dtype=torch.bfloat16, device=dev) for m in layer]
            calls = [B.gemm_batched_prepared([(packed[cp][j], m.n, m.k, I.TENSOR_SCALE, xw[j], yw[j])
                                              for j, m in enumerate(layer)], ws=ws_split)
                     for cp in range(dense_copies)]
            wbytes = sum(m.n * m.k * 9 // 16 + 2 * mw * m.k + 2 * mw * m.n for m in layer)
            extra_rows[r] = (calls, dense_copies, yw, wbytes, 2.0 * mw * sum(m.n * m.k for m in layer))
    if "head_b1" in rows:
        hc, hs = I.nvfp4_matrix(I.OUTPUT_HEAD, I.HEAD.matrix_id, I.HEAD.n, I.HEAD.k)
        head_packed = B.pack(u8(hc), u8(hs))
        del hc, hs
        xh = bf16(I.activations(I.OUTPUT_HEAD, 0, 1, I.HEAD.k)[0])
        yh = torch.empty(I.HEAD.n, dtype=torch.float32, device=dev)
        hbytes = I.HEAD.n * I.HEAD.k * 9 // 16 + 2 * I.HEAD.k + 4 * I.HEAD.n
        extra_rows["head_b1"] = ([B.gemv_batched_prepared([(head_packed, I.HEAD.n, I.HEAD.k, I.TENSOR_SCALE, xh, yh)],
                                                          ws=ws_split)], 1, [yh], hbytes, 2.0 * I.HEAD.n * I.HEAD.k)

    # ---- the single 1024 x 1024 GEMV (batch 1), one launch per step; 1800
    # copies of its 589,824 packed bytes (1.06 GB) so that no copy is read
    # twice within 1800 steps ----------------------------------------------
    g1k_copies, g1k_calls = 1800, []
    g1k_bytes = B.packed_bytes(1024, 1024) + 2 * 1024 + 4 * 1024
    if "gemv_1k" in rows:
        c, s_ = I.nvfp4_matrix(I.GEMV_1K, 0, 1024, 1024)
        g1k_p0 = B.pack(u8(c), u8(s_))
        g1k_x = bf16(I.activations(I.GEMV_1K, 0, 1, 1024)[0])
        g1k_y = torch.empty(1024, dtype=torch.float32, device=dev)
        g1k_ws = B.workspace(B.gemv_workspace_bytes(1024, 1024), dev)
        for cp in range(g1k_copies):
            pcp = g1k_p0 if cp == 0 else g1k_p0.clone()
            g1k_calls.append(B.gemv_batched_prepared([(pcp, 1024, 1024, I.TENSOR_SCALE, g1k_x, g1k_y)], ws=g1k_ws))

    def pre_items(cp):
        return [(pre_packed[cp][j], mat.n, mat.k, I.TENSOR_SCALE, pre_x[j], pre_y[j]) for j, mat in enumerate(pre)]

    pre_calls = []
    if "prefill" in rows:
        # The three prefill products share one stream-K launch; its workspace
        # (counters + cut-tile partial sums) is larger than the decode rows'.
        need = B.gemm_batched_workspace_bytes(pre_items(0), 512)
        if need > ws_split.numel():
            ws_split = B.workspace(need, dev)
        pre_calls = [B.gemm_batched_prepared(pre_items(cp), ws=ws_split) for cp in range(pre_copies)]

    def row_pre(cp):
        pre_calls[cp]()

    # ---- optional: the same three prefill products as W4A4 (both operands in
    # MX FP4 on the FP4 matrix cores; an approximation of the NVFP4 product) ---
    w4_mx, w4_x, w4_y = [[None] * len(pre) for _ in range(2)], [], []
    if "prefill_w4a4" in rows:
        for j, mat in enumerate(pre):
            c, s_ = I.nvfp4_matrix(I.PREFILL_512, mat.matrix_id, mat.n, mat.k)
            m0 = B.mx_pack(u8(c), u8(s_))
            w4_mx[0][j], w4_mx[1][j] = m0, m0.clone()
            w4_x.append(bf16(I.activations(I.PREFILL_512, mat.matrix_id, 512, mat.k)))
            w4_y.append(torch.empty((512, mat.n), dtype=torch.bfloat16, device=dev))
        w4_items = [[(w4_mx[cp][j], mat.n, mat.k, I.TENSOR_SCALE, w4_x[j], w4_y[j]) for j, mat in enumerate(pre)]
                    for cp in range(2)]
        ws_w4 = B.workspace(B.w4a4_batched_workspace_bytes(w4_items[0], 512), dev, kind="w4a4")
        w4_calls = [B.w4a4_batched_prepared(w4_items[cp], ws=ws_w4) for cp in range(2)]

    def row_w4(cp):
        w4_calls[cp]()

    # ---- optional: the NVFP4 quantiser over the layer's five matrices (bf16 in) ----
    q_w, q_out, q_bytes = [], [], 0
    if "quantize" in rows:
        gen = torch.Generator(device=dev)
        gen.manual_seed(1234)
        ws_q = B.workspace(B.quantize_workspace_bytes(), dev, kind="quantize")
        for m in layer:
            w = (torch.randn((m.n, m.k), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            q_w.append(w)
            q_out.append((torch.empty((m.n, m.k // 2), dtype=torch.uint8, device=dev),
                          torch.empty((m.n, m.k // 16), dtype=torch.uint8, device=dev),
                          torch.empty(1, dtype=torch.float32, device=dev)))
            q_bytes += m.n * m.k * 2 + m.n * m.k * 9 // 16 + 4   # bf16 read once, codes + scales + s_t written

    def row_q(cp):
        for w, (c, sc, st) in zip(q_w, q_out):
            B.quantize(w, c, sc, st, ws=ws_q)

    # Row order within a step: the compute-bound prefill first, the decode
    # rows after the memory-bound MoE.  A sustained matrix-core burst lowers
    # the clocks for tens of microseconds, and a GEMV launched straight after
    # the prefill runs ~15% slower (44 vs 38.5 us) -- a back-to-back pairing
    # that a decode loop does not have.
    plan_all = {
        "prefill": ("prefill", row_pre, pre_copies, lambda i: i % pre_copies, pre_y),
        "moe": ("moe", run_moe, 2 * moe_routings, lambda i: i % (2 * moe_routings), None),
        "gemv_1k": ("gemv_1k", lambda cp: g1k_calls[cp](), g1k_copies, lambda i: i % g1k_copies,
                    [g1k_y] if g1k_calls else None),
        "decode_b32": ("decode_b32", row_b32, dense_copies, lambda i: (2 * i + 1) % dense_copies, y32),
        "decode_b1": ("decode_b1", row_b1, dense_copies, lambda i: (2 * i) % dense_copies, y1),
        "quantize": ("quantize", row_q, 1, lambda i: 0, [c for c, _, _ in q_out]),
        "moe_stream": ("moe_stream", run_moe_stream, 64, lambda i: i % 64, None),
        "prefill_w4a4": ("prefill_w4a4", row_w4, 2, lambda i: i % 2, w4_y),
    }
    for r, (calls, ncp, outs, _, _) in extra_rows.items():
        plan_all[r] = (r, (lambda cp, c=calls: c[cp]()), ncp, (lambda i, n_=ncp: (2 * i + 1) % n_), outs)
    order = args.order.split(",") + [r for r in plan_all if r not in args.order.split(",")]
    plan = [plan_all[r] for r in order if r in rows]   # (row name, callable(copy), copies, copy for step i, outputs)
    # The rows that read the dense layer's weights take its copies in turn
    # (j-th such row of step i: copy (i * D + j) % 4), so a copy is read again
    # only after three others (558 MB) have passed through the 256 MB MALL.
    dense_names = [p_[0] for p_ in plan if p_[0] in ("decode_b1", "decode_b32") or p_[0].startswith("decode_m")]
    nd = len(dense_names)
    plan = [(nm, fn, ncp, (lambda i, j=dense_names.index(nm): (i * nd + j) % dense_copies) if nm in dense_names
             else pick, outs) for nm, fn, ncp, pick, outs in plan]
    # Eager reference outputs (copy 0), then (--graphs) capture.
    eager = {}
    for name, fn, ncp, _, outs in plan:
        fn(0)
        torch.cuda.synchronize()
        if outs is None:
            outs = [moe_out["y"]] if name == "moe" else [stream_state["out"]["y"]]
        eager[name] = [o.clone() for o in outs]
    graphs = {}
    if args.graphs and "moe_stream" in rows:
        raise SystemExit("--graphs: the moe_stream row synchronises with the host inside each call; run it without --graphs")
    if args.graphs:
        for name, fn, ncp, _, _ in plan:
            for cp in range(ncp):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    fn(cp)
                graphs[(name, cp)] = g
        torch.cuda.synchronize()
        # Every graph's replay must reproduce the eager result bit for bit.
        for name, fn, ncp, _, outs in plan:
            for cp in range(ncp):
                graphs[(name, cp)].replay()
                torch.cuda.synchronize()
                got = [o for o in outs] if outs is not None else [moe_out["y"]]
                for a_, b_ in zip(got, eager[name]):
                    if not torch.equal(a_.view(torch.uint8), b_.view(torch.uint8)):
                        raise SystemExit(f"graph replay of {name} (copy {cp}) differs from the eager run")
        log(f"captured {len(graphs)} graphs; replays match the eager runs")

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    hev = HipTimingEvents()
    stream = torch.cuda.current_stream().cuda_stream

    def step(i, timed):
        marks = {}
        for name, fn, ncp, pick, _ in plan:
            cp = pick(args.warmup + i if timed else i)
            a = hev.new()
            b = hev.new()
            hev.record(a, stream)
            if args.graphs:
                graphs[(name, cp)].replay()
            else:
                fn(cp)
            hev.record(b, stream)
            marks[name] = (a, b)
        return marks

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    log("warmup done")
    all_marks = []
    t0 = ev(); t1 = ev()
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        all_marks.append(step(i, True))
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    seg, seg_med = {}, {}
    for name in all_marks[0]:
        per = [hev.elapsed_ms(m[name][0], m[name][1]) for m in all_marks]
        seg[name] = sum(per) / args.steps
        seg_med[name] = statistics.median(per)
    hev.close()
    picks = {name: [pick(args.warmup + i) for i in range(args.steps)] for name, _, _, pick, _ in plan}
    ceil = {} if args.no_probes else probe_ceilings(dev, layer_weight_bytes=b1_weight_bytes)
    gemv_launches = args.steps if "decode_b1" in seg else 0   # one batched launch per step
    gemv_ms = seg.get("decode_b1", 0.0) * args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step; segments (ms): "
        + ", ".join(f"{k}={v:.4f}" for k, v in seg.items()))

    # ---- per-row results --------------------------------------------------
    result_rows = {}
    read_ceiling = ceil.get("hbm_read_GB/s")

    def hbm_row(gbs):
        d = {"frac_hbm": gbs / HBM_PEAK_GBS}
        if read_ceiling:
            d["frac_probe_read"] = gbs / read_ceiling
        return d

    if "decode_b1" in seg:
        s = seg["decode_b1"] * 1e-3
        result_rows["decode_b1"] = {"GB/s": b1_bytes / s / 1e9, "weight_GB/s": b1_weight_bytes / s / 1e9,
                                    "us": s * 1e6, "us_median": seg_med["decode_b1"] * 1e3,
                                    **hbm_row(b1_bytes / s / 1e9),
                                    "equiv_tok_s": b1_bytes / s / MODEL_27B_BYTES_PER_TOKEN,
                                    "inputs_sha256": b1_inputs.hexdigest()}
    if "decode_b32" in seg:
        s = seg["decode_b32"] * 1e-3
        result_rows["decode_b32"] = {"GB/s": b32_bytes / s / 1e9, "TFLOP/s": b32_flops / s / 1e12, "us": s * 1e6,
                                     "us_median": seg_med["decode_b32"] * 1e3, **hbm_row(b32_bytes / s / 1e9),
                                     "equiv_tok_s": 32 * b32_bytes / s / MODEL_27B_BYTES_PER_TOKEN}
    if "gemv_1k" in seg:
        s = seg["gemv_1k"] * 1e-3
        result_rows["gemv_1k"] = {"us": s * 1e6, "us_median": seg_med["gemv_1k"] * 1e3, "GB/s": g1k_bytes / s / 1e9,
                                  "algorithmic_bytes": g1k_bytes, **hbm_row(g1k_bytes / s / 1e9),
                                  "note": "latency-bound: 0.6 MB per launch; the 75 % bar applies to the layer"}
    if "moe" in seg:
        s = seg["moe"] * 1e-3
        moe_bytes = sum(moe_call_bytes[cp] for cp in picks["moe"]) / args.steps
        active = sum(moe_call_active[cp] for cp in picks["moe"]) / args.steps
        counts = moe_out["expert_counts"].cpu().numpy()
        result_rows["moe"] = {"GB/s": moe_bytes / s / 1e9, "us": s * 1e6, "us_median": seg_med["moe"] * 1e3,
                              "routings": moe_routings, "active_experts_mean": active,
                              "algorithmic_bytes_mean": moe_bytes, **hbm_row(moe_bytes / s / 1e9),
                              "layer_tok_s": shape.tokens / s, "max_tokens_per_expert_last": int(counts.max())}
    bf16_ceiling = ceil.get("mfma_bf16_TFLOP/s")
    if "prefill" in seg:
        s = seg["prefill"] * 1e-3
        tf = pre_flops / s / 1e12
        result_rows["prefill"] = {"TFLOP/s": tf, "us": s * 1e6, "us_median": seg_med["prefill"] * 1e3,
                                  "frac_mfma_bf16": tf / MFMA_BF16_PEAK_TFLOPS,
                                  **({"frac_probe_mfma_bf16": tf / bf16_ceiling} if bf16_ceiling else {}),
                                  "GB/s": pre_bytes / s / 1e9, "equiv_tok_s": pre_flops / s / (2 * 27e9)}

    if "prefill_w4a4" in seg:
        s = seg["prefill_w4a4"] * 1e-3
        tf = pre_flops / s / 1e12
        fp4_ceiling = ceil.get("mfma_fp4_TFLOP/s")
        result_rows["prefill_w4a4"] = {"TFLOP/s": tf, "us": s * 1e6, "us_median": seg_med["prefill_w4a4"] * 1e3,
                                       "frac_mfma_fp4": tf / 10100.0,
                                       **({"frac_probe_mfma_fp4": tf / fp4_ceiling} if fp4_ceiling else {}),
                                       "frac_mfma_bf16": tf / MFMA_BF16_PEAK_TFLOPS}
    if "moe_stream" in seg:
        s = seg["moe_stream"] * 1e-3
        st_timed = stream_state["stats"][-args.steps:]
        fetched = sum(x["fetched"] for x in st_timed) / len(st_timed)
        active = sum(x["active"] for x in st_timed) / len(st_timed)
        pcie = sum(x["bytes"] for x in st_timed) / len(st_timed)
        result_rows["moe_stream"] = {"us": s * 1e6, "cache_slots": 64, "active_experts": active,
                                     "fetched_experts": fetched, "hit_rate": 1.0 - fetched / active,
                                     "copied_bytes": pcie, "copied_GB/s": pcie / s / 1e9,
                                     "layer_tok_s": shape.tokens / s}
    for r, (_, _, _, nbytes, flops) in extra_rows.items():
        s = seg[r] * 1e-3
        result_rows[r] = {"GB/s": nbytes / s / 1e9, "TFLOP/s": flops / s / 1e12, "us": s * 1e6,
                          "us_median": seg_med[r] * 1e3, "algorithmic_bytes": nbytes, **hbm_row(nbytes / s / 1e9)}
    if "quantize" in seg:
        s = seg["quantize"] * 1e-3
        result_rows["quantize"] = {"GB/s": q_bytes / s / 1e9, "us": s * 1e6, "us_median": seg_med["quantize"] * 1e3,
                                   "algorithmic_bytes": q_bytes, **hbm_row(q_bytes / s / 1e9),
                                   "weights_per_s": sum(m.n * m.k for m in layer) / s}

    roofline = None
    if gemv_launches:
        bytes_per_launch = b1_bytes * args.steps / gemv_launches
        avg_launch_s = gemv_ms * 1e-3 / gemv_launches
        achieved = bytes_per_launch / avg_launch_s / 1e9
        roofline = {"kernel": "gemv_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": gemv_traffic(), "avg_launch_us": round(avg_launch_s * 1e6, 3),
                    "median_launch_us": round(seg_med["decode_b1"] * 1e3, 3),
                    "bytes_per_launch": int(bytes_per_launch)}
        if read_ceiling:
            roofline["probe_ceiling"] = round(read_ceiling, 1)
            roofline["frac_probe"] = round(achieved / read_ceiling, 4)

    cpu = None
    if not args.no_cpu_baseline and "decode_b1" in rows:
        cpu = cpu_baseline(args.cpu_seconds)

    value = result_rows.get("decode_b1", {}).get("GB/s")
    out = {
        "metric": "NVFP4 GEMV weight GB/s (% HBM peak) at B=1/32; MoE GB/s; prefill TFLOP/s",
        "value": round(value, 1) if value else None,
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 weights x bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded NVFP4 codes/scales, N(0,1) bf16 activations, Zipf-biased router logits)",
        "config": {"workload": "27B-class dense decode layer, batch 1: NVFP4 GEMVs gate/up 5120->17408, "
                               "down 17408->5120, QKV 5120->7168, O 5120->5120",
                   "batch": 1, "algorithmic_bytes_per_step": b1_bytes},
        "rows": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                 for k, v in result_rows.items()},
        "roofline": roofline,
        "ceilings": {k: round(v, 2) for k, v in ceil.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def gemv_traffic():
    """HBM bytes per gemv_kernel launch from the committed rocprofv3 counter
    summary, or None when the kernel's sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_kernel_layer_b1_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", " ", "#")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("gemv.hip", "device_common.h", "launchers.h"):
        with open(os.path.join(ROOT, "bit_quantized_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("sources_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def probe_ceilings(dev, layer_weight_bytes):
    """What this machine sustains, measured by libnvfp4_probes.so after the timed
    steps (median of timed launches, HIP events on the launch stream):
    a streaming read of the layer's packed-weight bytes in 9216-byte tiles
    (four rotating copies, so no copy is re-read from the 256 MB MALL), and the
    bf16 and FP4 matrix instructions with random operands."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "bit_quantized_decode_amd", "libnvfp4_probes.so")
    if not os.path.exists(path):
        log("ceiling probes skipped: libnvfp4_probes.so is not built")
        return {}
    L = ctypes.CDLL(path)
    P, i64, u32, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint, ctypes.c_int
    L.probe_hbm_read.argtypes = [P, i64, u32, P, P]
    L.probe_mfma_bf16.argtypes = [P, I32, I32, u32, P, P]
    L.probe_mfma_fp4.argtypes = [P, I32, I32, u32, P, P]
    magic = 0x9E3779B9
    stream = torch.cuda.current_stream().cuda_stream
    hev = HipTimingEvents()

    def timed(fn, reps):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        marks = []
        for i in range(reps):
            a, b = hev.new(), hev.new()
            hev.record(a, stream)
            fn(i)
            hev.record(b, stream)
            marks.append((a, b))
        torch.cuda.synchronize()
        return statistics.median(hev.elapsed_ms(a, b) for a, b in marks) * 1e-3

    nbytes = layer_weight_bytes
    bufs = [torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev) for _ in range(4)]
    sink = torch.zeros(256 * 4096, dtype=torch.int32, device=dev)

    def read(i):
        if L.probe_hbm_read(bufs[i % 4].data_ptr(), nbytes, magic, sink.data_ptr(), stream) != 0:
            raise RuntimeError("probe_hbm_read refused its arguments or failed to launch")
    t_read = timed(read, 20)
    del bufs
    # Launch shapes that gave each instruction its best sustained rate on
    # this box (a sweep of 256..2048 workgroups): bf16 2048 x 128
    # iterations, FP4 256 x 1024; operands N(0,1) bf16 / random FP4 codes.
    rnd_bf16 = torch.randn(256 * 6 * 1024 // 2, device=dev).to(torch.bfloat16)
    rnd_fp4 = torch.randint(0, 256, (256 * 6 * 1024,), dtype=torch.uint8, device=dev)

    def mfma(fn, buf, wgs, iters):
        def run(i):
            if fn(buf.data_ptr(), wgs, iters, magic, sink.data_ptr(), stream) != 0:
                raise RuntimeError("matrix-core probe refused its arguments or failed to launch")
        return run
    t_bf16 = timed(mfma(L.probe_mfma_bf16, rnd_bf16, 2048, 128), 10)
    t_fp4 = timed(mfma(L.probe_mfma_fp4, rnd_fp4, 256, 1024), 10)
    hev.close()
    flops = 2048 * 4 * 16 * 128 * 32768          # the same for both launches, in units of a bf16 instruction
    out = {"hbm_read_GB/s": nbytes / t_read / 1e9, "hbm_read_us": t_read * 1e6,
           "mfma_bf16_TFLOP/s": flops / t_bf16 / 1e12, "mfma_fp4_TFLOP/s": 4 * flops / t_fp4 / 1e12}
    log("ceilings: " + ", ".join(f"{k}={v:.1f}" for k, v in out.items()))
    return out


def cpu_baseline(target_s):
    """The oracle, untuned, on this host's cores: the batch-1 layer's five GEMVs, repeated
    until about `target_s` seconds of work, reported in the same unit (GB/s); then, on
    one thread, one pass of the layer and the 1024 x 1024 GEMV repeated for about a second."""
    import numpy as np

    import oracle
    from bit_quantized_decode_amd import inputs as I
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    mats = [(m, *I.nvfp4_matrix(I.DECODE_B1, m.matrix_id, m.n, m.k)) for m in I.DENSE_LAYER]
    xs = [I.activations(I.DECODE_B1, m.matrix_id, 1, m.k) for m in I.DENSE_LAYER]
    h = hashlib.sha256()
    for (m, c, s), x in zip(mats, xs):
        for a_ in (c, s, x[0]):
            h.update(np.ascontiguousarray(a_).tobytes())
    layer_bytes = sum(m.n * m.k * 9 // 16 + 2 * m.k + 4 * m.n for m in I.DENSE_LAYER)
    layer_flops = 2 * sum(m.n * m.k for m in I.DENSE_LAYER)
    oracle.gemm(mats[4][1], mats[4][2], I.TENSOR_SCALE, xs[4], nthreads=cores)  # warm-up
    reps, t0 = 0, time.time()
    while True:
        for (m, c, s), x in zip(mats, xs):
            oracle.gemm(c, s, I.TENSOR_SCALE, x, nthreads=cores)
        reps += 1
        if time.time() - t0 >= target_s or reps >= 200:
            break
    dt = time.time() - t0
    # One thread: one pass of the layer, and the 1024 x 1024 GEMV for about a second.
    t1 = time.time()
    for (m, c, s), x in zip(mats, xs):
        oracle.gemm(c, s, I.TENSOR_SCALE, x, nthreads=1)
    dt1 = time.time() - t1
    c0, s0 = I.nvfp4_matrix(I.GEMV_1K, 0, 1024, 1024)
    x0 = I.activations(I.GEMV_1K, 0, 1, 1024)
    oracle.gemm(c0, s0, I.TENSOR_SCALE, x0, nthreads=1)
    r0, t2 = 0, time.time()
    while time.time() - t2 < 1.0:
        oracle.gemm(c0, s0, I.TENSOR_SCALE, x0, nthreads=1)
        r0 += 1
    dt0 = (time.time() - t2) / r0
    log(f"cpu baseline ({model}): {reps} passes of the layer in {dt:.1f}s on {cores} threads; one thread: "
        f"layer {dt1:.2f}s, 1024x1024 GEMV {dt0 * 1e3:.2f} ms")
    return {"value": round(reps * layer_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} full passes of the batch-1 layer (5 GEMVs, 330,301,440 weights) in fp64, "
                      f"{dt:.1f} s wall; then one pass on one thread and the 1024 x 1024 GEMV on one thread",
            "cpu_model": model, "gflops_fp64": round(reps * layer_flops / dt / 1e9, 3),
            "single_thread": {"layer_b1_s": round(dt1, 3), "layer_b1_GB/s": round(layer_bytes / dt1 / 1e9, 4),
                              "layer_b1_gflops_fp64": round(layer_flops / dt1 / 1e9, 3),
                              "gemv_1k_ms": round(dt0 * 1e3, 3),
                              "gemv_1k_gflops_fp64": round(2 * 1024 * 1024 / dt0 / 1e9, 3)},
            "inputs_sha256": h.hexdigest()}


if __name__ == "__main__":
    main()
