#!/usr/bin/env python3
"""Benchmark of the QLoRA NF4 hot path on one MI355X.

One step is one pass of every stage of the path over one batch of seeded
synthetic input at Llama-7B shapes:

  attention projection 4096 x 4096 (W ~ N(0, 0.02), 0.1% outliers x20, r=16):
      nf4_quantize (fp32 in) + nf4_double_quant, nf4_dequantize (bf16 out),
      qlora_linear_fwd at T = 1 and T = 16 (dequant-GEMV)
  MLP gate / up 11008 x 4096 and down 4096 x 11008 (W ~ 0.02 t(5), r=16):
      nf4_quantize + nf4_double_quant of each,
      qlora_linear_fwd at T = 1024 (dequant-in-LDS MFMA GEMM + LoRA),
      qlora_linear_bwd at T = 1024 (dX, dA, dB)

The reported value is the step's roofline-ideal time (each stage's
algorithmic bytes at 8 TB/s or flops at 2.5 PFLOP/s dense bf16) divided by
the measured step time, in percent. Per-stage throughput (GB/s, TFLOP/s)
measured with cold caches is in "rows"; "roofline" is the dominant kernel
timed with HIP events inside the timed steps; "cpu_baseline" is the CPU
oracle on a bounded sample of the same step.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12  # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15  # flop/s, MI355X dense bf16 MFMA

BPW_QUANT_F32 = 4 + 0.5 + 4 / 64  # read fp32, write code nibble + absmax share
BPW_QUANT_BF16 = 2 + 0.5 + 4 / 64
BPW_DQ = (4 + 4 + 1 + 4 / 256) / 64  # absmax read twice, c8 + scale written
BPW_DEQUANT = 0.5 + 1 / 64 + 4 / (64 * 256) + 2  # codes + c8 + scale in, bf16 out
BPW_PACKED = 0.5 + 1 / 64 + 4 / (64 * 256)  # what a matmul reads per weight


def gemv_bytes(N, K, T, r):
    return BPW_PACKED * N * K + 2 * T * K + 2 * T * N + 2 * r * (K + N)


def fwd_flops(N, K, T, r):
    return 2 * T * N * K + 2 * T * K * r + 2 * T * r * N


def dx_flops(N, K, T, r):
    return 2 * T * N * K + 2 * T * N * r + 2 * T * r * K


def lora_grad_bytes(N, K, T, r):
    # dA = G^T X reads X and writes dA; dB = s dY^T U reads dY and writes dB
    return 2 * T * K + 2 * T * N + 4 * T * r * 2 + 4 * r * (K + N)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-stage cold-cache measurements")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as eager serial launches (default: replays of the step captured in a HIP "
                         "graph with its independent parts on two streams; the per-kernel timers always come from "
                         "an eager serial pass, since events inside a replayed graph give no elapsed times)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--cpu-suite", action="store_true",
                    help="host only: the oracle on 7B stack layer 0 (x32 extrapolated) and one 65B-shaped matrix of "
                         "each shape at T = 4096, one JSON line")
    ap.add_argument("--fwd-u", action="store_true",
                    help="instead of the step: the 7B gate forward at T = 1024, r = 16 with U inside the GEMM "
                         "launch and with a separate projection launch first (eager calls and graph replays), "
                         "one JSON line")
    ap.add_argument("--bwd-g", action="store_true",
                    help="instead of the step: the 7B down backward at T = 1024, r = 16 with G inside the dX GEMM "
                         "launch and with a separate projection launch first, one JSON line")
    ap.add_argument("--quantize-dq", action="store_true",
                    help="instead of the step: nf4_quantize_dq against nf4_quantize + nf4_double_quant at the 7B "
                         "weight shapes, fp32 and bf16 input, one JSON line")
    ap.add_argument("--grouped", action="store_true",
                    help="instead of the step: layers that read the same X (7B q/k/v, gate/up; r = 16) through "
                         "qlora_linear_fwd_group / qlora_linear_bwd_group against one call per layer, forward "
                         "and dX, T = 256 .. 4096, one JSON line")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the step: the wider measurement set (32-layer 7B stack, 65B linears, "
                         "a GEMV pass over the stack, residency, torch.matmul context), one JSON line")
    ap.add_argument("--suite-stack", action="store_true",
                    help="instead of the step: only the 7B stack passes of --suite (quantize, dequantize, decode "
                         "GEMV), e.g. under a kernel trace for the kernels' own durations, one JSON line")
    return ap.parse_args()


class Inputs:
    """Seeded synthetic inputs of one step, resident on the GPU."""

    def __init__(self, torch, workloads):
        attn = workloads.attn_proj_7b(T=16, seed=1)
        self.attn = attn
        self.W_attn = attn.W.cuda()
        self.X1 = attn.X[:1].contiguous().cuda()
        self.X16 = attn.X.cuda()
        self.A_attn, self.B_attn = attn.A.cuda(), attn.B.cuda()
        self.s_attn = attn.scale
        self.mlp = [workloads.mlp_7b(w, T=1024, seed=2) for w in ("gate", "up", "down")]
        # gate and up read the same activations, the MLP's input, as in the
        # model: their input gradients add up, in one grouped backward
        self.mlp[1].X = self.mlp[0].X
        self.mlp_dev = []
        for c in self.mlp:
            self.mlp_dev.append(dict(W=c.W.cuda(), X=c.X.cuda(), dY=c.dY.cuda(), A=c.A.cuda(), B=c.B.cuda(),
                                     s=c.scale, r=c.r, N=c.W.shape[0], K=c.W.shape[1], T=c.X.shape[0]))


def run_step(qn, inp):
    """One pass of the whole path. Returns nothing; results stay on device.
    The MLP: forward of gate, up and down; backward of down, then of gate
    and up together (they read the same X: one grouped call gives their
    summed dX and each one's dA, dB)."""
    wa = qn.quantize_weight(inp.W_attn)
    qn.nf4_dequantize(wa)
    wm = [qn.quantize_weight(m["W"]) for m in inp.mlp_dev]
    # the decode GEMVs run after the 0.5 GB of MLP quantization has streamed
    # through the caches, so the attention weight is read from HBM
    qn.qlora_linear_fwd(wa, inp.X1, inp.A_attn, inp.B_attn, inp.s_attn)
    qn.qlora_linear_fwd(wa, inp.X16, inp.A_attn, inp.B_attn, inp.s_attn)
    Us = [qn.qlora_linear_fwd(w, m["X"], m["A"], m["B"], m["s"])[1] for w, m in zip(wm, inp.mlp_dev)]
    gate, up, down = inp.mlp_dev
    qn.qlora_linear_bwd(wm[2], down["X"], down["dY"], down["A"], down["B"], down["s"], U=Us[2])
    qn.qlora_linear_bwd_group(wm[:2], gate["X"], [gate["dY"], up["dY"]], [gate["A"], up["A"]], [gate["B"], up["B"]],
                              gate["s"], Us=Us[:2])


def run_step_streams(torch, qn, inp, side):
    """The same step with its independent parts on two streams (both at the
    default priority): the side stream quantizes each MLP weight just ahead
    of its forward pass and then runs the attention weight's quantization,
    dequantization and decode GEMVs, while the current stream runs the MLP
    forward and backward passes, each waiting only for its own weight. The
    172-tile GEMMs leave a third of the CUs idle, which the HBM-bound side
    work fills. Same kernels, same inputs, same results as run_step.
    Unlike run_step, the decode GEMVs here follow the attention weight's own
    quantization and dequantization, so they read a cache-warm weight (8.4
    MB of a 256 MB last-level cache); moving them behind the MLP weights'
    quantization, as in run_step, made the replayed step 8 % slower (the
    GEMVs then wait for CUs behind the split-K GEMMs).
    Each backward is two calls of the library: dX on the current stream, and
    dA, dB (the adapter gradients need G^T, X, dY and the forward's U, not
    dX) on the side stream once the forward is done, so the gradient kernel
    overlaps the next GEMM instead of following the dX GEMM. The side call
    forms G again with its own projection (the ideal step counts it once);
    the outputs are those of run_step, bit for bit (measured 3-4 % faster
    per replayed step than one backward call). Gate and up take their
    backward together (one grouped dX call, their dA and dB in one grouped
    side call), after down's, as in run_step."""
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    ready = []
    wm = []
    with torch.cuda.stream(side):
        for m in inp.mlp_dev:
            wm.append(qn.quantize_weight(m["W"]))
            ev = torch.cuda.Event()
            ev.record(side)
            ready.append(ev)
        wa = qn.quantize_weight(inp.W_attn)
        qn.nf4_dequantize(wa)
        qn.qlora_linear_fwd(wa, inp.X1, inp.A_attn, inp.B_attn, inp.s_attn)
        qn.qlora_linear_fwd(wa, inp.X16, inp.A_attn, inp.B_attn, inp.s_attn)
    outs, fw = [], []
    for w, m, ev in zip(wm, inp.mlp_dev, ready):
        main.wait_event(ev)
        Y, U = qn.qlora_linear_fwd(w, m["X"], m["A"], m["B"], m["s"])
        done = torch.cuda.Event()
        done.record(main)
        fw.append((Y, U, done))
    gate, up, down = inp.mlp_dev
    (Yg, Ug, _), (Yu, Uu, done_gu), (Yd, Ud, done_d) = fw
    dX, _, _ = qn.qlora_linear_bwd(wm[2], down["X"], down["dY"], down["A"], down["B"], down["s"], U=Ud, need_da=False,
                                   need_db=False)
    side.wait_event(done_d)
    with torch.cuda.stream(side):
        _, dA, dB = qn.qlora_linear_bwd(wm[2], down["X"], down["dY"], down["A"], down["B"], down["s"], U=Ud,
                                        need_dx=False)
    grp = (wm[:2], gate["X"], [gate["dY"], up["dY"]], [gate["A"], up["A"]], [gate["B"], up["B"]], gate["s"])
    dXgu, _, _ = qn.qlora_linear_bwd_group(*grp, Us=[Ug, Uu], need_da=False, need_db=False)
    side.wait_event(done_gu)
    with torch.cuda.stream(side):
        _, dAs, dBs = qn.qlora_linear_bwd_group(*grp, Us=[Ug, Uu], need_dx=False)
    outs = [(Yg, Ug, Yu, Uu, dXgu, dAs[0], dBs[0], dAs[1], dBs[1]), (Yd, Ud, dX, dA, dB)]
    main.wait_stream(side)
    return outs


def ideal_step_seconds(inp):
    """Roofline-ideal time of one step, stage by stage."""
    t = 0.0
    na = 4096 * 4096
    t += (BPW_QUANT_F32 + BPW_DQ) * na / PEAK_HBM
    t += BPW_DEQUANT * na / PEAK_HBM
    r = inp.attn.r
    t += gemv_bytes(4096, 4096, 1, r) / PEAK_HBM + gemv_bytes(4096, 4096, 16, r) / PEAK_HBM
    for m in inp.mlp_dev:
        N, K, T, r = m["N"], m["K"], m["T"], m["r"]
        t += (BPW_QUANT_F32 + BPW_DQ) * N * K / PEAK_HBM
        t += fwd_flops(N, K, T, r) / PEAK_BF16
        t += dx_flops(N, K, T, r) / PEAK_BF16
        t += max(lora_grad_bytes(N, K, T, r) / PEAK_HBM, 4.0 * T * r * (N + K) / PEAK_BF16)
    return t


KERNELS = {
    "quantize": 1,
    "dq_encode": 2,
    "dequantize": 3,
    "gemv": 4,
    "gemm_fwd": 5,
    "gemm_dx": 6,
    "lora_grad": 7,
}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gemm_llama7b_mlp.json")


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` ("gemm_fwd" or "gemm_dx") from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when there is
    none or the GEMM sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
        entry = d["kernels"].get(kernel)
        if entry is None:
            return None
        h = hashlib.sha256()
        for src in d["source_files"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        return entry["bytes_per_launch"] if h.hexdigest() == d["source_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def per_launch_work(qn, inp):
    """Algorithmic work of one launch of each kernel in the step, averaged
    over the step's launches of it (the per-kernel timers come from eager
    steps: there U = X A^T runs inside the forward GEMM launch, and
    G = s dY B inside the dX GEMM launch, where the library says so, else in
    a separate projection launch). The dX of gate and up is one grouped
    launch (its G projections run apart)."""
    fwd, dx = [], []
    for m in inp.mlp_dev:
        N, K, T, r = m["N"], m["K"], m["T"], m["r"]
        u_in = qn.lib.qlora_linear_fwd_u_in_launch(N, K, T, r)
        fwd.append(fwd_flops(N, K, T, r) - (0 if u_in else 2 * T * K * r))
    gate, up, down = inp.mlp_dev
    dx.append(sum(dx_flops(m["N"], m["K"], m["T"], m["r"]) - 2 * m["T"] * m["N"] * m["r"] for m in (gate, up)))
    N, K, T, r = down["N"], down["K"], down["T"], down["r"]
    dx.append(dx_flops(N, K, T, r) - (0 if qn.lib.qlora_linear_bwd_g_in_launch(N, K, T, r) else 2 * T * N * r))
    return {
        "gemm_fwd": ("mfma", sum(fwd) / len(fwd), "TFLOP/s"),
        "gemm_dx": ("mfma", sum(dx) / len(dx), "TFLOP/s"),
    }


def measure_rows(torch, qn, inp, flush):
    """Cold-cache throughput of each stage: 5 untimed warm-up calls, then 20
    timed ones, each after a 1 GiB buffer is overwritten (L2 and the 256 MB
    last-level cache hold none of the inputs); the time of a call is the
    library's HIP-event timer of that stage's main kernel, recorded on the
    launch stream. Rows give the median (us) and the minimum (us_min); the
    throughput is from the median."""
    rows = {}
    reps = 20
    mins = {}

    def timed(kid, fn):
        t = qn.KernelTimer(kid)
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            flush()
            t.arm()
            fn()
            torch.cuda.synchronize()
            n, ms = t.read()
            t.disarm()
            ts.append(ms / max(n, 1) / 1e3)
        ts.sort()
        timed.last_min = ts[0]
        return ts[len(ts) // 2]

    na = 4096 * 4096
    W = inp.W_attn
    sec = timed(1, lambda: qn.nf4_quantize(W))
    rows["quantize_f32_4096x4096"] = _hbm_row(BPW_QUANT_F32 * na, sec, timed.last_min)
    Wb = W.to(torch.bfloat16)
    sec = timed(1, lambda: qn.nf4_quantize(Wb))
    rows["quantize_bf16_4096x4096"] = _hbm_row(BPW_QUANT_BF16 * na, sec, timed.last_min)
    Wm = inp.mlp_dev[0]["W"]
    sec = timed(1, lambda: qn.nf4_quantize(Wm))
    rows["quantize_f32_11008x4096"] = _hbm_row(BPW_QUANT_F32 * Wm.numel(), sec, timed.last_min)
    Wmb = Wm.to(torch.bfloat16)
    sec = timed(1, lambda: qn.nf4_quantize(Wmb))
    rows["quantize_bf16_11008x4096"] = _hbm_row(BPW_QUANT_BF16 * Wm.numel(), sec, timed.last_min)
    del Wmb
    _, absmax = qn.nf4_quantize(W)
    sec = timed(2, lambda: qn.nf4_double_quant(absmax))
    rows["dq_encode_4096x4096"] = _hbm_row((4 + 1 + 4 / 256) / 64 * na, sec, timed.last_min)
    wa = qn.quantize_weight(W)
    sec = timed(3, lambda: qn.nf4_dequantize(wa))
    rows["dequantize_bf16_4096x4096"] = _hbm_row(BPW_DEQUANT * na, sec, timed.last_min)
    r = inp.attn.r
    for T, X in ((1, inp.X1), (16, inp.X16)):
        sec = timed(4, lambda: qn.qlora_linear_fwd(wa, X, inp.A_attn, inp.B_attn, inp.s_attn))
        rows["gemv_T%d_4096x4096" % T] = _hbm_row(gemv_bytes(4096, 4096, T, r), sec, timed.last_min)
    m = inp.mlp_dev[0]
    w = qn.quantize_weight(m["W"])
    sec = timed(3, lambda: qn.nf4_dequantize(w))
    rows["dequantize_bf16_11008x4096"] = _hbm_row(BPW_DEQUANT * w.rows * w.cols, sec, timed.last_min)
    # decode GEMVs on the MLP shapes (x of the first T tokens of the layer's input)
    wd = qn.quantize_weight(inp.mlp_dev[2]["W"])
    for ww, mm in ((w, m), (wd, inp.mlp_dev[2])):
        for T in (1, 16):
            Xt = mm["X"][:T].contiguous()
            sec = timed(4, lambda: qn.qlora_linear_fwd(ww, Xt, mm["A"], mm["B"], mm["s"]))
            rows["gemv_T%d_%dx%d" % (T, ww.rows, ww.cols)] = _hbm_row(gemv_bytes(ww.rows, ww.cols, T, mm["r"]), sec,
                                                                      timed.last_min)
    del wd
    N, K, T, r = m["N"], m["K"], m["T"], m["r"]
    sec = timed(5, lambda: qn.qlora_linear_fwd(w, m["X"], m["A"], m["B"], m["s"]))
    # U = X A^T inside this launch (eager calls where the library says so),
    # else in a separate projection launch
    u_in = qn.lib.qlora_linear_fwd_u_in_launch(N, K, T, r)
    rows["gemm_fwd_T1024_11008x4096"] = dict(_mfma_row(fwd_flops(N, K, T, r) - (0 if u_in else 2 * T * K * r), sec,
                                                       timed.last_min), u_in_launch=bool(u_in))
    _, U = qn.qlora_linear_fwd(w, m["X"], m["A"], m["B"], m["s"])
    sec = timed(6, lambda: qn.qlora_linear_bwd(w, m["X"], m["dY"], m["A"], m["B"], m["s"], U=U,
                                              need_da=False, need_db=False))
    g_in = qn.lib.qlora_linear_bwd_g_in_launch(N, K, T, r)
    rows["gemm_dx_T1024_11008x4096"] = dict(_mfma_row(dx_flops(N, K, T, r) - (0 if g_in else 2 * T * N * r), sec,
                                                      timed.last_min), g_in_launch=bool(g_in))
    sec = timed(7, lambda: qn.qlora_linear_bwd(w, m["X"], m["dY"], m["A"], m["B"], m["s"], U=U, need_dx=False))
    rows["lora_grad_T1024_11008x4096"] = _hbm_row(lora_grad_bytes(N, K, T, r), sec, timed.last_min)  # dA and dB
    # adapter merge of the same weight: codes and constants in, bf16 out, A and B read once
    sec = timed(8, lambda: qn.qlora_merge(w, m["A"], m["B"], m["s"]))
    rows["merge_r%d_11008x4096" % r] = _hbm_row(BPW_DEQUANT * N * K + 2 * r * (N + K), sec, timed.last_min)
    # dropout (p = 0.05) on the adapter input of the same layer: the masking
    # pass (X and the keep bits in, X * keep out) and the masked adapter term
    # of dX (dX, G, the bits in, dX out; A is L2-resident)
    import workloads

    bits = workloads.pack_keep_bits(workloads.keep_mask(T, K, 0.05, 31)).cuda()
    sec = timed(10, lambda: qn.qlora_linear_fwd(w, m["X"], m["A"], m["B"], m["s"], keep=bits, p=0.05))
    rows["dropout_keep_apply_T1024_K4096"] = _hbm_row(T * K * (2 + 2 + 1 / 8), sec, timed.last_min)
    sec = timed(11, lambda: qn.qlora_linear_bwd(w, m["X"], m["dY"], m["A"], m["B"], m["s"], U=U, need_da=False,
                                               need_db=False, keep=bits, p=0.05))
    rows["dropout_dx_term_T1024_K4096"] = _hbm_row(T * K * (2 + 2 + 1 / 8) + 2 * T * 64 + 2 * r * K, sec,
                                                   timed.last_min)
    # quantization-error measurement on the uniform grid, fp32 weight read once
    sec = timed(9, lambda: qn.q4_quant_error(m["W"], "uniform"))
    rows["quant_error_uniform_f32_11008x4096"] = _hbm_row(4 * N * K, sec, timed.last_min)
    rows.update(measure_adamw_rows(torch, qn, flush))
    # dispatch floor: the same HIP-event timing around a kernel that does
    # nothing measurable (a one-element fill), cold cache as above
    tiny = torch.empty(1, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    floor = []
    for _ in range(reps):
        flush()
        e0.record()
        tiny.fill_(0.0)
        e1.record()
        torch.cuda.synchronize()
        floor.append(e0.elapsed_time(e1))
    rows["launch_floor_us"] = round(sorted(floor)[len(floor) // 2] * 1e3, 2)
    # Beside each HBM row's event time, the same row less that floor: an
    # estimate of the kernel's own time (the kernel trace of these launches
    # gives the measured one)
    fl = rows["launch_floor_us"] * 1e-6
    for name, row in rows.items():
        if isinstance(row, dict) and "GB/s" in row and row["us"] * 1e-6 > fl:
            sec = row["us"] * 1e-6 - fl
            nbytes = row["GB/s"] * 1e9 * row["us"] * 1e-6
            row["us_less_floor"] = round(sec * 1e6, 2)
            row["frac_less_floor"] = round(nbytes / sec / PEAK_HBM, 4)
    return rows


def measure_adamw_rows(torch, qn, flush):
    """The paged AdamW step of every adapter of the 32-layer 7B-shaped stack at
    r = 16 (A and B of its 224 linears: 40.0 M fp32 parameters), with the
    state in device memory (HBM-bound: 16 B read, 14 B written per
    parameter with the bf16 copy) and paged out to pinned host memory (the
    host link bounds it: 8 B in and 8 B out per parameter; a plain pinned
    copy of the same bytes in each direction, timed the same way, is the
    measured ceiling). Library HIP-event timer over the whole call."""
    n = 32 * sum(16 * (nn + kk) for _, nn, kk in LLAMA7B_LAYER)
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    P = torch.randn(n, device="cuda", generator=g) * 0.02
    G = torch.randn(n, device="cuda", generator=g) * 1e-3
    P16 = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    Md, Vd = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    Mh, Vh = torch.zeros(n, pin_memory=True), torch.zeros(n, pin_memory=True)
    cs = torch.cuda.Stream()
    rows = {}

    def timed(fn, reps=3):
        t = qn.KernelTimer(12)
        fn(1)
        torch.cuda.synchronize()
        t.arm()
        for i in range(reps):
            flush()
            fn(2 + i)
        cnt, ms = t.read()
        t.disarm()
        return ms / max(cnt, 1) / 1e3

    sec = timed(lambda t: qn.paged_adamw_step(P, G, Md, Vd, t, weight_decay=0.01, param_bf16=P16))
    rows["adamw_device_state_7b_r16"] = dict(_hbm_row(30 * n, sec), params=n)
    sec_p = timed(lambda t: qn.paged_adamw_step(P, G, Mh, Vh, t, weight_decay=0.01, param_bf16=P16, copy_stream=cs))
    # the host link's ceiling: the same bytes as plain pinned copies, in and out at once on two streams
    Dm, Dv = torch.empty(n, device="cuda"), torch.empty(n, device="cuda")
    Hm, Hv = torch.empty(n, pin_memory=True), torch.empty(n, pin_memory=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cps = []
    for _ in range(3):
        torch.cuda.synchronize()
        e0.record()
        cs.wait_stream(torch.cuda.current_stream())
        Dm.copy_(Mh, non_blocking=True)
        Dv.copy_(Vh, non_blocking=True)
        with torch.cuda.stream(cs):
            Hm.copy_(Md, non_blocking=True)
            Hv.copy_(Vd, non_blocking=True)
        torch.cuda.current_stream().wait_stream(cs)
        e1.record()
        torch.cuda.synchronize()
        cps.append(e0.elapsed_time(e1) / 1e3)
    cp = sorted(cps)[1]
    rows["adamw_paged_state_7b_r16"] = {"us": round(sec_p * 1e6, 1), "host_link_GB/s": round(16 * n / sec_p / 1e9, 1),
                                        "plain_copy_us": round(cp * 1e6, 1),
                                        "frac_of_plain_copy": round(cp / sec_p, 4), "params": n}
    del P, G, P16, Md, Vd, Mh, Vh, Dm, Dv, Hm, Hv
    return rows


def _hbm_row(nbytes, sec, sec_min=None):
    gbs = nbytes / sec / 1e9
    row = {"us": round(sec * 1e6, 2), "GB/s": round(gbs, 1), "frac": round(gbs * 1e9 / PEAK_HBM, 4)}
    if sec_min is not None:
        row["us_min"] = round(sec_min * 1e6, 2)
    return row


def _mfma_row(flops, sec, sec_min=None):
    tf = flops / sec / 1e12
    row = {"us": round(sec * 1e6, 2), "TFLOP/s": round(tf, 1), "frac": round(tf * 1e12 / PEAK_BF16, 4)}
    if sec_min is not None:
        row["us_min"] = round(sec_min * 1e6, 2)
    return row


def _host_threads():
    try:
        from threadpoolctl import threadpool_info

        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    return len(os.sched_getaffinity(0)), blas


def _oracle_weight(W):
    """The oracle's quantize + double quant + dequantize of fp32 numpy W:
    returns the dequantized bf16 values as fp32 [N, K]."""
    import oracle

    packed, absmax = oracle.quantize(W)
    c8, scale, mean = oracle.double_quant(absmax)
    a_eff = oracle.dequant_absmax(c8, scale, mean)
    return oracle.bf16_bits_to_f32(oracle.dequantize(packed, a_eff, W.size)).reshape(W.shape)


def cpu_baseline(inp, ideal_s):
    """The CPU oracle runs one whole step of the benchmark on the host, every
    stage on the full tensors (no sampling, no extrapolation): the 4096 x 4096
    attention weight's quantize + double quant + dequantize and its decode
    forward at T = 1 and 16, and for each 7B MLP weight quantize + double
    quant + dequantize, forward and backward at T = 1024. The 256 x 256
    configuration is timed alongside. Same unit as the GPU line."""
    import numpy as np

    import oracle
    import workloads

    cores, blas = _host_threads()
    per = {}

    def tick():
        return time.perf_counter()

    c1 = workloads.tiny_256()
    t0 = tick()
    wd = _oracle_weight(c1.W.numpy())
    X, dY, A, B = (t.float().numpy() for t in (c1.X, c1.dY, c1.A, c1.B))
    oracle.lora_forward(X, wd, A, B, c1.scale)
    oracle.lora_backward(X, dY, wd, A, B, c1.scale)
    per["c1_256x256_T4_r8"] = {"s": round(tick() - t0, 4)}

    step = 0.0
    t0 = tick()
    wd = _oracle_weight(inp.attn.W.numpy())
    tq = tick() - t0
    X16 = inp.attn.X.float().numpy()
    A, B = inp.attn.A.float().numpy(), inp.attn.B.float().numpy()
    t1 = tick()
    oracle.lora_forward(X16[:1], wd, A, B, inp.attn.scale)
    oracle.lora_forward(X16, wd, A, B, inp.attn.scale)
    tg = tick() - t1
    per["c2_attn_4096x4096"] = {"quantize_dq_dequant_s": round(tq, 3), "decode_fwd_T1_T16_s": round(tg, 3)}
    step += tq + tg
    for c in inp.mlp:
        t0 = tick()
        wd = _oracle_weight(c.W.numpy())
        tq = tick() - t0
        X, dY, A, B = (t.float().numpy() for t in (c.X, c.dY, c.A, c.B))
        t1 = tick()
        oracle.lora_forward(X, wd, A, B, c.scale)
        tf = tick() - t1
        t1 = tick()
        oracle.lora_backward(X, dY, wd, A, B, c.scale)
        tb = tick() - t1
        N, K = c.W.shape
        T, r = c.X.shape[0], c.r
        per["c3_%s" % c.name] = {"quantize_dq_dequant_s": round(tq, 3), "fwd_s": round(tf, 3), "bwd_s": round(tb, 3),
                                 "fwd_GFLOP/s": round(fwd_flops(N, K, T, r) / tf / 1e9, 1),
                                 "bwd_GFLOP/s": round(bwd_flops(N, K, T, r) / tb / 1e9, 1),
                                 "quantize_GB/s": round((BPW_QUANT_F32 + BPW_DQ + BPW_DEQUANT) * N * K / tq / 1e9, 3)}
        step += tq + tf + tb
    return {
        "value": round(100.0 * ideal_s / step, 6),
        "unit": "% of MI355X roofline",
        "cores": int(blas) if blas > 1 else 1,
        "kind": "oracle",
        "sample": "the whole benchmark step on the numpy oracle, full tensors, run once (%.1f s): elementwise "
                  "numpy single-threaded, fp64 matmuls on %d BLAS threads; %d host cores" % (step, blas, cores),
        "step_seconds": round(step, 3),
        "configs": per,
    }


def cpu_suite():
    """--cpu-suite: the oracle on the larger configurations, run once each:
    layer 0 of the 32-layer 7B-shaped stack at T = 4096, r = 64 (its seven
    linears: quantize + double quant + dequantize, forward, backward; the
    stack's time is 32 x that, extrapolated) and one 65B-shaped matrix of each
    shape at T = 4096, r = 64. Host-only; prints one JSON line."""
    import oracle
    import workloads

    cores, blas = _host_threads()
    res = {"host_cores": cores, "blas_threads": blas}

    def run(case):
        N, K = case.W.shape
        T, r = case.X.shape[0], case.r
        t0 = time.perf_counter()
        wd = _oracle_weight(case.W.numpy())
        tq = time.perf_counter() - t0
        X, dY, A, B = (t.float().numpy() for t in (case.X, case.dY, case.A, case.B))
        t1 = time.perf_counter()
        oracle.lora_forward(X, wd, A, B, case.scale)
        tf = time.perf_counter() - t1
        t1 = time.perf_counter()
        oracle.lora_backward(X, dY, wd, A, B, case.scale)
        tb = time.perf_counter() - t1
        return {"quantize_dq_dequant_s": round(tq, 2), "fwd_s": round(tf, 2), "bwd_s": round(tb, 2),
                "fwd_GFLOP/s": round(fwd_flops(N, K, T, r) / tf / 1e9, 1),
                "bwd_GFLOP/s": round(bwd_flops(N, K, T, r) / tb / 1e9, 1)}

    layer = {}
    for name, _, _ in LLAMA7B_LAYER:
        print("cpu suite: 7B layer 0 %s" % name, file=sys.stderr, flush=True)
        layer[name] = run(workloads.llama7b_layer_linear(name))
    tot = sum(v["quantize_dq_dequant_s"] + v["fwd_s"] + v["bwd_s"] for v in layer.values())
    res["c4_layer0_T4096_r64"] = layer
    res["c4_stack_x32_extrapolated_s"] = round(32 * tot, 1)
    c5 = {}
    for name, _, _ in LLAMA65B:
        print("cpu suite: 65B %s" % name, file=sys.stderr, flush=True)
        c5[name] = run(workloads.llama65b_linear(name))
    res["c5_one_matrix_each_T4096_r64"] = c5
    return res


def clock_samples(torch, replay, seconds=1.5):
    """The shader clock while the step runs: the replayed step is run back to
    back for ``seconds`` while a thread samples `amd-smi metric -c` (current
    clocks) every ~0.2 s. Returns the GFX clock readings in MHz (and the
    first raw sample's clock lines)."""
    import re
    import subprocess
    import threading

    samples, raw = [], []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c"], capture_output=True, text=True, timeout=10)
            except (OSError, subprocess.SubprocessError):
                return
            lines = r.stdout.splitlines()
            if not raw:
                raw.extend(ln.strip() for ln in lines if ln.strip())
            # the GFX block's "CLK:" lines in MHz
            gfx = False
            for ln in lines:
                t = ln.strip()
                if t.upper().startswith("GFX"):
                    gfx = True
                elif t and t.endswith(":") and not t.upper().startswith("GFX") and not t.upper().startswith("CLK"):
                    gfx = False
                m = re.match(r"CLK:\s*([0-9.]+)\s*MHz", t)
                if gfx and m:
                    samples.append(float(m.group(1)))
            stop.wait(0.2)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            replay()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    busy = [x for x in samples if x > 0]
    out = {"gfx_clk_MHz_samples": len(busy), "raw_first_sample": raw[:40]}
    if busy:
        busy.sort()
        out.update({"gfx_clk_MHz_median": busy[len(busy) // 2], "gfx_clk_MHz_min": busy[0],
                    "gfx_clk_MHz_max": busy[-1]})
    return out


# ---------------------------------------------------------------------------
# --suite: the wider measurement set. Weights are generated on the device
# (seeded torch generator); nothing here is compared with the oracle (the
# tests do that at these shapes on sampled outputs).
# ---------------------------------------------------------------------------
LLAMA7B_LAYER = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                 ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
LLAMA65B = [("sq", 8192, 8192), ("up", 22016, 8192), ("down", 8192, 22016)]


def bwd_flops(N, K, T, r):
    return 2 * T * N * K + 2 * T * N * r + 2 * T * r * K + 2 * r * T * K + 2 * N * T * r


def clock_info():
    import subprocess
    out = {}
    for cmd in (["amd-smi", "metric", "-g", "0", "-c"], ["rocm-smi", "--showclocks"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
            lines = [ln.strip() for ln in r.stdout.splitlines() if "clk" in ln.lower() or "CLK" in ln]
            out[cmd[0]] = lines[:12]
        except (OSError, subprocess.SubprocessError):
            out[cmd[0]] = None
    return out


def run_suite(torch, qn, stack_only=False):
    res = {}
    prop = torch.cuda.get_device_properties(0)
    res["device"] = {"name": prop.name, "compute_units": prop.multi_processor_count,
                     "memory_GiB": round(prop.total_memory / 2 ** 30, 1), "clocks": clock_info()}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps=5, warm=1):
        for _ in range(warm):
            fn()
        ts = []
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        ts.sort()
        return ts[len(ts) // 2]

    g = torch.Generator(device="cuda")

    def dev_randn(shape, std, seed, dtype=torch.float32):
        g.manual_seed(seed)
        return (torch.randn(shape, device="cuda", generator=g) * std).to(dtype)

    # (1) the 32-layer 7B-shaped stack quantized end to end (fp32 in, DQ).
    # Times are the library's HIP-event kernel timers summed over the calls:
    # the quantize launch, and the double quantization from its tree-level
    # launch (where the quantize launch has not folded that level in) to the
    # end of its encoder: GPU time, without the host's launch gaps.
    print("suite: quantizing the 7B stack", file=sys.stderr, flush=True)
    tq, td = qn.KernelTimer(1), qn.KernelTimer(2)
    stack, nweights = [], 0
    tq.arm()
    td.arm()
    for layer in range(32):
        for i, (name, n, k) in enumerate(LLAMA7B_LAYER):
            W = dev_randn((n, k), 0.02, 1000 * layer + i)
            w = qn.quantize_weight(W)
            nweights += n * k
            stack.append((name, n, k, w))
            del W
    torch.cuda.synchronize()
    nq, msq = tq.read()
    nd, msd = td.read()
    tq.disarm()
    td.disarm()
    qsec = (msq + msd) / 1e3
    qbytes = (BPW_QUANT_F32 + BPW_DQ) * nweights
    res["c4_stack_quantize"] = {"weights": nweights, "quantize_ms": round(msq, 3), "double_quant_ms": round(msd, 3),
                                "timed_calls": nq + nd, "GB/s": round(qbytes / qsec / 1e9, 1),
                                "frac": round(qbytes / qsec / PEAK_HBM, 4),
                                "quantize_alone_GB/s": round(BPW_QUANT_F32 * nweights / (msq / 1e3) / 1e9, 1)}
    packed_bytes = sum(w.packed.numel() + w.c8.numel() + 4 * w.dq_scale.numel() for _, _, _, w in stack)
    res["c4_stack_resident_GB"] = round(packed_bytes / 1e9, 3)

    # (1b) the same stack from bf16 weights (the same seeded values rounded
    # to bf16), quantize + double quant; outputs discarded
    print("suite: quantizing the 7B stack from bf16", file=sys.stderr, flush=True)
    tq.arm()
    td.arm()
    for layer in range(32):
        for i, (name, n, k) in enumerate(LLAMA7B_LAYER):
            Wb = dev_randn((n, k), 0.02, 1000 * layer + i, torch.bfloat16)
            qn.quantize_weight(Wb)
            del Wb
    torch.cuda.synchronize()
    nqb, msqb = tq.read()
    ndb, msdb = td.read()
    tq.disarm()
    td.disarm()
    qbytes_b = (BPW_QUANT_BF16 + BPW_DQ) * nweights
    res["c4_stack_quantize_bf16"] = {"quantize_ms": round(msqb, 3), "double_quant_ms": round(msdb, 3),
                                     "timed_calls": nqb + ndb,
                                     "GB/s": round(qbytes_b / ((msqb + msdb) / 1e3) / 1e9, 1),
                                     "frac": round(qbytes_b / ((msqb + msdb) / 1e3) / PEAK_HBM, 4),
                                     "quantize_alone_GB/s": round(BPW_QUANT_BF16 * nweights / (msqb / 1e3) / 1e9, 1),
                                     "quantize_alone_frac": round(BPW_QUANT_BF16 * nweights / (msqb / 1e3) / PEAK_HBM,
                                                                  4)}

    # (1c) the whole packed stack dequantized to bf16 (3.3 GB in, 13 GB out):
    # one output buffer per shape, overwritten; the library's dequantize timer
    # summed over the 224 launches
    print("suite: dequantizing the 7B stack", file=sys.stderr, flush=True)
    outs_dq = {(n, k): torch.empty(n, k, dtype=torch.bfloat16, device="cuda") for _, n, k in LLAMA7B_LAYER}
    tdq = qn.KernelTimer(3)
    tdq.arm()
    for _, n, k, w in stack:
        qn.nf4_dequantize(w, out=outs_dq[(n, k)])
    torch.cuda.synchronize()
    ndq, msdq = tdq.read()
    tdq.disarm()
    dq_bytes = BPW_DEQUANT * nweights

    # the same 224 launches captured once into a HIP graph and replayed: the
    # pass's wall time without host-side gaps or per-launch timer events
    def dequant_pass():
        for _, n, k, w in stack:
            qn.nf4_dequantize(w, out=outs_dq[(n, k)])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dequant_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dequant_pass()
    dq_graph_s = timed(graph.replay, reps=5)
    del graph
    res["c4_stack_dequantize_bf16"] = {"launches": ndq, "kernel_ms": round(msdq, 3), "GB": round(dq_bytes / 1e9, 2),
                                       "GB/s": round(dq_bytes / (msdq / 1e3) / 1e9, 1),
                                       "frac": round(dq_bytes / (msdq / 1e3) / PEAK_HBM, 4),
                                       "graph_ms": round(dq_graph_s * 1e3, 3),
                                       "graph_GB/s": round(dq_bytes / dq_graph_s / 1e9, 1),
                                       "graph_frac": round(dq_bytes / dq_graph_s / PEAK_HBM, 4)}
    del outs_dq

    # (2) one decode GEMV pass over all 224 linears, r = 16, T in {1, 16}:
    # the sum of the GEMV kernel times, and the wall time of the pass
    print("suite: GEMV pass", file=sys.stderr, flush=True)
    lora = {}
    for _, n, k in LLAMA7B_LAYER:
        if (n, k) not in lora:
            lora[(n, k)] = (dev_randn((16, k), 1.0 / k, n + k, torch.bfloat16),
                            dev_randn((n, 16), 0.01, n + 2 * k, torch.bfloat16))
    for T in (1, 16):
        Xs = {k: dev_randn((T, k), 1.0, k + T, torch.bfloat16) for k in (4096, 11008)}
        outs = [torch.empty(T, n, dtype=torch.bfloat16, device="cuda") for _, n, _, _ in stack]

        def gemv_pass():
            for (_, n, k, w), Y in zip(stack, outs):
                A, B = lora[(n, k)]
                qn.qlora_linear_fwd(w, Xs[k], A, B, 2.0, save_u=False, out=Y)

        wall = timed(gemv_pass, reps=3)
        tg = qn.KernelTimer(4)
        tg.arm()
        gemv_pass()
        torch.cuda.synchronize()
        ng, msg = tg.read()
        tg.disarm()
        sec = msg / 1e3
        # the same pass captured once into a HIP graph and replayed, as a
        # decode loop would run it: no host-side gap between the launches
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            gemv_pass()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            gemv_pass()
        graph_s = timed(graph.replay, reps=5)
        del graph
        nbytes = sum(gemv_bytes(n, k, T, 16) for _, n, k, _ in stack)
        res["c4_gemv_pass_T%d" % T] = {"calls": ng, "kernel_ms": round(msg, 3), "wall_ms": round(wall * 1e3, 3),
                                       "GB": round(nbytes / 1e9, 3), "GB/s": round(nbytes / sec / 1e9, 1),
                                       "frac": round(nbytes / sec / PEAK_HBM, 4),
                                       "kernel_us_per_call": round(msg * 1e3 / max(ng, 1), 2),
                                       "graph_ms": round(graph_s * 1e3, 3),
                                       "graph_GB/s": round(nbytes / graph_s / 1e9, 1),
                                       "graph_frac": round(nbytes / graph_s / PEAK_HBM, 4)}

        # the same pass with the layers that read the same x grouped into one
        # launch (q/k/v and gate/up): 4 launches per transformer layer, not 7
        groups = []
        for layer in range(32):
            ws_ = [w for _, _, _, w in stack[7 * layer:7 * layer + 7]]
            groups += [ws_[0:3], ws_[3:4], ws_[4:6], ws_[6:7]]

        def grouped_pass():
            for ws_ in groups:
                k = ws_[0].cols
                qn.qlora_linear_fwd_group(ws_, Xs[k], [lora[(w.rows, k)][0] for w in ws_],
                                          [lora[(w.rows, k)][1] for w in ws_], 2.0, save_u=False)

        tg.arm()
        grouped_pass()
        torch.cuda.synchronize()
        ngg, msgg = tg.read()
        tg.disarm()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            grouped_pass()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            grouped_pass()
        ggraph_s = timed(graph.replay, reps=5)
        del graph
        res["c4_gemv_pass_T%d" % T].update({"grouped_launches": ngg, "grouped_kernel_ms": round(msgg, 3),
                                            "grouped_graph_ms": round(ggraph_s * 1e3, 3),
                                            "grouped_graph_GB/s": round(nbytes / ggraph_s / 1e9, 1),
                                            "grouped_graph_frac": round(nbytes / ggraph_s / PEAK_HBM, 4)})
        del outs
    if stack_only:
        return res

    def gemm_rows(shapes, T, r, alpha, std, seed0, weights=None):
        rows, tf_f, tf_b, t_f, t_b = {}, 0.0, 0.0, 0.0, 0.0
        for i, (name, n, k) in enumerate(shapes):
            w = weights[i] if weights is not None else qn.quantize_weight(dev_randn((n, k), std, seed0 + i))
            X = dev_randn((T, k), 1.0, seed0 + 100 + i, torch.bfloat16)
            dY = dev_randn((T, n), 1.0, seed0 + 200 + i, torch.bfloat16)
            A = dev_randn((r, k), 1.0 / k, seed0 + 300 + i, torch.bfloat16)
            B = dev_randn((n, r), 0.01, seed0 + 400 + i, torch.bfloat16)
            s = alpha / r
            sf = timed(lambda: qn.qlora_linear_fwd(w, X, A, B, s))
            _, U = qn.qlora_linear_fwd(w, X, A, B, s)
            sb = timed(lambda: qn.qlora_linear_bwd(w, X, dY, A, B, s, U=U))
            ff, fb = fwd_flops(n, k, T, r), bwd_flops(n, k, T, r)
            rows[name] = {"shape": [n, k], "fwd_us": round(sf * 1e6, 1), "fwd_TFLOP/s": round(ff / sf / 1e12, 1),
                          "fwd_frac": round(ff / sf / PEAK_BF16, 4), "bwd_us": round(sb * 1e6, 1),
                          "bwd_TFLOP/s": round(fb / sb / 1e12, 1), "bwd_frac": round(fb / sb / PEAK_BF16, 4)}
            tf_f += ff
            tf_b += fb
            t_f += sf
            t_b += sb
            del X, dY, A, B, U
        rows["aggregate"] = {"fwd_ms": round(t_f * 1e3, 3), "fwd_TFLOP/s": round(tf_f / t_f / 1e12, 1),
                             "fwd_frac": round(tf_f / t_f / PEAK_BF16, 4), "bwd_ms": round(t_b * 1e3, 3),
                             "bwd_TFLOP/s": round(tf_b / t_b / 1e12, 1), "bwd_frac": round(tf_b / t_b / PEAK_BF16, 4)}
        return rows

    # (3) GEMMs of one 7B layer at T = 4096, r = 64, alpha = 16 (layer 0 of the
    # stack); the stack's 32 layers take 32x that time
    print("suite: 7B layer GEMMs", file=sys.stderr, flush=True)
    layer0 = [w for _, _, _, w in stack[:7]]
    rows = gemm_rows(LLAMA7B_LAYER, 4096, 64, 16.0, 0.02, 7000, weights=layer0)
    agg = rows["aggregate"]
    agg["stack_fwd_bwd_ms_x32"] = round(32 * (agg["fwd_ms"] + agg["bwd_ms"]), 1)
    res["c4_layer_T4096_r64"] = rows
    del stack, layer0
    torch.cuda.empty_cache()

    # (4) the 65B-shaped linears at T = 4096, r = 64
    print("suite: 65B linears", file=sys.stderr, flush=True)
    res["c5_T4096_r64"] = gemm_rows(LLAMA65B, 4096, 64, 16.0, 0.015, 8000)
    torch.cuda.empty_cache()

    # (5) residency: 80 layers of 65B-shaped packed weights + constants
    per_layer = 4 * 8192 * 8192 + 2 * 22016 * 8192 + 8192 * 22016
    nbytes = per_layer * 80 * (0.5 + 1 / 64 + 4 / (64 * 256))
    buf = torch.empty(int(nbytes), dtype=torch.uint8, device="cuda")
    free, total = torch.cuda.mem_get_info()
    res["c5_80_layer_residency"] = {"packed_GB": round(nbytes / 1e9, 2), "allocated": True,
                                    "free_after_GB": round(free / 1e9, 1), "total_GB": round(total / 1e9, 1)}
    del buf
    torch.cuda.empty_cache()

    # (6) context: the fused NF4 GEMM against torch.matmul (hipBLASLt) on the
    # dequantized bf16 weight, 7B gate shape, T = 1024
    n, k, T = 11008, 4096, 1024
    w = qn.quantize_weight(dev_randn((n, k), 0.02, 9000))
    Wd = qn.nf4_dequantize(w)
    X = dev_randn((T, k), 1.0, 9001, torch.bfloat16)
    s_nf4 = timed(lambda: qn.qlora_linear_fwd(w, X, save_u=False), reps=11)
    s_mm = timed(lambda: torch.matmul(X, Wd.t()), reps=11)
    fl = 2 * T * n * k
    res["context_vs_torch_matmul_11008x4096_T1024"] = {
        "nf4_fused_us": round(s_nf4 * 1e6, 1), "nf4_fused_TFLOP/s": round(fl / s_nf4 / 1e12, 1),
        "torch_matmul_bf16_us": round(s_mm * 1e6, 1), "torch_matmul_TFLOP/s": round(fl / s_mm / 1e12, 1),
        "nf4_over_bf16_time": round(s_nf4 / s_mm, 3)}
    del w, Wd, X
    torch.cuda.empty_cache()

    # (7) NF4 against the uniform 4-bit grid: quantization error (sum of
    # squares relative to sum w^2, max |w - w'|) of 11008 x 4096 weights with
    # normal, Student-t (3 degrees of freedom) and outlier entries, and the
    # error kernel's throughput (cold cache, library timer)
    print("suite: NF4 vs uniform 4-bit error", file=sys.stderr, flush=True)
    import workloads

    flush = torch.empty(512 * 1024 * 1024 // 4, device="cuda")
    dists = {
        "normal_sd0.02": lambda: workloads.normal_weight(n, k, 0.02, seed=1),
        "student_t3_scale0.02": lambda: workloads.student_t_weight(n, k, 3.0, 0.02, seed=2),
        "normal_sd0.02_outliers_1e-3_x20": lambda: workloads.normal_weight(n, k, 0.02, seed=3, outlier_frac=1e-3,
                                                                          outlier_scale=20.0),
    }
    qe = {}
    for name, make in dists.items():
        W = make().cuda()
        row = {}
        for grid in ("nf4", "uniform"):
            tmr = qn.KernelTimer(9)
            qn.q4_quant_error(W, grid)
            torch.cuda.synchronize()
            tmr.arm()
            for _ in range(5):
                flush.fill_(1)
                st = qn.q4_quant_error(W, grid)
            cnt, ms = tmr.read()
            tmr.disarm()
            sse, ssw, mx = st.cpu().tolist()
            sec = ms / cnt / 1e3
            row[grid] = {"rel_mse": sse / ssw, "max_abs_err": mx, "kernel_us": round(sec * 1e6, 2),
                         "GB/s": round(4 * n * k / sec / 1e9, 1)}
        row["uniform_over_nf4_mse"] = round(row["uniform"]["rel_mse"] / row["nf4"]["rel_mse"], 4)
        qe[name] = row
        del W
    res["q4_error_nf4_vs_uniform_11008x4096_f32"] = qe

    # (8) adapter merge of a 7B MLP weight at ranks 16, 64 and 128 (cold cache)
    print("suite: adapter merge", file=sys.stderr, flush=True)
    w = qn.quantize_weight(dev_randn((n, k), 0.02, 9100))
    out = torch.empty(n, k, dtype=torch.bfloat16, device="cuda")
    mg = {}
    for r in (16, 64, 128):
        A = dev_randn((r, k), 1.0 / k, 9101 + r, torch.bfloat16)
        B = dev_randn((n, r), 0.01, 9201 + r, torch.bfloat16)
        tmr = qn.KernelTimer(8)
        qn.qlora_merge(w, A, B, 2.0, out=out)
        torch.cuda.synchronize()
        tmr.arm()
        for _ in range(5):
            flush.fill_(1)
            qn.qlora_merge(w, A, B, 2.0, out=out)
        cnt, ms = tmr.read()
        tmr.disarm()
        sec = ms / cnt / 1e3
        nbytes = BPW_DEQUANT * n * k + 2 * r * (n + k)
        mg["r%d" % r] = {"us": round(sec * 1e6, 2), "GB/s": round(nbytes / sec / 1e9, 1),
                         "frac": round(nbytes / sec / PEAK_HBM, 4)}
    res["merge_11008x4096"] = mg

    # (9) dropout (p = 0.05, r = 16) on the 7B gate projection at T = 1024:
    # forward and backward time with and without it (warm)
    print("suite: dropout", file=sys.stderr, flush=True)
    T, r = 1024, 16
    X = dev_randn((T, k), 1.0, 9301, torch.bfloat16)
    dY = dev_randn((T, n), 1.0, 9302, torch.bfloat16)
    A = dev_randn((r, k), 1.0 / k, 9303, torch.bfloat16)
    B = dev_randn((n, r), 0.01, 9304, torch.bfloat16)
    bits = workloads.pack_keep_bits(workloads.keep_mask(T, k, 0.05, 9305)).cuda()
    _, U = qn.qlora_linear_fwd(w, X, A, B, 2.0)
    _, Ud = qn.qlora_linear_fwd(w, X, A, B, 2.0, keep=bits, p=0.05)
    res["dropout_11008x4096_T1024_r16_p0.05"] = {
        "fwd_us": round(timed(lambda: qn.qlora_linear_fwd(w, X, A, B, 2.0), reps=11) * 1e6, 1),
        "fwd_dropout_us": round(timed(lambda: qn.qlora_linear_fwd(w, X, A, B, 2.0, keep=bits, p=0.05), reps=11) * 1e6, 1),
        "bwd_us": round(timed(lambda: qn.qlora_linear_bwd(w, X, dY, A, B, 2.0, U=U), reps=11) * 1e6, 1),
        "bwd_dropout_us": round(timed(lambda: qn.qlora_linear_bwd(w, X, dY, A, B, 2.0, U=Ud, keep=bits, p=0.05),
                                      reps=11) * 1e6, 1)}
    return res

def replay_us_per_call(torch, fn, calls=10, replays=5):
    """fn() captured `calls` times into one HIP graph (after a warm-up call on
    a side stream), replayed 3 times untimed, then `replays` times between
    HIP events: microseconds per captured call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (calls * replays) * 1e3


def compare_fwd_u(torch, qn):
    """The forward of the 7B gate projection (11008 x 4096, T = 1024, r = 16)
    issued both ways, in alternating rounds: U = X A^T computed by the
    GEMM's first workgroups (one launch) and by a separate projection launch
    before the GEMM (QLORA_NF4_FWD_U=prepass). HIP events around 20
    back-to-back eager calls, then around replays of 10 calls captured in a
    HIP graph (a captured in-launch call also records its epoch kernel)."""
    N, K, T, r = 11008, 4096, 1024, 16
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    W = torch.randn(N, K, device="cuda", generator=g) * 0.02
    X = torch.randn(T, K, device="cuda", generator=g).to(torch.bfloat16)
    A = (torch.randn(r, K, device="cuda", generator=g) / K).to(torch.bfloat16)
    B = (torch.randn(N, r, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    w = qn.quantize_weight(W)
    Y = torch.empty(T, N, dtype=torch.bfloat16, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"shape": [N, K], "T": T, "r": r, "in_launch_applies": qn.lib.qlora_linear_fwd_u_in_launch(N, K, T, r)}
    times = {"in_launch": [], "separate_projection": []}
    outs = {}
    for rnd in range(3):
        for mode in ("in_launch", "separate_projection"):
            if mode == "separate_projection":
                os.environ["QLORA_NF4_FWD_U"] = "prepass"
            else:
                os.environ.pop("QLORA_NF4_FWD_U", None)
            for _ in range(3):
                qn.qlora_linear_fwd(w, X, A, B, 2.0, out=Y)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(20):
                qn.qlora_linear_fwd(w, X, A, B, 2.0, out=Y)
            e1.record()
            torch.cuda.synchronize()
            times[mode].append(e0.elapsed_time(e1) / 20 * 1e3)
            outs[mode] = Y.clone()
    graph = {"in_launch": [], "separate_projection": []}
    for rnd in range(3):
        for mode in graph:
            if mode == "separate_projection":
                os.environ["QLORA_NF4_FWD_U"] = "prepass"
            else:
                os.environ.pop("QLORA_NF4_FWD_U", None)
            graph[mode].append(replay_us_per_call(torch, lambda: qn.qlora_linear_fwd(w, X, A, B, 2.0, out=Y)))
    os.environ.pop("QLORA_NF4_FWD_U", None)
    for mode, v in times.items():
        res[mode + "_us"] = round(sorted(v)[1], 1)
        res[mode + "_rounds_us"] = [round(x, 1) for x in v]
        res[mode + "_graph_rounds_us"] = [round(x, 1) for x in graph[mode]]
    res["same_bits"] = bool(torch.equal(outs["in_launch"], outs["separate_projection"]))
    return res


def compare_bwd_g(torch, qn):
    """The backward of the 7B down projection (4096 x 11008, T = 1024,
    r = 16; its dX GEMM runs 172 unsplit tiles) issued both ways, in
    alternating rounds: G = s dY B computed by the dX GEMM's first
    workgroups (one launch) and by a separate projection launch before it
    (QLORA_NF4_FWD_U=prepass); dX alone and dX with dA and dB. HIP events
    around 20 back-to-back eager calls, then around replays of 10 calls
    captured in a HIP graph."""
    N, K, T, r = 4096, 11008, 1024, 16
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    W = torch.randn(N, K, device="cuda", generator=g) * 0.02
    X = torch.randn(T, K, device="cuda", generator=g).to(torch.bfloat16)
    dY = torch.randn(T, N, device="cuda", generator=g).to(torch.bfloat16)
    A = (torch.randn(r, K, device="cuda", generator=g) / K).to(torch.bfloat16)
    B = (torch.randn(N, r, device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    w = qn.quantize_weight(W)
    _, U = qn.qlora_linear_fwd(w, X, A, B, 2.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"shape": [N, K], "T": T, "r": r, "in_launch_applies": qn.lib.qlora_linear_bwd_g_in_launch(N, K, T, r)}
    for kind, kw in (("dx", dict(need_da=False, need_db=False)), ("dx_da_db", {})):
        times = {"in_launch": [], "separate_projection": []}
        outs = {}
        for rnd in range(3):
            for mode in ("in_launch", "separate_projection"):
                if mode == "separate_projection":
                    os.environ["QLORA_NF4_FWD_U"] = "prepass"
                else:
                    os.environ.pop("QLORA_NF4_FWD_U", None)
                for _ in range(3):
                    qn.qlora_linear_bwd(w, X, dY, A, B, 2.0, U=U, **kw)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(20):
                    o = qn.qlora_linear_bwd(w, X, dY, A, B, 2.0, U=U, **kw)
                e1.record()
                torch.cuda.synchronize()
                times[mode].append(e0.elapsed_time(e1) / 20 * 1e3)
                outs[mode] = [t.clone() for t in o if t is not None]
        graph = {"in_launch": [], "separate_projection": []}
        for rnd in range(3):
            for mode in graph:
                if mode == "separate_projection":
                    os.environ["QLORA_NF4_FWD_U"] = "prepass"
                else:
                    os.environ.pop("QLORA_NF4_FWD_U", None)
                graph[mode].append(replay_us_per_call(torch, lambda: qn.qlora_linear_bwd(w, X, dY, A, B, 2.0, U=U, **kw)))
        os.environ.pop("QLORA_NF4_FWD_U", None)
        sub = {}
        for mode, v in times.items():
            sub[mode + "_us"] = round(sorted(v)[1], 1)
            sub[mode + "_rounds_us"] = [round(x, 1) for x in v]
            sub[mode + "_graph_rounds_us"] = [round(x, 1) for x in graph[mode]]
        sub["same_bits"] = all(torch.equal(a, b) for a, b in zip(outs["in_launch"], outs["separate_projection"]))
        res[kind] = sub
    return res


def compare_grouped(torch, qn):
    """--grouped: the 7B layers that read the same X (q/k/v 3 x 4096x4096,
    gate/up 2 x 11008x4096), r = 16, alpha = 32, at T in {256, 512, 1024,
    2048, 4096}: the forward as one qlora_linear_fwd_group call against one
    qlora_linear_fwd per layer, and dX alone as one qlora_linear_bwd_group
    call against one qlora_linear_bwd per layer. HIP events around 20
    back-to-back calls after 3 untimed ones, three alternating rounds (us
    per call); `fwd_one_launch` is what qlora_linear_fwd_group_one_launch
    says (0: the grouped forward runs one call per layer itself)."""
    import ctypes

    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / 20 * 1e3, 1)

    res = {}
    r = 16
    for name, N, K, m in (("qkv", 4096, 4096, 3), ("gate_up", 11008, 4096, 2)):
        ws = [qn.quantize_weight(torch.randn(N, K, device="cuda", generator=g) * 0.02) for _ in range(m)]
        As = [(torch.randn(r, K, device="cuda", generator=g) / K).to(torch.bfloat16) for _ in range(m)]
        Bs = [(torch.randn(N, r, device="cuda", generator=g) * 0.01).to(torch.bfloat16) for _ in range(m)]
        for T in (256, 512, 1024, 2048, 4096):
            print("grouped: %s T=%d" % (name, T), file=sys.stderr, flush=True)
            X = torch.randn(T, K, device="cuda", generator=g).to(torch.bfloat16)
            dYs = [torch.randn(T, N, device="cuda", generator=g).to(torch.bfloat16) for _ in range(m)]
            ways = {
                "fwd_separate": lambda: [qn.qlora_linear_fwd(ws[i], X, As[i], Bs[i], 2.0) for i in range(m)],
                "fwd_grouped": lambda: qn.qlora_linear_fwd_group(ws, X, As, Bs, 2.0),
                "dx_separate": lambda: [qn.qlora_linear_bwd(ws[i], X, dYs[i], As[i], Bs[i], 2.0, need_da=False,
                                                            need_db=False) for i in range(m)],
                "dx_grouped": lambda: qn.qlora_linear_bwd_group(ws, X, dYs, As, Bs, 2.0, need_da=False,
                                                                need_db=False),
            }
            row = {"fwd_one_launch": qn.lib.qlora_linear_fwd_group_one_launch((ctypes.c_int64 * m)(*[N] * m), m, K,
                                                                              T, r)}
            for _ in range(3):
                for k, fn in ways.items():
                    row.setdefault(k + "_us", []).append(timed(fn))
            res["%s_T%d" % (name, T)] = row
            del X, dYs
        del ws
        torch.cuda.empty_cache()
    return res


def compare_quantize_dq(torch, qn):
    """Quantize + double quantization of the 7B weight shapes, fp32 and bf16
    input, both ways in alternating rounds: nf4_quantize_dq (one call; two
    launches where the quantize launch folds in the mean tree's first level)
    and nf4_quantize followed by nf4_double_quant (three launches). HIP
    events around 20 back-to-back eager calls; bitwise equality of the five
    outputs."""
    g = torch.Generator(device="cuda")
    g.manual_seed(2)
    res = {}
    for rows, cols in ((4096, 4096), (11008, 4096)):
        Wf = torch.randn(rows, cols, device="cuda", generator=g) * 0.02
        for name, W in (("f32", Wf), ("bf16", Wf.to(torch.bfloat16))):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            times = {"one_call": [], "two_calls": []}
            outs = {}
            for rnd in range(3):
                for mode in ("one_call", "two_calls"):
                    def run():
                        if mode == "one_call":
                            return qn.nf4_quantize_dq(W)
                        packed, absmax = qn.nf4_quantize(W)
                        return (packed, absmax) + qn.nf4_double_quant(absmax)

                    for _ in range(3):
                        run()
                    torch.cuda.synchronize()
                    e0.record()
                    for _ in range(20):
                        o = run()
                    e1.record()
                    torch.cuda.synchronize()
                    times[mode].append(e0.elapsed_time(e1) / 20 * 1e3)
                    outs[mode] = o
            sub = {"fold": lib_fold_applies(qn, rows, cols, name)}
            for mode, v in times.items():
                sub[mode + "_us"] = round(sorted(v)[1], 1)
                sub[mode + "_rounds_us"] = [round(x, 1) for x in v]
            sub["same_bits"] = all(torch.equal(a, b) for a, b in zip(outs["one_call"], outs["two_calls"]))
            res["%dx%d_%s" % (rows, cols, name)] = sub
    return res


def lib_fold_applies(qn, rows, cols, dtype):
    """Whether nf4_quantize_dq folds the tree level into its quantize launch
    at this size (its workspace is then one fp64 node per quantize
    workgroup, smaller than the tree levels' own)."""
    dt = {"f32": qn._lib.QL_F32, "bf16": qn._lib.QL_BF16}[dtype]
    n1 = -(-rows * cols // 64)
    return qn.lib.nf4_quantize_dq_workspace(rows, cols, dt) != qn.lib.nf4_double_quant_workspace(n1)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU (--gpus 1); it has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.cpu_suite:
        print(json.dumps({"cpu_suite": cpu_suite()}), flush=True)
        return
    import torch

    import bit_nf4_quantized_16_amd as qn
    import workloads

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)
    if args.suite or args.suite_stack:
        print(json.dumps({"suite": run_suite(torch, qn, stack_only=args.suite_stack)}), flush=True)
        return
    if args.fwd_u:
        print(json.dumps({"fwd_u": compare_fwd_u(torch, qn)}), flush=True)
        return
    if args.bwd_g:
        print(json.dumps({"bwd_g": compare_bwd_g(torch, qn)}), flush=True)
        return
    if args.quantize_dq:
        print(json.dumps({"quantize_dq": compare_quantize_dq(torch, qn)}), flush=True)
        return
    if args.grouped:
        print(json.dumps({"grouped": compare_grouped(torch, qn)}), flush=True)
        return
    print("bench: generating inputs", file=sys.stderr, flush=True)
    inp = Inputs(torch, workloads)
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("bench: copy calibration 268435456 bytes read + written", file=sys.stderr, flush=True)

    print("bench: warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run_step(qn, inp)
    torch.cuda.synchronize()

    # eager steps with the library's kernel timers armed: the per-kernel
    # durations of the roofline (HIP events on the launch stream)
    timers = {k: qn.KernelTimer(v) for k, v in KERNELS.items()}
    for t in timers.values():
        t.arm()
    print("bench: timing %d eager steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(qn, inp)
    torch.cuda.synchronize()
    elapsed_eager = time.perf_counter() - t0
    kstats = {}
    for k, t in timers.items():
        n, ms = t.read()
        t.disarm()
        kstats[k] = (n, ms)
    ms_per_step_eager = elapsed_eager * 1e3 / args.steps
    if args.eager:
        ms_per_step = ms_per_step_eager
    else:
        # the same step captured once into a HIP graph (every call of the
        # library issues only kernel launches) and replayed: the launch gaps
        # of the host-side calls are gone, the work is the same
        side = torch.cuda.Stream()
        warm = torch.cuda.Stream()
        warm.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(warm):
            ref = [tuple(t.clone() for t in o) for o in run_step_streams(torch, qn, inp, side)]
        torch.cuda.current_stream().wait_stream(warm)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            outs = run_step_streams(torch, qn, inp, side)
        for _ in range(args.warmup):
            graph.replay()
        print("bench: timing %d graph replays of the step" % args.steps, file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        # the replayed two-stream step gives the eager serial step's results
        same = all(torch.equal(a, b) for o, r in zip(outs, ref) for a, b in zip(o, r))
        if not same:
            raise SystemExit("bench: the replayed step's outputs differ from the eager step's")
        print("bench: sampling the clock under the replayed step", file=sys.stderr, flush=True)
        clock = clock_samples(torch, graph.replay)
    ideal = ideal_step_seconds(inp)
    value = 100.0 * ideal / (ms_per_step / 1e3)

    # dominant kernel: the largest total time in the timed steps
    dom = max(kstats, key=lambda k: kstats[k][1])
    work = per_launch_work(qn, inp)
    roof = None
    if dom in work:
        bound, per_launch, unit = work[dom]
        n, ms = kstats[dom]
        avg_s = ms / n / 1e3
        achieved = per_launch / avg_s / 1e12
        tb = measured_traffic(dom)
        roof = {"bound": bound, "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16 / 1e12,
                "unit": unit, "frac": round(achieved / (PEAK_BF16 / 1e12), 4),
                "traffic": round(tb / avg_s / 1e9, 1) if tb else None, "traffic_unit": "GB/s",
                "traffic_bytes_per_launch": tb,
                "avg_launch_us": round(avg_s * 1e6, 2), "launches": n}
    out = {
        "metric": "dequant-GEMM TFLOP/s + quant/GEMV GB/s at 7B shapes, % of MI355X roofline",
        "value": round(value, 2),
        "unit": "% of MI355X roofline",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_eager": round(ms_per_step_eager, 4),
        "step_launch": "eager" if args.eager else "hip_graph_replay_two_streams",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the 7B workloads)",
        "config": {
            "workload": "llama7b_qlora_step: attn 4096x4096 quantize+DQ+dequant+GEMV T=1,16 (r=16); "
                        "MLP 11008x4096 x2 + 4096x11008 quantize+DQ+fwd+bwd at T=1024 (r=16; gate and up read "
                        "the same X, their backward one grouped call)",
            "ideal_step_ms": round(ideal * 1e3, 4),
            "blocksize": 64,
            "dq_blocksize": 256,
        },
        "roofline": roof,
        "kernels_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in kstats.items()},
    }
    if not args.eager:
        out["clock"] = clock
    if not args.no_rows:
        flushbuf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        print("bench: per-stage cold-cache rows", file=sys.stderr, flush=True)
        out["rows"] = measure_rows(torch, qn, inp, lambda: flushbuf.fill_(1))
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, ideal)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
