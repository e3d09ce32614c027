"""Benchmark of the MI355X quantized linear layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass over every stage of the quantized linear layer on synthetic inputs resident in HBM:
  quantize   Llama-70B-shaped decoder layer (q, k, v, o, gate, up, down; 855.6 M bf16 weights) to symmetric
             INT4, g = 128, packed                                                  (range, scale, codes, pack)
  dequantize the packed layer back to bf16                                          (standalone dequantize)
  w4a16_m1   the seven projections at batch 1 (decode) in one grouped launch (pqg_qlinear_w4a16_grouped),
             four such launches back to back, alternating between this step's copy and a fourth copy of
             the layer kept for it                           <- the headline weight-stream GB/s
             (by step, four other forms of the same pass are measured and reported apart: the seven
             launches back to back; the seven launches with events between them, for per-projection times;
             four launches over q|k|v and gate|up stored as concatenated matrices sharing their input, as
             serving engines store them; and a third copy of the layer with 16-bit metadata)
  w4a16_m32  the layer at batch 32, four launches over the concatenated layout (q|k|v, o, gate|up, down;
             every fifth step the seven projections instead, and in the steps whose decode pass runs as four
             launches the four products in one grouped launch; both reported apart)
  w4a16_m8   the same at batch 8
  smooth     SmoothQuant factor, alpha = 0.5, X 2048x4096 (41 channels x50), W 11008x4096
  wquant     W' = W diag(s) -> INT8 per output channel
  w8a8       dynamic per-token INT8 activations + INT8 GEMM + s_x*s_w epilogue, 2048x11008x4096
                                                             <- the INT8 GEMM TOPS
  w8a8_static_actquant  the pages' static variant: X' = X diag(s)^-1 in bf16 (as a LayerNorm with s folded
             into its gain emits it) to INT8 with one calibrated per-tensor scale (the GEMM is the same)
  w4a8       the same layer with the smoothed weights as INT4, g = 128 (quantized once, offline), times the
             step's per-token INT8 activation codes                                    <- the W4A8 TOPS
  kv         one layer's KV cache of 32 sequences x 4096 tokens (8 KV heads x 128 = 1024 channels, bf16):
             keys per channel over groups of 128 tokens, values per token; then one online append step for
             the 32 sequences with no group completing, and one where every sequence completes its group
The packed layer exists twice. A step re-quantizes into one copy, runs the dequantize and the W8A8 layer,
then the batch-32 and batch-8 passes over the other copy (clean 455 MB reads that also drain the dirty lines
the 1.7 GB dequantize left in the 256 MB last-level cache), and last the batch-1 decode pass over the copy
quantized at the start of the step: cold weights streamed from HBM behind a clean cache, as in a decode
loop where each layer's weight stream follows the previous one. In the headline form the decode launch runs
four times back to back, over that copy and a fourth one in turn, so that every launch streams 455 MB the
launch before it has pushed out of the last-level cache, and no launch waits on the host or on an event.

After the timed steps, the Llama-7B attention and FFN configurations are measured on their own (quantize and
W4A16 throughput over device copies rotated past the last-level cache, metadata bytes against weight bytes),
then the tiny 256 x 512 configuration (quantize, dequantize and GEMV times: launch-bound, no roofline claim),
and the oracle is timed on the host: the decode sample (cpu_baseline) and each function on all threads and on
one.

Output: one JSON line. `value` = the decode weight stream (packed INT4 bytes + fp32 scales of all seven
projections) divided by the mean duration of the grouped launch that streams it (the four back-to-back
launches between two HIP events recorded on the stream the kernel runs on), in GB/s. The roofline entry uses
the same measurement (one launch, all the bytes), which agrees with the kernel trace.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA, 5.0 POP/s
DECODE_REPS = 4                # grouped decode launches timed back to back per headline step
GEMV_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a16_gemv_l70b_m1_traffic.md")
GEMV_SOURCE = os.path.join(ROOT, "post_quantization_group_amd", "csrc", "w4a16.hip")
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_i8_w8a8_2048x11008x4096_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "post_quantization_group_amd", "csrc", "gemm_i8.hip")


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--cpu-function-seconds", type=float, default=1.5,
                    help="target CPU time per oracle function and thread count")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--m8-paths", action="store_true",
                    help="only time the 70B gate projection at M = 8 on the matrix-core kernel (one launch) and on "
                         "the vector kernel (two launches of 4 tokens), for counter runs; prints one JSON line")
    return ap.parse_args()


def device_record(dev):
    """The properties the runtime reports for the GPU the bench ran on."""
    import torch

    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
            "total_memory_gib": round(p.total_memory / 2 ** 30, 1), "l2_cache_bytes": p.L2_cache_size,
            "warp_size": p.warp_size}


def stream_reference(pqg, dev, reps=6):
    """Measured streaming rates on this GPU, to set the kernels' rates beside: one streaming read of 1 GiB
    (pqg_stream_read_probe: 16-byte non-temporal loads, four in flight per lane) and a device copy of 1 GiB
    (torch's copy, reads + writes), event-timed, medians over `reps` after one warm-up; both buffers are far
    larger than the 256 MB last-level cache. Also the int8 matrix-core rate with no memory traffic
    (pqg_mfma_i8_probe), which the chip's clock under that load sets."""
    import numpy as np
    import torch

    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, fn, nbytes in (("read_gbs", lambda: pqg.stream_read_probe(src, sink), 4 * n),
                             ("copy_gbs", lambda: dst.copy_(src), 8 * n)):
        ts = []
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            if r:
                ts.append(e0.elapsed_time(e1))
        out[name] = round(nbytes / (float(np.median(ts)) * 1e-3) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    # int8 matrix-core rate from registers alone (pqg_mfma_i8_probe), on the GEMM's 232-block grid and on one
    # block per CU, as 4 launches back to back between two events: each wave issuing as many instructions as
    # a GEMM wave does (3072 per SIMD, about the GEMM's duration), and 16 times as many (the rate the chip
    # settles at once its clock has risen under the load; shorter runs include the ramp)
    for _ in range(4):  # bring the clock up under matrix load first, as the GEMM finds it inside a step
        pqg.mfma_i8_probe(256, 2048, sink)
    for blocks in (232, 256):
        for iters, tag in ((128, ""), (2048, "_long")):
            ts = []
            for r in range(reps + 1):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(4):
                    pqg.mfma_i8_probe(blocks, iters, sink)
                e1.record(stream)
                e1.synchronize()
                if r:
                    ts.append(e0.elapsed_time(e1) / 4)
            ops = blocks * 8 * 12 * iters * 65536
            out["mfma_i8_tops_%d_blocks%s" % (blocks, tag)] = round(ops / (float(np.median(ts)) * 1e-3) / 1e12, 1)
    return out


def m8_paths(pqg, W, dev, bf16, reps=10):
    """The 70B gate projection (28672 x 8192, symmetric INT4, g = 128) at M = 8: the matrix-core kernel the
    library takes for 5 <= M <= 64, against the vector (decode) kernel run as two launches of 4 tokens (it
    takes at most 4 per launch), over four weight copies taken in turn (each streamed from HBM)."""
    import numpy as np
    import torch

    i = [p[0] for p in W.L70B_PROJ].index("gate")
    w = bf16(W.l70b_weight(i))
    x = bf16(W.l70b_x(i, 8))
    copies = [pqg.quantize(w, 4, True, pqg.GROUP, 128) for _ in range(4)]  # 500 MB: past the 256 MB cache
    del w
    y = torch.empty((8, copies[0][0].shape[0]), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {"projection": "gate 28672x8192 sym g128", "M": 8}
    for name, fn in (("matrix_one_launch", lambda c: pqg.qlinear_w4a16(x, c[0], c[1], None, 128, True, out=y)),
                     ("vector_two_launches", lambda c: (pqg.qlinear_w4a16(x[:4], c[0], c[1], None, 128, True, out=y[:4]),
                                                        pqg.qlinear_w4a16(x[4:], c[0], c[1], None, 128, True, out=y[4:])))):
        ts = []
        for r in range(reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(copies[r % 4])
            e1.record(stream)
            e1.synchronize()
            if r >= 2:
                ts.append(e0.elapsed_time(e1))
        out[name + "_us"] = round(float(np.median(ts)) * 1e3, 2)
    return out


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(summary, source):
    """HBM bytes per launch measured with rocprofv3 counters (a summary under profiles/), or None when the
    summary is missing or was taken on a different version of the kernel source."""
    try:
        text = open(summary).read()
    except OSError:
        return None
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != source_hash(source):
        return None
    return float(t.group(1))


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (each GPU would run the same "
              "kernels on its own shard of the output rows); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import post_quantization_group_amd as pqg
    import workloads as W

    pqg.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.m8_paths:
        print(json.dumps(m8_paths(pqg, W, dev, bf16)), flush=True)
        return

    t_setup = time.time()
    # ---------------------------------------------------------------- inputs (resident in HBM)
    # Each copy of the packed layer holds q|k|v and gate|up as concatenated matrices (rows of one group are
    # independent, so the per-projection tensors are row views of them and quantize into them unchanged).
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    fused = []
    for g in groups:
        n_sum, k = sum(W.L70B_PROJ[i][1] for i in g), W.L70B_PROJ[g[0]][2]
        fused.append(dict(members=g, n=n_sum, k=k,
                          packed=[torch.empty((n_sum, k // 2), dtype=torch.uint8, device=dev) for _ in range(2)],
                          scales=[torch.empty(n_sum * k // 128, dtype=torch.float32, device=dev) for _ in range(2)],
                          y1=torch.empty((1, n_sum), dtype=torch.bfloat16, device=dev),
                          y8=torch.empty((8, n_sum), dtype=torch.bfloat16, device=dev),
                          y32=torch.empty((32, n_sum), dtype=torch.bfloat16, device=dev)))
    projs = []
    for f in fused:
        r0 = 0
        for i in f["members"]:
            name, n, k = W.L70B_PROJ[i]
            w = bf16(W.l70b_weight(i))
            x = bf16(W.l70b_x(i, 32))
            packed = [f["packed"][c][r0:r0 + n] for c in range(2)]
            scales = [f["scales"][c][r0 * (k // 128):(r0 + n) * (k // 128)] for c in range(2)]
            r0 += n
            for c in range(2):
                pqg.quantize(w, 4, True, pqg.GROUP, 128, out=(packed[c], scales[c], None))
            packed16, s16, _ = pqg.quantize_meta16(w, True, 128)  # the third copy, 16-bit metadata
            # the fourth copy: the decode headline alternates between it and copy c
            packed_d, scales_d, _ = pqg.quantize(w, 4, True, pqg.GROUP, 128)
            projs.append(dict(name=name, n=n, k=k, w=w, x=x, packed=packed, scales=scales, packed16=packed16, s16=s16,
                              packed_d=packed_d, scales_d=scales_d,
                              y1=torch.empty((1, n), dtype=torch.bfloat16, device=dev),
                              y8=torch.empty((8, n), dtype=torch.bfloat16, device=dev),
                              y32=torch.empty((32, n), dtype=torch.bfloat16, device=dev)))
    for f in fused:
        f["x"] = projs[f["members"][0]]["x"]  # the group's shared input
    deq = torch.empty(max(p["n"] * p["k"] for p in projs), dtype=torch.bfloat16, device=dev)
    d8 = W.w8a8()
    X8, W8 = bf16(d8["x"]), bf16(d8["w"])
    M8, K8 = X8.shape
    N8 = W8.shape[0]
    s8 = pqg.smooth(X8, W8, 0.5)
    wq8, sw8, _ = pqg.quantize(W8, 8, True, pqg.ROW, 0, s8, pqg.SMOOTH_MUL)
    y8 = torch.empty((M8, N8), dtype=torch.bfloat16, device=dev)
    xq8 = torch.empty((M8, K8), dtype=torch.int8, device=dev)
    sx8 = torch.empty(M8, dtype=torch.float32, device=dev)
    # static variant: X' stands in for the output of the previous LayerNorm with s folded into its gain, and
    # the per-tensor activation scale is calibrated once on a second batch
    Xp8 = (X8.float() / s8).to(torch.bfloat16)
    Xcal = (bf16(W.w8a8_calibration(512, K8)).float() / s8).to(torch.bfloat16)
    s_static = float(pqg.quantize(Xcal, 8, True, pqg.TENSOR)[1].cpu()[0])
    xq8s = torch.empty((M8, K8), dtype=torch.int8, device=dev)
    wq4, sw4, _ = pqg.quantize(W8, 4, True, pqg.GROUP, 128, s8, pqg.SMOOTH_MUL)
    y4 = torch.empty((M8, N8), dtype=torch.bfloat16, device=dev)
    KV_B, KV_S, KV_T = 32, 4096, 128
    dkv = W.kv_cache(KV_B * KV_S, W.KV_CHANNELS)
    Kkv, Vkv = bf16(dkv["k"]), bf16(dkv["v"])
    del dkv
    KV_C = Kkv.shape[1]
    kvk = (torch.empty_like(Kkv, dtype=torch.int8), torch.empty((KV_B * KV_S // KV_T, KV_C), dtype=torch.float32,
                                                                 device=dev), None)
    kvv = (torch.empty_like(Vkv, dtype=torch.int8), torch.empty(KV_B * KV_S, dtype=torch.float32, device=dev), None)
    kv_cache = pqg.kv_cache_alloc(KV_B, KV_S, KV_C, KV_T, 0, True, torch.bfloat16, dev)
    kv_new_k, kv_new_v = Kkv[:KV_B].clone(), Vkv[:KV_B].clone()
    kv_pos_none = torch.full((KV_B,), 1000, dtype=torch.int64, device=dev)  # slot 1000 % 128 = 104
    kv_pos_all = torch.full((KV_B,), 1023, dtype=torch.int64, device=dev)   # slot 127: every group completes
    sx8s = torch.empty(M8, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    gemv_bytes = sum(p["n"] * p["k"] // 2 + p["n"] * (p["k"] // 128) * 4 for p in projs)
    gemv_bytes16 = sum(p["n"] * p["k"] // 2 + p["n"] * (p["k"] // 128) * 2 for p in projs)
    gemv_bytes_total = gemv_bytes + sum(p["k"] * 2 + p["n"] * 2 for p in projs)  # + x and y
    # bytes the quantize stage moves (bf16 weights in, packed codes + scales out) and the dequantize the reverse
    quant_bytes = sum(p["n"] * p["k"] * 2 for p in projs) + gemv_bytes
    w8a8_ops = 2.0 * M8 * N8 * K8

    parts = ["quantize", "dequantize", "smooth", "wquant", "w8a8_actquant", "w8a8_gemm", "w8a8_static_actquant",
             "w4a8_gemm", "kv_keys", "kv_values", "kv_append", "kv_append_groups", "w4a16_m32", "w4a16_m8",
             "w4a16_m1"]
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def run_step(i, rec):
        # Offline stages and the W8A8 layer first; this step re-quantizes the layer into copy c. Then the
        # batch-32 and batch-8 passes stream copy o (clean reads, which also drain the dirty lines the
        # dequantize left in the last-level cache), and the batch-1 decode pass streams copy c, last touched
        # more than 2 GB of traffic earlier: cold weights and a clean cache, as in a decode loop.
        c, o = i % 2, 1 - i % 2
        mode = i % 5
        marks = {}
        if rec:
            marks["start"] = ev()
            marks["start"].record(stream)
        for p in projs:  # S1-S4: range, scale, codes, pack
            pqg.quantize(p["w"], 4, True, pqg.GROUP, 128, out=(p["packed"][c], p["scales"][c], None))
        if rec:
            marks["quantize"] = ev()
            marks["quantize"].record(stream)
        for p in projs:  # S5: standalone dequantize
            out = deq[: p["n"] * p["k"]].view(p["n"], p["k"])
            pqg.dequantize(p["packed"][c], p["scales"][c], None, p["n"], p["k"], 4, True, pqg.GROUP, 128, out=out)
        if rec:
            marks["dequantize"] = ev()
            marks["dequantize"].record(stream)
        s = pqg.smooth(X8, W8, 0.5)  # S8
        if rec:
            marks["smooth"] = ev()
            marks["smooth"].record(stream)
        pqg.quantize(W8, 8, True, pqg.ROW, 0, s, pqg.SMOOTH_MUL, out=(wq8, sw8, None))  # S9
        if rec:
            marks["wquant"] = ev()
            marks["wquant"].record(stream)
        # S10: dynamic per-token INT8 activations after X diag(s)^-1
        pqg.quantize(X8, 8, True, pqg.ROW, 0, s, pqg.SMOOTH_DIV, out=(xq8, sx8, None))
        if rec:
            marks["w8a8_actquant"] = ev()
            marks["w8a8_actquant"].record(stream)
        pqg.qlinear_w8a8(None, None, wq8, sw8, out=y8, x_q=xq8, x_scales=sx8)  # S11-S12: INT8 GEMM + epilogue
        if rec:
            marks["w8a8_gemm"] = ev()
            marks["w8a8_gemm"].record(stream)
        pqg.quantize_static(Xp8, 8, True, s_static, out=xq8s, row_scales=sx8s)  # static per-tensor activations
        if rec:
            marks["w8a8_static_actquant"] = ev()
            marks["w8a8_static_actquant"].record(stream)
        pqg.qlinear_w4a8(xq8, sx8, wq4, sw4, None, 128, True, out=y4)  # INT4 g = 128 weights x INT8 activations
        if rec:
            marks["w4a8_gemm"] = ev()
            marks["w4a8_gemm"].record(stream)
        pqg.kv_quantize_keys(Kkv, KV_T, True, out=kvk)  # keys per channel over groups of 128 tokens
        if rec:
            marks["kv_keys"] = ev()
            marks["kv_keys"].record(stream)
        pqg.quantize(Vkv, 8, True, pqg.ROW, out=kvv)  # values per token
        if rec:
            marks["kv_values"] = ev()
            marks["kv_values"].record(stream)
        pqg.kv_append(kv_cache, kv_new_k, kv_new_v, kv_pos_none, KV_T, 0, True)
        if rec:
            marks["kv_append"] = ev()
            marks["kv_append"].record(stream)
        pqg.kv_append(kv_cache, kv_new_k, kv_new_v, kv_pos_all, KV_T, 0, True)
        if rec:
            marks["kv_append_groups"] = ev()
            marks["kv_append_groups"].record(stream)
        # the batched passes run over the concatenated layout (q|k|v, o, gate|up, down: four launches), or
        # over the seven projections in mode 4
        batched = projs if mode == 4 else fused
        if mode == 2:  # S7: batch 32, the four products in one grouped launch
            pqg.qlinear_w4a16_grouped([f["x"] for f in fused], [f["packed"][o] for f in fused],
                                      [f["scales"][o] for f in fused], None, 128, True, outs=[f["y32"] for f in fused])
        else:
            for p in batched:  # S7: batch 32
                pqg.qlinear_w4a16(p["x"], p["packed"][o], p["scales"][o], None, 128, True, out=p["y32"])
        if rec:
            marks["w4a16_m32"] = ev()
            marks["w4a16_m32"].record(stream)
        if mode == 2:  # S7: batch 8, same copy, the four products in one grouped launch
            pqg.qlinear_w4a16_grouped([f["x"][:8] for f in fused], [f["packed"][o] for f in fused],
                                      [f["scales"][o] for f in fused], None, 128, True, outs=[f["y8"] for f in fused])
        else:
            for p in batched:  # S7: batch 8, same copy
                pqg.qlinear_w4a16(p["x"][:8], p["packed"][o], p["scales"][o], None, 128, True, out=p["y8"])
        if rec:
            marks["w4a16_m8"] = ev()
            marks["w4a16_m8"].record(stream)
        # The decode pass takes one of five forms by step: the seven projections in one grouped launch (mode
        # 0: value), the seven launches with events between them (mode 1: per-kernel durations; the events
        # break back-to-back dispatch), the four launches of the concatenated layout (mode 2), the seven
        # launches over the copy with 16-bit metadata (mode 3), or the seven launches back to back (mode 4).
        gemv_ev = []
        if mode == 0:
            # DECODE_REPS grouped launches back to back, as the layers of a decode step run, alternating between
            # copy c and the fourth copy: each launch streams 455 MB that the one before it has pushed out of the
            # 256 MB last-level cache
            for r in range(DECODE_REPS):
                pk, sc = ("packed", "scales") if r % 2 == 0 else ("packed_d", "scales_d")
                pqg.qlinear_w4a16_grouped([p["x"][:1] for p in projs],
                                          [p[pk][c] if r % 2 == 0 else p[pk] for p in projs],
                                          [p[sc][c] if r % 2 == 0 else p[sc] for p in projs], None, 128, True,
                                          outs=[p["y1"] for p in projs])
        elif mode == 3:
            for p in projs:  # S6 with binary16 scales
                pqg.qlinear_w4a16_meta16(p["x"][:1], p["packed16"], p["s16"], None, 128, True, out=p["y1"])
        elif mode == 2:
            for f in fused:  # S6 over the concatenated layout
                pqg.qlinear_w4a16(f["x"][:1], f["packed"][c], f["scales"][c], None, 128, True, out=f["y1"])
        else:
            for p in projs:  # S6: decode GEMV, batch 1
                if rec and mode == 1:
                    e0 = ev()
                    e0.record(stream)
                pqg.qlinear_w4a16(p["x"][:1], p["packed"][c], p["scales"][c], None, 128, True, out=p["y1"])
                if rec and mode == 1:
                    e1 = ev()
                    e1.record(stream)
                    gemv_ev.append((e0, e1))
        if rec:
            marks["w4a16_m1"] = ev()
            marks["w4a16_m1"].record(stream)
        return marks, gemv_ev, mode

    for i in range(args.warmup):
        run_step(i, False)
    torch.cuda.synchronize()

    records = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        records.append(run_step(args.warmup + i, True))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_part = {k: [] for k in parts}
    gemv_launch_ms = []
    seven_seq_ms = []
    fused_seq_ms = []
    meta16_seq_ms = []
    batched_seven = {"w4a16_m32": [], "w4a16_m8": []}
    batched_grouped_m8 = []
    batched_grouped_m32 = []
    for marks, gemv_ev, mode in records:
        prev = marks["start"]
        for k in parts:
            t = prev.elapsed_time(marks[k])
            prev = marks[k]
            if k in batched_seven and mode == 4:
                batched_seven[k].append(t)
            elif k == "w4a16_m8" and mode == 2:
                batched_grouped_m8.append(t)
            elif k == "w4a16_m32" and mode == 2:
                batched_grouped_m32.append(t)
            elif k != "w4a16_m1" or mode == 0:
                per_part[k].append(t)
            elif mode == 2:
                fused_seq_ms.append(t)
            elif mode == 3:
                meta16_seq_ms.append(t)
            elif mode == 4:
                seven_seq_ms.append(t)
        if mode == 1:  # per-launch kernel durations
            gemv_launch_ms.append([a.elapsed_time(b) for a, b in gemv_ev])
    # mode 0: DECODE_REPS grouped launches back to back between the surrounding marks
    gemv_seq_ms = [t / DECODE_REPS for t in per_part["w4a16_m1"]]
    med = lambda v: float(np.median(v))  # noqa: E731
    part_ms = {k: med(v) for k, v in per_part.items()}
    launch_ms = np.median(np.array(gemv_launch_ms), axis=0)  # per projection
    seq_ms = med(gemv_seq_ms)
    gemm_ms = part_ms["w8a8_gemm"]  # one launch per step: event pair around the GEMM + epilogue kernel

    value = gemv_bytes / (seq_ms * 1e-3) / 1e9
    avg_launch_ms = seq_ms  # one grouped launch streams the whole layer (mean of DECODE_REPS back to back)
    achieved = gemv_bytes / (avg_launch_ms * 1e-3) / 1e9
    tops = w8a8_ops / (gemm_ms * 1e-3) / 1e12
    traffic = read_traffic(GEMV_TRAFFIC_FILE, GEMV_SOURCE)
    gemm_traffic = read_traffic(GEMM_TRAFFIC_FILE, GEMM_SOURCE)

    out = {
        "metric": "W4A16 GEMV weight GB/s (% HBM peak); W8A8 GEMM TOPS (% int8 MFMA peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xbf16->f32 (W4A16); int8xint8->int32 (W8A8)",
        "data": "synthetic (seeded N(0, 0.02) weights / N(0, 1) activations; no trained weights)",
        "config": {
            "workload": "llama70b_layer_w4a16_decode_m1 + w8a8_2048x11008x4096",
            "w4a16": {"projections": [[p["name"], p["n"], p["k"]] for p in projs], "M": 1, "group_size": 128,
                      "symmetric": True, "weight_bytes_per_step": gemv_bytes},
            "w8a8": {"M": M8, "N": N8, "K": K8, "alpha": 0.5, "outlier_channels": int(d8["outlier_chans"].size)},
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "k_w4a16_gemv_grouped (M=1, the seven 70B-layer projections in one launch)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": gemv_bytes,
            "avg_launch_us": round(avg_launch_ms * 1e3, 3),
        },
        "w8a8_gemm": {
            "value": round(tops, 1),
            "unit": "TOPS",
            "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                         "frac": round(tops / INT8_PEAK_TOPS, 4), "traffic": gemm_traffic,
                         "ops_per_launch": w8a8_ops, "avg_launch_us": round(gemm_ms * 1e3, 2)},
        },
        # the W4A8 layer: one launch over the same activation codes; its weights take half the INT8 GEMM's
        # bytes (4 bits against 8) plus one fp32 scale per 128 weights
        "w4a8_gemm": {
            "value": round(w8a8_ops / (part_ms["w4a8_gemm"] * 1e-3) / 1e12, 1),
            "unit": "TOPS",
            "frac": round(w8a8_ops / (part_ms["w4a8_gemm"] * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "avg_launch_us": round(part_ms["w4a8_gemm"] * 1e3, 2),
            "group_size": 128,
            "weight_bytes": N8 * K8 // 2 + N8 * (K8 // 128) * 4,
        },
        # the KV cache of one layer (32 x 4096 tokens, 1024 channels): bulk key and value quantization as
        # bytes moved (bf16 in, INT8 codes and fp32 scales out), and one online append step for 32 sequences
        "kv_int8": {
            "tokens": KV_B * KV_S, "channels": KV_C, "block_tokens": KV_T,
            "keys_us": round(part_ms["kv_keys"] * 1e3, 2),
            "keys_gbs": round((KV_B * KV_S * KV_C * 3 + KV_B * KV_S // KV_T * KV_C * 4) / (part_ms["kv_keys"] * 1e-3)
                              / 1e9, 1),
            "values_us": round(part_ms["kv_values"] * 1e3, 2),
            "values_gbs": round((KV_B * KV_S * KV_C * 3 + KV_B * KV_S * 4) / (part_ms["kv_values"] * 1e-3) / 1e9, 1),
            "append_us": round(part_ms["kv_append"] * 1e3, 2),
            "append_completing_groups_us": round(part_ms["kv_append_groups"] * 1e3, 2),
        },
        "per_projection_event_us": {p["name"]: round(float(t) * 1e3, 2) for p, t in zip(projs, launch_ms)},
        "stage_ms": {k: round(v, 4) for k, v in part_ms.items()},
        # the 70B layer's quantize (bf16 in, packed INT4 + scales out) and dequantize (the reverse): bytes moved
        # per second, against 8 TB/s
        "layer_quantize_gbs": round(quant_bytes / (part_ms["quantize"] * 1e-3) / 1e9, 1),
        "layer_dequantize_gbs": round(quant_bytes / (part_ms["dequantize"] * 1e-3) / 1e9, 1),
        # the batched passes over the same weight stream (packed codes + scales), as weight GB/s: over the
        # concatenated layout (four launches), the same four products in one grouped launch (steps of mode 2), and
        # over the seven projections (steps of mode 4)
        "w4a16_batched_weight_gbs": {m: round(gemv_bytes / (part_ms["w4a16_m%d" % m] * 1e-3) / 1e9, 1)
                                     for m in (8, 32)},
        "w4a16_batched_layout": ["+".join(W.L70B_PROJ[i][0] for i in g) for g in groups],
        "w4a16_batched_grouped_gbs": {m: (round(gemv_bytes / (med(v) * 1e-3) / 1e9, 1) if v else None)
                                      for m, v in ((8, batched_grouped_m8), (32, batched_grouped_m32))},
        "w4a16_batched_seven_launches_gbs": {
            m: (round(gemv_bytes / (med(batched_seven["w4a16_m%d" % m]) * 1e-3) / 1e9, 1)
                if batched_seven["w4a16_m%d" % m] else None) for m in (8, 32)},
        # the static per-tensor activation quantize of the W8A8 layer (bf16 X' in, INT8 codes and the per-token
        # copy of the scale out), and the static layer = it plus the same GEMM + epilogue launch
        "w8a8_static": {"actquant_us": round(part_ms["w8a8_static_actquant"] * 1e3, 2),
                        "actquant_gbs": round((M8 * K8 * 3 + M8 * 4) / (part_ms["w8a8_static_actquant"] * 1e-3) / 1e9,
                                              1),
                        "layer_us": round((part_ms["w8a8_static_actquant"] + gemm_ms) * 1e3, 2),
                        "calibrated_scale": s_static},
        # the same decode weight stream as four launches (q|k|v, o, gate|up, down), each group stored as one
        # concatenated matrix and sharing its input
        # the same decode pass over a third copy of the layer quantized with 16-bit metadata (binary16 scales;
        # the codes use the stored scales), as weight-stream GB/s over its own bytes
        "w4a16_m1_meta16": {"bytes": gemv_bytes16,
                            "value": round(gemv_bytes16 / (med(meta16_seq_ms) * 1e-3) / 1e9, 1) if meta16_seq_ms else None,
                            "unit": "GB/s", "ms": round(med(meta16_seq_ms), 4) if meta16_seq_ms else None},
        "w4a16_m1_seven_launches": {"value": round(gemv_bytes / (med(seven_seq_ms) * 1e-3) / 1e9, 1),
                                    "unit": "GB/s",
                                    "hbm_frac": round(gemv_bytes / (med(seven_seq_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                    "ms": round(med(seven_seq_ms), 4)},
        "w4a16_m1_fused_layout": {"launches": ["+".join(W.L70B_PROJ[i][0] for i in g) for g in groups],
                                  "value": round(gemv_bytes / (med(fused_seq_ms) * 1e-3) / 1e9, 1),
                                  "unit": "GB/s",
                                  "hbm_frac": round(gemv_bytes / (med(fused_seq_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "ms": round(med(fused_seq_ms), 4)},
        "setup_s": round(setup_s, 1),
    }
    out["device"] = device_record(dev)
    ref = stream_reference(pqg, dev)
    out["stream_reference"] = dict(ref, decode_frac_of_read=round(value / ref["read_gbs"], 4),
                                   gemm_frac_of_mfma_probe=round(out["w8a8_gemm"]["value"]
                                                                 / ref["mfma_i8_tops_232_blocks"], 4),
                                   gemm_frac_of_mfma_probe_long=round(out["w8a8_gemm"]["value"]
                                                                      / ref["mfma_i8_tops_232_blocks_long"], 4),
                                   quantize_frac_of_copy=round((quant_bytes / (part_ms["quantize"] * 1e-3) / 1e9)
                                                               / ref["copy_gbs"], 4),
                                   dequantize_frac_of_copy=round((quant_bytes / (part_ms["dequantize"] * 1e-3) / 1e9)
                                                                 / ref["copy_gbs"], 4))
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = 1 << 30
    out["llama7b_configs"] = llama7b_configs(pqg, W, dev, bf16)
    out["tiny_config"] = tiny_config(pqg, W, dev, bf16)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        out["cpu_oracle_per_function"] = cpu_per_function(args.cpu_function_seconds)
    print(json.dumps(out), flush=True)


def llama7b_configs(pqg, W, dev, bf16, reps=8, rounds=6):
    """The Llama-7B attention (4096 x 4096, symmetric INT4 g = 128) and FFN (11008 x 4096 with 41 input columns
    x10, asymmetric UINT4 at g = 32 and g = 128) configurations: quantize and W4A16 throughput with the
    weights rotated over R device copies (R x packed bytes >= 512 MB, twice the last-level cache), so every
    timed call streams its copy from HBM. `reps` launches back to back on consecutive copies are timed as one
    event pair and averaged; the median over `rounds` such blocks is reported. A call through the binding
    costs the host about as long as these kernels run, so the same calls are also captured once into a HIP
    graph over all R copies and replayed (`graph_*`: the kernels back to back without host dispatch in
    between). Also the metadata bytes
    against the packed weight bytes, as stored (fp32 scales + uint8 zero points) and with 16-bit metadata
    (binary16 scales + 4-bit zero points)."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream(dev)
    out = {}

    def timed(fn):
        ts = []
        for r in range(rounds + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for j in range(reps):
                fn(r * reps + j)
            e1.record(stream)
            e1.synchronize()
            if r:
                ts.append(e0.elapsed_time(e1) / reps)
        return float(np.median(ts))

    def graphed(fn, count):
        """`count` calls captured once into a HIP graph (through torch's capture of the current stream), then
        the graph replayed between two events: per-call time without the host's dispatch of each launch."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(count):
                fn(j)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for r in range(rounds + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            if r:
                ts.append(e0.elapsed_time(e1) / count)
        del g
        return float(np.median(ts))

    cases = [("attn7b_4096x4096_sym_g128", W.attn7b(ms=(16,)), True, 128, (1, 16)),
             ("ffn7b_11008x4096_asym_g32", W.ffn7b(ms=(64,)), False, 32, (1, 8, 64)),
             ("ffn7b_11008x4096_asym_g128", None, False, 128, (1, 8, 64))]
    ffn = cases[1][1]
    for name, d, sym, g, ms in cases:
        d = d if d is not None else ffn
        w = bf16(d["w"])
        x = bf16(d["x"])
        n, k = w.shape
        packed_b = n * k // 2
        meta_b = n * (k // g) * (4 + (0 if sym else 1))
        meta16_b = n * (k // g) * 2 + (0 if sym else (n * (k // g) + 1) // 2)
        R = max(2, -(-512 * 2 ** 20 // (packed_b + meta_b)))
        wr = [w] + [w.clone() for _ in range(min(R, 24) - 1)]  # bf16 inputs: 32-86 MiB each, >= 24 copies
        codes = [torch.empty((n, k // 2), dtype=torch.uint8, device=dev) for _ in range(R)]
        scales = [torch.empty(n * k // g, dtype=torch.float32, device=dev) for _ in range(R)]
        zeros = [None if sym else torch.empty(n * k // g, dtype=torch.uint8, device=dev) for _ in range(R)]
        for c in range(R):
            pqg.quantize(w, 4, sym, pqg.GROUP, g, out=(codes[c], scales[c], zeros[c]))
        ys = {m: torch.empty((m, n), dtype=torch.bfloat16, device=dev) for m in ms}
        torch.cuda.synchronize()
        q_ms = timed(lambda i: pqg.quantize(wr[i % len(wr)], 4, sym, pqg.GROUP, g,
                                            out=(codes[i % R], scales[i % R], zeros[i % R])))
        q_bytes = n * k * 2 + packed_b + meta_b
        qg_ms = graphed(lambda i: pqg.quantize(wr[i % len(wr)], 4, sym, pqg.GROUP, g,
                                               out=(codes[i % R], scales[i % R], zeros[i % R])), len(wr))
        e = {"N": n, "K": k, "symmetric": sym, "group_size": g, "copies": R,
             "quantize_us": round(q_ms * 1e3, 2), "quantize_gbs": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
             "quantize_hbm_frac": round(q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "quantize_graph_us": round(qg_ms * 1e3, 2),
             "quantize_graph_gbs": round(q_bytes / (qg_ms * 1e-3) / 1e9, 1),
             "weight_bytes": packed_b + meta_b, "packed_bytes": packed_b, "metadata_bytes": meta_b,
             "metadata_share": round(meta_b / packed_b, 5), "metadata16_bytes": meta16_b,
             "metadata16_share": round(meta16_b / packed_b, 5), "w4a16": {}}
        for m in ms:
            t = timed(lambda i, m=m: pqg.qlinear_w4a16(x[:m], codes[i % R], scales[i % R], zeros[i % R], g, sym,
                                                        out=ys[m]))
            gbs = (packed_b + meta_b) / (t * 1e-3) / 1e9
            tg = graphed(lambda i, m=m: pqg.qlinear_w4a16(x[:m], codes[i % R], scales[i % R], zeros[i % R], g,
                                                           sym, out=ys[m]), R)
            gg = (packed_b + meta_b) / (tg * 1e-3) / 1e9
            e["w4a16"][str(m)] = {"us": round(t * 1e3, 2), "weight_gbs": round(gbs, 1),
                                  "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                                  "graph_us": round(tg * 1e3, 2), "graph_weight_gbs": round(gg, 1),
                                  "graph_hbm_frac": round(gg / HBM_PEAK_GBS, 4)}
        out[name] = e
        del wr, codes, scales, zeros, ys, w
        torch.cuda.empty_cache()
    return out


def tiny_config(pqg, W, dev, bf16, reps=20, rounds=6):
    """The tiny configuration (fp32 weight 256 x 512 with 0.5 % outliers, symmetric INT4 g = 128; x in R^512):
    quantize, dequantize to fp32 and the W4A16 GEMV with fp32 output, each timed as `reps` launches back to
    back between two events (median of `rounds`), both as calls through the binding and as the same calls
    replayed from a HIP graph. 71 KB of data: the times are launch and latency, reported without a roofline
    fraction."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream(dev)
    d = W.tiny()
    w = torch.from_numpy(d["w"]).to(dev)
    x = bf16(d["x"])
    n, k = w.shape
    codes, scales, _ = pqg.quantize(w, 4, True, pqg.GROUP, 128)
    deq = torch.empty((n, k), dtype=torch.float32, device=dev)
    y = torch.empty((1, n), dtype=torch.float32, device=dev)

    def timed(fn):
        ts = []
        for r in range(rounds + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            e1.synchronize()
            if r:
                ts.append(e0.elapsed_time(e1) / reps)
        return round(float(np.median(ts)) * 1e3, 2)

    def graphed(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for r in range(rounds + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            if r:
                ts.append(e0.elapsed_time(e1) / reps)
        del g
        return round(float(np.median(ts)) * 1e3, 2)

    ops = {"quantize": lambda: pqg.quantize(w, 4, True, pqg.GROUP, 128, out=(codes, scales, None)),
           "dequantize": lambda: pqg.dequantize(codes, scales, None, n, k, 4, True, pqg.GROUP, 128, out=deq),
           "w4a16_m1_f32": lambda: pqg.qlinear_w4a16(x, codes, scales, None, 128, True, out_dtype=torch.float32,
                                                     out=y)}
    r = {"N": n, "K": k, "group_size": 128, "symmetric": True,
         "note": "per call through the Python binding, back to back: host dispatch sets these times; the "
                 "graph_us figures replay the same calls captured in a HIP graph (kernels back to back)"}
    for name, fn in ops.items():
        r[name + "_us"] = timed(fn)
        r[name + "_graph_us"] = graphed(fn)
    return r


def cpu_baseline(target_s):
    """The oracle timed on the host cores over a bounded sample of the decode workload: INT4 group quantize
    of the first rows of each 70B projection, then the binary64 W4A16 product at M=1, in weight GB/s."""
    import numpy as np

    import oracle
    import workloads as W

    threads = oracle.num_threads()
    rows = 2048
    sample = [(W.l70b_weight(i, rows=np.arange(min(rows, n))), W.l70b_x(i, 1), k)
              for i, (name, n, k) in enumerate(W.L70B_PROJ)]
    done_bytes = 0
    t_total = 0.0
    passes = 0
    while t_total < target_s:
        for w, x, k in sample:
            t0 = time.perf_counter()
            q, s, _ = oracle.quantize(w, 4, True, oracle.GROUP, 128)
            oracle.w4a16(x, q, s, None, 128)
            t_total += time.perf_counter() - t0
            done_bytes += w.shape[0] * k // 2 + w.shape[0] * (k // 128) * 4
        passes += 1
    return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "first %d rows of each of the seven 70B projections (all of k and v), INT4 g=128 quantize "
                      "+ binary64 W4A16 at M=1, %d passes, %.1f s" % (rows, passes, t_total)}


def cpu_per_function(target_s):
    """Each oracle function timed on bounded samples of the workloads, on all the host threads and on one:
    quantize (INT4 g = 128, 70B q projection rows), dequantize, smooth (W8A8 layer rows), the W4A16 product at
    M = 1 and the W8A8 pipeline (smooth, both quantizations, the int64 GEMM, the epilogue) on a token sample.
    Rates in the unit of each function's own bytes (GB/s) or integer multiply-adds (GMAC/s)."""
    import numpy as np

    import oracle
    import workloads as W

    w70 = W.l70b_weight(0, rows=np.arange(512))   # 512 x 8192 bf16
    x70 = W.l70b_x(0, 1)
    q70, s70, _ = oracle.quantize(w70, 4, True, oracle.GROUP, 128)
    d8 = W.w8a8(m=64, n=1024, k=4096)
    nw = w70.size
    funcs = {
        "quantize_int4_g128": (lambda: oracle.quantize(w70, 4, True, oracle.GROUP, 128),
                               nw * 2 + nw // 2 + nw // 128 * 4, "GB/s"),
        "dequantize_int4_g128": (lambda: oracle.dequantize(q70, s70, None, oracle.GROUP, 128),
                                 nw // 2 + nw // 128 * 4 + nw * 2, "GB/s"),
        "w4a16_m1": (lambda: oracle.w4a16(x70, q70, s70, None, 128), nw // 2 + nw // 128 * 4, "GB/s"),
        "smooth_alpha05": (lambda: oracle.smooth(d8["x"], d8["w"], 0.5), (d8["x"].size + d8["w"].size) * 2, "GB/s"),
        "w8a8_pipeline": (lambda: oracle.w8a8(d8["x"], d8["w"], 0.5), 64 * 1024 * 4096, "GMAC/s"),
    }
    all_threads = oracle.num_threads()
    res = {"threads_all": all_threads, "sample": "512 x 8192 rows of the 70B q projection; W8A8 64 tokens x 1024 "
           "channels x 4096", "functions": {}}
    for name, (fn, units, unit) in funcs.items():
        row = {"unit": unit}
        for label, nt in (("all", all_threads), ("one", 1)):
            oracle.set_num_threads(nt)
            n, t_total = 0, 0.0
            while t_total < target_s or n == 0:
                t0 = time.perf_counter()
                fn()
                t_total += time.perf_counter() - t0
                n += 1
            row[label] = round(units * n / t_total / 1e9, 4)
        res["functions"][name] = row
    oracle.set_num_threads(all_threads)
    return res


if __name__ == "__main__":
    main()
