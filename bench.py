#!/usr/bin/env python
"""MLA paged decode benchmark on one MI355X.

Workload: DeepSeek-V3 per-GPU decode in bf16 -- B=64 requests, H=128 heads,
every sequence 8192 tokens, kv_lora_rank 512 + rope_dim 64 (576-wide cache
rows), block_size 64, random physical blocks, N(0,1) inputs, sm_scale
1/sqrt(192), num_kv_splits = ceil(8192/512) = 16.

One step is the whole hot path for one decode iteration: the paged cache
write of the B new tokens (one per request) followed by the split-KV decode
(stage 1 + stage 2).  Inputs are resident in HBM before timing starts.

Prints one JSON line.  Extra fields: per-stage times from HIP events recorded
on the launch stream, the bulk cache-write bandwidth, the batch-invariant
(num_kv_splits = 1) step time (library default, and with requests of 4096
tokens or more on the token-split stage 1), and the CPU oracle's time on a
bounded sample.
"""

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode µs/step, KV-read HBM GB/s and % roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


class HipEvent:
    """A raw HIP event (timing enabled).  The library records it on the
    stream it launches on; torch.cuda.Event cannot be used for that because
    torch creates its event lazily on its own record().  The events only
    time work (they are read after a device synchronisation), so they skip
    the system-scope fence a default event performs when it completes: that
    fence writes back and invalidates the caches, which costs the step time
    and adds to the interval the event measures."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so.7")
        self.handle = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.handle),
                                                 ctypes.c_uint(HipEvent.DISABLE_SYSTEM_FENCE)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    @property
    def cuda_event(self):
        return self.handle.value

    def ms_until(self, other) -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.handle, other.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        hip = type(self)._hip          # module globals may already be gone at interpreter exit
        if hip is not None and self.handle:
            hip.hipEventDestroy(self.handle)


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_v3_b64_h128_n8192_hbm_traffic.txt")


# the sources that define the stage-1 kernel and its launch (plan, grid)
STAGE1_SOURCES = ["api.hip", "decode_mfma.hip", "mla_device.h", "mla_launch.h"]


def code_tokens(text: str) -> str:
    """C++ source without comments and with whitespace collapsed, so that a
    comment edit does not count as a kernel change."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_sources_sha256() -> str:
    """sha256 over the stage-1 kernel's sources (file names and code)."""
    import hashlib
    h = hashlib.sha256()
    for name in STAGE1_SOURCES:
        h.update(name.encode())
        with open(os.path.join(ROOT, "mla_paged_decode_concat_amd", "csrc", name)) as f:
            h.update(code_tokens(f.read()).encode())
    return h.hexdigest()


def measured_traffic():
    """Stage-1 HBM bytes per launch (read + write) from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary, calibrated against a plain
    device copy; None when the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            line = [l for l in f if l.startswith("machine:")][-1]
    except (OSError, IndexError):
        return None
    kv = dict(t.split("=", 1) for t in line.split()[1:] if "=" in t)
    if kv.get("source_sha256") != kernel_sources_sha256():
        return None
    return int(kv["stage1_read_bytes"]) + int(kv["stage1_write_bytes"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # ~20 ms of untimed steps: the board's clocks take a few hundred steps
    # to settle (measured: the first 50 steps of a fresh process ran 238 us
    # against 197 us a few hundred steps later)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--min-untimed-steps", type=int, default=100,
                    help="untimed steps before the timed ones: the --warmup steps, topped up to this many "
                         "(the board's clocks dip after the first few dispatches and settle over the next "
                         "~100 steps; fewer time that transient, not the kernels)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="bound on the CPU oracle's timed work (0 = skip)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--kernel", type=int, default=0, help="stage-1 kernel: 0 auto, 1 vector ALU, 2 MFMA, 3 MFMA token split (16- or 32-head groups)")
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--heads-per-group", type=int, default=0)
    ap.add_argument("--partition", type=int, default=0)
    ap.add_argument("--no-invariant", action="store_true", help="skip the num_kv_splits=1 timing")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload runs")
    ap.add_argument("--main-only", action="store_true",
                    help="run only the warmup and timed step loop (profiler runs: every decode launch is a step's)")
    ap.add_argument("--num-kv-splits", type=int, default=0,
                    help="splits per request in the step loop (0 = the library's rule; 1 = the batch-invariant step)")
    ap.add_argument("--data", choices=["workload", "zeros", "ones"], default="workload",
                    help="contents of the cache and queries in the step loop: the workload's N(0,1) values "
                         "(default), or all 0.0 / all 1.0 after the bulk write (a check of how the stage-1 "
                         "time depends on the data the matrix cores see; not the benchmark)")
    ap.add_argument("--configs-only", action="store_true",
                    help="run only the per-workload runs (profiler runs: one bulk cache write opens each workload)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mla_paged_decode_concat_amd as M
    from mla_paged_decode_concat_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M.load_library()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    if args.configs_only:
        configs = config_runs(M, W, torch, dev, cus, min(3.0, args.cpu_seconds))
        copy_probe(torch, dev, args.copy_probe_mb)
        print(json.dumps({"configs": configs}), flush=True)
        return
    spec = W.SPECS[2]
    bt = W.make_batch(2, dev, pad_table_with_spare=False)
    B, H, R, D = bt.B, spec.H, spec.R, spec.D
    N = sum(bt.seq_lens_list)
    S = args.num_kv_splits or M.num_kv_splits(max(bt.seq_lens_list), cus)

    # bulk write of the whole context (reported separately), timed warm and
    # beside a device-to-device copy of the same payload (torch's copy_), the
    # practical ceiling of a read-once, write-once kernel
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    copy_src = torch.empty(N * D, dtype=torch.bfloat16, device=dev).normal_()
    copy_dst = torch.empty_like(copy_src)
    bulk_ms, copy_ms = [], []
    for i in range(13):
        for fn, out in ((lambda: M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, "auto"), bulk_ms),
                        (lambda: copy_dst.copy_(copy_src), copy_ms)):
            ev_a.record()
            fn()
            ev_b.record()
            torch.cuda.synchronize()
            if i >= 3:
                out.append(ev_a.elapsed_time(ev_b))
    del copy_src, copy_dst
    bulk_bytes = N * (D * 2 + D * 2 + 8)
    bulk_gbs = bulk_bytes / (statistics.median(bulk_ms) * 1e-3) / 1e9
    copy_gbs = N * D * 2 * 2 / (statistics.median(copy_ms) * 1e-3) / 1e9

    def timed_us(fn, n=10):
        """GPU time per call: the stream is held by a spin kernel while
        the n calls are queued behind the start event, so host-side
        launch overhead does not show as idle time between them."""
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(5_000_000)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    # per-step inputs: the newest token of every request
    idx = bt.last_token_rows
    step_kv_c = bt.kv_c.index_select(0, idx).contiguous()
    step_k_pe = bt.k_pe.index_select(0, idx).contiguous()
    step_slots = bt.slot_mapping.index_select(0, idx).contiguous()
    if args.data != "workload":
        # constant contents: the same work and bytes, no bit toggling in the data paths
        val = 0.0 if args.data == "zeros" else 1.0
        for t in (bt.cache, bt.q, step_kv_c, step_k_pe):
            t.fill_(val)
    ws = torch.empty(M.decode_workspace_bytes(B, H, S, R) // 4, dtype=torch.float32, device=dev)
    o = torch.empty((B, H, R), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    kw = dict(kernel=args.kernel, grid=args.grid, heads_per_group=args.heads_per_group, partition=args.partition)
    # the per-step write of the B new tokens alone (GPU time)
    step_write_us = timed_us(lambda: M.cache_write(step_kv_c, step_k_pe, bt.cache, step_slots, "auto"), n=20)

    def step(S_, evs=None):
        M.cache_write(step_kv_c, step_k_pe, bt.cache, step_slots, "auto")
        M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, W.SM_SCALE, S_, R, workspace=ws, o=o, lse=lse,
                 stage_events=evs, **kw)

    untimed = max(args.warmup, args.min_untimed_steps)
    for _ in range(untimed):
        step(S)
    torch.cuda.synchronize()
    K = args.steps
    # stage events on every EVERY-th timed step: an event record costs the
    # step about a microsecond of queue time (measured: 4.5 us per step with
    # the three on every step), which is measurement, not work
    EVERY = 4
    evs = [[HipEvent() for _ in range(3)] if k % EVERY == 0 else None for k in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step(S, evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    evs = [e for e in evs if e is not None]
    st1 = [e[0].ms_until(e[1]) for e in evs]
    st2 = [e[1].ms_until(e[2]) for e in evs]
    st1_ms = statistics.mean(st1)
    st2_ms = statistics.mean(st2)
    dec_us = sorted((a + b) * 1e3 for a, b in zip(st1, st2))

    # decode with the 256 MB last-level cache flushed before every step (a
    # 512 MB write outside the timed region), per-step events
    fl_us = None
    if not args.main_only:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        n_fl = max(5, K // 2)
        evf = [[HipEvent() for _ in range(3)] for _ in range(n_fl)]
        for k in range(n_fl):
            flush.fill_(k & 0xFF)
            step(S, evf[k])
        torch.cuda.synchronize()
        fl_us = sorted((e[0].ms_until(e[1]) + e[1].ms_until(e[2])) * 1e3 for e in evf)
        del flush

    # batch-invariant run: one split per request, with the library's default
    # stage 1 (requests of 4096 tokens or more on the token-split kernel), and
    # with that length rule off (every request on the shared-tile kernel)
    inv_us = inv_off_us = inv_pieces_us = None
    if not (args.no_invariant or args.main_only):
        ws1 = torch.empty(M.decode_workspace_bytes(B, H, 1, R) // 4, dtype=torch.float32, device=dev)

        def inv_run(S_, wsx, **kx):
            for _ in range(3):
                M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, W.SM_SCALE, S_, R, workspace=wsx, o=o, lse=lse,
                         **kx)
            torch.cuda.synchronize()
            ta = time.perf_counter()
            n_inv = max(5, K // 5)
            for _ in range(n_inv):
                M.cache_write(step_kv_c, step_k_pe, bt.cache, step_slots, "auto")
                M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, W.SM_SCALE, S_, R, workspace=wsx, o=o, lse=lse,
                         **kx)
            torch.cuda.synchronize()
            return (time.perf_counter() - ta) * 1e6 / n_inv

        inv_us = inv_run(1, ws1, **kw)
        inv_off_us = inv_run(1, ws1, split_len=-1, **kw)
        # fixed pieces of 2048 tokens (partition 3): batch-invariant with four
        # partials per V3 request; the workspace slots of num_kv_splits = 4
        S_pc = -(-bt.block_table.shape[1] * spec.block_size // 2048)
        ws_pc = torch.empty(M.decode_workspace_bytes(B, H, S_pc, R) // 4, dtype=torch.float32, device=dev)
        inv_pieces_us = inv_run(S_pc, ws_pc, **dict(kw, partition=3, piece_len=2048))
        del ws_pc

    extras = None
    if not args.main_only:
        # the rows beyond the single-token step, each timed on its own with events
        # non-causal multi-token decode: 2 query tokens per request on the same
        # cache, run as 2*H rows of one request
        q2 = W.multi_token_q(bt, 2)
        S2 = S
        ws2 = torch.empty(M.decode_workspace_bytes(B, 2 * H, S2, R) // 4, dtype=torch.float32, device=dev)
        o2 = torch.empty((B, 2, H, R), dtype=torch.bfloat16, device=dev)
        lse2 = torch.empty((B, 2, H), dtype=torch.float32, device=dev)
        mtok_us = timed_us(lambda: M.decode(q2, bt.cache, bt.block_table, bt.seq_lens, W.SM_SCALE, S2, R,
                                            workspace=ws2, o=o2, lse=lse2))
        dec1_us = timed_us(lambda: M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, W.SM_SCALE, S, R,
                                            workspace=ws, o=o, lse=lse))
        del q2, ws2, o2, lse2
        # merge of 8 shard results of this batch's shape (bf16 o, fp32 lse)
        G8 = 8
        o_parts = torch.randn((G8, B, H, R), device=dev).to(torch.bfloat16)
        lse_parts = torch.randn((G8, B, H), device=dev)
        om = torch.empty((B, H, R), dtype=torch.bfloat16, device=dev)
        lm = torch.empty((B, H), dtype=torch.float32, device=dev)
        merge_us = timed_us(lambda: M.merge_partials(o_parts, lse_parts, om, lm), n=20)
        merge_bytes = G8 * B * H * (R * 2 + 4) + B * H * (R * 2 + 4)
        del o_parts, lse_parts
        # RoPE fused into the write: the whole context, and the step's 64
        # tokens with the query's rope part rotated at the newest positions
        tab = W.rope_table(8192, spec.P).to(dev)
        pos = W.token_positions(bt)
        rope_bulk_us = timed_us(lambda: M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, "auto",
                                                      positions=pos, cos_sin_cache=tab), n=3)
        step_pos = pos.index_select(0, idx)
        qr = bt.q.clone()
        rope_step_us = timed_us(lambda: (M.cache_write(step_kv_c, step_k_pe, bt.cache, step_slots, "auto",
                                                       positions=step_pos, cos_sin_cache=tab),
                                         M.rope_q(qr, step_pos, tab, R)), n=20)
        del qr
        M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, "auto")   # back to the unrotated cache
        # absorbed projections at the DeepSeek-V3 per-GPU shape, batch 64:
        # q_c [64, 1536] x W_Q_UK^T -> [64, 128*512]; o [64, 128*512] x W_UV_O^T -> [64, 7168]
        gq = torch.Generator(device=dev).manual_seed(7)
        lin = {}
        for name, (Nf, Kf) in {"q_absorbed": (H * R, 1536), "o_absorbed": (7168, H * R)}.items():
            Aq = torch.randn((B, Kf), generator=gq, device=dev).to(torch.bfloat16)
            Wq = torch.randn((Nf, Kf), generator=gq, device=dev).to(torch.bfloat16)
            Cq = torch.empty((B, Nf), dtype=torch.bfloat16, device=dev)
            wsq = torch.empty(max(1, M.linear_workspace_bytes(B, Nf, Kf) // 4), dtype=torch.float32, device=dev)
            us = timed_us(lambda: M.linear(Aq, Wq, out=Cq, workspace=wsq), n=10)
            lin[name] = (us, (Nf * Kf + B * Kf + B * Nf) * 2)
            del Aq, Wq, Cq, wsq
        extras = {
            "decode_us_q_len1": round(dec1_us, 2),
            "decode_us_q_len2_noncausal": round(mtok_us, 2),
            "shard_merge_g8_us": round(merge_us, 2),
            "shard_merge_g8_gbps": round(merge_bytes / (merge_us * 1e-6) / 1e9, 1),
            "cache_write_rope_bulk_gbps": round((bulk_bytes + N * 8) / (rope_bulk_us * 1e-6) / 1e9, 1),
            "step_write_rope_plus_q_rope_us": round(rope_step_us, 2),
            "linear_q_absorbed_us": round(lin["q_absorbed"][0], 2),
            "linear_q_absorbed_gbps": round(lin["q_absorbed"][1] / (lin["q_absorbed"][0] * 1e-6) / 1e9, 1),
            "linear_o_absorbed_us": round(lin["o_absorbed"][0], 2),
            "linear_o_absorbed_gbps": round(lin["o_absorbed"][1] / (lin["o_absorbed"][0] * 1e-6) / 1e9, 1),
        }

    copy_probe(torch, dev, args.copy_probe_mb)

    # algorithmic bytes and flops of one stage-1 launch
    kv_bytes = N * D * 2
    tab_bytes = sum(-(-n // spec.block_size) for n in bt.seq_lens_list) * 4 + B * 4
    st1_bytes = kv_bytes + B * H * D * 2 + tab_bytes
    flops = 2.0 * H * (D + R) * N
    st1_s = st1_ms * 1e-3
    achieved = st1_bytes / st1_s / 1e9
    mfma_tflops = flops / st1_s / 1e12

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(bt, step_kv_c, step_k_pe, step_slots, args.cpu_seconds)

    configs = None
    if not (args.main_only or args.no_configs):
        del ws, o, lse
        torch.cuda.empty_cache()
        configs = config_runs(M, W, torch, dev, cus, min(3.0, args.cpu_seconds))

    out = {
        "metric": METRIC,
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "untimed_steps": untimed,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic" if args.data == "workload" else f"synthetic, cache and q all {args.data} (data check)",
        "config": {
            "workload": "DeepSeek-V3 per-GPU MLA decode, bf16: B=64, H=128, seq_len 8192 each, kv_lora_rank 512, "
                        "rope_dim 64, block_size 64, random block table, N(0,1) inputs, sm_scale 1/sqrt(192); "
                        "step = cache write of 64 new tokens + split-KV decode",
            "global_batch": B,
            "seq_len": 8192,
            "num_heads": H,
            "num_kv_splits": S,
            "partition": "balanced" if S > 1 else "one split per request",
            "partials_per_request": effective_splits(bt.seq_lens_list, S, cus),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode stage 1",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
        },
        "kv_read_gbps": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "stage1_us": round(st1_ms * 1e3, 2),
        "stage2_us": round(st2_ms * 1e3, 2),
        "mfma_tflops": round(mfma_tflops, 1),
        "mfma_frac": round(mfma_tflops / BF16_PEAK_TFLOPS, 4),
        "hbm_floor_us": round(kv_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
        "bulk_write_gbps": round(bulk_gbs, 1),
        "bulk_write_vs_device_copy": round(bulk_gbs / copy_gbs, 3),
        "step_cache_write_us": round(step_write_us, 2),
        "batch_invariant_us_per_step": round(inv_us, 2) if inv_us else None,
        "batch_invariant_shared_tile_only_us_per_step": round(inv_off_us, 2) if inv_off_us else None,
        "batch_invariant_pieces_2048_us_per_step": round(inv_pieces_us, 2) if inv_pieces_us else None,
        "decode_us_p10_p50_p90": [round(pct(dec_us, q), 2) for q in (10, 50, 90)],
        "decode_us_llc_flushed_p10_p50_p90": [round(pct(fl_us, q), 2) for q in (10, 50, 90)] if fl_us else None,
        "num_kv_splits_effective": effective_splits(bt.seq_lens_list, S, cus),
        "beyond_single_token": extras,
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


# binding roofline per workload (algorithmic bytes vs flops at the spec peaks):
# an fp8 cache keeps q in bf16, so its contractions run on bf16 matrix cores
# and its arithmetic intensity (~484 flop/B of KV) is past the bf16 ridge
BINDING = {0: "hbm", 1: "hbm", 2: "hbm", 3: "hbm", 4: "mfma"}


def config_runs(M, W, torch, dev, cus, cpu_seconds):
    """Every workload at full size in the benchmark's launch configuration
    (num_kv_splits from the library's rule, default kernel and partition),
    plus the V3 shape under the pages' literal partition at S = 16.  Each
    entry: stage times (HIP events on the launch stream, median of 20
    decodes after about 40 ms of untimed ones), KV-read GB/s and MFMA TFLOP/s of the
    decode, the binding roofline's fraction, and the oracle on a bounded
    sample of the same batch."""
    out = {}
    runs = [(0, {}), (1, {}), (2, {}), (2, {"partition": 1}), (3, {}), (4, {})]
    for index, kw in runs:
        spec = W.SPECS[index]
        bt = W.make_batch(index, dev, pad_table_with_spare=False)
        M.cache_write(bt.kv_c, bt.k_pe, bt.cache, bt.slot_mapping, "fp8" if spec.cache_dtype == "fp8" else "auto",
                      bt.scale)
        N = sum(bt.seq_lens_list)
        S = M.num_kv_splits(max(bt.seq_lens_list), cus)
        ws = torch.empty(max(1, M.decode_workspace_bytes(bt.B, bt.H, S, spec.R) // 4), dtype=torch.float32,
                         device=dev)

        def dec(evs=None):
            return M.decode(bt.q, bt.cache, bt.block_table, bt.seq_lens, W.SM_SCALE, S, spec.R, kv_scale=bt.scale,
                            workspace=ws, stage_events=evs, **kw)
        # untimed calls for about 40 ms of GPU time: the board's clocks
        # settle over the first tens of milliseconds of load (a V3-shape
        # decode measured 201 us after 5 untimed calls, 164 us after 100)
        for _ in range(5):
            dec()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        dec()
        torch.cuda.synchronize()
        for _ in range(min(400, int(0.04 / max(time.perf_counter() - t0, 1e-5)))):
            dec()
        evs = [[HipEvent() for _ in range(3)] for _ in range(20)]
        for e in evs:
            dec(e)
        torch.cuda.synchronize()
        s1 = statistics.median(e[0].ms_until(e[1]) * 1e3 for e in evs)
        s2 = statistics.median(e[1].ms_until(e[2]) * 1e3 for e in evs)
        tot = statistics.median(e[0].ms_until(e[2]) * 1e3 for e in evs)
        kv_b = N * spec.D * {"f32": 4, "bf16": 2, "fp8": 1}[spec.cache_dtype]
        flops = 2.0 * bt.H * (spec.D + spec.R) * N
        kv_gbps = kv_b / (tot * 1e-6) / 1e9
        tflops = flops / (tot * 1e-6) / 1e12
        bound = BINDING[index]
        frac = kv_gbps / HBM_PEAK_GBS if bound == "hbm" else tflops / BF16_PEAK_TFLOPS
        name = spec.name + ("_literal_S" + str(S) if kw.get("partition") == 1 else "")
        entry = {
            "B": bt.B, "H": bt.H, "R": spec.R, "cache": spec.cache_dtype, "tokens": N, "num_kv_splits": S,
            "partition": "literal" if kw.get("partition") == 1 or S == 1 else "balanced",
            "partials_per_request_max": S if kw.get("partition") == 1 else effective_splits(bt.seq_lens_list, S, cus),
            "stage1_us": round(s1, 2), "stage2_us": round(s2, 2), "decode_us": round(tot, 2),
            "kv_read_gbps": round(kv_gbps, 1), "mfma_tflops": round(tflops, 1),
            "roofline": {"bound": bound, "frac": round(frac, 4)},
        }
        if cpu_seconds > 0 and not kw:
            entry["cpu_oracle"] = cpu_decode_sample(bt, cpu_seconds)
        out[name] = entry
        del bt, ws
        torch.cuda.empty_cache()
    return out


def copy_probe(torch, dev, mb):
    """One plain device copy of `mb` MiB: its FETCH_SIZE and WRITE_SIZE
    readings calibrate the counters against bytes known to move."""
    if not mb:
        return
    src = torch.empty(mb * (1 << 20) // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def cpu_decode_sample(bt, seconds):
    """The oracle's fp64 decode of as many requests of the batch as fit in
    `seconds` (from the GPU-written cache copied back), scaled to the batch."""
    from mla_paged_decode_concat_amd import workloads as W
    from oracle import mla_oracle as O
    from threadpoolctl import threadpool_info
    spec = bt.spec
    cache = W.bits(bt.cache)
    q = W.bits(bt.q)
    table = bt.block_table.cpu().numpy()
    lens = bt.seq_lens.cpu().numpy()
    scale = float(bt.scale[0].cpu()) if bt.scale is not None else None
    t0 = time.perf_counter()
    done = 0
    for b in range(bt.B):
        O.decode(q[b:b + 1], cache, table[b:b + 1], lens[b:b + 1], W.SM_SCALE, spec.in_dtype, spec.cache_dtype,
                 spec.R, scale)
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(el / done * bt.B * 1e6, 1), "unit": "us/decode", "cores": int(threads),
            "sample": f"{done} of {bt.B} requests, scaled"}


def pct(sorted_vals, q):
    """q-th percentile (nearest rank) of an ascending list."""
    i = min(len(sorted_vals) - 1, max(0, int(math.ceil(q / 100.0 * len(sorted_vals))) - 1))
    return sorted_vals[i]


def effective_splits(lens, S, cus, groups=1):
    """Most partials any request gets from the library's balanced partition
    with the MFMA kernel's default grid (the rule is stated with the
    library's split-partition code): requests padded to 32 tokens are laid
    end to end and cut into G = min(CUs / head groups, B (S - 1)) chunks of
    Q = pad32(ceil(total / G)) tokens."""
    if S == 1:
        return 1
    pad = [-(-n // 32) * 32 for n in lens]
    total = sum(pad)
    G = max(1, min(cus // groups, len(lens) * (S - 1)))
    Q = max(32, -(-(-(-total // G)) // 32) * 32)
    start, most = 0, 0
    for n, p in zip(lens, pad):
        if n > 0:
            most = max(most, (start + n - 1) // Q - start // Q + 1)
        start += p
    return most


def cpu_baseline(bt, step_kv_c, step_k_pe, step_slots, seconds):
    """The oracle as it stands, on the host: the per-step write of the B new
    tokens plus the decode of as many requests as fit in `seconds`, scaled to
    the full batch (µs/step)."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from mla_paged_decode_concat_amd import workloads as W
    from oracle import mla_oracle as O

    spec = bt.spec
    slots = bt.slot_mapping.cpu().numpy()
    cache = O.cache_write(W.bits(W.nan_cache(spec, bt.num_blocks, "cpu")), W.bits(bt.kv_c), W.bits(bt.k_pe),
                          slots, spec.in_dtype, spec.cache_dtype)
    q = W.bits(bt.q)
    table = bt.block_table.cpu().numpy()
    lens = bt.seq_lens.cpu().numpy()
    skv, skp, ssl = W.bits(step_kv_c), W.bits(step_k_pe), step_slots.cpu().numpy()
    t0 = time.perf_counter()
    cache = O.cache_write(cache, skv, skp, ssl, spec.in_dtype, spec.cache_dtype)
    t_write = time.perf_counter() - t0
    # the GPU cache after every timed step, copied back, against the oracle's write
    write_exact = bool(np.array_equal(W.bits(bt.cache), cache))
    t0 = time.perf_counter()
    done = 0
    for b in range(bt.B):
        O.decode(q[b:b + 1], cache, table[b:b + 1], lens[b:b + 1], W.SM_SCALE, spec.in_dtype, spec.cache_dtype,
                 spec.R)
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": round((t_write + el / done * bt.B) * 1e6, 1),
        "unit": "us/step",
        "cores": int(threads),
        "kind": "oracle",
        "gpu_cache_write_bit_exact": write_exact,
        "sample": f"oracle per-step write of {bt.B} tokens + fp64 decode of {done} of {bt.B} requests "
                  f"(8192 tokens x 128 heads each), time scaled to {bt.B} requests; host os.cpu_count()="
                  f"{os.cpu_count()}",
    }


if __name__ == "__main__":
    main()
