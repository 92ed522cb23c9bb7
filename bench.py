"""Benchmark of the DPO LM-head hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input with
inputs already resident in HBM: completion-position indexing, the fused
LM-head forward with online log-sum-exp, the fp64 combine and row sums, the
sigmoid DPO loss, and the fused backward (recompute, dlogits, dHidden,
dW_vocab).  Default workload: 4 pairs x 2,048 tokens at H=4096, V=128,256
(the Llama-3.1-8B head shapes).  --workload 5 times the materialised-logits
variant instead, --workload 3 the offline reference scoring.

Prints one JSON line: throughput in completion tokens/s, the roofline of the
dominant kernel (the library's HIP event timing on the stream the kernels run
on: only that kernel is bracketed inside the timed region, after two untimed
steps with every kernel bracketed have picked it and given the per-kernel
breakdown), and the CPU oracle timed on a bounded sample of the same workload
on this host.
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

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (published figure)
# the same peak from the unit counts: 256 CUs x 2.4 GHz x 4,096 bf16 flop per clock per CU
PEAK_BF16_TFLOPS_UNITS = 256 * 2.4e9 * 4096 / 1e12  # 2,516.6
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

METRICS = {
    2: "completion tokens/s, fused head logp fwd+bwd @H4096 V128256; % MFMA peak",
    4: "completion tokens/s, fused head logp fwd+bwd @H2048 V151936; % MFMA peak",
    3: "completion tokens/s, reference scoring (forward only) @H4096 V128256; % MFMA peak",
    5: "completion tokens/s, materialised bf16 logits fwd+bwd @V128256; % HBM peak",
}


# Kernel families whose sources decide a kernel's HBM traffic; the counter
# table under profiles/ records the digest of the family it was measured on.
CSRC = os.path.join(ROOT, "preference_alignment_amd", "csrc")
FAMILIES = {"head": ["dpo_common.h", "gemm_core.h", "kernels_head.hip", "launch.h"],
            "stream": ["dpo_common.h", "kernels_stream.hip", "launch.h"]}
KERNEL_FAMILY = {"fwd_gemm": "head", "dlogits_gemm": "head", "dhidden_gemm": "head", "dw_gemm": "head",
                 "stream_fwd": "stream", "stream_bwd": "stream", "stream_fwd_f32": "stream",
                 "stream_bwd_f32": "stream"}
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")


def source_digest(family):
    import hashlib
    h = hashlib.sha256()
    for n in FAMILIES[family]:
        h.update(n.encode()); h.update(b"\0")
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` (a label such as "2" or
    "5 f32") from the committed counter table; see _measured_traffic."""
    return _measured_traffic(kernel, str(workload))


def _measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE counters,
    scaled by the copy calibration; None when absent or when the kernel's
    sources changed since the counters were taken."""
    fam = KERNEL_FAMILY.get(kernel)
    if fam is None or not os.path.exists(TRAFFIC_TABLE):
        return None
    scale = {}
    rows = {}
    with open(TRAFFIC_TABLE) as f:
        for line in f:
            line = line.strip()
            for key in ("fetch_scale", "write_scale"):
                if line.startswith(key + ":"):
                    scale[key] = float(line.split(":", 1)[1])
            if line.startswith("|") and not line.startswith("|---"):
                c = [x.strip() for x in line.strip("|").split("|")]
                if len(c) >= 6 and c[0] in KERNEL_FAMILY:
                    rows[(c[0], c[1])] = (c[2], c[3], float(c[4]), float(c[5]))
    r = rows.get((kernel, workload))
    if r is None or len(scale) != 2 or r[0] != fam or r[1] != source_digest(fam):
        return None
    return (r[2] * scale["fetch_scale"] + r[3] * scale["write_scale"]) * 1024.0


ROWS = ["main", "loss-variant", "vocab-shard", "f32-logits", "logits-means"]
ROW_METRICS = {
    "loss-variant": "completion tokens/s, fused head fwd+bwd with the length-normalised loss and NLL term "
                    "@H{H} V{V}; % MFMA peak",
    "vocab-shard": "completion tokens/s, one GPU's V/4 vocabulary shard (TP=4 share) fwd+combine+bwd "
                   "@H{H} V{Vs} of {V}; % MFMA peak",
    "f32-logits": "completion tokens/s, materialised fp32 logits fwd+bwd @V{V}; % HBM peak",
    "logits-means": "completion tokens/s, fused head fwd+bwd with logits-mean sums @H{H} V{V}; % MFMA peak",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=0,
                   help="completion positions per sampled row for the CPU baseline (0 = all: whole pairs)")
    p.add_argument("--cpu-sample-pairs", type=int, default=None,
                   help="whole pairs in the CPU baseline sample; default 1 for the fused head's fwd+bwd, "
                        "2 for reference scoring (forward only) and for given logits")
    p.add_argument("--no-kernel-timing", action="store_true")
    p.add_argument("--all-kernel-timing", action="store_true",
                   help="bracket every kernel with events inside the timed region (default: only the dominant "
                        "kernel there; the per-kernel breakdown comes from an untimed pass)")
    p.add_argument("--profile-steps", type=int, default=2,
                   help="untimed steps with every kernel timed, run before the timed region")
    p.add_argument("--out", default=None, help="also write the JSON line to this file")
    p.add_argument("--no-also", action="store_true",
                   help="skip the logits-path measurement that the default workload-2 run adds under 'also'")
    p.add_argument("--row", default="main", choices=ROWS,
                   help="main: the fused step (or the streaming step for workload 5); loss-variant: "
                        "length-normalised loss with an NLL term (alpha 1); vocab-shard: one GPU's quarter "
                        "of the vocabulary (TP=4 share) with the shard combine; f32-logits: the streaming "
                        "step on fp32 logits of workload 5's shape; logits-means: the fused step with the "
                        "logits-mean sums")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of this many MiB (5 times), to scale "
                        "hardware byte counters")
    return p.parse_args()


def bf(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


class HeadStep:
    """Buffers and the call sequence of one fused step (all work in the HIP library)."""

    def __init__(self, x, dev, forward_only=False, loss_variant=False, metrics=False):
        import torch
        from preference_alignment_amd import dpo_head as D
        self.D, self.x, self.fwd_only = D, x, forward_only
        self.loss_variant, self.metrics = loss_variant, metrics
        R, T, H, V = x.rows, x.T, x.H, x.V
        self.hidden, self.w = bf(x.hidden, dev), bf(x.w_vocab, dev)
        self.targets = torch.from_numpy(x.targets).to(dev)
        self.mask = torch.from_numpy(x.mask).to(dev)
        op = D.DPO_OP_REF_SCORE if forward_only else D.DPO_OP_SEQ_LOGPS
        if metrics:
            op = D.DPO_OP_SEQ_LOGPS_METRICS
        self.ws_f = D.alloc_workspace(op, R, T, H, V, dev)
        self.s32 = torch.empty(R, dtype=torch.float32, device=dev)
        if forward_only:
            return
        self.ws_b = D.alloc_workspace(D.DPO_OP_HEAD_BACKWARD, R, T, H, V, dev)
        self.s64 = torch.empty(R, dtype=torch.float64, device=dev)
        self.lse = torch.empty(R, T, dtype=torch.float32, device=dev)
        self.loss = torch.empty(1, dtype=torch.float32, device=dev)
        self.weight = torch.empty(R, dtype=torch.float32, device=dev)
        self.dh = torch.empty(R, T, H, dtype=torch.float32, device=dev)
        self.dw = torch.empty(V, H, dtype=torch.float32, device=dev)
        self.ntok = torch.empty(R, dtype=torch.int32, device=dev)
        self.zsum = torch.empty(R, dtype=torch.float64, device=dev)
        self.means = torch.empty(2, dtype=torch.float32, device=dev)
        # reference sums: the policy sums of this batch plus N(0,1) noise
        D.dpo_seq_logps(self.hidden, self.w, self.targets, self.mask, self.s32, self.s64, self.lse,
                        self.ntok, workspace=self.ws_f)
        D.dpo_device_status(self.ws_f)
        self.ref = (self.s64 + torch.from_numpy(x.ref_noise).to(dev)).float()

    def step(self):
        D, x = self.D, self.x
        if self.fwd_only:
            D.dpo_ref_score(self.hidden, self.w, self.targets, self.mask, self.s32, workspace=self.ws_f)
            return
        if self.metrics:
            D.dpo_seq_logps_metrics(self.hidden, self.w, self.targets, self.mask, self.s32, self.zsum,
                                    self.s64, self.lse, self.ntok, workspace=self.ws_f)
            D.dpo_logits_mean(self.zsum, self.ntok, x.V, x.layout, self.means)
        else:
            D.dpo_seq_logps(self.hidden, self.w, self.targets, self.mask, self.s32, self.s64, self.lse,
                            self.ntok, workspace=self.ws_f)
        if self.loss_variant:
            D.dpo_loss_ex(self.s64, self.ref, self.ntok, x.beta, x.layout, D.DPO_LOSS_LENGTH_NORM, 1.0,
                          self.loss, self.weight)
        else:
            D.dpo_loss(self.s64, self.ref, x.beta, x.layout, self.loss, self.weight)
        D.dpo_head_backward(self.hidden, self.w, self.targets, self.mask, self.lse, self.weight, self.dh,
                            self.dw, 0, workspace=self.ws_b)


class LogitsStep:
    def __init__(self, x, dev, logits_dev=None):
        import torch
        from preference_alignment_amd import dpo_head as D
        self.D, self.x = D, x
        R, T, V = x.rows, x.T, x.V
        if logits_dev is not None:
            self.f32 = logits_dev.dtype == torch.float32
            self.logits = logits_dev
        else:
            self.f32 = x.logits.dtype == np.float32
            self.logits = torch.from_numpy(x.logits).to(dev) if self.f32 else bf(x.logits, dev)
        fwd = D.dpo_logits_f32_seq_logps if self.f32 else D.dpo_logits_seq_logps
        self.fwd, self.bwd = fwd, (D.dpo_logits_f32_backward if self.f32 else D.dpo_logits_backward)
        self.targets = torch.from_numpy(x.targets).to(dev)
        self.mask = torch.from_numpy(x.mask).to(dev)
        self.ws_f = D.alloc_workspace(D.DPO_OP_LOGITS_SEQ_LOGPS, R, T, 0, V, dev)
        self.ws_b = D.alloc_workspace(D.DPO_OP_LOGITS_BACKWARD, R, T, 0, V, dev)
        self.s32 = torch.empty(R, dtype=torch.float32, device=dev)
        self.s64 = torch.empty(R, dtype=torch.float64, device=dev)
        self.lse = torch.empty(R, T, dtype=torch.float32, device=dev)
        self.loss = torch.empty(1, dtype=torch.float32, device=dev)
        self.weight = torch.empty(R, dtype=torch.float32, device=dev)
        self.dl = torch.empty(R, T, V, dtype=torch.float32 if self.f32 else torch.bfloat16, device=dev)
        self.fwd(self.logits, self.targets, self.mask, self.s32, self.s64, self.lse, workspace=self.ws_f)
        D.dpo_device_status(self.ws_f)
        self.ref = (self.s64 + torch.from_numpy(x.ref_noise).to(dev)).float()

    def step(self):
        D, x = self.D, self.x
        self.fwd(self.logits, self.targets, self.mask, self.s32, self.s64, self.lse, workspace=self.ws_f)
        D.dpo_loss(self.s64, self.ref, x.beta, x.layout, self.loss, self.weight)
        self.bwd(self.logits, self.targets, self.mask, self.lse, self.weight, self.dl, workspace=self.ws_b)


class ShardStep:
    """One GPU's share of a head whose vocabulary is split in `shards` equal
    slices: this GPU's slice forward, the combine of all slices' partials
    (the other slices' partials stand for what an all-gather would bring and
    are computed once at set-up), the loss, and this slice's backward."""

    def __init__(self, x, dev, shards=4):
        import torch
        from preference_alignment_amd import dpo_head as D
        self.D, self.x = D, x
        R, T, H, V = x.rows, x.T, x.H, x.V
        assert V % (8 * shards) == 0
        self.Vs = V // shards
        w = bf(x.w_vocab, dev)
        self.w_shard = w[:self.Vs].contiguous()
        self.hidden = bf(x.hidden, dev)
        self.targets = torch.from_numpy(x.targets).to(dev)
        self.mask = torch.from_numpy(x.mask).to(dev)
        self.ws_f = D.alloc_workspace(D.DPO_OP_SEQ_LOGPS, R, T, H, self.Vs, dev)
        self.ws_c = D.alloc_workspace(D.DPO_OP_SHARD_COMBINE, R, T, 0, V, dev)
        self.ws_b = D.alloc_workspace(D.DPO_OP_HEAD_BACKWARD, R, T, H, self.Vs, dev)
        self.pm = torch.empty(shards, R, T, dtype=torch.float32, device=dev)
        self.ps = torch.empty_like(self.pm)
        self.pt = torch.empty_like(self.pm)
        for s in range(shards):
            ws = self.ws_f
            D.dpo_seq_logps_shard(self.hidden, w[s * self.Vs:(s + 1) * self.Vs].contiguous(), self.targets,
                                  self.mask, s * self.Vs, V, self.pm[s], self.ps[s], self.pt[s], workspace=ws)
        del w
        self.s32 = torch.empty(R, dtype=torch.float32, device=dev)
        self.s64 = torch.empty(R, dtype=torch.float64, device=dev)
        self.lse = torch.empty(R, T, dtype=torch.float32, device=dev)
        self.loss = torch.empty(1, dtype=torch.float32, device=dev)
        self.weight = torch.empty(R, dtype=torch.float32, device=dev)
        self.dh = torch.empty(R, T, H, dtype=torch.float32, device=dev)
        self.dw = torch.empty(self.Vs, H, dtype=torch.float32, device=dev)
        D.dpo_shard_combine(self.pm, self.ps, self.pt, self.targets, self.mask, V, self.s32, self.s64, self.lse,
                            workspace=self.ws_c)
        D.dpo_device_status(self.ws_c)
        self.ref = (self.s64 + torch.from_numpy(x.ref_noise).to(dev)).float()

    def step(self):
        D, x = self.D, self.x
        D.dpo_seq_logps_shard(self.hidden, self.w_shard, self.targets, self.mask, 0, x.V, self.pm[0], self.ps[0],
                              self.pt[0], workspace=self.ws_f)
        D.dpo_shard_combine(self.pm, self.ps, self.pt, self.targets, self.mask, x.V, self.s32, self.s64, self.lse,
                            workspace=self.ws_c)
        D.dpo_loss(self.s64, self.ref, x.beta, x.layout, self.loss, self.weight)
        D.dpo_head_backward_shard(self.hidden, self.w_shard, self.targets, self.mask, 0, x.V, self.lse,
                                  self.weight, self.dh, self.dw, 0, workspace=self.ws_b)


def logits_workload_on_device(dev, seed=5):
    """Workload 5's shapes, mask and targets (host generator), with its
    N(0, 3) bf16 logits drawn on the GPU from a seeded torch generator, so
    that the default run can also time the logits path in seconds."""
    import torch
    from preference_alignment_amd import workloads as W
    _, kw = W.WORKLOADS[5]
    R, T, V, c0, std = kw["rows"], kw["T"], kw["V"], kw["comp_start"], kw["logit_std"]
    rng = np.random.default_rng(seed)
    mask = np.zeros((R, T), dtype=np.uint8)
    mask[:, c0:] = 1
    targets = np.where(mask != 0, rng.integers(0, V, size=(R, T), dtype=np.int32), W.IGNORE_INDEX).astype(np.int32)
    x = W.HeadInputs(name="workload5-device", rows=R, T=T, H=0, V=V, beta=0.1, layout=W.PAIRS_ADJACENT,
                     targets=targets, mask=mask, ref_noise=rng.standard_normal(R))
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    logits = torch.empty(R, T, V, dtype=torch.bfloat16, device=dev)
    for r in range(R):
        logits[r] = (torch.randn(T, V, generator=g, device=dev) * std).to(torch.bfloat16)
    return x, logits


def also_logits_path(dev, steps=20, warmup=3):
    """The materialised-logits path (workload 5's shape) timed the same way as
    the main line: per-step events, then an untimed pass for the kernel split."""
    import torch
    from preference_alignment_amd import dpo_head as D
    x, logits = logits_workload_on_device(dev)
    runner = LogitsStep(x, dev, logits_dev=logits)
    for _ in range(warmup):
        runner.step()
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        runner.step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / steps
    med = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]))
    D.dpo_profile_select(None)
    D.dpo_profile_enable(True)
    for _ in range(2):
        runner.step()
    torch.cuda.synchronize()
    kern = D.dpo_profile_read()
    D.dpo_profile_enable(False)
    n_c, V, E = x.n_completion, x.V, x.rows * x.T * x.V
    step_bytes = n_c * V * 2.0 * 2 + E * 2.0
    out = {"metric": METRICS[5], "value": n_c / (ms / 1e3), "ms_per_step": ms, "ms_per_step_median": med,
           "steps": steps, "warmup": warmup, "completion_tokens": n_c,
           "step_hbm_frac": step_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
           "step_hbm_frac_median": step_bytes / (med / 1e3) / 1e9 / PEAK_HBM_GBS,
           "kernels_ms_per_step": {k: round(v[0] / 2, 4) for k, v in kern.items()},
           "inputs": "workload 5 shapes, mask and targets; N(0,3) bf16 logits drawn on the GPU (seeded)"}
    for k, b in (("stream_fwd", n_c * V * 2.0), ("stream_bwd", n_c * V * 2.0 + E * 2.0)):
        if k in kern:
            out[k + "_GBs"] = b / (kern[k][0] / kern[k][1] / 1e3) / 1e9
    del runner, logits
    torch.cuda.empty_cache()
    return out


def cpu_baseline(x, k, sample_tokens, row="main", shard_rows=None, sample_pairs=1):
    """The oracle, as it stands, on a bounded sample: the first `sample_pairs`
    pairs of the workload, each row cut to its first `sample_tokens` completion
    positions (0 = all of them)."""
    from oracle import dpo_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    rows = list(range(2 * sample_pairs))
    mask = x.mask[rows].copy()
    if sample_tokens > 0:
        for r in range(len(rows)):
            on = np.flatnonzero(mask[r])
            mask[r, on[sample_tokens:]] = 0
    tg = np.where(mask != 0, x.targets[rows], -100)
    n = int(mask.astype(np.int64).sum())
    t0 = time.perf_counter()
    if x.logits is not None and x.logits.dtype == np.float32:
        fwd = O.logits_f32_seq_logps(x.logits[rows], tg, mask)
        loss = O.dpo_loss(fwd["logp_sum"], fwd["logp_sum"] + x.ref_noise[rows], x.beta, x.layout)
        for c in range(0, len(rows) * x.T, 256):  # dlogits of 256 positions at a time
            O.logits_f32_backward_rows(x.logits[rows], tg, mask, fwd["lse"], loss["weight"], np.arange(c, c + 256))
        what = "fp32 logits fwd+loss+bwd"
    elif x.logits is not None:
        fwd = O.logits_seq_logps(x.logits[rows], tg, mask)
        loss = O.dpo_loss(fwd["logp_sum"], fwd["logp_sum"] + x.ref_noise[rows], x.beta, x.layout)
        for c in range(0, len(rows) * x.T, 256):  # dlogits of 256 positions at a time
            O.logits_backward_rows(x.logits[rows], tg, mask, fwd["lse"], loss["weight"], np.arange(c, c + 256))
        what = "fwd+loss+bwd"
    elif row == "vocab-shard":
        hid = O.bf16_to_f64(x.hidden[rows])
        ws = O.bf16_to_f64(x.w_vocab[:shard_rows])
        O.shard_partials_f64(hid, ws, tg, mask, 0, x.V)
        t_fwd = time.perf_counter() - t0
        # the other shards' share of the combined lse, untimed
        fwd = O.seq_logps(x.hidden[rows], x.w_vocab, tg, mask)
        t1 = time.perf_counter()
        loss = O.dpo_loss(fwd["logp_sum"], fwd["logp_sum"] + x.ref_noise[rows], x.beta, x.layout)
        O.head_backward_shard_f64(hid, ws, tg, mask, fwd["lse"], loss["weight"], 0, x.V)
        t0 = t1 - t_fwd
        what = "one V/4 shard: fwd partials + loss + bwd (the whole-vocabulary lse it needs is computed untimed)"
    elif k == 3:
        O.seq_logps(x.hidden[rows], x.w_vocab, tg, mask)
        what = "fwd"
    else:
        fwd = O.seq_logps(x.hidden[rows], x.w_vocab, tg, mask)
        if row == "logits-means":
            sums = O.logit_row_sums_f64(O.bf16_to_f64(x.hidden[rows]), O.bf16_to_f64(x.w_vocab), mask)
            O.logits_means(sums, fwd["n_tokens"], x.V, x.layout)
        if row == "loss-variant":
            loss = O.dpo_loss_variant(fwd["logp_sum"], fwd["logp_sum"] + x.ref_noise[rows], fwd["n_tokens"], x.beta,
                                      x.layout, length_normalise=True, sft_alpha=1.0)
        else:
            loss = O.dpo_loss(fwd["logp_sum"], fwd["logp_sum"] + x.ref_noise[rows], x.beta, x.layout)
        O.head_backward(x.hidden[rows], x.w_vocab, tg, mask, fwd["lse"], loss["weight"])
        what = "fwd+loss+bwd" + ({"logits-means": " with logits-mean sums",
                                   "loss-variant": " with the length-normalised loss and NLL term"}.get(row, ""))
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "completion tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {'pair' if sample_pairs == 1 else f'{sample_pairs} pairs'}, "
                      f"{f'{sample_tokens} completion positions per row' if sample_tokens > 0 else 'every completion position'} "
                      f"({n} tokens), {what}, {dt:.1f} s"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    from preference_alignment_amd import dpo_head as D
    from preference_alignment_amd import workloads as W

    dev = torch.device("cuda:0")
    if a.copy_calibration:
        n = a.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return
    D.lib()  # fail loudly if the HIP library is missing
    row = a.row
    if row == "f32-logits":
        a.workload = 5
    if row in ("loss-variant", "vocab-shard", "logits-means") and a.workload not in (2, 4):
        print(json.dumps({"error": f"--row {row} runs on the fused head workloads 2 or 4"}))
        sys.exit(2)
    if row == "f32-logits":
        _, kw = W.WORKLOADS[5]
        kw = {k: v for k, v in kw.items() if k != "kind"}
        x = W.make_logits_inputs(name="workload5", seed=5, logits_dtype="f32", **kw)
    else:
        x = W.make_workload(a.workload)
    n_c = x.n_completion
    print(f"[bench] workload {a.workload}: {W.WORKLOADS[a.workload][0]}; N_c={n_c}; row {row}", file=sys.stderr,
          flush=True)
    shards = 4
    if a.workload == 5:
        runner = LogitsStep(x, dev)
    elif row == "vocab-shard":
        runner = ShardStep(x, dev, shards)
    else:
        runner = HeadStep(x, dev, forward_only=(a.workload == 3), loss_variant=(row == "loss-variant"),
                          metrics=(row == "logits-means"))

    for _ in range(a.warmup):
        runner.step()
    torch.cuda.synchronize()

    # the kernels the roofline may name: the contractions, or the two streams
    sfx = "_f32" if row == "f32-logits" else ""
    if a.workload == 5:
        candidates = ["stream_fwd" + sfx, "stream_bwd" + sfx]
    elif a.workload == 3:
        candidates = ["fwd_gemm"]
    else:
        candidates = ["fwd_gemm", "dlogits_gemm", "dhidden_gemm", "dw_gemm"]
    kernels, kernels_steps, dom = {}, a.steps, candidates[-1]
    if not a.no_kernel_timing:
        if a.all_kernel_timing:
            D.dpo_profile_select(None)
        else:
            # an untimed pass with every kernel bracketed by events gives the
            # per-kernel breakdown and the dominant kernel (the most time per
            # step); only that kernel carries events in the timed region
            D.dpo_profile_select(None)
            D.dpo_profile_enable(True)
            for _ in range(a.profile_steps):
                runner.step()
            torch.cuda.synchronize()
            kernels, kernels_steps = D.dpo_profile_read(), a.profile_steps
            D.dpo_profile_enable(False)
            tot = {k: kernels[k][0] for k in candidates if k in kernels}
            dom = max(tot, key=tot.get) if tot else candidates[-1]
            D.dpo_profile_select(dom)
        D.dpo_profile_enable(True)
    stream = torch.cuda.current_stream(dev)
    # an event between consecutive steps gives each step's time (for the
    # median) while the first and last bracket the whole timed region
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    ev[0].record(stream)
    for i in range(a.steps):
        runner.step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host
    ms = ev[0].elapsed_time(ev[-1])
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(a.steps))
    ms_median = float(np.median(step_ms))
    timed_kernels = {}
    if not a.no_kernel_timing:
        timed_kernels = D.dpo_profile_read()
        D.dpo_profile_enable(False)
        D.dpo_profile_select(None)
        if a.all_kernel_timing:
            kernels, kernels_steps = timed_kernels, a.steps
            tot = {k: kernels[k][0] for k in candidates if k in kernels}
            dom = max(tot, key=tot.get) if tot else candidates[-1]
    ms_step = ms / a.steps
    value = n_c * a.steps / (ms / 1e3)

    H, V = x.H, x.V
    label = str(a.workload) + {"main": "", "f32-logits": " f32", "vocab-shard": " shard4",
                               "loss-variant": " loss-variant", "logits-means": " logits-means"}[row]
    kern_avg = {k: (v[0] / v[1], v[1]) for k, v in kernels.items()}
    # the dominant kernel's average launch time over the timed region
    avg = timed_kernels[dom][0] / timed_kernels[dom][1] if dom in timed_kernels else None
    dom_launches = timed_kernels[dom][1] / a.steps if dom in timed_kernels else 1.0
    if a.workload == 5:
        E = x.rows * x.T * V
        eb = 4.0 if row == "f32-logits" else 2.0
        per_kernel_bytes = {"stream_fwd" + sfx: n_c * V * eb, "stream_bwd" + sfx: n_c * V * eb + E * eb}
        ach = per_kernel_bytes[dom] / (avg / 1e3) / 1e9 if avg else None
        roof = {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS if ach else None,
                "traffic": measured_traffic(dom, label), "avg_ms": avg,
                "algorithmic_bytes_per_launch": per_kernel_bytes[dom]}
        step_bytes = n_c * V * eb * 2 + E * eb
        extra = {"step_hbm_frac": step_bytes / (ms_step / 1e3) / 1e9 / PEAK_HBM_GBS,
                 "step_hbm_frac_median": step_bytes / (ms_median / 1e3) / 1e9 / PEAK_HBM_GBS,
                 "kernels_ms_per_step": {k: round(v[0] / kernels_steps, 4) for k, v in kernels.items()}}
    else:
        gemms = candidates
        Vw = runner.Vs if row == "vocab-shard" else V
        flops_step = 2.0 * n_c * H * Vw   # each contraction, per step
        # the backward contractions run once per vocabulary slice: the dominant
        # one is the one with the most time per step, and its algorithmic flops
        # per launch are its per-step flops over its launches per step
        flops = flops_step / dom_launches
        ach = flops / (avg / 1e3) / 1e12 if avg else None
        roof = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS if ach else None,
                "frac_of_unit_count_peak": ach / PEAK_BF16_TFLOPS_UNITS if ach else None,
                "traffic": measured_traffic(dom, label), "avg_ms": avg,
                "algorithmic_flops_per_launch": flops}
        # the step's contractions: 4 x 2 H V flops per completion token for the
        # fused step (the recomputed forward included), 3 x 2 H V useful
        step_flops = flops_step * len(gemms)
        useful = flops_step * (1 if a.workload == 3 else 3)
        tf = 1.0 / (ms_step / 1e3) / 1e12
        tf_med = 1.0 / (ms_median / 1e3) / 1e12
        extra = {"step_mfma_frac": step_flops * tf / PEAK_BF16_TFLOPS,
                 "step_useful_mfma_frac": useful * tf / PEAK_BF16_TFLOPS,
                 "step_mfma_frac_of_unit_count_peak": step_flops * tf / PEAK_BF16_TFLOPS_UNITS,
                 "step_useful_mfma_frac_of_unit_count_peak": useful * tf / PEAK_BF16_TFLOPS_UNITS,
                 "step_mfma_frac_median": step_flops * tf_med / PEAK_BF16_TFLOPS,
                 "peaks_tflops": {"published": PEAK_BF16_TFLOPS, "unit_count": round(PEAK_BF16_TFLOPS_UNITS, 1)},
                 "kernels_ms_per_step": {k: round(v[0] / kernels_steps, 4) for k, v in kernels.items()}}

    also = None
    if a.workload == 2 and row == "main" and not a.no_also:
        print("[bench] also: the materialised-logits path at workload 5's shape", file=sys.stderr, flush=True)
        also = {"workload5_logits_path": also_logits_path(dev)}

    cpu = None
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        given_logits = x.logits is not None
        pairs = a.cpu_sample_pairs if a.cpu_sample_pairs is not None else (
            min(2, x.num_pairs) if (given_logits or a.workload == 3) else 1)
        cpu = cpu_baseline(x, a.workload, a.cpu_sample_tokens, row, runner.Vs if row == "vocab-shard" else None,
                           pairs)

    metric = METRICS[a.workload] if row == "main" else ROW_METRICS[row].format(
        H=H, V=V, Vs=getattr(runner, "Vs", V))
    line = {
        "metric": metric, "value": value, "unit": "completion tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_step, "ms_per_step_median": ms_median,
        "ms_per_step_min": step_ms[0], "ms_per_step_max": step_ms[-1],
        "value_median": n_c / (ms_median / 1e3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if row == "f32-logits" else "bf16",
        "data": "synthetic",
        "config": {"workload": f"workload{a.workload}: {W.WORKLOADS[a.workload][0]}"
                               + ("" if row == "main" else f"; row {row}"), "rows": x.rows,
                   "seq_len": x.T, "hidden": H, "vocab": V, "completion_tokens": n_c,
                   "parallelism": "single GPU" if row != "vocab-shard" else
                   f"one GPU's share of a {shards}-way vocabulary split (V/{shards} = {runner.Vs})"},
        "roofline": roof, "cpu_baseline": cpu,
        "kernels_ms_avg": {k: round(v[0], 4) for k, v in kern_avg.items()},
        "kernel_timing": None if a.no_kernel_timing else {
            "events_in_timed_region": "every kernel" if a.all_kernel_timing else dom,
            "breakdown_from": "timed region" if a.all_kernel_timing else f"{kernels_steps} untimed steps"},
        "host_wall_s": t_host,
    }
    line.update(extra)
    if also is not None:
        line["also"] = also
    s = json.dumps(line)
    print(s, flush=True)
    if a.out:
        with open(a.out, "w") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
