"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the whole path over one batch: the host allocator
appends the step's tokens (one per sequence for decode, the chunk for
prefill) and packs block tables, slots and lengths into pinned buffers; they
are copied to the device; copy-on-write copies run if any; the new K/V rows
are written with pa_reshape_and_cache; then pa_decode (or pa_prefill_chunk)
runs.  Inputs (pool contents, new rows, queries) are resident in HBM before
the timed region.  The default workload is the LLaMA-13B-shaped decode
batch.  One JSON line is printed.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_kv_cache_166_amd as pa  # noqa: E402
import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "pa_decode KV GB/s and % of HBM peak; decode tokens/s at LLaMA-13B shape"
ELEM = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Pinned:
    """Two sets of pinned host buffers (alternating steps) and one device set."""

    def __init__(self, shapes, device):
        self.host = [{k: torch.empty(s, dtype=d, pin_memory=True) for k, (s, d) in shapes.items()}
                     for _ in range(2)]
        self.np = [{k: t.numpy() for k, t in h.items()} for h in self.host]
        self.dev = {k: torch.empty(s, dtype=d, device=device) for k, (s, d) in shapes.items()}
        self.done = [torch.cuda.Event(), torch.cuda.Event()]
        for e in self.done:
            e.record()

    def begin(self, k):
        b = k % 2
        self.done[b].synchronize()     # copies out of this buffer (two steps ago) finished
        return self.np[b]

    def upload(self, k):
        b = k % 2
        for name, t in self.host[b].items():
            self.dev[name].copy_(t, non_blocking=True)
        self.done[b].record()
        return self.dev


# ------------------------------------------------------------------ decode

class DecodeBench:
    """Decode steps over a batch: one new token per sequence per step."""

    def __init__(self, workload, steps, warmup, device):
        self.name = workload
        cfg = W.CONFIGS[workload]
        self.cfg = cfg
        self.device = device
        self.kv = cfg["kv_dtype"]
        self.qdt = cfg["q_dtype"]
        self.H, self.D, self.bs = cfg["num_heads"], cfg["head_dim"], cfg["block_size"]
        total = steps + warmup
        if workload == "llama13b_decode":
            self.B = cfg["batch"]
            lens0 = [int(x) for x in W.uniform_ints(cfg["seed"], self.B, cfg["len_lo"], cfg["len_hi"])]
            self.N = cfg["num_blocks"]
            self.pb = 0
        elif workload == "prefix_cow":
            self.B = cfg["batch"]
            suffix = W.uniform_ints(cfg["seed"], self.B, cfg["suffix_lo"], cfg["suffix_hi"])
            lens0 = [cfg["prefix"] + int(s) + 1 for s in suffix]
            self.N = cfg["num_blocks"]
            self.pb = 0
        elif workload == "long_fp8_decode":
            self.B = cfg["batch"]
            lens0 = [cfg["context"]] * self.B
            # room for the timed steps' growth beyond the 16384 blocks of the context
            self.N = cfg["num_blocks"] + self.B * (-(-total // self.bs) + 1)
            self.pb = cfg["partition_blocks"]
        else:
            raise ValueError(workload)
        self.lens0 = lens0
        self.alloc = pa.Allocator(self.N, self.bs, W.free_order(cfg["seed"], self.N))
        self.pool = pa.PagedPool.empty(self.N, self.H, self.bs, self.D, self.kv, device)
        g = torch.Generator(device=device)
        g.manual_seed(cfg["seed"])
        for t in (self.pool.k_cache, self.pool.v_cache):
            if self.kv == "fp8":
                # codes of N(0,1)/scale values: draw normal values, take the codes
                for i in range(0, self.N, 1024):
                    x = torch.randn((min(1024, self.N - i),) + tuple(t.shape[1:]), generator=g,
                                    device=device) * 40.0
                    t[i:i + x.shape[0]] = x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
            else:
                t.copy_(torch.randn(t.shape, generator=g, device=device).to(t.dtype))
        if self.kv == "fp8":
            self.pool.k_scale.fill_(1.0 / 40.0)
            self.pool.v_scale.fill_(1.0 / 40.0)
        # sequences: the prompt holds every token but the step's own
        if workload == "prefix_cow":
            self.alloc.alloc_prompt(0, cfg["prefix"])
            for i in range(1, self.B):
                self.alloc.fork(0, i)
            for i in range(self.B):
                self.alloc.append_tokens(i, lens0[i] - 1 - cfg["prefix"])
        else:
            for i in range(self.B):
                self.alloc.alloc_prompt(i, lens0[i] - 1)
        self.ids = np.arange(self.B, dtype=np.int64)
        self.maxb = -(-(max(lens0) + total) // self.bs)
        self.bufs = Pinned({"slots": ((self.B, 1), torch.int64),
                            "tables": ((self.B, self.maxb), torch.int32),
                            "lens": ((self.B,), torch.int32),
                            "cow": ((self.B, 2), torch.int32)}, device)
        tdt = pa.TORCH_DTYPE
        in_dt = tdt["bf16"] if self.kv == "fp8" else tdt[self.kv]
        self.knew = [torch.randn((self.B, self.H, self.D), generator=g, device=device).to(in_dt)
                     for _ in range(4)]
        self.vnew = [torch.randn((self.B, self.H, self.D), generator=g, device=device).to(in_dt)
                     for _ in range(4)]
        self.q = [torch.randn((self.B, self.H, self.D), generator=g, device=device).to(tdt[self.qdt])
                  for _ in range(4)]
        self.out = torch.empty((self.B, self.H, self.D), dtype=tdt[self.qdt], device=device)
        self.ws = pa.decode_workspace(self.pool, self.B, self.maxb, self.pb)
        self.scale = 1 / math.sqrt(self.D)
        self.ev = []
        self.step_bytes = []
        self.cows = 0

    def step(self, k, timed):
        h = self.bufs.begin(k)
        _, _, ncow = self.alloc.append_tokens_batch(self.ids, 1, slots_out=h["slots"],
                                                     cow_out=h["cow"])
        self.alloc.pack(self.ids, self.maxb, tables_out=h["tables"], lens_out=h["lens"])
        lens = h["lens"].copy()
        d = self.bufs.upload(k)
        if ncow:
            pairs = d["cow"][torch.from_numpy(h["cow"][:, 0] >= 0).to(self.device)]
            pa.pa_copy_blocks(self.pool, pairs.contiguous())
            self.cows += ncow
        pa.pa_reshape_and_cache(self.pool, self.knew[k % 4], self.vnew[k % 4], d["slots"].view(-1))
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        pa.pa_decode(self.out, self.q[k % 4], self.pool, d["tables"], d["lens"], self.scale, self.pb,
                     self.ws)
        if timed:
            e1.record()
            self.ev.append((e0, e1))
            self.step_bytes.append(self.decode_bytes(lens))

    def decode_bytes(self, lens):
        """Algorithmic bytes of one pa_decode launch: every cached K and V row
        once, q, out, the table entries read and the lengths."""
        row = self.H * self.D * ELEM[self.kv]
        kv = 2 * int(np.sum(lens)) * row
        qo = self.B * self.H * self.D * (ELEM[self.qdt] * 2)
        tables = int(np.sum(-(-lens // self.bs))) * 4 + self.B * 4
        scales = 0
        if self.kv == "fp8":
            scales = 2 * int(np.sum(-(-lens // self.bs))) * self.H * 4
        return kv + qo + tables + scales

    def kernel_stats(self):
        times = [a.elapsed_time(b) * 1e-3 for a, b in self.ev]
        t = float(np.mean(times))
        bytes_ = float(np.mean(self.step_bytes))
        return t, bytes_

    def workload_config(self):
        c = self.cfg
        d = {"workload": self.name, "batch": self.B, "num_heads": self.H, "head_dim": self.D,
             "block_size": self.bs, "kv_dtype": self.kv, "q_dtype": self.qdt,
             "pool_blocks": self.N, "mean_context": float(np.mean(self.lens0))}
        if self.name == "llama13b_decode":
            d["context_lens"] = f"uniform[{c['len_lo']},{c['len_hi']}] seed {c['seed']}"
        d["partition_blocks"] = self.pb or pa.pa_decode_auto_partition_blocks(self.pool, self.B,
                                                                              self.maxb)
        return d

    def cpu_baseline(self, budget_s=12.0):
        """The oracle on the same shape: (sequence, head) decodes of the batch
        at the prompt lengths (pool rows filled by torch before any library
        write), in order, until the budget is spent; only the oracle call is
        timed."""
        from oracle import attention as A
        rng = np.random.default_rng(0)
        pairs = [(i, h) for h in range(self.H) for i in range(self.B)]
        done_bytes, n, spent = 0, 0, 0.0
        for i, h in pairs:
            L = self.lens0[i] - 1
            nb = -(-L // self.bs)
            idx = torch.tensor(self.alloc.block_table(i)[:nb], dtype=torch.int64, device=self.device)
            kp = _bits(self.pool.k_cache[idx, h:h + 1])
            vp = _bits(self.pool.v_cache[idx, h:h + 1])
            ks = vs = None
            if self.kv == "fp8":
                ks = self.pool.k_scale[idx, h:h + 1].cpu().numpy()
                vs = self.pool.v_scale[idx, h:h + 1].cpu().numpy()
            q = rng.standard_normal((1, 1, self.D))
            t0 = time.perf_counter()
            A.decode(q, kp, vp, self.kv, [list(range(nb))], [L], self.bs, self.scale, ks, vs)
            spent += time.perf_counter() - t0
            done_bytes += 2 * L * self.D * ELEM[self.kv]
            n += 1
            if spent >= budget_s:
                break
        return {"value": done_bytes / spent / 1e9, "unit": "GB/s", "cores": _cores(),
                "kind": "oracle",
                "sample": f"{n} of {len(pairs)} (sequence, head) decodes of this workload's batch, "
                          f"{spent:.1f} s of oracle time, float64 NumPy"}


# ------------------------------------------------------------------ prefill

class PrefillBench:
    """Chunked prefill: each step allocates a batch (context + chunk), writes
    the chunk's K/V, runs pa_prefill_chunk, then frees the batch."""

    def __init__(self, steps, warmup, device):
        cfg = W.CONFIGS["chunked_prefill"]
        self.cfg, self.name, self.device = cfg, "chunked_prefill", device
        self.B, self.S, self.H, self.D, self.bs = (cfg["batch"], cfg["chunk"], cfg["num_heads"],
                                                   cfg["head_dim"], cfg["block_size"])
        self.kv = "bf16"
        self.ctx = [int(c) for c in W.uniform_ints(cfg["seed"], self.B, cfg["ctx_lo"], cfg["ctx_hi"])]
        self.N = cfg["num_blocks"]
        self.alloc = pa.Allocator(self.N, self.bs, W.free_order(cfg["seed"], self.N))
        self.pool = pa.PagedPool.empty(self.N, self.H, self.bs, self.D, "bf16", device)
        g = torch.Generator(device=device)
        g.manual_seed(cfg["seed"])
        for t in (self.pool.k_cache, self.pool.v_cache):
            t.copy_(torch.randn(t.shape, generator=g, device=device).to(torch.bfloat16))
        T = self.B * self.S
        self.knew = torch.randn((T, self.H, self.D), generator=g, device=device).to(torch.bfloat16)
        self.vnew = torch.randn((T, self.H, self.D), generator=g, device=device).to(torch.bfloat16)
        self.q = torch.randn((T, self.H, self.D), generator=g, device=device).to(torch.bfloat16)
        self.out = torch.empty((T, self.H, self.D), dtype=torch.bfloat16, device=device)
        self.maxb = -(-(max(self.ctx) + self.S) // self.bs)
        self.bufs = Pinned({"slots": ((self.B, self.S), torch.int64),
                            "tables": ((self.B, self.maxb), torch.int32),
                            "lens": ((self.B,), torch.int32)}, device)
        self.qsl = torch.tensor(np.arange(self.B + 1) * self.S, dtype=torch.int32, device=device)
        self.scale = 1 / math.sqrt(self.D)
        self.ev, self.next_id = [], 0

    def step(self, k, timed):
        h = self.bufs.begin(k)
        ids = np.arange(self.next_id, self.next_id + self.B, dtype=np.int64)
        self.next_id += self.B
        for j, s in enumerate(ids):
            self.alloc.alloc_prompt(int(s), self.ctx[j])
        self.alloc.append_tokens_batch(ids, self.S, slots_out=h["slots"])
        self.alloc.pack(ids, self.maxb, tables_out=h["tables"], lens_out=h["lens"])
        d = self.bufs.upload(k)
        pa.pa_reshape_and_cache(self.pool, self.knew, self.vnew, d["slots"].view(-1))
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        pa.pa_prefill_chunk(self.out, self.q, self.pool, d["tables"], d["lens"], self.qsl, self.S,
                            self.scale)
        if timed:
            e1.record()
            self.ev.append((e0, e1))
        for s in ids:
            self.alloc.free_seq(int(s))

    def flops(self):
        """Causal FLOPs of one launch: 4*D*H per (query, visible key) pair."""
        pairs = sum(self.S * c + self.S * (self.S + 1) // 2 for c in self.ctx)
        return 4.0 * self.D * self.H * pairs

    def kernel_stats(self):
        t = float(np.mean([a.elapsed_time(b) * 1e-3 for a, b in self.ev]))
        return t, self.flops()

    def workload_config(self):
        c = self.cfg
        return {"workload": self.name, "batch": self.B, "chunk": self.S, "num_heads": self.H,
                "head_dim": self.D, "block_size": self.bs, "kv_dtype": "bf16",
                "context": f"uniform[{c['ctx_lo']},{c['ctx_hi']}] seed {c['seed']}: {self.ctx}",
                "pool_blocks": self.N}

    def cpu_baseline(self, budget_s=12.0):
        from oracle import attention as A
        rng = np.random.default_rng(0)
        t0 = time.perf_counter()
        flops = 0.0
        i = 0
        while time.perf_counter() - t0 < budget_s:
            L = self.ctx[i % self.B] + self.S
            K = rng.standard_normal((L, self.D))
            V = rng.standard_normal((L, self.D))
            qh = rng.standard_normal((self.S, self.D))
            A.attend(qh, K, V, self.scale, A.chunk_visible(L, self.S))
            flops += 4.0 * self.D * (self.S * (L - self.S) + self.S * (self.S + 1) // 2)
            i += 1
        dt = time.perf_counter() - t0
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": _cores(), "kind": "oracle",
                "sample": f"{i} (sequence, head) chunk attentions of this workload, {dt:.1f} s, "
                          "float64 NumPy"}


def _bits(t):
    t = t.cpu()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.uint8).numpy()


def _cores():
    n = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        return int(min(n, blas))
    except Exception:
        return n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama13b_decode",
                    choices=["llama13b_decode", "prefix_cow", "chunked_prefill", "long_fp8_decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(each GPU would hold its own pool and batch; see the sharding notes).",
              file=sys.stderr)
        sys.exit(2)
    device = "cuda:0"
    torch.cuda.set_device(0)
    log(f"bench: workload={args.workload} steps={args.steps} warmup={args.warmup}")
    if args.workload == "chunked_prefill":
        b = PrefillBench(args.steps, args.warmup, device)
    else:
        b = DecodeBench(args.workload, args.steps, args.warmup, device)
    torch.cuda.synchronize()
    for k in range(args.warmup):
        b.step(k, False)
    torch.cuda.synchronize()
    log("bench: warmup done")
    t0 = time.perf_counter()
    for k in range(args.warmup, args.warmup + args.steps):
        b.step(k, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("bench: timed steps done")
    ms = wall / args.steps * 1e3
    kt, work = b.kernel_stats()
    res = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "data": "synthetic",
           "config": b.workload_config()}
    if args.workload == "chunked_prefill":
        res.update(metric="pa_prefill_chunk TFLOP/s (causal) at the chunked-prefill workload",
                   value=work / (wall / args.steps) / 1e12, unit="TFLOP/s", dtype="bf16")
        ach = work / kt / 1e12
        res["roofline"] = {"bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS, "traffic": None,
                           "kernel": "prefill_kernel", "kernel_us": kt * 1e6}
    else:
        kv_bytes = work
        res.update(metric=METRIC if args.workload == "llama13b_decode"
                   else f"pa_decode KV GB/s at the {args.workload} workload",
                   value=kv_bytes / (wall / args.steps) / 1e9, unit="GB/s", dtype=b.kv)
        ach = kv_bytes / kt / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS, "traffic": None, "kernel": "decode_kernel",
                           "kernel_us": kt * 1e6, "bytes_per_launch": kv_bytes}
        res["decode_tokens_per_s"] = b.B / (wall / args.steps)
        res["decode_tokens_per_s_40_layers"] = b.B / (40 * wall / args.steps)
        res["pa_decode_tokens_per_s"] = b.B / kt
    if not args.no_cpu_baseline:
        log("bench: cpu baseline")
        res["cpu_baseline"] = b.cpu_baseline()
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
