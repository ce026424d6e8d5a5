"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the whole path over one batch: the host allocator
appends the step's tokens (one per sequence for decode, the chunk for
prefill) and packs block tables, slots and lengths into one pinned buffer,
which is copied to the device once; then, for every attention layer the step
serves, copy-on-write block copies (if any) and one decode launch that also
stores the step's new K/V rows into that layer's pool (pa_decode_append;
pa_decode_shared_prefix_append for the shared-prefix batch) -- or, for
prefill, pa_reshape_and_cache of the chunk and pa_prefill_chunk.  The default workload is a decode step of an
attention-only model with the LLaMA-13B shape (40 layers of 40 heads x 128,
fp16 KV, 16-token blocks, 32 sequences of 128..2048 tokens); the block
tables are shared by all layers, each layer has its own pool.  Pool contents,
new rows and queries are resident in HBM before the timed region.  One JSON
line is printed.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--layers N] [--partition-blocks P] [--no-cpu-baseline]
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


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` at `workload` from the rocprofv3 PMC
    summaries in profiles/ (FETCH_SIZE + WRITE_SIZE, scaled by a plain-copy
    calibration), or None when there is none or the kernel's sources changed
    since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if "<!-- traffic:" not in line:
                continue
            rec = json.loads(line.split("<!-- traffic:", 1)[1].rsplit("-->", 1)[0])
            if rec.get("workload") != workload or kernel not in rec.get("kernel", ""):
                continue
            h = hashlib.sha256()
            for f in rec["src"]:
                h.update(open(os.path.join(ROOT, f), "rb").read())
            if h.hexdigest()[:16] != rec["src_sha256"]:
                return None
            return rec["traffic_bytes_per_launch"]
    return None


def spread(seconds):
    """Median, 10th and 90th percentile of event-timed launches, in us."""
    us = np.asarray(seconds) * 1e6
    return {"launches": int(us.size), "p10": float(np.percentile(us, 10)),
            "median": float(np.median(us)), "p90": float(np.percentile(us, 90))}


class Timer:
    """HIP events (torch.cuda.Event, timing enabled) recorded on the launch
    stream immediately before and after one call."""

    def __init__(self):
        self.e0 = torch.cuda.Event(enable_timing=True)
        self.e1 = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.e0.record()

    def stop(self):
        self.e1.record()

    def seconds(self):
        return self.e0.elapsed_time(self.e1) * 1e-3


def warm_clocks(call, seconds=2.0):
    """Back-to-back calls for about `seconds` before a timed series.  The GPU
    lowers its clocks while it idles (the CPU baseline, host work between
    series) and needs a second or more of load to return to its sustained
    clocks; a series of a few milliseconds right after an idle period would
    time the ramp (up to 20% slower)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            call()
        torch.cuda.synchronize()


def loop_seconds(call, n, warm=2, warm_s=2.0):
    """Mean duration of one call over n back-to-back calls on the current
    stream, bracketed by one event pair (no event between launches: an event
    record waits for the caches' write-back and would add its cost to every
    launch it brackets), after warm_clocks(call, warm_s)."""
    warm_clocks(call, warm_s)
    for _ in range(warm):
        call()
    tm = Timer()
    tm.start()
    for _ in range(n):
        call()
    tm.stop()
    torch.cuda.synchronize()
    return tm.seconds() / n


class Staging:
    """Per-step host->device inputs (slots, tables, lengths, copy pairs)
    packed into one pinned buffer and sent with one copy on the compute
    stream.  Two pinned buffers alternate steps so the host never rewrites
    one that a queued copy has not read yet."""

    def __init__(self, shapes, device):
        self.layout, off = {}, 0
        for k, (shape, dt) in shapes.items():
            n = int(np.prod(shape)) * torch.empty((), dtype=dt).element_size()
            self.layout[k] = (off, shape, dt, n)
            off += (n + 255) // 256 * 256
        self.host = [torch.empty(off, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        self.devb = torch.empty(off, dtype=torch.uint8, device=device)
        self.np = [self._views(h, numpy=True) for h in self.host]
        self.dev = self._views(self.devb)
        self.copied = [torch.cuda.Event(), torch.cuda.Event()]
        for e in self.copied:
            e.record()

    def _views(self, buf, numpy=False):
        out = {}
        for k, (off, shape, dt, n) in self.layout.items():
            v = buf[off:off + n].view(dt).view(shape)
            out[k] = v.numpy() if numpy else v
        return out

    def begin(self, k):
        b = k % 2
        self.copied[b].synchronize()     # the copy out of this pinned buffer has run
        return self.np[b]

    def upload(self, k):
        b = k % 2
        self.devb.copy_(self.host[b], non_blocking=True)
        self.copied[b].record()
        return self.dev



# ------------------------------------------------------------------ decode

class DecodeBench:
    """Decode steps over a batch: one new token per sequence per step.

    A step serves `layers` attention layers: one host allocation and one
    upload of slots / tables / lengths (shared by every layer, as block tables
    are), then, per layer, one decode launch over that layer's pool that also
    stores the step's K/V rows (fused=False: pa_reshape_and_cache, then
    pa_decode)."""

    def __init__(self, workload, steps, warmup, device, partition_blocks=None, layers=None,
                 stream_kv=None, fused=None):
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
            self.layers = 40 if layers is None else layers   # LLaMA-13B has 40 layers
        elif workload == "prefix_cow":
            self.B = cfg["batch"]
            suffix = W.uniform_ints(cfg["seed"], self.B, cfg["suffix_lo"], cfg["suffix_hi"])
            lens0 = [cfg["prefix"] + int(s) + 1 for s in suffix]
            self.N = cfg["num_blocks"]
            self.pb = 0
            self.layers = 1 if layers is None else layers
        elif workload == "long_fp8_decode":
            self.B = cfg["batch"]
            lens0 = [cfg["context"]] * self.B
            # room for the timed steps' growth beyond the 16384 blocks of the context
            self.N = cfg["num_blocks"] + self.B * (-(-total // self.bs) + 1)
            self.pb = cfg["partition_blocks"]
            self.layers = 1 if layers is None else layers
        else:
            raise ValueError(workload)
        if partition_blocks is not None:
            self.pb = partition_blocks
        # the pools' stream flag: only when no block is shared by two sequences
        # (every workload but the shared-prefix one)
        self.stream_kv = (workload != "prefix_cow") if stream_kv is None else stream_kv
        # fp8: the step's appended tokens keep each block's scale at its amax / 448
        self.auto_scale = self.kv == "fp8"
        # the step's new rows are stored by the decode launch itself
        # (pa_decode_append; fp8 pools quantise them there, with scale upkeep),
        # or (fused=False) written by pa_reshape_and_cache first
        self.fused = True if fused is None else fused
        self.lens0 = lens0
        self.alloc = pa.Allocator(self.N, self.bs, W.free_order(cfg["seed"], self.N))
        g = torch.Generator(device=device)
        g.manual_seed(cfg["seed"])
        self.pools = [self._filled_pool(g) for _ in range(self.layers)]
        self.pool = self.pools[0]
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
        self.bufs = Staging({"slots": ((self.B, 1), torch.int64),
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
        # tables that begin with the same blocks (the shared-prefix workload):
        # the step decodes with pa_decode_shared_prefix_append, the prefix
        # read once for the whole batch
        self.shared = 0
        if self.fused and workload == "prefix_cow":
            t, ln = self.alloc.pack(self.ids, self.maxb)
            self.shared = pa.shared_prefix_blocks(t, ln + 1, self.bs)
            self.ws_sp = pa.shared_prefix_workspace(self.pool, self.B, self.maxb, self.shared,
                                                    self.pb)
        self.scale = 1 / math.sqrt(self.D)
        self.ev = []
        self.step_bytes = []
        self.step_unique = []
        self.cows = 0

    def _filled_pool(self, g):
        pool = pa.PagedPool.empty(self.N, self.H, self.bs, self.D, self.kv, self.device,
                                  stream_kv=self.stream_kv, fp8_auto_scale=self.auto_scale)
        for t in (pool.k_cache, pool.v_cache):
            for i in range(0, self.N, 1024):
                n = min(1024, self.N - i)
                x = torch.randn((n,) + tuple(t.shape[1:]), generator=g, device=self.device)
                if self.kv == "fp8":
                    # codes of values drawn N(0, 40^2) with scale 1/40: N(0,1) after scaling
                    t[i:i + n] = (x * 40.0).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
                else:
                    t[i:i + n] = x.to(t.dtype)
        if self.kv == "fp8":
            pool.k_scale.fill_(1.0 / 40.0)
            pool.v_scale.fill_(1.0 / 40.0)
        return pool

    def step(self, k, timed):
        h = self.bufs.begin(k)
        _, _, ncow = self.alloc.append_tokens_batch(self.ids, 1, slots_out=h["slots"],
                                                     cow_out=h["cow"])
        self.alloc.pack(self.ids, self.maxb, tables_out=h["tables"], lens_out=h["lens"])
        lens = h["lens"].copy()
        d = self.bufs.upload(k)
        pairs = None
        if ncow:
            pairs = d["cow"][torch.from_numpy(h["cow"][:, 0] >= 0).to(self.device)].contiguous()
            self.cows += ncow
        if pairs is not None:
            for pool in self.pools:
                pa.pa_copy_blocks(pool, pairs)
        # 16-bit pools: one event pair around the step's layers, one launch
        # (pa_decode_append: decode kernel + merge kernel) per layer back to
        # back, so the mean launch is the bracket / layers with no event
        # inside it.  fp8 pools (a cache write before each decode): the pair
        # brackets one decode launch of a middle layer.
        if timed and self.fused:
            tm_all = Timer()
            tm_all.start()
        for li, pool in enumerate(self.pools):
            if not self.fused:
                pa.pa_reshape_and_cache(pool, self.knew[(k + li) % 4], self.vnew[(k + li) % 4],
                                        d["slots"].view(-1))
            timing = timed and not self.fused and li == len(self.pools) // 2
            if timing:
                tm = Timer()
                tm.start()
            j = (k + li) % 4
            if self.shared:
                call = lambda pool=pool, j=j: pa.pa_decode_shared_prefix_append(
                    self.out, self.q[j], pool, self.knew[j], self.vnew[j], d["slots"].view(-1),
                    d["tables"], d["lens"], self.shared, self.scale, self.pb, self.ws_sp)
            elif self.fused:
                call = lambda pool=pool, j=j: pa.pa_decode_append(
                    self.out, self.q[j], pool, self.knew[j], self.vnew[j], d["slots"].view(-1),
                    d["tables"], d["lens"], self.scale, self.pb, self.ws)
            else:
                call = lambda pool=pool, j=j: pa.pa_decode(
                    self.out, self.q[j], pool, d["tables"], d["lens"], self.scale, self.pb, self.ws)
            call()
            # the call again stores the same rows at the same slots: a replay
            # leaves the pool as the step left it
            self.last_call = call
            if timing:
                tm.stop()
                self.ev.append(tm)
        if timed and self.fused:
            tm_all.stop()
            self.ev.append(tm_all)
        if timed:
            self.step_bytes.append(self.decode_bytes(lens))
            self.step_unique.append(self.unique_bytes(lens))
        self.last = (d, lens)

    def unique_bytes(self, lens):
        """Bytes of the distinct K/V rows a launch reads: for the shared-prefix
        workload the prefix once plus every sequence's own tokens; otherwise
        every row (nothing is shared)."""
        row = self.H * self.D * ELEM[self.kv]
        if self.name != "prefix_cow":
            return self.decode_bytes(lens)
        prefix = self.cfg["prefix"]
        return 2 * row * (prefix + int(np.sum(lens - prefix)))

    def fp8_write_series(self, tokens=4096, reps=20):
        """A prefill-sized fp8 write: `tokens` bf16 rows of K and V into fresh
        blocks of a separate pool, with scale upkeep and with caller-set
        scales (the plain write), event-timed; algorithmic bytes = the input
        rows read once + the codes and scales written."""
        H, D, bs = self.H, self.D, self.bs
        nb = -(-tokens // bs)
        res = {"tokens": tokens}
        g = torch.Generator(device=self.device)
        g.manual_seed(1)
        k = torch.randn((tokens, H, D), generator=g, device=self.device).to(torch.bfloat16)
        v = torch.randn((tokens, H, D), generator=g, device=self.device).to(torch.bfloat16)
        slots = torch.arange(tokens, dtype=torch.int64, device=self.device)
        nbytes = 2 * tokens * H * D * (2 + 1) + 2 * nb * H * 4
        for name, auto in (("upkeep", True), ("plain", False)):
            pool = pa.PagedPool.empty(nb, H, bs, D, "fp8", self.device, fp8_auto_scale=auto)
            ts = []
            for r in range(reps + 3):
                tm = Timer()
                tm.start()
                pa.pa_reshape_and_cache(pool, k, v, slots)
                tm.stop()
                torch.cuda.synchronize()
                if r >= 3:
                    ts.append(tm.seconds())
            t = float(np.median(ts))
            res[name] = {"us": t * 1e6, "GBps": nbytes / t / 1e9}
            del pool
        res["bytes"] = nbytes
        return res

    def block_sizes(self, reps=20):
        """pa_decode of the batch at its current lengths with other block
        sizes: one pool per fixed size (8, 16, 32, 64; same shuffled-pool
        construction), and one arena whose sequences take the size the size
        rule gives their length (one pa_decode per size, back to back on the
        stream, timed as one).  Event-timed medians, warm caches; bytes =
        this launch's algorithmic bytes (K/V rows, q, out; tables at each
        size).  Memory: tokens reserved (whole blocks) against tokens held.
        The pools here do not set the stream flag (ordinary loads for K and
        V), so these launches are kernels of their own in a profile, apart
        from the steps' pa_decode."""
        lens = self.lens_now()
        H, D, B = self.H, self.D, self.B
        row = H * D * ELEM[self.kv]
        tokens = int(np.sum(lens))
        g = torch.Generator(device=self.device)
        g.manual_seed(7)
        tdt = pa.TORCH_DTYPE[self.qdt]
        q = torch.randn((B, H, D), generator=g, device=self.device).to(tdt)

        def fill(*ts):
            for t in ts:
                for i in range(0, t.shape[0], 1024):
                    x = torch.randn((min(1024, t.shape[0] - i),) + tuple(t.shape[1:]), generator=g,
                                    device=self.device)
                    t[i:i + x.shape[0]] = x.to(t.dtype)

        def timed(calls):
            ts = []
            for r in range(reps + 3):
                tm = Timer()
                tm.start()
                for c in calls:
                    c()
                tm.stop()
                torch.cuda.synchronize()
                if r >= 3:
                    ts.append(tm.seconds())
            return float(np.median(ts))

        def nbytes(groups):
            b = 2 * tokens * row + B * H * D * ELEM[self.qdt] * 2 + B * 4
            return b + sum(int(np.sum(-(-ln // bs))) * 4 for bs, ln in groups)

        res = {"tokens": tokens, "fixed": {}}
        for bs in (8, 16, 32, 64):
            N = int(np.sum(-(-lens // bs))) + 64
            alloc = pa.Allocator(N, bs, W.free_order(self.cfg["seed"] + bs, N))
            for i in range(B):
                alloc.alloc_prompt(i, int(lens[i]))
            pool = pa.PagedPool.empty(N, H, bs, D, self.kv, self.device)
            fill(pool.k_cache, pool.v_cache)
            maxb = int(np.max(-(-lens // bs)))
            t, ln = alloc.pack(self.ids, maxb)
            td, lnd = torch.from_numpy(t).to(self.device), torch.from_numpy(ln).to(self.device)
            out = torch.empty_like(q)
            ws = pa.decode_workspace(pool, B, maxb, 0)
            sec = timed([lambda: pa.pa_decode(out, q, pool, td, lnd, self.scale, 0, ws)])
            nb = nbytes([(bs, lens)])
            res["fixed"][bs] = {"us": sec * 1e6, "GBps": nb / sec / 1e9,
                                "reserved_tokens": int(np.sum(-(-lens // bs) * bs))}
            del pool, alloc
        arena_tokens = -(-int(np.sum(-(-lens // 64) * 64)) // 64) * 64 + 64 * 64
        ba = pa.BuddyAllocator(arena_tokens, W.free_order(self.cfg["seed"], arena_tokens // 64))
        sizes = np.array([ba.alloc_prompt(i, int(lens[i]))[0] for i in range(B)])
        arena = pa.ArenaPool(arena_tokens, H, D, self.kv, self.device)
        fill(arena.k, arena.v)
        calls, groups, keep = [], [], []
        mpools, mtabs, mbegin, mrows = [], [], [0], []
        for bs in sorted(set(sizes.tolist())):
            idx = np.nonzero(sizes == bs)[0]
            ids = self.ids[idx]
            maxb = int(np.max(-(-lens[idx] // bs)))
            t, ln = ba.pack(ids, maxb)
            td, lnd = torch.from_numpy(t).to(self.device), torch.from_numpy(ln).to(self.device)
            qg = q[torch.from_numpy(idx).to(self.device)].contiguous()
            og = torch.empty_like(qg)
            view = arena.view(bs)
            ws = pa.decode_workspace(view, len(ids), maxb, 0)
            keep.append((td, lnd, qg, og, ws))
            calls.append(lambda v=view, qg=qg, og=og, td=td, lnd=lnd, ws=ws:
                         pa.pa_decode(og, qg, v, td, lnd, self.scale, 0, ws))
            groups.append((bs, lens[idx]))
            mpools.append(view)
            mtabs.append(td)
            mbegin.append(mbegin[-1] + len(ids))
            mrows.append(idx)
        sec = timed(calls)
        # the same batch in one pa_decode_multi launch (rows grouped by size)
        rows = torch.from_numpy(np.concatenate(mrows)).to(self.device)
        qm = q[rows].contiguous()
        om = torch.empty_like(qm)
        lm = torch.from_numpy(lens[np.concatenate(mrows)].astype(np.int32)).to(self.device)
        wsm = pa.decode_multi_workspace(mpools, [t.shape[1] for t in mtabs], B, 0)
        sec_m = timed([lambda: pa.pa_decode_multi(om, qm, mpools, mtabs, lm, mbegin, self.scale, 0,
                                                  wsm)])
        res["by_length"] = {"us": sec_m * 1e6, "GBps": nbytes(groups) / sec_m / 1e9,
                            "launch": "pa_decode_multi (one launch)",
                            "us_one_launch_per_size": sec * 1e6, "sizes": len(calls),
                            "sequences_per_size": {int(b): int(np.sum(sizes == b)) for b in set(sizes.tolist())},
                            "reserved_tokens": int(sum(int(np.sum(-(-ln // bs) * bs)) for bs, ln in groups))}
        del arena, ba, keep, qm, om, wsm
        torch.cuda.empty_cache()
        return res

    def cold_series(self, reps=10, flush_mib=512):
        """pa_decode on the middle layer with the caches cold: a read of
        flush_mib MiB (twice the 256 MB Infinity Cache) before each timed
        call, outside the event pair.  A read, not a write: a written flush
        buffer stays dirty in the Infinity Cache and the decode would then pay
        for writing it back."""
        d, lens = self.last
        pool = self.pools[len(self.pools) // 2]
        scratch = torch.ones((flush_mib << 20) // 4, dtype=torch.float32, device=self.device)
        for _ in range(2):
            scratch.sum()                 # its own dirty lines written back
        torch.cuda.synchronize()
        ts = []
        for r in range(reps):
            scratch.sum()
            tm = Timer()
            tm.start()
            pa.pa_decode(self.out, self.q[0], pool, d["tables"], d["lens"], self.scale, self.pb,
                         self.ws)
            tm.stop()
            torch.cuda.synchronize()
            ts.append(tm.seconds())
        del scratch
        t = float(np.median(ts))
        return {"kernel_us": t * 1e6, "logical_GBps": self.decode_bytes(lens) / t / 1e9,
                "unique_GBps": self.unique_bytes(lens) / t / 1e9,
                "flush": f"{flush_mib} MiB device read before each of {reps} calls"}

    def prefix_reuse(self, reps=5):
        """Prefill of the workload's 64 prompts (the shared 1024-token prefix,
        then each sequence's own tokens; token ids drawn from the seed) in
        two ways on one pool: every prompt in full, and through the prefix
        index -- request 0 in full and inserted, the other 63 allocated from
        the cache and prefilled on their own tokens only (queries against the
        whole prompt's context).  Event-timed prefill per way; host time per
        index call (C++ through ctypes)."""
        cfg = self.cfg
        H, D, bs, B, P = self.H, self.D, self.bs, self.B, cfg["prefix"]
        rng = np.random.default_rng(cfg["seed"])
        system = [int(t) for t in rng.integers(0, 32000, P)]
        own = W.uniform_ints(cfg["seed"], B, cfg["suffix_lo"], cfg["suffix_hi"])
        prompts = [system + [int(t) for t in rng.integers(0, 32000, int(n))] for n in own]
        N = sum(-(-len(p) // bs) for p in prompts) + 8
        pool = pa.PagedPool.empty(N, H, bs, D, "bf16", self.device)
        pool.k_cache.normal_()
        pool.v_cache.normal_()
        tdt = pa.TORCH_DTYPE["bf16"]

        def run(seqs, alloc, qlens):
            t, ln = alloc.pack(seqs, max(len(alloc.block_table(s_)) for s_ in seqs))
            qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
            q = torch.randn((int(qsl[-1]), H, D), device=self.device).to(tdt)
            out = torch.empty_like(q)
            args = (out, q, pool, torch.from_numpy(t).to(self.device),
                    torch.from_numpy(ln).to(self.device), torch.from_numpy(qsl).to(self.device),
                    int(max(qlens)), self.scale)
            pa.pa_prefill_chunk(*args)
            ts = []
            for _ in range(reps):
                tm = Timer()
                tm.start()
                pa.pa_prefill_chunk(*args)
                tm.stop()
                torch.cuda.synchronize()
                ts.append(tm.seconds())
            return float(np.median(ts)), int(qsl[-1])

        a_full = pa.Allocator(N, bs)
        for i, p_ in enumerate(prompts):
            a_full.alloc_prompt(i, len(p_))
        t_full, q_full = run(list(range(B)), a_full, [len(p_) for p_ in prompts])
        del a_full

        a = pa.Allocator(N, bs)
        x = pa.PrefixIndex(a)
        a.alloc_prompt(0, len(prompts[0]))
        t0 = time.perf_counter()
        x.insert(0, prompts[0])
        t_insert = time.perf_counter() - t0
        t_match = t_alloc = 0.0
        hits = []
        for i in range(1, B):
            t0 = time.perf_counter()
            x.match(prompts[i])
            t_match += time.perf_counter() - t0
            t0 = time.perf_counter()
            hit, _, _ = x.alloc_prompt_cached(i, prompts[i])
            t_alloc += time.perf_counter() - t0
            hits.append(hit)
        qlens = [len(prompts[0])] + [len(prompts[i]) - hits[i - 1] for i in range(1, B)]
        t_cached, q_cached = run(list(range(B)), a, qlens)
        del x, a, pool
        torch.cuda.empty_cache()
        return {"requests": B, "prefix_tokens": P, "hits": sorted(set(hits)),
                "query_tokens": {"full": q_full, "cached": q_cached},
                "prefill_us": {"full": t_full * 1e6, "cached": t_cached * 1e6},
                "speedup": t_full / t_cached,
                "host_us_per_call": {"insert": t_insert * 1e6, "match": t_match / (B - 1) * 1e6,
                                     "alloc_prompt_cached": t_alloc / (B - 1) * 1e6}}

    def eviction_churn(self, requests=2000, systems=16, live_max=16, generated=128):
        """Host-side serving churn on the workload's pool geometry (block 16,
        4096 blocks): requests are one of `systems` 1024-token system prompts
        plus 1..256 own tokens; each is allocated through the prefix index,
        grows by `generated` tokens, and when it finishes (oldest first, at
        most live_max in flight) is inserted whole and freed.  Finished
        conversations fill the pool with cached blocks; with automatic
        eviction the least recently used leaves make room, without it the
        allocator refuses.  Host time per index call (C++ through ctypes)."""
        cfg, bs, N = self.cfg, self.bs, self.cfg["num_blocks"]
        rng = np.random.default_rng(cfg["seed"] + 1)
        sys_prompts = [[int(t) for t in rng.integers(0, 32000, cfg["prefix"])] for _ in range(systems)]
        reqs = [(int(rng.integers(0, systems)), [int(t) for t in rng.integers(0, 32000, int(n))])
                for n in rng.integers(cfg["suffix_lo"], cfg["suffix_hi"] + 1, requests)]
        out = {"requests": requests, "systems": systems, "pool_blocks": N, "live_max": live_max}
        for mode in ("evict", "no_evict"):
            a = pa.Allocator(N, bs)
            x = pa.PrefixIndex(a, auto_evict=(mode == "evict"))
            live, toks = [], {}
            refused = hit_tok = prompt_tok = 0
            t_alloc = t_ins = 0.0
            n_alloc = n_ins = 0
            for i, (sp, own) in enumerate(reqs):
                if len(live) >= live_max:
                    s = live.pop(0)
                    t0 = time.perf_counter()
                    x.insert(s, toks.pop(s))
                    t_ins += time.perf_counter() - t0
                    n_ins += 1
                    a.free_seq(s)
                p = sys_prompts[sp] + own
                t0 = time.perf_counter()
                try:
                    hit, _, _ = x.alloc_prompt_cached(i, p)
                except RuntimeError:
                    refused += 1
                    continue
                finally:
                    t_alloc += time.perf_counter() - t0
                    n_alloc += 1
                hit_tok += hit
                prompt_tok += len(p)
                try:
                    a.append_tokens(i, generated)
                except RuntimeError:
                    refused += 1
                    a.free_seq(i)
                    continue
                live.append(i)
                toks[i] = p + [int(t) for t in rng.integers(0, 32000, generated)]
            st = x.stats()
            out[mode] = {"refused": refused, "evicted_leaves": st["evicted"],
                         "hit_token_fraction": hit_tok / max(prompt_tok, 1),
                         "host_us_per_call": {"alloc_prompt_cached": t_alloc / max(n_alloc, 1) * 1e6,
                                              "insert": t_ins / max(n_ins, 1) * 1e6}}
            del x, a
        return out

    def cow_copy_us(self, reps=10):
        """One copy-on-write block copy as the allocator issues it: fork a
        sequence whose last block is partly filled, append one token (one
        (src, dst) pair), time pa_copy_blocks of that pair, free the fork."""
        partial = np.nonzero(self.lens_now() % self.bs != 0)[0]
        if len(partial) == 0:
            return None
        src = int(self.ids[partial[0]])
        ts = []
        for r in range(reps):
            child = 1_000_000 + r
            self.alloc.fork(src, child)
            _, pair = self.alloc.append_tokens(child, 1)
            assert pair is not None
            pairs = torch.tensor([pair], dtype=torch.int32, device=self.device)
            tm = Timer()
            tm.start()
            pa.pa_copy_blocks(self.pools[0], pairs)
            tm.stop()
            torch.cuda.synchronize()
            ts.append(tm.seconds())
            self.alloc.free_seq(child)
        tile = self.H * self.bs * self.D * ELEM[self.kv]
        t = float(np.median(ts))
        return {"us": t * 1e6, "bytes": 2 * 2 * tile, "GBps": 2 * 2 * tile / t / 1e9}

    def shared_prefix_series(self, reps=20):
        """The batch at its current lengths on the middle layer's pool, warm,
        decoded two ways with the same inputs: pa_decode (every sequence
        reads the shared prefix itself) and pa_decode_shared_prefix (the
        prefix read once for the whole batch on MFMA, each sequence's own
        blocks by the decode kernel, one merge).  Mean of back-to-back calls
        under one event pair; GB/s over the logical bytes (every sequence's
        full context) and over the unique bytes (the prefix once), and the
        fraction of the HBM peak on the unique bytes."""
        lens = self.lens_now()
        t, ln = self.alloc.pack(self.ids, self.maxb)
        shared = pa.shared_prefix_blocks(t, ln, self.bs)
        if shared == 0:
            return None
        pool = self.pools[len(self.pools) // 2]
        td = torch.from_numpy(t).to(self.device)
        lnd = torch.from_numpy(ln).to(self.device)
        q = self.q[0]
        out = torch.empty_like(q)
        ws_sp = pa.shared_prefix_workspace(pool, self.B, self.maxb, shared, 0)

        def timed(call):
            return loop_seconds(call, reps, warm=3)

        fused, self.fused = self.fused, False
        logical = self.decode_bytes(lens)      # no new rows stored in these calls
        self.fused = fused
        unique = self.unique_bytes(lens)       # K/V rows, the prefix once
        sec_d = timed(lambda: pa.pa_decode(out, q, pool, td, lnd, self.scale, self.pb, self.ws))
        sec_s = timed(lambda: pa.pa_decode_shared_prefix(out, q, pool, td, lnd, shared, self.scale,
                                                         0, ws_sp))
        res = {"shared_blocks": shared, "logical_bytes": logical, "unique_bytes": unique}
        for name, sec in (("pa_decode", sec_d), ("pa_decode_shared_prefix", sec_s)):
            res[name] = {"us": sec * 1e6, "logical_GBps": logical / sec / 1e9,
                         "unique_GBps": unique / sec / 1e9,
                         "hbm_frac_unique": unique / sec / 1e9 / HBM_PEAK_GBS}
        res["speedup"] = sec_d / sec_s
        return res

    def lens_now(self):
        return np.array([self.alloc.seq_len(int(i)) for i in self.ids], dtype=np.int64)

    def warm(self, seconds=2.0):
        """warm_clocks with the step's decode on the state the last step left
        (no rows written, so the workload is unchanged)."""
        if getattr(self, "last", None) is None:
            return
        d, _ = self.last
        pool = self.pools[0]
        if self.shared:
            call = lambda: pa.pa_decode_shared_prefix(self.out, self.q[0], pool, d["tables"],
                                                      d["lens"], self.shared, self.scale, self.pb,
                                                      self.ws_sp)
        else:
            call = lambda: pa.pa_decode(self.out, self.q[0], pool, d["tables"], d["lens"],
                                        self.scale, self.pb, self.ws)
        warm_clocks(call, seconds)

    def decode_bytes(self, lens):
        """Algorithmic bytes of one pa_decode launch: every cached K and V row
        once, q, out, the table entries read and the lengths (and, for
        pa_decode_append, the new rows stored)."""
        row = self.H * self.D * ELEM[self.kv]
        kv = 2 * int(np.sum(lens)) * row
        qo = self.B * self.H * self.D * (ELEM[self.qdt] * 2)
        tables = int(np.sum(-(-lens // self.bs))) * 4 + self.B * 4
        scales = 0
        if self.kv == "fp8":
            scales = 2 * int(np.sum(-(-lens // self.bs))) * self.H * 4
        new_rows = 2 * self.B * self.H * self.D * ELEM[self.kv] if self.fused else 0
        return kv + qo + tables + scales + new_rows

    def launch_seconds(self):
        """Mean launch time of each timed step (s): the layer-loop bracket
        over the layers (fused), or the one bracketed launch."""
        per = self.layers if self.fused else 1
        return [t.seconds() / per for t in self.ev]

    def kernel_stats(self):
        """Mean pa_decode launch time (s) and mean algorithmic bytes per launch."""
        return float(np.mean(self.launch_seconds())), float(np.mean(self.step_bytes))

    def kernel_spread(self):
        return spread(self.launch_seconds())

    def mean_unique_bytes(self):
        """Mean distinct K/V bytes per launch over the timed steps (the
        contexts grow by one token a step)."""
        return float(np.mean(self.step_unique))

    def workload_config(self):
        c = self.cfg
        d = {"workload": self.name, "layers_per_step": self.layers, "batch": self.B,
             "num_heads": self.H, "head_dim": self.D,
             "block_size": self.bs, "kv_dtype": self.kv, "q_dtype": self.qdt,
             "pool_blocks": self.N, "mean_context": float(np.mean(self.lens0))}
        if self.name == "llama13b_decode":
            d["context_lens"] = f"uniform[{c['len_lo']},{c['len_hi']}] seed {c['seed']}"
        d["partition_blocks"] = self.pb or pa.pa_decode_auto_partition_blocks(self.pool, self.B,
                                                                              self.maxb)
        d["stream_kv"] = self.stream_kv
        d["fp8_auto_scale"] = self.auto_scale
        return d

    def merge_kernel(self):
        """The merge launch behind a split decode: one thread per output
        element when the workspace holds at most 8 partitions per (sequence,
        head), the strided LDS merge beyond that."""
        pb = self.pb or pa.pa_decode_auto_partition_blocks(self.pool, self.B, self.maxb)
        parts = -(-self.maxb // pb)
        return "decode_merge_small_kernel" if parts <= 8 else "decode_merge_kernel"

    def cpu_baseline(self, budget_s=10.0):
        """The oracle on the same shape: (sequence, head) decodes of the batch
        at the prompt lengths (pool rows filled by torch before any library
        write), cycling over the pairs until the budget is spent; only the
        oracle call is timed."""
        from oracle import attention as A
        rng = np.random.default_rng(0)
        pairs = [(i, h) for h in range(self.H) for i in range(self.B)]
        done_bytes, n, spent = 0, 0, 0.0
        cache = {}
        c0, w0 = time.process_time(), time.perf_counter()
        while spent < budget_s:
            i, h = pairs[n % len(pairs)]
            L = self.lens0[i] - 1
            nb = -(-L // self.bs)
            if (i, h) not in cache:
                idx = torch.tensor(self.alloc.block_table(i)[:nb], dtype=torch.int64,
                                   device=self.device)
                kp = _bits(self.pool.k_cache[idx, h:h + 1])
                vp = _bits(self.pool.v_cache[idx, h:h + 1])
                ks = vs = None
                if self.kv == "fp8":
                    ks = self.pool.k_scale[idx, h:h + 1].cpu().numpy()
                    vs = self.pool.v_scale[idx, h:h + 1].cpu().numpy()
                cache[(i, h)] = (kp, vp, ks, vs)
                if len(cache) > 256:
                    cache.pop(next(iter(cache)))
            kp, vp, ks, vs = cache[(i, h)]
            q = rng.standard_normal((1, 1, self.D))
            t0 = time.perf_counter()
            A.decode(q, kp, vp, self.kv, [list(range(nb))], [L], self.bs, self.scale, ks, vs)
            spent += time.perf_counter() - t0
            done_bytes += 2 * L * self.D * ELEM[self.kv]
            n += 1
        used = _cores_used(time.process_time() - c0, time.perf_counter() - w0)
        return {"value": done_bytes / spent / 1e9, "unit": "GB/s", "cores": used,
                "cores_available": _cores(),
                "kind": "oracle",
                "sample": f"{n} (sequence, head) decodes cycling over this workload's "
                          f"{len(pairs)} pairs at the prompt lengths, {spent:.1f} s of oracle "
                          "time, float64 NumPy"}


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
        self.bufs = Staging({"slots": ((self.B, self.S), torch.int64),
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
            tm = Timer()
            tm.start()
        pa.pa_prefill_chunk(self.out, self.q, self.pool, d["tables"], d["lens"], self.qsl, self.S,
                            self.scale)
        if timed:
            tm.stop()
            self.ev.append(tm)
        for s in ids:
            self.alloc.free_seq(int(s))

    def flops(self):
        """Causal FLOPs of one launch: 4*D*H per (query, visible key) pair."""
        pairs = sum(self.S * c + self.S * (self.S + 1) // 2 for c in self.ctx)
        return 4.0 * self.D * self.H * pairs

    def kernel_stats(self):
        t = float(np.mean([tm.seconds() for tm in self.ev]))
        return t, self.flops()

    def kernel_spread(self):
        return spread([tm.seconds() for tm in self.ev])

    def fp8_series(self, reps=20):
        """The workload's launch over an fp8 E4M3 pool (codes drawn N(0, 40^2)
        with scale 1/40 per (block, head), so values are N(0,1)) with the same
        bf16 queries, tables and lengths: mean of back-to-back calls, causal TFLOP/s,
        and the K/V bytes (one byte per element)."""
        N, H, D, bs = self.N, self.H, self.D, self.bs
        pool = pa.PagedPool.empty(N, H, bs, D, "fp8", self.device)
        g = torch.Generator(device=self.device)
        g.manual_seed(5)
        for t in (pool.k_cache, pool.v_cache):
            for i in range(0, N, 1024):
                n = min(1024, N - i)
                x = torch.randn((n,) + tuple(t.shape[1:]), generator=g, device=self.device)
                t[i:i + n] = (x * 40.0).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        pool.k_scale.fill_(1.0 / 40.0)
        pool.v_scale.fill_(1.0 / 40.0)
        ids = np.arange(self.next_id, self.next_id + self.B, dtype=np.int64)
        self.next_id += self.B
        for j, sid in enumerate(ids):
            self.alloc.alloc_prompt(int(sid), self.ctx[j] + self.S)
        t, ln = self.alloc.pack(ids, self.maxb)
        td, ld = torch.from_numpy(t).to(self.device), torch.from_numpy(ln).to(self.device)
        out = torch.empty_like(self.out)
        sec = loop_seconds(lambda: pa.pa_prefill_chunk(out, self.q, pool, td, ld, self.qsl, self.S,
                                                       self.scale), reps, warm=3)
        for sid in ids:
            self.alloc.free_seq(int(sid))
        del pool
        return {"kv_dtype": "fp8", "q_dtype": "bf16", "us": sec * 1e6,
                "TFLOPs": self.flops() / sec / 1e12,
                "kv_bytes": 2 * H * D * sum(c + self.S for c in self.ctx)}

    def warm(self, seconds=2.0):
        """warm_clocks with the workload's launch (a batch allocated for it
        and freed again, so the pool's state is unchanged)."""
        self.loop_us(1, warm_s=seconds)

    def loop_us(self, reps=20, warm_s=2.0):
        """The workload's launch (bf16 pool, the batch allocated once), mean
        of back-to-back calls under one event pair, in us."""
        ids = np.arange(self.next_id, self.next_id + self.B, dtype=np.int64)
        self.next_id += self.B
        for j, sid in enumerate(ids):
            self.alloc.alloc_prompt(int(sid), self.ctx[j] + self.S)
        t, ln = self.alloc.pack(ids, self.maxb)
        td, ld = torch.from_numpy(t).to(self.device), torch.from_numpy(ln).to(self.device)
        sec = loop_seconds(lambda: pa.pa_prefill_chunk(self.out, self.q, self.pool, td, ld,
                                                       self.qsl, self.S, self.scale), reps,
                           warm_s=warm_s)
        for sid in ids:
            self.alloc.free_seq(int(sid))
        return sec * 1e6

    def hbm_bytes(self):
        """Algorithmic bytes of one launch: every context and chunk K/V row
        once, q and out."""
        row = self.H * self.D * 2
        return 2 * row * sum(c + self.S for c in self.ctx) + 2 * row * self.B * self.S

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
        c0 = time.process_time()
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
        used = _cores_used(time.process_time() - c0, dt)
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": used,
                "cores_available": _cores(), "kind": "oracle",
                "sample": f"{i} (sequence, head) chunk attentions of this workload, {dt:.1f} s, "
                          "float64 NumPy"}


def _bits(t):
    t = t.cpu()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.uint8).numpy()


def _cores_used(cpu_s, wall_s):
    """Threads the baseline kept busy on average: process CPU time (all
    threads) over wall time."""
    return round(cpu_s / wall_s, 2) if wall_s > 0 else None


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
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed steps: no cold-cache series, block-size, fp8-write, "
                         "prefix-reuse or eviction measurements (for counter runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (the reference "
                         "for scaling HBM byte counters) and exit")
    ap.add_argument("--layers", type=int, default=None,
                    help="attention layers per decode step (default: 40 for the LLaMA-13B shape)")
    ap.add_argument("--partition-blocks", type=int, default=None,
                    help="decode split-K partition size in blocks (default: the library's choice, "
                         "or the workload's own)")
    ap.add_argument("--stream-kv", choices=["auto", "on", "off"], default="auto",
                    help="decode pools' PA_POOL_STREAM_KV flag (auto: on unless blocks are shared)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(each GPU would hold its own pools and sub-batch).",
              file=sys.stderr)
        sys.exit(2)
    device = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return
    log(f"bench: workload={args.workload} steps={args.steps} warmup={args.warmup}")
    if args.workload == "chunked_prefill":
        b = PrefillBench(args.steps, args.warmup, device)
    else:
        b = DecodeBench(args.workload, args.steps, args.warmup, device, args.partition_blocks,
                        args.layers, {"auto": None, "on": True, "off": False}[args.stream_kv])
    torch.cuda.synchronize()
    for k in range(args.warmup):
        b.step(k, False)
    b.warm()
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
                           "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                           "traffic": measured_traffic(args.workload, "prefill_kernel"),
                           "kernel": "prefill_kernel", "kernel_us": kt * 1e6,
                           "kernel_us_spread": b.kernel_spread()}
        hb = b.hbm_bytes()
        res["hbm"] = {"bytes_per_launch": hb, "GBps": hb / kt / 1e9,
                      "frac": hb / kt / 1e9 / HBM_PEAK_GBS}
        if not args.no_extras:
            log("bench: fp8 pool")
            res["fp8_pool"] = b.fp8_series()
    else:
        kv_bytes = work                   # per launch (one layer), logical
        step_s = wall / args.steps
        res.update(metric=METRIC if args.workload == "llama13b_decode"
                   else f"pa_decode KV GB/s at the {args.workload} workload",
                   value=kv_bytes * b.layers / step_s / 1e9, unit="GB/s", dtype=b.kv)
        # the HBM has to deliver each distinct row once: with a shared prefix
        # (the same blocks in every table) the unique bytes are the basis,
        # the logical ones (the prefix counted per sequence) are reported apart
        hbm_bytes = b.mean_unique_bytes() if args.workload == "prefix_cow" else kv_bytes
        ach = hbm_bytes / kt / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": ach / HBM_PEAK_GBS,
                           "traffic": measured_traffic(args.workload, "decode_kernel"),
                           "kernel": ("pa_decode_shared_prefix_append (prefill_kernel prefix "
                                      "pass + decode_kernel with the merge fused)"
                                      if getattr(b, "shared", 0) else
                                      ("pa_decode_append" if b.fused else "pa_decode")
                                      + f" (decode_kernel + {b.merge_kernel()})"),
                           "kernel_us": kt * 1e6, "kernel_us_spread": b.kernel_spread(),
                           "bytes_per_launch": hbm_bytes,
                           "basis": "unique bytes" if args.workload == "prefix_cow"
                           else "algorithmic bytes"}
        if args.workload == "prefix_cow":
            res["roofline"]["logical_bytes_per_launch"] = kv_bytes
            res["roofline"]["logical_GBps"] = kv_bytes / kt / 1e9
        assert res["roofline"]["frac"] <= 1.0, res["roofline"]
        res["hbm_frac_step"] = kv_bytes * b.layers / step_s / 1e9 / HBM_PEAK_GBS
        res["decode_tokens_per_s"] = b.B / step_s
        res["pa_decode_us_per_layer"] = kt * 1e6
    if args.workload != "chunked_prefill" and not args.no_extras:
        log("bench: cold-cache series")
        res["cold"] = b.cold_series()
        if args.workload == "llama13b_decode":
            log("bench: block sizes")
            res["block_sizes"] = b.block_sizes()
        if args.workload == "long_fp8_decode":
            res["fp8_write"] = b.fp8_write_series()
        if args.workload == "prefix_cow":
            ub = b.mean_unique_bytes()
            res["unique_bytes_per_launch"] = ub
            res["unique_GBps"] = ub / kt / 1e9
            res["cow_copy"] = b.cow_copy_us()
            log("bench: shared-prefix decode")
            res["shared_prefix_decode"] = b.shared_prefix_series()
            log("bench: prefix reuse")
            res["prefix_reuse"] = b.prefix_reuse()
            log("bench: eviction churn (host)")
            res["eviction"] = b.eviction_churn()
    if not args.no_cpu_baseline:
        log("bench: cpu baseline")
        res["cpu_baseline"] = b.cpu_baseline()
    else:
        res["cpu_baseline"] = None
    if args.workload == "llama13b_decode" and not args.no_extras:
        del b
        torch.cuda.empty_cache()
        res["other_workloads"] = other_workloads(device)
    print(json.dumps(res), flush=True)


def other_workloads(device, reps=20):
    """The other full-size workloads, one launch configuration each, so that
    the default line carries all of them: the chunked prefill (MFMA), the
    131072-token fp8 decode (HBM) and the shared-prefix decode (HBM on the
    unique bytes).  Kernel times are means of back-to-back launches under one
    event pair (the fp8 decode: its bench steps, a cache write with scale
    upkeep and then the decode, the event pair around the decode)."""
    out = {}
    log("bench: other workloads: chunked prefill")
    p = PrefillBench(4, 2, device)
    us = p.loop_us(reps)
    fl = p.flops()
    out["chunked_prefill"] = {
        "kernel": "prefill_kernel (pa_prefill_chunk)", "kernel_us": us,
        "flops_per_launch": fl, "TFLOPs": fl / us / 1e6,
        "mfma_frac": fl / us / 1e6 / BF16_PEAK_TFLOPS, "peak_TFLOPs": BF16_PEAK_TFLOPS,
        "hbm_bytes_per_launch": p.hbm_bytes(), "config": p.workload_config(),
        "fp8_pool": p.fp8_series(reps)}
    del p
    torch.cuda.empty_cache()
    log("bench: other workloads: long fp8 decode")
    steps, warm = 6, 2
    d = DecodeBench("long_fp8_decode", steps, warm, device)
    for k in range(warm):
        d.step(k, False)
    d.warm()
    for k in range(warm, warm + steps):
        d.step(k, True)
    torch.cuda.synchronize()
    kt, nb = d.kernel_stats()
    out["long_fp8_decode"] = {
        "kernel": ("pa_decode_append (the step's rows quantised with scale upkeep in the decode "
                   f"launch; decode_kernel + {d.merge_kernel()}), 256 partitions" if d.fused else
                   f"pa_decode (decode_kernel + {d.merge_kernel()}), 256 partitions"),
        "kernel_us": kt * 1e6, "kernel_us_spread": d.kernel_spread(), "bytes_per_launch": nb,
        "GBps": nb / kt / 1e9, "hbm_frac": nb / kt / 1e9 / HBM_PEAK_GBS,
        "config": d.workload_config()}
    del d
    torch.cuda.empty_cache()
    log("bench: other workloads: shared-prefix decode")
    steps, warm = 30, 5
    d = DecodeBench("prefix_cow", steps, warm, device)
    for k in range(warm):
        d.step(k, False)
    d.warm()
    for k in range(warm, warm + steps):
        d.step(k, True)
    torch.cuda.synchronize()
    kt, logical = d.kernel_stats()
    unique = d.mean_unique_bytes()
    sp = d.shared_prefix_series(reps)
    # the workload's decode step as the bench runs it: the new rows stored
    # and the prefix read once (pa_decode_shared_prefix_append)
    # the last step's call replayed back to back (its new rows stored again
    # at the same slots): the launch pair's own duration, without the gap
    # between the step's start event and a launch the host is still issuing
    # (the steps are host-bound: the GPU idles between them)
    last_unique = d.step_unique[-1]
    rep = loop_seconds(d.last_call, reps)
    sp["step"] = {"call": "pa_decode_shared_prefix_append", "kernel_us": kt * 1e6,
                  "kernel_us_spread": d.kernel_spread(), "unique_bytes": unique,
                  "unique_GBps": unique / kt / 1e9,
                  "hbm_frac_unique": unique / kt / 1e9 / HBM_PEAK_GBS,
                  "logical_bytes": logical,
                  "last_step_back_to_back": {"us": rep * 1e6, "unique_bytes": last_unique,
                                             "hbm_frac_unique": last_unique / rep / 1e9
                                             / HBM_PEAK_GBS}}
    assert sp["step"]["hbm_frac_unique"] <= 1.0, sp["step"]
    sp["config"] = d.workload_config()
    for name in ("pa_decode", "pa_decode_shared_prefix"):
        assert sp[name]["hbm_frac_unique"] <= 1.0, sp
    out["prefix_cow"] = sp
    del d
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
