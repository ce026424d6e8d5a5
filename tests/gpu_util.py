"""Helpers for the GPU parity tests: one scenario drives the library (C++
allocator + HIP kernels) and the oracle side by side on the same seeded
inputs, and checks the integer state bit for bit as it goes."""
import numpy as np
import torch

import paged_kv_cache_166_amd as pa
from oracle import cache as C
from oracle.allocator import OracleAllocator

BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}
SENTINEL = {"f32": 0xFFFFFFFF, "f16": 0xFFFF, "bf16": 0xFFFF, "fp8": 0x7F}   # NaN patterns
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3, "fp8": 2e-2}


def to_bits(x_f32, dt):
    """float32 host array -> storage bits of dtype dt (RNE casts)."""
    x_f32 = np.ascontiguousarray(x_f32, dtype=np.float32)
    if dt == "f32":
        return x_f32.view(np.uint32).copy()
    if dt == "f16":
        return x_f32.astype(np.float16).view(np.uint16)
    if dt == "bf16":
        return torch.from_numpy(x_f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dt)


def bits_to_device(bits, dt, device):
    t = torch.from_numpy(np.ascontiguousarray(bits))
    if dt == "f32":
        t = t.view(torch.int32).view(torch.float32)
    elif dt == "f16":
        t = t.view(torch.int16).view(torch.float16)
    elif dt == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def device_bits(t):
    """Device tensor -> host numpy array of its raw bits."""
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return t.view(torch.uint8).numpy()
    raise ValueError(t.dtype)


def values_f64(bits, dt):
    return C.to_float64(bits, dt)


class Scenario:
    """A pool plus both allocators.  K/V rows are written through the library
    on the GPU and through the oracle on the host, from the same inputs."""

    def __init__(self, num_blocks, num_heads, block_size, head_dim, kv, seed, device="cuda",
                 in_dtype=None, scale_range=(0.004, 0.02), fp8_auto_scale=False):
        self.N, self.H, self.bs, self.D, self.kv = num_blocks, num_heads, block_size, head_dim, kv
        self.in_dtype = in_dtype or ("bf16" if kv == "fp8" else kv)
        self.rng = np.random.default_rng(seed)
        order = self.rng.permutation(num_blocks).astype(np.int32)
        self.alloc = pa.Allocator(num_blocks, block_size, order)
        self.ora = OracleAllocator(num_blocks, block_size, order)
        self.device = device
        self.auto_scale = fp8_auto_scale
        self.pool = pa.PagedPool.empty(num_blocks, num_heads, block_size, head_dim, kv, device,
                                       fp8_auto_scale=fp8_auto_scale)
        shape = (num_blocks, num_heads, block_size, head_dim)
        self.ok = np.full(shape, SENTINEL[kv], dtype=BITS[kv])
        self.ov = self.ok.copy()
        self._fill_device_sentinel()
        self.oks = self.ovs = None
        if kv == "fp8":
            lo, hi = scale_range
            self.oks = self.rng.uniform(lo, hi, (num_blocks, num_heads)).astype(np.float32)
            self.ovs = self.rng.uniform(lo, hi, (num_blocks, num_heads)).astype(np.float32)
            self.pool.k_scale.copy_(torch.from_numpy(self.oks))
            self.pool.v_scale.copy_(torch.from_numpy(self.ovs))
        self.seqs = []

    def _fill_device_sentinel(self):
        for t in (self.pool.k_cache, self.pool.v_cache):
            if t.dtype == torch.float32:
                t.view(torch.int32).fill_(-1)
            elif t.dtype in (torch.float16, torch.bfloat16):
                t.view(torch.int16).fill_(-1)
            else:
                t.fill_(SENTINEL["fp8"])

    # -- writes ---------------------------------------------------------------
    def _write(self, slots, n, amp=1.0):
        """Draw n rows of K and V (N(0, amp^2)), write them at slots on both
        sides.  amp may be an array broadcast over [n, H, 1]."""
        if n == 0:
            return
        a = np.asarray(amp, dtype=np.float32)
        k32 = self.rng.standard_normal((n, self.H, self.D), dtype=np.float32) * a
        v32 = self.rng.standard_normal((n, self.H, self.D), dtype=np.float32) * a
        kb, vb = to_bits(k32, self.in_dtype), to_bits(v32, self.in_dtype)
        kd = bits_to_device(kb, self.in_dtype, self.device)
        vd = bits_to_device(vb, self.in_dtype, self.device)
        sd = torch.from_numpy(np.asarray(slots, dtype=np.int64)).to(self.device)
        pa.pa_reshape_and_cache(self.pool, kd, vd, sd)
        if self.kv == "fp8":
            kf = values_f64(kb, self.in_dtype).astype(np.float32)
            vf = values_f64(vb, self.in_dtype).astype(np.float32)
            w = C.write_rows_fp8_upkeep if self.auto_scale else C.write_rows_fp8
            w(self.ok, kf, slots, self.oks, self.bs)
            w(self.ov, vf, slots, self.ovs, self.bs)
        else:
            C.write_rows(self.ok, kb, slots, self.bs)
            C.write_rows(self.ov, vb, slots, self.bs)

    def prompt(self, seq, n, amp=1.0):
        s_lib = self.alloc.alloc_prompt(seq, n)
        s_ora = self.ora.alloc_prompt(seq, n)
        assert list(s_lib) == s_ora
        self.seqs.append(seq)
        self._write(s_ora, n, amp)

    def append(self, seq, n=1, amp=1.0):
        s_lib, cow_lib = self.alloc.append_tokens(seq, n)
        s_ora, cow_ora = self.ora.append_tokens(seq, n)
        assert list(s_lib) == s_ora and cow_lib == cow_ora
        if cow_ora is not None:
            pairs = torch.tensor([cow_ora], dtype=torch.int32, device=self.device)
            pa.pa_copy_blocks(self.pool, pairs)
            C.copy_blocks(self.ok, [cow_ora], self.oks)
            C.copy_blocks(self.ov, [cow_ora], self.ovs)
        self._write(s_ora, n, amp)
        return cow_ora

    def write_batch(self, seqs, n=1, amp=1.0):
        """Append n tokens (or n[i] to seqs[i]) and write them in one call (the
        slot mapping of a batched decode or prefill step)."""
        slots = []
        ns = n if isinstance(n, (list, tuple)) else [n] * len(seqs)
        for sq, k in zip(seqs, ns):
            s_lib, cow = self.alloc.append_tokens(sq, k)
            s_ora, cow_o = self.ora.append_tokens(sq, k)
            assert list(s_lib) == s_ora and cow is None and cow_o is None
            slots += s_ora
        self._write(slots, len(slots), amp)

    def fork(self, parent, child):
        self.alloc.fork(parent, child)
        self.ora.fork(parent, child)
        self.seqs.append(child)

    # -- views ----------------------------------------------------------------
    def tables(self, seqs, max_blocks=None):
        if max_blocks is None:
            max_blocks = max(1, max(len(self.ora.block_table(s)) for s in seqs))
        t, ln = self.alloc.pack(seqs, max_blocks)
        assert t.tolist() == self.ora.padded_tables(seqs, max_blocks)
        assert ln.tolist() == [self.ora.seq_len(s) for s in seqs]
        return t, ln

    def device_tables(self, seqs, max_blocks=None):
        t, ln = self.tables(seqs, max_blocks)
        return (torch.from_numpy(t).to(self.device), torch.from_numpy(ln).to(self.device), t, ln)

    def check_pool_bits(self):
        torch.cuda.synchronize()
        assert np.array_equal(device_bits(self.pool.k_cache), self.ok)
        assert np.array_equal(device_bits(self.pool.v_cache), self.ov)
        if self.kv == "fp8":
            assert np.array_equal(self.pool.k_scale.cpu().numpy(), self.oks)
            assert np.array_equal(self.pool.v_scale.cpu().numpy(), self.ovs)

    def oracle_tables(self, seqs):
        return [self.ora.block_table(s) for s in seqs], [self.ora.seq_len(s) for s in seqs]

    def random_q(self, n, dtype):
        q32 = self.rng.standard_normal((n, self.H, self.D), dtype=np.float32)
        qb = to_bits(q32, dtype)
        return bits_to_device(qb, dtype, self.device), values_f64(qb, dtype)


def assert_close(got, ref, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    worst = float(np.nanmax(err)) if err.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert worst <= tol, f"{what}: max abs error {worst:.3e} > {tol:.1e}"
    return worst


def half_ulp(dt, ref):
    """Half a unit in the last place of dtype dt at |ref| (output rounding)."""
    a = np.maximum(np.abs(ref), 2.0 ** -14)
    bits = {"f16": 10, "bf16": 7, "f32": 23}[dt]
    return 2.0 ** (np.floor(np.log2(a)) - bits - 1)
