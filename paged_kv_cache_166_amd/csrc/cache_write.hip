// pa_reshape_and_cache and pa_copy_blocks kernels.
//
// reshape_and_cache writes token t's K and V rows into physical slot s:
// block s / bs, row s % bs of every head's tile (vLLM course ch. 4 attention
// pseudocode: block table -> physical block, offset inside it).  One thread
// moves 8 elements of one (token, head) row; a row of 128 elements is 16
// threads, so each wave writes 4 whole rows with contiguous 16-byte (or
// 8-byte for fp8) stores.  fp8 pools store RNE-saturate(x / scale) with the
// block's existing per-head scale (the blog article's mixed-precision KV), or,
// with scale upkeep, keep each block's scale at the amax of its rows / 448.
//
// copy_blocks copies whole (block, head) tiles of K and V, and the fp8
// scales, for the copy-on-write step (DataWhale notes section 4).
#include "device.h"
#include "kernels.h"

namespace pa {
namespace {

// 8 elements of dtype dt at p -> float32.
__device__ __forceinline__ void load8_f32(const void* p, int dt, float* x) {
  if (dt == PA_F32) {
    const float4 a = ((const float4*)p)[0];
    const float4 b = ((const float4*)p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const uint4 r = *(const uint4*)p;
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = dt == PA_F16 ? f16_lo(w[i]) : bf16_lo(w[i]);
      x[2 * i + 1] = dt == PA_F16 ? f16_hi(w[i]) : bf16_hi(w[i]);
    }
  }
}

// kNarrow: the call's (token, head, chunk) count fits 32 bits, so the index
// splits in 32-bit arithmetic (64-bit division is a long instruction
// sequence).  head_dim / 8 and block_size are powers of two (checked on the
// host): shifts and masks.
template <bool kNarrow>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheWriteArgs a) {
  const int cl = __builtin_ctz(unsigned(a.head_dim) / 8u);   // log2(chunks per row)
  const int bl = __builtin_ctz(unsigned(a.block_size));
  int c, h;
  int64_t t;
  if constexpr (kNarrow) {
    const uint32_t n = (uint32_t(a.num_tokens) * uint32_t(a.num_heads)) << cl;
    const uint32_t idx = blockIdx.x * 256u + threadIdx.x;
    if (idx >= n) return;
    c = int(idx & ((1u << cl) - 1u));
    const uint32_t th = idx >> cl;
    h = int(th % uint32_t(a.num_heads));
    t = int64_t(th / uint32_t(a.num_heads));
  } else {
    const int64_t n = (int64_t(a.num_tokens) * a.num_heads) << cl;
    const int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (idx >= n) return;
    c = int(idx & ((int64_t(1) << cl) - 1));
    const int64_t th = idx >> cl;
    h = int(th % a.num_heads);
    t = th / a.num_heads;
  }
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  const int64_t blk = slot >> bl;
  const int64_t off = slot & (a.block_size - 1);
  const int64_t src_e = (t * a.num_heads + h) * a.head_dim + c * 8;
  const int64_t dst_e = ((blk * a.num_heads + h) * a.block_size + off) * a.head_dim + c * 8;
  const int in_b = dtype_bytes(a.in_dtype);
  if (a.kv_dtype != PA_FP8_E4M3) {
    const char* ks = (const char*)a.key + src_e * in_b;
    const char* vs = (const char*)a.value + src_e * in_b;
    char* kd = (char*)a.k_cache + dst_e * in_b;
    char* vd = (char*)a.v_cache + dst_e * in_b;
    *(uint4*)kd = *(const uint4*)ks;
    *(uint4*)vd = *(const uint4*)vs;
    if (in_b == 4) {
      *(uint4*)(kd + 16) = *(const uint4*)(ks + 16);
      *(uint4*)(vd + 16) = *(const uint4*)(vs + 16);
    }
    return;
  }
  const float kscale = a.k_scale[blk * a.num_heads + h];
  const float vscale = a.v_scale[blk * a.num_heads + h];
  float x[8], y[8];
  load8_f32((const char*)a.key + src_e * in_b, a.in_dtype, x);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fp8_prep(x[i], kscale);
  *(uint2*)((uint8_t*)a.k_cache + dst_e) = make_uint2(pack4_fp8(y), pack4_fp8(y + 4));
  load8_f32((const char*)a.value + src_e * in_b, a.in_dtype, x);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fp8_prep(x[i], vscale);
  *(uint2*)((uint8_t*)a.v_cache + dst_e) = make_uint2(pack4_fp8(y), pack4_fp8(y + 4));
}

// Largest value over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// fp8 write with scale upkeep (PA_POOL_FP8_AUTO_SCALE).  Grid (window of
// tokens, head), one wave each.  The call's tokens form runs: consecutive
// tokens writing consecutive positions of one block.  The wave whose window
// holds a run's first token does the whole run for its head: amax of the run's rows, new scale
// max(old, amax / 448) (old = 0 when the run starts the block), the block's
// earlier rows requantised if the scale grew, the run's rows stored, the
// scale written -- K, then V (a window's runs one after another).  Runs of
// different blocks touch disjoint tiles and scales, so no wave waits for
// another.  Every step issues all its loads at once (a run is at most one
// block of rows of at most 128 elements: kMaxChunksPerLane chunks of 8 per
// lane, 8 for blocks up to 32 rows, 16 for 64), so a run costs a few memory
// round trips, not one per row.
template <int kMaxChunksPerLane>
__device__ __forceinline__ void upkeep_one(const CacheWriteArgs& a, const void* in, uint8_t* tile,
                                           float* scale, int64_t t, int h, int p0, int n,
                                           int lane) {
  const int D = a.head_dim;
  const int chunks = D / 8;
  const int in_b = dtype_bytes(a.in_dtype);
  const int H = a.num_heads;
  const int total = n * chunks;
  float x[kMaxChunksPerLane][8];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxChunksPerLane; ++k) {
    const int i = lane + 64 * k;
    if (i < total) {
      const int r = i / chunks, c = i % chunks;
      load8_f32((const char*)in + (((t + r) * H + h) * D + c * 8) * in_b, a.in_dtype, x[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[k][e]));
    }
  }
  amax = wave_max(amax);
  const float s_old = p0 == 0 ? 0.f : *scale;
  const float s_new = fmaxf(s_old, __fdiv_rn(amax, 448.f));
  const float d = s_new > 0.f ? s_new : 1.f;
  if (p0 > 0 && s_new > s_old) {
    uint2 w[kMaxChunksPerLane];
#pragma unroll
    for (int k = 0; k < kMaxChunksPerLane; ++k) {
      const int i = lane + 64 * k;
      if (i < p0 * chunks) w[k] = *(const uint2*)(tile + i * 8);
    }
#pragma unroll
    for (int k = 0; k < kMaxChunksPerLane; ++k) {
      const int i = lane + 64 * k;
      if (i < p0 * chunks) *(uint2*)(tile + i * 8) = requant8(w[k], s_old, d);
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxChunksPerLane; ++k) {
    const int i = lane + 64 * k;
    if (i < total) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = fp8_prep(x[k][e], d);
      *(uint2*)(tile + p0 * D + i * 8) = make_uint2(pack4_fp8(y), pack4_fp8(y + 4));
    }
  }
  if (lane == 0) *scale = s_new;
}

template <int kMaxChunksPerLane>
__global__ __launch_bounds__(64) void reshape_fp8_upkeep_kernel(CacheWriteArgs a, int window) {
  const int64_t t0 = int64_t(blockIdx.x) * window;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int bs = a.block_size;
  // Run heads among this wave's tokens t0 .. t0 + window - 1 (window <= 64):
  // a token with a slot whose previous token did not write the previous
  // position of the same block.
  const int64_t tl = t0 + lane;
  bool head = false;
  if (lane < window && tl < a.num_tokens) {
    const int64_t s = a.slots[tl];
    head = s >= 0 && !(tl > 0 && s % bs > 0 && a.slots[tl - 1] == s - 1);
  }
  uint64_t heads = __ballot(head);
  while (heads) {
    const int64_t t = t0 + __builtin_ctzll(heads);
    heads &= heads - 1;
    const int64_t s = a.slots[t];
    const int64_t blk = s / bs;
    const int p0 = int(s % bs);
    // Run length in one round trip: lane i checks token t + i (i < bs - p0).
    const bool cont = lane < bs - p0 && t + lane < a.num_tokens && a.slots[t + lane] == s + lane;
    const uint64_t run = __ballot(cont);
    const int n = run == ~uint64_t(0) ? 64 : int(__builtin_ctzll(~run));   // leading run of ones
    const int64_t si = blk * a.num_heads + h;
    const int64_t tile = si * bs * a.head_dim;
    upkeep_one<kMaxChunksPerLane>(a, a.key, (uint8_t*)a.k_cache + tile, a.k_scale + si, t, h, p0,
                                  n, lane);
    upkeep_one<kMaxChunksPerLane>(a, a.value, (uint8_t*)a.v_cache + tile, a.v_scale + si, t, h,
                                  p0, n, lane);
  }
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int pair = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t src = a.src_dst[2 * pair];
  const int64_t dst = a.src_dst[2 * pair + 1];
  const int64_t so = (src * a.num_heads + h) * a.tile_bytes;
  const int64_t d_o = (dst * a.num_heads + h) * a.tile_bytes;
  for (int64_t b = threadIdx.x * 16; b < a.tile_bytes; b += blockDim.x * 16) {
    *(uint4*)((char*)a.k_cache + d_o + b) = *(const uint4*)((const char*)a.k_cache + so + b);
    *(uint4*)((char*)a.v_cache + d_o + b) = *(const uint4*)((const char*)a.v_cache + so + b);
  }
  if (threadIdx.x == 0 && a.k_scale) {
    a.k_scale[dst * a.num_heads + h] = a.k_scale[src * a.num_heads + h];
    a.v_scale[dst * a.num_heads + h] = a.v_scale[src * a.num_heads + h];
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const CacheWriteArgs& a, hipStream_t stream) {
  const int64_t n = int64_t(a.num_tokens) * a.num_heads * (a.head_dim / 8);
  if (n == 0) return hipSuccess;
  if (a.kv_dtype == PA_FP8_E4M3 && a.scale_upkeep) {
    // One wave per (window of tokens, head).  Large calls are mostly runs of
    // a whole block (prefill chunks): a window of one block keeps every wave
    // busy.  Small calls are mostly one-token runs (decode): one token per
    // wave runs them all at once.
    const int window = a.num_tokens > 1024 ? a.block_size : 1;
    const unsigned waves = unsigned((int64_t(a.num_tokens) + window - 1) / window);
    if (a.block_size * a.head_dim > 32 * 128)
      hipLaunchKernelGGL(reshape_fp8_upkeep_kernel<16>, dim3(waves, unsigned(a.num_heads)),
                         dim3(64), 0, stream, a, window);
    else
      hipLaunchKernelGGL(reshape_fp8_upkeep_kernel<8>, dim3(waves, unsigned(a.num_heads)),
                         dim3(64), 0, stream, a, window);
    return hipGetLastError();
  }
  const int64_t groups = (n + 255) / 256;
  if (groups > 0x7fffffff) return hipErrorInvalidValue;   // the grid's x limit
  if (n <= 0xffffffffll)
    hipLaunchKernelGGL(reshape_and_cache_kernel<true>, dim3(unsigned(groups)), dim3(256), 0, stream,
                       a);
  else
    hipLaunchKernelGGL(reshape_and_cache_kernel<false>, dim3(unsigned(groups)), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  if (a.num_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs, a.num_heads), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
