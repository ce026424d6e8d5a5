// pa_reshape_and_cache and pa_copy_blocks kernels.
//
// reshape_and_cache writes token t's K and V rows into physical slot s:
// block s / bs, row s % bs of every head's tile (vLLM course ch. 4 attention
// pseudocode: block table -> physical block, offset inside it).  One thread
// moves 8 elements of one (token, head) row; a row of 128 elements is 16
// threads, so each wave writes 4 whole rows with contiguous 16-byte (or
// 8-byte for fp8) stores.  fp8 pools store RNE-saturate(x / scale) with the
// block's existing per-head scale (the blog article's mixed-precision KV).
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

// x / s rounded once in float32, then RNE to E4M3FN saturating at +-448.
// Clamping first is exact: every |x/s| >= 448 rounds to 448 when saturating.
__device__ __forceinline__ float fp8_prep(float x, float s) {
  const float y = __fdiv_rn(x, s);
  return __builtin_isnan(y) ? y : fminf(fmaxf(y, -448.f), 448.f);
}

__device__ __forceinline__ uint32_t pack4_fp8(const float* y) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
  return (uint32_t)w;
}

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheWriteArgs a) {
  const int chunks = a.head_dim / 8;
  const int64_t n = int64_t(a.num_tokens) * a.num_heads * chunks;
  const int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (idx >= n) return;
  const int c = int(idx % chunks);
  const int64_t th = idx / chunks;
  const int h = int(th % a.num_heads);
  const int64_t t = th / a.num_heads;
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  const int64_t blk = slot / a.block_size;
  const int64_t off = slot % a.block_size;
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
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  if (a.num_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(a.num_pairs, a.num_heads), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
