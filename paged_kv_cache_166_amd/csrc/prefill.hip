// pa_prefill_chunk: causal attention of a chunk of query tokens against the
// sequence's paged K/V, on gfx950 matrix cores.
//
// What is computed (blog article section 3.2.2 forward pass: gather through
// the block table, Q K^T * scale, causal mask, softmax, times V): the chunk's
// S rows are the last S positions of a sequence of L tokens, so row r sees
// keys 0 .. L - S + r.
//
// How: a workgroup of 4 wavefronts owns 128 query rows of one (sequence,
// head); wave w owns 32 of them.  The keys are walked in tiles of 32 tokens
// (one to eight blocks, found through the block table):
//  * the K tile is staged in LDS as rows; the V tile is staged transposed
//    (dimension-major) and converted to fp16; two LDS buffers, the next
//    tile's global loads in flight while the current tile is consumed;
//  * S^T = K Q^T on v_mfma_f32_32x32x16 (bf16 or fp16 inputs, fp32
//    accumulate): A = K rows from LDS, B = the wave's Q rows, held in
//    registers for the whole walk;
//  * the accumulator layout of S^T gives every lane one query column and 16
//    of the tile's keys, so the online softmax (running max m, running sum
//    l, exp2 of log2-scaled scores) is lane-local plus one exchange between
//    the two half-waves;
//  * O^T += V^T P^T on v_mfma_f32_32x32x16_f16: P (rounded to fp16) is used
//    straight from the S^T accumulators as the B operand -- the contraction
//    index is permuted to match the accumulator layout and V^T is read from
//    LDS in the same permuted key order -- so P never leaves registers;
//  * tiles wholly above the causal diagonal are skipped per wave; only
//    tiles that cross it are masked.
// Workgroups are mapped so that all query tiles of one (sequence, head) run
// on the same XCD (its L2 holds that head's K/V); the last query tile, which
// sees the most keys, is dispatched first.
#include "device.h"
#include "kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kQW = 32;                 // query rows per wave
constexpr int kBM = kWaves * kQW;       // query rows per workgroup
constexpr int kBN = 32;                 // keys per tile
constexpr int kVtStride = 72;           // bytes per dimension row of V^T in LDS
constexpr int kXcds = 8;

template <int KV>
__device__ __forceinline__ f32x16_t mfma_qk(uint4 a, uint4 b, f32x16_t c) {
  if constexpr (KV == PA_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma_pv(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Two 16-bit values of the pool's type -> packed fp16 pair (RNE).
template <int KV>
__device__ __forceinline__ uint32_t to_f16x2(uint32_t w) {
  if constexpr (KV == PA_F16) return w;
  const uint32_t lo = f32_to_f16_bits(bf16_lo(w));
  const uint32_t hi = f32_to_f16_bits(bf16_hi(w));
  return lo | (hi << 16);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return uint32_t(f32_to_f16_bits(a)) | (uint32_t(f32_to_f16_bits(b)) << 16);
}

template <int KV, int D, int BS>
__global__ __launch_bounds__(kWaves * 64) void prefill_kernel(PrefillArgs a, int num_qtiles,
                                                              int num_pairs) {
  constexpr int kKStride = D * 2 + 16;       // bytes per key row of K in LDS
  constexpr int kKSteps = D / 16;            // S^T contraction steps
  constexpr int kDBlocks = D / 32;           // O^T row blocks
  constexpr int kKBytes = kBN * kKStride;
  constexpr int kVBytes = D * kVtStride;
  constexpr int kKChunks = kBN * D / 8;      // 16-byte chunks of a K tile
  constexpr int kVItems = (kBN / 2) * (D / 8);  // (key pair, 8 dims) items of a V tile
  constexpr int kKPer = (kKChunks + 255) / 256;
  constexpr int kVPer = (kVItems + 255) / 256;
  static_assert(kBN % BS == 0 || BS > kBN, "tile / block");

  __shared__ __attribute__((aligned(16))) char lds[2][kKBytes + kVBytes];

  // Work item: (pair = seq * H + head, query tile); pairs are dealt to XCDs
  // round robin by pair, the query tiles of a pair go to the same XCD, last
  // tile first.
  const int lin = blockIdx.x;
  const int xcd = lin % kXcds;
  const int g = lin / kXcds;
  const int pair = xcd + kXcds * (g / num_qtiles);
  if (pair >= num_pairs) return;
  const int qtile = num_qtiles - 1 - (g % num_qtiles);
  const int seq = pair / a.num_heads;
  const int head = pair % a.num_heads;
  const int H = a.num_heads;

  const int qs = a.query_start_loc[seq];
  const int S = a.query_start_loc[seq + 1] - qs;
  const int q_begin = qtile * kBM;
  if (q_begin >= S) return;
  const int L = a.context_lens[seq];
  const int ctx = L - S;  // tokens before the chunk

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // This wave's query rows and the last key any of the workgroup's rows sees.
  const int wq0 = q_begin + wave * kQW;
  const int wg_last_row = min(q_begin + kBM, S) - 1;
  const int n_keys = ctx + wg_last_row + 1;
  const int n_tiles = (n_keys + kBN - 1) / kBN;
  const int wave_last_key = wq0 < S ? ctx + min(wq0 + kQW, S) - 1 : -1;

  // Q^T fragments: lane holds query wq0 + col, dims kk*16 + 8*half .. +8.
  uint4 qf[kKSteps];
  {
    const int r = wq0 + col;
    const bool ok = r < S;
    const uint16_t* qrow = (const uint16_t*)a.q + (int64_t(qs + (ok ? r : 0)) * H + head) * D;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk)
      qf[kk] = ok ? *(const uint4*)(qrow + kk * 16 + 8 * half) : make_uint4(0, 0, 0, 0);
  }

  const int32_t* table = a.block_tables + int64_t(seq) * a.max_blocks_per_seq;
  const int64_t tile_elems = int64_t(BS) * D;
  const uint16_t* kpool = (const uint16_t*)a.k_cache;
  const uint16_t* vpool = (const uint16_t*)a.v_cache;

  // Global -> register staging of one KV tile.
  uint4 kreg[kKPer], vreg[kVPer][2];
  auto load_tile = [&](int t) {
    const int kb = t * kBN;
#pragma unroll
    for (int i = 0; i < kKPer; ++i) {
      const int c = tid + i * 256;
      const int key = c / (D / 8);
      const int dc = c % (D / 8);
      const int kabs = kb + key;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (c < kKChunks && kabs < L) {
        const int64_t blk = table[kabs / BS];
        v = *(const uint4*)(kpool + (blk * H + head) * tile_elems + (kabs % BS) * D + dc * 8);
      }
      kreg[i] = v;
    }
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      const int w = tid + i * 256;
      const int kp = w % (kBN / 2);
      const int dc = w / (kBN / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int kabs = kb + 2 * kp + e;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (w < kVItems && kabs < L) {
          const int64_t blk = table[kabs / BS];
          v = *(const uint4*)(vpool + (blk * H + head) * tile_elems + (kabs % BS) * D + dc * 8);
        }
        vreg[i][e] = v;
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* kl = lds[buf];
    char* vl = lds[buf] + kKBytes;
#pragma unroll
    for (int i = 0; i < kKPer; ++i) {
      const int c = tid + i * 256;
      if (c < kKChunks) {
        const int key = c / (D / 8);
        const int dc = c % (D / 8);
        *(uint4*)(kl + key * kKStride + dc * 16) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
      const int w = tid + i * 256;
      if (w < kVItems) {
        const int kp = w % (kBN / 2);
        const int dc = w / (kBN / 2);
        const uint32_t a0[4] = {vreg[i][0].x, vreg[i][0].y, vreg[i][0].z, vreg[i][0].w};
        const uint32_t a1[4] = {vreg[i][1].x, vreg[i][1].y, vreg[i][1].z, vreg[i][1].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t x = to_f16x2<KV>(a0[j]);  // key 2kp: dims 2j, 2j+1
          const uint32_t y = to_f16x2<KV>(a1[j]);  // key 2kp+1
          const uint32_t lo = (x & 0xffffu) | (y << 16);          // dim 2j: keys 2kp, 2kp+1
          const uint32_t hi = (x >> 16) | (y & 0xffff0000u);      // dim 2j+1
          const int d = dc * 8 + 2 * j;
          *(uint32_t*)(vl + d * kVtStride + kp * 4) = lo;
          *(uint32_t*)(vl + (d + 1) * kVtStride + kp * 4) = hi;
        }
      }
    }
  };

  f32x16_t o[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m = kNoMax, l = 0.f;
  const int my_row = wq0 + col;           // query row of this lane's column
  const int my_lim = ctx + my_row;        // last key it sees

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const int kb = t * kBN;
    if (kb <= wave_last_key) {
      const char* kl = lds[buf];
      const char* vl = lds[buf] + kKBytes;
      // S^T = K Q^T : rows = keys of the tile, columns = this wave's queries.
      f32x16_t s;
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        const uint4 kf = *(const uint4*)(kl + col * kKStride + kk * 32 + half * 16);
        s = mfma_qk<KV>(kf, qf[kk], s);
      }
      // Register v of this lane holds key 8*(v/4) + 4*half + v%4 of the tile.
      const bool crosses = kb + kBN - 1 > ctx + wq0;
      float mx = kNoMax;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = s[v] * a.scale_log2;
        if (crosses) {
          const int key = kb + 8 * (v / 4) + 4 * half + (v % 4);
          x = key <= my_lim ? x : -INFINITY;
        }
        s[v] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      float psum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s[v] = __builtin_amdgcn_exp2f(s[v] - m_new);
        psum += s[v];
      }
      l = fmaf(l, alpha, psum);
      m = m_new;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
      // P^T as B operands: k-step tt takes accumulator registers 8tt .. 8tt+7,
      // i.e. keys 16tt + 8*(e/4) + 4*half + e%4 for e = 0..7.
      uint4 pf[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        pf[tt] = make_uint4(pack_f16(s[8 * tt + 0], s[8 * tt + 1]),
                            pack_f16(s[8 * tt + 2], s[8 * tt + 3]),
                            pack_f16(s[8 * tt + 4], s[8 * tt + 5]),
                            pack_f16(s[8 * tt + 6], s[8 * tt + 7]));
      // O^T += V^T P^T : A = V^T rows (dims) with the same key order.
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
        const char* vrow = vl + (db * 32 + col) * kVtStride;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const uint2 lo = *(const uint2*)(vrow + (16 * tt + 4 * half) * 2);
          const uint2 hi = *(const uint2*)(vrow + (16 * tt + 8 + 4 * half) * 2);
          o[db] = mfma_pv(make_uint4(lo.x, lo.y, hi.x, hi.y), pf[tt], o[db]);
        }
      }
    }
    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Normalise and store: lane holds query my_row, dims 8*(v/4) + 4*half + v%4.
  l += __shfl_xor(l, 32);
  if (my_row < S && wq0 < S) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t ob = (int64_t(qs + my_row) * H + head) * D;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int d = db * 32 + 8 * (v / 4) + 4 * half + (v % 4);
        store_from_f32(a.out, ob + d, a.out_dtype, o[db][v] * inv);
      }
  }
}

template <int KV, int D, int BS>
hipError_t launch_t(const PrefillArgs& a, int max_query_len, hipStream_t stream) {
  const int num_qtiles = (max_query_len + kBM - 1) / kBM;
  const int num_pairs = a.num_seqs * a.num_heads;
  const int padded_pairs = (num_pairs + kXcds - 1) / kXcds * kXcds;
  const int64_t blocks = int64_t(padded_pairs) * num_qtiles;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<KV, D, BS>), dim3(unsigned(blocks)), dim3(kWaves * 64), 0,
                     stream, a, num_qtiles, num_pairs);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_bs(const PrefillArgs& a, int bs, int mq, hipStream_t stream) {
  switch (bs) {
    case 4: return launch_t<KV, D, 4>(a, mq, stream);
    case 8: return launch_t<KV, D, 8>(a, mq, stream);
    case 16: return launch_t<KV, D, 16>(a, mq, stream);
    case 32: return launch_t<KV, D, 32>(a, mq, stream);
  }
  return hipErrorInvalidValue;
}

template <int KV>
hipError_t launch_d(const PrefillArgs& a, int d, int bs, int mq, hipStream_t stream) {
  if (d == 64) return launch_bs<KV, 64>(a, bs, mq, stream);
  if (d == 128) return launch_bs<KV, 128>(a, bs, mq, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, int head_dim, int block_size,
                          int max_query_len, hipStream_t stream) {
  if (kv_dtype == PA_BF16) return launch_d<PA_BF16>(a, head_dim, block_size, max_query_len, stream);
  if (kv_dtype == PA_F16) return launch_d<PA_F16>(a, head_dim, block_size, max_query_len, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
