// pa_decode: one query token per sequence against its paged K/V, on gfx950.
//
// What is computed (blog article section 3.2.2 forward pass at a single query
// row; vLLM course ch. 4 attention pseudocode): for each sequence i and head
// h, softmax(scale * q K^T) V over the L_i cached tokens, with K and V read
// block by block through the sequence's block table.
//
// How (decode is a gather-GEMV: ~1 flop per byte, so HBM bandwidth bounds it
// and MFMA has nothing to do here):
//  * grid (head, sequence, partition); a workgroup of NW wavefronts owns one
//    partition of `part_blocks` blocks (up to 256) of one (sequence, head);
//    wave w takes blocks w, w+NW, ... of the partition;
//  * a wave's block-table entries are read once into one VGPR (lane t holds
//    the id of the wave's t-th block) and each id is moved to an SGPR with
//    readlane, so every tile address is uniform;
//  * one (block, head) tile is contiguous in the [N][H][bs][D] pool; a
//    wave-wide 16-byte-per-lane load covers 1 KiB of it, so K and V tiles are
//    read with fully coalesced dwordx4 loads straight into registers (each
//    lane consumes exactly the bytes it loads, so staging through LDS would
//    only add traffic);
//  * lanes form groups of `lanes per row` (16 for a 128 x 16-bit row): a
//    group holds one key/value row per load, the q.k partial sums are reduced
//    inside the group with DPP, and each group keeps its own running max and
//    sum (online softmax) over the rows it sees -- no cross-group traffic in
//    the loop;
//  * with the pool's stream flag (no block shared by two sequences of the
//    batch) V is read with non-temporal loads, which skip the cache fills a
//    read-once stream does not need; K keeps ordinary loads (measured: one
//    stream non-temporal beats both, and shared blocks want both cached);
//  * the next block's K and V loads are issued before the current block is
//    consumed (two register buffers), unconditionally: past the wave's last
//    block they re-read its K tile (an L2 hit), so the number of loads in
//    flight is the same on every path and the compiler's waits keep exactly
//    one block outstanding while the current one is consumed;
//  * at the end the groups, then the waves, merge their (max, sum, acc)
//    triples; a sequence that fits one partition writes its output directly,
//    otherwise each partition writes its triple to the workspace and a small
//    second kernel merges the triples of each (sequence, head).  (Merging in
//    the last partition to finish would need device-scope release/acquire
//    fences per workgroup; on this chip they write back and invalidate the
//    whole L2 and cost far more than a second launch.)
// Scores live in the log2 domain: s = log2(e) * scale * q.k, p = exp2(s - m).
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace pa {
namespace {

// MaxL: wave-loads per sub-tile at most (see kLoads).
template <int KV, int D, int BS, int MaxL>
struct Geo {
  static constexpr int kElem = dtype_bytes(KV);
  static constexpr int kRowBytes = D * kElem;
  static constexpr int kLpr = kRowBytes / 16;        // lanes per K/V row
  static constexpr int kEpl = 16 / kElem;            // elements per lane per load
  static constexpr int kRows = 64 / kLpr;            // rows one wave-load covers
  static constexpr bool kIdleGroups = BS < kRows;    // groups past the block's rows
  static constexpr int kTileLoads = kIdleGroups ? 1 : BS / kRows;  // wave-loads per tile
  // A tile is consumed in sub-tiles of at most MaxL wave-loads: 8 (two
  // buffers of K and V within 128 registers), 4 for 64-row blocks, which
  // then run like 16-row blocks of 16-bit elements with a quarter of the
  // table lookups (and 4 for every size in the several-pool kernel, whose
  // register budget is that of its largest branch).
  static constexpr int kLoads = kTileLoads < MaxL ? kTileLoads : MaxL;
  static constexpr int kSubs = kTileLoads / kLoads;
  static constexpr int kSubRows = kIdleGroups ? BS : kLoads * kRows;
  static constexpr int64_t kSubBytes = int64_t(kSubRows) * kRowBytes;
  static constexpr int64_t kTileBytes = int64_t(BS) * kRowBytes;
  static_assert(kLpr >= 4 && kLpr <= 32, "row must span 4..32 lanes");
};

// Per-lane arithmetic of one KV type; QT is the query's type where the
// kernel is instantiated for it (fp8 pools with 16-bit queries), else KV.
template <int KV, int QT = KV>
struct KvOps;

template <>
struct KvOps<PA_F32> {
  static constexpr int kEpl = 4;
  struct Q { float v[4]; };
  __device__ static Q load_q(const void* q, int64_t off, int) {
    float4 x = *(const float4*)((const float*)q + off);
    return Q{{x.x, x.y, x.z, x.w}};
  }
  __device__ static float dot(const Q& q, uint4 k) {
    float s = q.v[0] * __uint_as_float(k.x);
    s = fmaf(q.v[1], __uint_as_float(k.y), s);
    s = fmaf(q.v[2], __uint_as_float(k.z), s);
    return fmaf(q.v[3], __uint_as_float(k.w), s);
  }
  __device__ static void axpy(float* acc, float p, uint4 v) {
    acc[0] = fmaf(p, __uint_as_float(v.x), acc[0]);
    acc[1] = fmaf(p, __uint_as_float(v.y), acc[1]);
    acc[2] = fmaf(p, __uint_as_float(v.z), acc[2]);
    acc[3] = fmaf(p, __uint_as_float(v.w), acc[3]);
  }
};

template <>
struct KvOps<PA_F16> {
  static constexpr int kEpl = 8;
  struct Q { uint4 raw; };  // q in the pool's format: exact products in v_dot2
  __device__ static Q load_q(const void* q, int64_t off, int) {
    return Q{*(const uint4*)((const uint16_t*)q + off)};
  }
  __device__ static float dot(const Q& q, uint4 k) {
    float s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.raw.x),
                                     __builtin_bit_cast(half2_t, k.x), 0.f, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.raw.y),
                               __builtin_bit_cast(half2_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.raw.z),
                               __builtin_bit_cast(half2_t, k.z), s, false);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.raw.w),
                                  __builtin_bit_cast(half2_t, k.w), s, false);
  }
  __device__ static void axpy(float* acc, float p, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(p, f16_lo(w[i]), acc[2 * i]);
      acc[2 * i + 1] = fmaf(p, f16_hi(w[i]), acc[2 * i + 1]);
    }
  }
};

template <>
struct KvOps<PA_BF16> {
  static constexpr int kEpl = 8;
  struct Q { uint4 raw; };
  __device__ static Q load_q(const void* q, int64_t off, int) {
    return Q{*(const uint4*)((const uint16_t*)q + off)};
  }
  __device__ static float dot(const Q& q, uint4 k) {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.raw.x),
                                              __builtin_bit_cast(bf162_t, k.x), 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.raw.y),
                                        __builtin_bit_cast(bf162_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.raw.z),
                                        __builtin_bit_cast(bf162_t, k.z), s, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.raw.w),
                                           __builtin_bit_cast(bf162_t, k.w), s, false);
  }
  __device__ static void axpy(float* acc, float p, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(p, bf16_lo(w[i]), acc[2 * i]);
      acc[2 * i + 1] = fmaf(p, bf16_hi(w[i]), acc[2 * i + 1]);
    }
  }
};

// fp8 codes against a 16-bit query kept in its own type: two codes per
// exact conversion (v_cvt_scalef32_pk_{f16,bf16}_fp8, scale 1: every E4M3
// value is an f16 and a bf16 value) into a v_dot2 with two query elements,
// as the 16-bit pools do.
template <int QT>
struct Fp8Dot {
  static constexpr int kEpl = 16;
  struct Q { uint4 raw[2]; };  // 16 elements of QT
  __device__ static Q load_q(const void* q, int64_t off, int) {
    const uint4* p = (const uint4*)((const uint16_t*)q + off);
    return Q{{p[0], p[1]}};
  }
  __device__ static float dot(const Q& q, uint4 k) {
    const uint32_t w[4] = {k.x, k.y, k.z, k.w};
    const uint32_t qw[8] = {q.raw[0].x, q.raw[0].y, q.raw[0].z, q.raw[0].w,
                            q.raw[1].x, q.raw[1].y, q.raw[1].z, q.raw[1].w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (QT == PA_BF16) {
        const bf162_t k0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
        const bf162_t k1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, qw[2 * i]), k0, s, false);
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, qw[2 * i + 1]), k1, s,
                                            false);
      } else {
        const half2_t k0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false);
        const half2_t k1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true);
        s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qw[2 * i]), k0, s, false);
        s = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, qw[2 * i + 1]), k1, s, false);
      }
    }
    return s;
  }
};

template <int QT>
struct KvOps<PA_FP8_E4M3, QT> {
  static constexpr int kEpl = 16;
  struct Q { float v[16]; };  // q converted to float32 once
  __device__ static Q load_q(const void* q, int64_t off, int q_dtype) {
    Q r;
#pragma unroll
    for (int e = 0; e < 16; ++e) r.v[e] = load_as_f32(q, off + e, q_dtype);
    return r;
  }
  __device__ static float dot(const Q& q, uint4 k) {
    const uint32_t w[4] = {k.x, k.y, k.z, k.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float2_t a = fp8x2_lo(w[i]);
      float2_t b = fp8x2_hi(w[i]);
      s = fmaf(q.v[4 * i], a.x, s);
      s = fmaf(q.v[4 * i + 1], a.y, s);
      s = fmaf(q.v[4 * i + 2], b.x, s);
      s = fmaf(q.v[4 * i + 3], b.y, s);
    }
    return s;
  }
  __device__ static void axpy(float* acc, float p, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float2_t a = fp8x2_lo(w[i]);
      float2_t b = fp8x2_hi(w[i]);
      acc[4 * i] = fmaf(p, a.x, acc[4 * i]);
      acc[4 * i + 1] = fmaf(p, a.y, acc[4 * i + 1]);
      acc[4 * i + 2] = fmaf(p, b.x, acc[4 * i + 2]);
      acc[4 * i + 3] = fmaf(p, b.y, acc[4 * i + 3]);
    }
  }
};

template <>
struct KvOps<PA_FP8_E4M3, PA_BF16> : Fp8Dot<PA_BF16> {
  __device__ static void axpy(float* acc, float p, uint4 v) {
    KvOps<PA_FP8_E4M3, PA_FP8_E4M3>::axpy(acc, p, v);
  }
};

template <>
struct KvOps<PA_FP8_E4M3, PA_F16> : Fp8Dot<PA_F16> {
  __device__ static void axpy(float* acc, float p, uint4 v) {
    KvOps<PA_FP8_E4M3, PA_FP8_E4M3>::axpy(acc, p, v);
  }
};


__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kMaxPartBlocks = 256;

constexpr int default_max_loads(int bs) { return bs >= 64 ? 4 : 8; }

// 16 codes requantised from scale s_old to divisor d (see requant8).
__device__ __forceinline__ uint4 requant16(uint4 w, float s_old, float d) {
  const uint2 a = requant8(make_uint2(w.x, w.y), s_old, d);
  const uint2 b = requant8(make_uint2(w.z, w.w), s_old, d);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// A new row stored into an fp8 pool from the decode launch: codes (16 per
// lane, this lane's part of the row), the block's scale before (s_old) and
// after (s_new) the row, the divisor of the quantisation, and whether the
// block's earlier rows are requantised.  Without scale upkeep the row is
// quantised with the block's scale, which stays.  With it (the same float32
// operations as pa_reshape_and_cache's upkeep write, one-row runs): s_run =
// amax(|row|) / 448, s_old = 0 when the row starts its block (position 0),
// else the block's scale, s_new = max(s_old, s_run), divisor s_new (1 while
// it is 0), the earlier rows requantised when s_new > s_old.  A row of 128
// elements spans kLpr lanes; each of the wave's groups of kLpr lanes holds
// the whole row, so the amax is a group maximum.
struct Fp8Row {
  uint4 codes;
  float s_old, s_new, div;
  bool requant;
};

template <int kLpr>
__device__ __forceinline__ Fp8Row fp8_new_row(const void* src, int64_t off, int in_dtype,
                                              const float* scale, int p, int upkeep) {
  float x[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) x[e] = load_as_f32(src, off + e, in_dtype);
  Fp8Row r;
  const float s_cur = *scale;
  if (upkeep) {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int m = 1; m < kLpr; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    r.s_old = p == 0 ? 0.f : s_cur;
    r.s_new = fmaxf(r.s_old, __fdiv_rn(amax, 448.f));
    r.div = r.s_new > 0.f ? r.s_new : 1.f;
    r.requant = p > 0 && r.s_new > r.s_old;
  } else {
    r.s_old = r.s_new = r.div = s_cur;
    r.requant = false;
  }
  // the same in every lane: keep them in scalar registers
  r.s_old = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, r.s_old)));
  r.s_new = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, r.s_new)));
  r.div = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, r.div)));
  r.requant = __builtin_amdgcn_readfirstlane(int(r.requant)) != 0;
  float y[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) y[e] = fp8_prep(x[e], r.div);
  r.codes = make_uint4(pack4_fp8(y), pack4_fp8(y + 4), pack4_fp8(y + 8), pack4_fp8(y + 12));
  return r;
}

// Output element d of (seq, head) from the shared prefix's partials (max,
// sum, unnormalised output of partitions 0 .. prefix_parts - 1, written by
// the prefix pass that ran before this launch) and one more partial (M, S,
// A): the log-sum-exp merge, M' = max(M, m_c), S' = S 2^(M - M') + l_c
// 2^(m_c - M'), likewise A.
template <int D>
__device__ __forceinline__ void merge_prefix_partials(const DecodeArgs& a, int seq, int head,
                                                      int d, float M, float S, float A) {
  const int64_t base = (int64_t(seq) * a.num_heads + head) * a.ws_parts;
#pragma unroll 4
  for (int c = 0; c < a.prefix_parts; ++c) {
    const float mc = a.ws_ml[2 * (base + c)], lc = a.ws_ml[2 * (base + c) + 1];
    const float xc = a.ws_acc[(base + c) * D + d];
    const float Mn = fmaxf(M, mc);
    const float fo = __builtin_amdgcn_exp2f(M - Mn), fn = __builtin_amdgcn_exp2f(mc - Mn);
    S = S * fo + lc * fn;
    A = A * fo + xc * fn;
    M = Mn;
  }
  store_from_f32(a.out, (int64_t(seq) * a.num_heads + head) * D + d, a.out_dtype,
                 S > 0.f ? A / S : 0.f);
}

// One workgroup's work: (head, sequence, partition) = blockIdx (x, y, z).
// kAppend: the step's new K/V row of each sequence (position L - 1) comes
// with the call; the workgroup of the last partition stores it at its slot
// (fp8 pools: quantised there, see fp8_new_row) and uses it from registers
// for that position, so no wave reads the row while it is being written.
template <int KV, int D, int BS, int NW, bool kStreamV, int MaxL, bool kAppend = false,
          int QT = KV>
__device__ __forceinline__ void decode_body(const DecodeArgs& a) {
  using G = Geo<KV, D, BS, MaxL>;
  using Ops = KvOps<KV, QT>;
  constexpr int E = G::kEpl;
  static_assert(E == Ops::kEpl, "lane element count");

  // Heads of one (sequence, partition) are adjacent in the dispatch order
  // (they read the same blocks, one tile apart); the highest partitions,
  // which only the longest sequences have, are dispatched first.
  const int head = blockIdx.x;
  const int seq = blockIdx.y;
  const int part = a.max_parts - 1 - int(blockIdx.z);
  const int H = a.num_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // The block-table row and q do not depend on the context length: their
  // loads go out together with it, so a workgroup waits for one round trip
  // before it can address its first tile, not two.  Lane t of wave w reads
  // entry w + NW t of the partition (bounded by the table's row length; the
  // entries past the sequence's blocks are never used).
  const int64_t out_off = (int64_t(seq) * H + head) * D;
  const int blk0 = a.first_block + part * a.part_blocks;
  const int32_t* table = a.block_tables + int64_t(seq) * a.max_blocks_per_seq + blk0;
  const int t_idx = wave + NW * lane;
  const int tab = (t_idx < a.part_blocks && blk0 + t_idx < a.max_blocks_per_seq) ? table[t_idx] : 0;
  static_assert(kMaxPartBlocks <= 64 * NW, "one table register per wave");
  const int grp = lane / G::kLpr;
  const int col = lane % G::kLpr;
  const typename Ops::Q q = Ops::load_q(a.q, out_off + col * E, a.q_dtype);

  const int L = a.context_lens[seq];
  if (L <= 0) {
    if (part == 0)
      for (int d = tid; d < D; d += NW * 64) store_from_f32(a.out, out_off + d, a.out_dtype, 0.f);
    return;
  }
  const int nblocks = (L + BS - 1) / BS;
  const int nparts = nblocks > a.first_block
                         ? (nblocks - a.first_block + a.part_blocks - 1) / a.part_blocks
                         : 0;
  if (part >= nparts) {
    // a sequence with no blocks past the shared prefix: its output is the
    // merge of the prefix's partials alone
    if (a.fuse_merge && part == 0 && tid < D)
      merge_prefix_partials<D>(a, seq, head, tid, kNoMax, 0.f, 0.f);
    return;
  }
  const int nb = min(a.part_blocks, nblocks - blk0);
  const bool row_ok = !G::kIdleGroups || grp < BS;

  // The new row (kAppend): the wave that owns the partition's last block
  // (the one holding position L - 1) loads it, 16 bytes per lane (this
  // lane's column), and stores it after the loop (a store here would wait
  // for these loads before any tile load could go out).
  uint4 knew = make_uint4(0, 0, 0, 0), vnew = make_uint4(0, 0, 0, 0);
  int64_t new_slot = -1;
  // fp8 pools: the new row's block and position in it, the scales before
  // (s_old) and after (s_new) the row, the divisors of its quantisation, and
  // whether the block's earlier rows are requantised (scale upkeep).
  Fp8Row fk{}, fv{};
  int64_t new_blk = -1;
  int new_p = 0;
  if constexpr (kAppend) {
    if (part == nparts - 1 && wave == (nb - 1) % NW) new_slot = a.new_slots[seq];
    if (new_slot >= 0) {
      if constexpr (KV == PA_FP8_E4M3) {
        new_blk = new_slot / BS;
        new_p = int(new_slot % BS);
        const int64_t si = new_blk * H + head;
        fk = fp8_new_row<G::kLpr>(a.k_new, out_off + col * E, a.q_dtype, a.k_scale + si, new_p,
                                  a.fp8_upkeep);
        fv = fp8_new_row<G::kLpr>(a.v_new, out_off + col * E, a.q_dtype, a.v_scale + si, new_p,
                                  a.fp8_upkeep);
        knew = fk.codes;
        vnew = fv.codes;
      } else {
        const int64_t off = (out_off + col * E) * G::kElem;
        knew = *(const uint4*)((const char*)a.k_new + off);
        vnew = *(const uint4*)((const char*)a.v_new + off);
      }
    }
  }
  const bool has_new = new_slot >= 0;

  // This wave's blocks are wave, wave + NW, ... of the partition (n_w <= 64
  // of them); lane t of `tab` holds the block id of the wave's t-th block.
  // Its work units are their sub-tiles in order: unit u is sub-tile
  // u % kSubs of its (u / kSubs)-th block.
  const int n_w = wave < nb ? (nb - wave + NW - 1) / NW : 0;
  const int n_u = n_w * G::kSubs;
  const int64_t blk_stride = int64_t(H) * G::kTileBytes;
  char* const kbase = (char*)a.k_cache + int64_t(head) * G::kTileBytes + lane * 16;
  char* const vbase = (char*)a.v_cache + int64_t(head) * G::kTileBytes + lane * 16;

  // fp8 scale upkeep: when the new row grows its block's scale, the block's
  // earlier rows are requantised in place before the loop reads them.  Each
  // lane rewrites exactly the 16 bytes it loads from that block in the loop,
  // so its own later loads see the new codes (same lane, program order).
  if constexpr (kAppend && KV == PA_FP8_E4M3) {
    if (has_new && (fk.requant || fv.requant)) {
#pragma unroll
      for (int sub = 0; sub < G::kSubs; ++sub)
#pragma unroll
        for (int i = 0; i < G::kLoads; ++i) {
          const int row = sub * G::kSubRows + i * G::kRows + grp;
          if (row_ok && row < new_p) {
            const int64_t off = new_blk * blk_stride + sub * G::kSubBytes + i * 1024;
            if (fk.requant) {
              uint4* kp = (uint4*)(kbase + off);
              *kp = requant16(*kp, fk.s_old, fk.div);
            }
            if (fv.requant) {
              uint4* vp = (uint4*)(vbase + off);
              *vp = requant16(*vp, fv.s_old, fv.div);
            }
          }
        }
    }
  }

  float m = kNoMax, l = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  uint4 k0[G::kLoads], v0[G::kLoads], k1[G::kLoads], v1[G::kLoads];
  int p0 = 0, p1 = 0;

  // Loads of the wave's unit u.  Past its last unit (the pipeline's
  // prefetch after the final one, never consumed) both K and V re-read the
  // last unit's K sub-tile: K loads are ordinary ones, so it is still in the
  // L2, whereas a streamed V sub-tile would come from HBM again.
  auto issue = [&](uint4* kr, uint4* vr, int& phys, int u) {
    const bool past = u >= n_u;
    const int ue = past ? n_u - 1 : u;
    phys = __builtin_amdgcn_readlane(tab, ue / G::kSubs);
    const int64_t sub = int64_t(ue % G::kSubs) * G::kSubBytes;
    const char* kp = kbase + int64_t(phys) * blk_stride + sub;
    const char* vp = past ? kp : vbase + int64_t(phys) * blk_stride + sub;
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      if (row_ok) {
        kr[i] = *(const uint4*)(kp + i * 1024);
        if constexpr (kStreamV) {
          const u32x4_t x = __builtin_nontemporal_load((const u32x4_t*)(vp + i * 1024));
          vr[i] = make_uint4(x.x, x.y, x.z, x.w);
        } else {
          vr[i] = *(const uint4*)(vp + i * 1024);
        }
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto consume = [&](uint4* kr, uint4* vr, int phys, int u) {
    float mul_k = a.scale_log2;
    float mul_v = 1.f;
    const int jl = wave + (u / G::kSubs) * NW;  // block of the partition
    const int r0 = (blk0 + jl) * BS + (u % G::kSubs) * G::kSubRows;  // first token of the unit
    const int tok0 = r0 + grp;                    // token of load 0 in this lane's group
    const bool full = r0 + G::kSubRows <= L;
    if constexpr (KV == PA_FP8_E4M3) {
      if (kAppend && has_new && phys == new_blk) {
        // the new row's block: its scales after the row (its earlier rows
        // were requantised before the loop when a scale grew)
        mul_k *= fk.s_new;
        mul_v = fv.s_new;
      } else {
        mul_k *= a.k_scale[int64_t(phys) * H + head];
        mul_v = a.v_scale[int64_t(phys) * H + head];
      }
    }
    if constexpr (kAppend) {
      if (has_new && r0 + G::kSubRows >= L) {   // the unit holding position L - 1
#pragma unroll
        for (int i = 0; i < G::kLoads; ++i) {
          if (tok0 + i * G::kRows == L - 1) {
            kr[i] = knew;
            vr[i] = vnew;
          }
        }
      }
    }
    float s[G::kLoads];
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      s[i] = group_sum<G::kLpr>(Ops::dot(q, kr[i])) * mul_k;
      if constexpr (G::kIdleGroups) s[i] = row_ok ? s[i] : -INFINITY;
    }
    if (!full) {
#pragma unroll
      for (int i = 0; i < G::kLoads; ++i) {
        if (tok0 + i * G::kRows >= L) {
          s[i] = -INFINITY;
          vr[i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    float mx = m;
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) mx = fmaxf(mx, s[i]);
    const float alpha = fast_exp2(m - mx);
    float psum = 0.f;
    float p[G::kLoads];
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) {
      p[i] = fast_exp2(s[i] - mx);
      psum += p[i];
    }
    l = fmaf(l, alpha, psum);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < G::kLoads; ++i) Ops::axpy(acc, p[i] * mul_v, vr[i]);
    m = mx;
  };

  // Two-deep software pipeline over this wave's n_u units (the prefetch
  // after the last one is a dummy, see issue()).
  if (n_u > 0) {
    issue(k0, v0, p0, 0);
    for (int i = 0;;) {
      issue(k1, v1, p1, i + 1);
      consume(k0, v0, p0, i);
      if (++i >= n_u) break;
      issue(k0, v0, p0, i + 1);
      consume(k1, v1, p1, i);
      if (++i >= n_u) break;
    }
  }

  if constexpr (kAppend) {
    if (has_new && lane < G::kLpr) {   // one lane group stores the row
      const int64_t dst =
          ((new_slot / BS * H + head) * BS + new_slot % BS) * G::kRowBytes + lane * 16;
      *(uint4*)((char*)a.k_cache + dst) = knew;
      *(uint4*)((char*)a.v_cache + dst) = vnew;
    }
    if constexpr (KV == PA_FP8_E4M3) {
      if (has_new && a.fp8_upkeep && lane == 0) {
        // (the pool's scales are writable; the decode reads them through
        // const pointers)
        const_cast<float*>(a.k_scale)[new_blk * H + head] = fk.s_new;
        const_cast<float*>(a.v_scale)[new_blk * H + head] = fv.s_new;
      }
    }
  }

  // Merge the groups of this wave (lanes with equal col, different grp).
#pragma unroll
  for (int mask = G::kLpr; mask < 64; mask <<= 1) {
    const float mo = __shfl_xor(m, mask);
    const float lo = __shfl_xor(l, mask);
    const float mx = fmaxf(m, mo);
    const float sa = fast_exp2(m - mx);
    const float sb = fast_exp2(mo - mx);
    l = l * sa + lo * sb;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = acc[e] * sa + __shfl_xor(acc[e], mask) * sb;
    m = mx;
  }

  // Merge the waves through LDS.
  __shared__ float sm_acc[NW][D];
  __shared__ float sm_m[NW], sm_l[NW];
  if (lane < G::kLpr) {
#pragma unroll
    for (int e = 0; e < E; ++e) sm_acc[wave][col * E + e] = acc[e];
  }
  if (lane == 0) {
    sm_m[wave] = m;
    sm_l[wave] = l;
  }
  __syncthreads();

  float A = 0.f, M = kNoMax, S = 0.f;
  if (tid < D) {
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w]);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(sm_m[w] - M);
      S = fmaf(sm_l[w], f, S);
      A = fmaf(sm_acc[w][tid], f, A);
    }
  }

  if (nparts == 1 && a.prefix_parts == 0) {
    if (tid < D) store_from_f32(a.out, out_off + tid, a.out_dtype, S > 0.f ? A / S : 0.f);
    return;
  }
  if (a.fuse_merge) {  // this is the sequence's only partition past the prefix
    if (tid < D) merge_prefix_partials<D>(a, seq, head, tid, M, S, A);
    return;
  }

  // Split-K: publish this partition's (max, sum, acc) for the merge kernel.
  const int64_t pidx = (int64_t(seq) * H + head) * a.ws_parts + a.prefix_parts + part;
  if (tid < D) a.ws_acc[pidx * D + tid] = A;
  if (tid == 0) {
    a.ws_ml[2 * pidx] = M;
    a.ws_ml[2 * pidx + 1] = S;
  }
}

template <int KV, int D, int BS, int NW, bool kStreamV, bool kAppend, int QT = KV>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  decode_body<KV, D, BS, NW, kStreamV, default_max_loads(BS), kAppend, QT>(a);
}

// A batch over several pools (same heads, head_dim and KV type; e.g. the
// block-size views of one arena): the sequences of group g are rows
// [seq_begin, next group's seq_begin) of the batch and use group g's pool
// and block table.  Each workgroup finds its group (a uniform scan of at most
// kMaxGroups entries), then runs the body of its group's block size with
// sub-tiles of at most 4 wave-loads, so that every branch fits the same
// register budget.  Partitions are part_tokens long in every group.
template <int KV, int D, int NW, bool kStreamV, int QT = KV>
__global__ __launch_bounds__(NW * 64) void decode_multi_kernel(DecodeMultiArgs m) {
  const int seq = blockIdx.y;
  int g = 0;
  for (int i = 1; i < m.num_groups; ++i)
    if (seq >= m.g[i].seq_begin) g = i;
  const DecodeGroup& grp = m.g[g];
  DecodeArgs a = m.base;
  a.k_cache = grp.k_cache;
  a.v_cache = grp.v_cache;
  a.k_scale = grp.k_scale;
  a.v_scale = grp.v_scale;
  // the body indexes rows by the batch-wide sequence number
  a.block_tables = grp.block_tables - int64_t(grp.seq_begin) * grp.max_blocks_per_seq;
  a.max_blocks_per_seq = grp.max_blocks_per_seq;
  a.block_size = grp.block_size;
  a.part_blocks = m.part_tokens / grp.block_size;
  switch (grp.block_size) {
    case 4: decode_body<KV, D, 4, NW, kStreamV, 4, false, QT>(a); break;
    case 8: decode_body<KV, D, 8, NW, kStreamV, 4, false, QT>(a); break;
    case 16: decode_body<KV, D, 16, NW, kStreamV, 4, false, QT>(a); break;
    case 32: decode_body<KV, D, 32, NW, kStreamV, 4, false, QT>(a); break;
    case 64: decode_body<KV, D, 64, NW, kStreamV, 4, false, QT>(a); break;
  }
}

// Merge the partitions of each (sequence, head) that has more than one:
// M = max_p m_p, out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
// R threads per output element take every R-th partition with a running
// maximum (all their loads can be in flight together), then combine in LDS.
// A workgroup covers DC of the D output elements (blockIdx.z picks which):
// many partitions take more threads per element and so more workgroups.
template <int D, int R, int DC>
__global__ __launch_bounds__(DC * R) void decode_merge_kernel(DecodeArgs a) {
  const int head = blockIdx.x;
  const int seq = blockIdx.y;
  const int H = a.num_heads;
  const int d = int(blockIdx.z) * DC + int(threadIdx.x) % DC;
  const int r = threadIdx.x / DC;
  const int64_t sh = int64_t(seq) * H + head;
  const float* ml = a.ws_ml + 2 * sh * a.ws_parts;
  const float* pa = a.ws_acc + sh * a.ws_parts * D + d;
  // Partition r's triple is loaded before the context length is known (it
  // lies inside the workspace whenever r < ws_parts, and is used only if
  // the partition exists), so the common case of at most R partitions waits
  // for one round trip to memory, not two.
  float m0 = kNoMax, l0 = 0.f, x0 = 0.f;
  if (r < a.ws_parts) {
    m0 = ml[2 * r];
    l0 = ml[2 * r + 1];
    x0 = pa[int64_t(r) * D];
  }
  const int L = a.context_lens[seq];
  const int nblocks = (L + a.block_size - 1) / a.block_size;
  const int nparts = a.prefix_parts + (nblocks > a.first_block
                                           ? (nblocks - a.first_block + a.part_blocks - 1) /
                                                 a.part_blocks
                                           : 0);
  if (nparts <= 1 && a.prefix_parts == 0) return;
  float M = kNoMax, A = 0.f, S = 0.f;
  if (r < nparts) {
    M = m0;
    S = l0;
    A = x0;
  }
#pragma unroll 4
  for (int p = r + R; p < nparts; p += R) {
    const float m = ml[2 * p], l = ml[2 * p + 1], x = pa[int64_t(p) * D];
    const float Mn = fmaxf(M, m);
    const float fo = fast_exp2(M - Mn), fn = fast_exp2(m - Mn);
    S = S * fo + l * fn;
    A = A * fo + x * fn;
    M = Mn;
  }
  const int dl = int(threadIdx.x) % DC;
  __shared__ float sm_a[R][DC], sm_m[R][DC], sm_s[R][DC];
  sm_a[r][dl] = A;
  sm_m[r][dl] = M;
  sm_s[r][dl] = S;
  __syncthreads();
  if (r != 0) return;
  float Mg = kNoMax;
#pragma unroll
  for (int i = 0; i < R; ++i) Mg = fmaxf(Mg, sm_m[i][dl]);
  float Ag = 0.f, Sg = 0.f;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const float f = fast_exp2(sm_m[i][dl] - Mg);
    Ag = fmaf(sm_a[i][dl], f, Ag);
    Sg = fmaf(sm_s[i][dl], f, Sg);
  }
  store_from_f32(a.out, sh * D + d, a.out_dtype, Sg > 0.f ? Ag / Sg : 0.f);
}

// The merge for workspaces of at most P partitions per sequence: one thread
// per output element, with every partition's triple loaded before the
// context length is known (one round trip to memory).  Same operations, in
// the same order, as decode_merge_kernel<D, R, D> for sequences of at most
// R partitions.
template <int D, int P>
__global__ __launch_bounds__(D) void decode_merge_small_kernel(DecodeArgs a) {
  const int head = blockIdx.x;
  const int seq = blockIdx.y;
  const int H = a.num_heads;
  const int d = threadIdx.x;
  const int64_t sh = int64_t(seq) * H + head;
  const float* ml = a.ws_ml + 2 * sh * a.ws_parts;
  const float* pa = a.ws_acc + sh * a.ws_parts * D + d;
  float m[P], l[P], x[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    m[p] = kNoMax;
    l[p] = 0.f;
    x[p] = 0.f;
    if (p < a.ws_parts) {
      m[p] = ml[2 * p];
      l[p] = ml[2 * p + 1];
      x[p] = pa[int64_t(p) * D];
    }
  }
  const int L = a.context_lens[seq];
  const int nblocks = (L + a.block_size - 1) / a.block_size;
  const int nparts = a.prefix_parts + (nblocks > a.first_block
                                           ? (nblocks - a.first_block + a.part_blocks - 1) /
                                                 a.part_blocks
                                           : 0);
  if (nparts <= 1 && a.prefix_parts == 0) return;
  float M = kNoMax;
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < nparts) M = fmaxf(M, m[p]);
  float A = 0.f, S = 0.f;
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < nparts) {
      const float f = fast_exp2(m[p] - M);
      A = fmaf(x[p], f, A);
      S = fmaf(l[p], f, S);
    }
  store_from_f32(a.out, sh * D + d, a.out_dtype, S > 0.f ? A / S : 0.f);
}

constexpr int kWaves = 4;

// The merge launch: up to 8 partitions, one thread per element; up to 16,
// 512 / D threads per element over all D elements in one workgroup; more,
// 16 threads per element over 64 elements per workgroup.
template <int D>
void launch_merge(const DecodeArgs& a, int num_seqs, hipStream_t stream) {
  if (a.ws_parts <= 8) {
    hipLaunchKernelGGL((decode_merge_small_kernel<D, 8>), dim3(a.num_heads, num_seqs), dim3(D), 0,
                       stream, a);
  } else if (a.ws_parts <= 16) {
    constexpr int R = 512 / D;
    hipLaunchKernelGGL((decode_merge_kernel<D, R, D>), dim3(a.num_heads, num_seqs), dim3(D * R),
                       0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_merge_kernel<D, 16, 64>), dim3(a.num_heads, num_seqs, D / 64),
                       dim3(64 * 16), 0, stream, a);
  }
}

template <int KV, int D, int BS, int QT>
void launch_q(const DecodeArgs& a, bool stream_v, dim3 grid, hipStream_t stream) {
  if (a.k_new) {
    if (stream_v)
      hipLaunchKernelGGL((decode_kernel<KV, D, BS, kWaves, true, true, QT>), grid,
                         dim3(kWaves * 64), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<KV, D, BS, kWaves, false, true, QT>), grid,
                         dim3(kWaves * 64), 0, stream, a);
  } else if (stream_v) {
    hipLaunchKernelGGL((decode_kernel<KV, D, BS, kWaves, true, false, QT>), grid,
                       dim3(kWaves * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<KV, D, BS, kWaves, false, false, QT>), grid,
                       dim3(kWaves * 64), 0, stream, a);
  }
}

template <int KV, int D, int BS>
hipError_t launch_t(const DecodeArgs& a, bool stream_v, int num_seqs, hipStream_t stream) {
  dim3 grid(a.num_heads, num_seqs, a.max_parts);
  // fp8 pools: the body for the query's type (16-bit queries in v_dot2)
  if constexpr (KV == PA_FP8_E4M3) {
    if (a.q_dtype == PA_BF16)
      launch_q<KV, D, BS, PA_BF16>(a, stream_v, grid, stream);
    else if (a.q_dtype == PA_F16)
      launch_q<KV, D, BS, PA_F16>(a, stream_v, grid, stream);
    else
      launch_q<KV, D, BS, KV>(a, stream_v, grid, stream);
  } else {
    launch_q<KV, D, BS, KV>(a, stream_v, grid, stream);
  }
  if ((a.max_parts > 1 || a.prefix_parts > 0) && !a.fuse_merge) launch_merge<D>(a, num_seqs, stream);
  return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_bs(const DecodeArgs& a, int bs, bool sv, int num_seqs, hipStream_t stream) {
  switch (bs) {
    case 4: return launch_t<KV, D, 4>(a, sv, num_seqs, stream);
    case 8: return launch_t<KV, D, 8>(a, sv, num_seqs, stream);
    case 16: return launch_t<KV, D, 16>(a, sv, num_seqs, stream);
    case 32: return launch_t<KV, D, 32>(a, sv, num_seqs, stream);
    case 64: return launch_t<KV, D, 64>(a, sv, num_seqs, stream);
  }
  return hipErrorInvalidValue;
}

template <int KV>
hipError_t launch_d(const DecodeArgs& a, int d, int bs, bool sv, int num_seqs,
                    hipStream_t stream) {
  if (d == 64) return launch_bs<KV, 64>(a, bs, sv, num_seqs, stream);
  if (d == 128) return launch_bs<KV, 128>(a, bs, sv, num_seqs, stream);
  return hipErrorInvalidValue;
}

template <int KV, int D>
hipError_t launch_multi_t(const DecodeMultiArgs& m, bool stream_v, int num_seqs,
                          hipStream_t stream) {
  dim3 grid(m.base.num_heads, num_seqs, m.base.max_parts);
  // fp8 pools: the body for the query's type, as launch_t picks it (the
  // same arithmetic as pa_decode, bit for bit)
  auto go = [&](auto qt_c) {
    constexpr int QT = decltype(qt_c)::value;
    if (stream_v)
      hipLaunchKernelGGL((decode_multi_kernel<KV, D, kWaves, true, QT>), grid, dim3(kWaves * 64),
                         0, stream, m);
    else
      hipLaunchKernelGGL((decode_multi_kernel<KV, D, kWaves, false, QT>), grid,
                         dim3(kWaves * 64), 0, stream, m);
  };
  if constexpr (KV == PA_FP8_E4M3) {
    if (m.base.q_dtype == PA_BF16)
      go(std::integral_constant<int, PA_BF16>{});
    else if (m.base.q_dtype == PA_F16)
      go(std::integral_constant<int, PA_F16>{});
    else
      go(std::integral_constant<int, KV>{});
  } else {
    go(std::integral_constant<int, KV>{});
  }
  if (m.base.max_parts > 1) {
    // The merge kernel counts a sequence's partitions as ceil(L / block_size
    // / part_blocks): in tokens, with block_size 1.
    DecodeArgs a = m.base;
    a.block_size = 1;
    a.part_blocks = m.part_tokens;
    launch_merge<D>(a, num_seqs, stream);
  }
  return hipGetLastError();
}

template <int KV>
hipError_t launch_multi_d(const DecodeMultiArgs& m, int d, bool sv, int num_seqs,
                          hipStream_t stream) {
  if (d == 64) return launch_multi_t<KV, 64>(m, sv, num_seqs, stream);
  if (d == 128) return launch_multi_t<KV, 128>(m, sv, num_seqs, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_multi(const DecodeMultiArgs& m, int kv_dtype, int head_dim,
                               bool stream_v, int num_seqs, hipStream_t stream) {
  switch (kv_dtype) {
    case PA_F32: return launch_multi_d<PA_F32>(m, head_dim, stream_v, num_seqs, stream);
    case PA_F16: return launch_multi_d<PA_F16>(m, head_dim, stream_v, num_seqs, stream);
    case PA_BF16: return launch_multi_d<PA_BF16>(m, head_dim, stream_v, num_seqs, stream);
    case PA_FP8_E4M3: return launch_multi_d<PA_FP8_E4M3>(m, head_dim, stream_v, num_seqs, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, int head_dim, int block_size,
                         bool stream_v, int num_seqs, hipStream_t stream) {
  const int d = head_dim, bs = block_size;
  const bool sv = stream_v;
  switch (kv_dtype) {
    case PA_F32: return launch_d<PA_F32>(a, d, bs, sv, num_seqs, stream);
    case PA_F16: return launch_d<PA_F16>(a, d, bs, sv, num_seqs, stream);
    case PA_BF16: return launch_d<PA_BF16>(a, d, bs, sv, num_seqs, stream);
    case PA_FP8_E4M3: return launch_d<PA_FP8_E4M3>(a, d, bs, sv, num_seqs, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
