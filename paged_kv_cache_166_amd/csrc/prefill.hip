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
//  * K and V tiles travel through registers into LDS rows: each wave loads
//    its part of a tile with global_load_dwordx4 a tile ahead of the LDS
//    ring, converts it in registers where needed and stores it with
//    ds_write_b128 into a three-stage ring (the tile consumed, the next one,
//    the one being filled); one workgroup barrier per tile;
//  * S^T = K Q^T on v_mfma_f32_32x32x16 (bf16 or fp16 inputs, fp32
//    accumulate): A = K rows from LDS, B = the wave's Q rows, held in
//    registers for the whole walk;
//  * the accumulator layout of S^T gives every lane one query column and 16
//    of the tile's keys, so the online softmax (running max m, running sum
//    l, exp2 of log2-scaled scores) is lane-local plus one exchange between
//    the two half-waves; a row's reference maximum (and so the accumulator
//    rescale) moves only when the row maximum grows by more than 2^8;
//  * O^T += V^T P^T on v_mfma_f32_32x32x16: P is used straight from the S^T
//    accumulators as the B operand (the contraction index is permuted to
//    match the accumulator layout) so P never leaves registers; the V^T
//    operand is read from the V rows by gfx950's transposing LDS read
//    (ds_read_b64_tr_b16) in the same permuted key order.  P is rounded to
//    fp16 (bf16's 8 bits would cost up to ~5e-3 on rows of a few keys); for
//    bf16 pools V is converted to fp16 in registers, between its load and
//    its store into LDS;
//  * tiles wholly above the causal diagonal are skipped per wave; only
//    tiles that cross it are masked.
// Workgroups are mapped so that all query tiles of one (sequence, head) run
// on the same XCD (its L2 holds that head's K/V).  In batches of up to 64
// (sequence, query tile) classes each XCD takes its work items longest
// first (a longest-processing-time order over the classes' key-tile
// counts, which each workgroup ranks in its prologue), so the short items
// fill the end of the launch; larger batches go pair by pair, the last query
// tile of a pair (it sees the most keys) first.
#include <type_traits>

#include "device.h"
#include "kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kQW = 32;                 // query rows per wave
constexpr int kBM = kWaves * kQW;       // query rows per workgroup
constexpr int kBN = 32;                 // keys per tile
constexpr int kXcds = 8;
// Buffer resource flags (dword 3) for plain 32-bit raw buffer loads.
constexpr int kBufferFlags = 0x00020000;
// Longest work first: batches of at most this many (sequence, query tile)
// classes have their workgroups dispatched in order of decreasing key-tile
// count (each workgroup ranks the classes in its prologue).
constexpr int kMaxLptClasses = 64;

__host__ __device__ inline bool lpt_order(int num_seqs, int num_qtiles) {
  return num_seqs * num_qtiles <= kMaxLptClasses;
}

// Heads h in [0, H) whose pair seq * H + h is dealt to XCD x (pair % 8 == x):
// the first one and how many.
__device__ __forceinline__ int first_head_on(int x, int seq, int H) {
  return ((x - seq * H) % kXcds + kXcds) % kXcds;
}
__device__ __forceinline__ int heads_on(int x, int seq, int H) {
  const int h0 = first_head_on(x, seq, H);
  return h0 < H ? (H - 1 - h0) / kXcds + 1 : 0;
}

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

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed fp16 pair, RNE (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}

// Eight bf16 values -> eight fp16 values (RNE), in place in a 16-byte word.
__device__ __forceinline__ u32x4_t bf16x8_to_f16x8(u32x4_t w) {
  return u32x4_t{pack_f16(bf16_lo(w.x), bf16_hi(w.x)), pack_f16(bf16_lo(w.y), bf16_hi(w.y)),
                 pack_f16(bf16_lo(w.z), bf16_hi(w.z)), pack_f16(bf16_lo(w.w), bf16_hi(w.w))};
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// gfx950 transposing LDS read (ds_read_b64_tr_b16), 8 bytes per lane: in each
// group of 16 lanes, lane i receives 16-bit element i % 4 of the 8-byte
// pieces addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12 (in that
// order).  So if lane j addresses 4 consecutive dimensions d0 + 4 (j % 4) ..
// of row r0 + j / 4, lane i gets dimension d0 + i of rows r0 .. r0 + 3.
//
// Issued as inline assembly with an immediate offset: the compiler's wait
// insertion cannot tell the ring stages apart for this instruction and would
// otherwise wait for every memory operation in flight before some of these
// reads.  The caller waits with lds_wait_tr() before using the results.
template <int kOffset>
__device__ __forceinline__ uint2 lds_read_tr16(uint32_t lds_addr) {
  static_assert(kOffset >= 0 && kOffset < 65536, "ds offset field");
  uint2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(lds_addr), "i"(kOffset));
  return r;
}

// n 16-byte LDS reads at a, a + 1024, ... (inline assembly, waited for
// before returning) and the matching writes (complete at the next wait for
// LDS operations, such as the one in wg_barrier()).
template <int n>
__device__ __forceinline__ void lds_read_b128_x(uint32_t a, u32x4_t (&w)[n]) {
  static_assert(n == 1 || n == 2, "one or two chunks per lane");
  asm volatile("ds_read_b128 %0, %1" : "=v"(w[0]) : "v"(a));
  if constexpr (n == 2) {
    asm volatile("ds_read_b128 %0, %1 offset:1024" : "=v"(w[1]) : "v"(a));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]));
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]));
  }
}
template <int n>
__device__ __forceinline__ void lds_write_b128_x(uint32_t a, const u32x4_t (&w)[n]) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(w[0]) : "memory");
  if constexpr (n == 2) asm volatile("ds_write_b128 %0, %1 offset:1024" : : "v"(a), "v"(w[1]) : "memory");
}

// Wait for every LDS read issued so far (the transposing reads above among
// them); the values pass through the statement so no use of them can be
// scheduled before the wait.
__device__ __forceinline__ void lds_wait_tr(uint2 (&v)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}

// The running maximum a query row's weights are taken against moves only
// when the row's maximum grows by more than this (log2 units): weights stay
// below 2^8, well inside fp16, and the accumulator is rescaled rarely.
constexpr float kRescaleSlack = 8.0f;

// s_waitcnt immediate: at most n vector-memory operations outstanding, the
// other counters unconstrained (vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] << 14).
constexpr int wait_vm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }

// (v[l mod 32], v[l mod 32 + 32]) in lane l: this lane's value and its
// partner's in the other half-wave, by gfx950's v_permlane32_swap (a VALU
// exchange, no LDS round trip).
__device__ __forceinline__ float2 half_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// a ^ b with b uniform (v_xor_b32 with an SGPR operand).  With the lane
// constant a redefined once per tile (redefine() below), an LDS offset that
// is a lane constant XOR a per-step constant is rebuilt with one VALU
// operation per use instead of being kept, per step, in a register of its
// own (the compiler would hoist all of them out of the loop).
__device__ __forceinline__ uint32_t xor_here(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_xor_b32 %0, %1, %2" : "=v"(r) : "s"(b), "v"(a));
  return r;
}

// Makes v opaque to the compiler from here on (same value): expressions of
// it computed after this point are not hoisted above it.
__device__ __forceinline__ void redefine(uint32_t& v) { asm volatile("" : "+v"(v)); }

typedef __attribute__((address_space(3))) void lds_t;

// s_waitcnt immediate: all LDS / scalar-memory operations done, vector
// memory unconstrained.
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);

// Workgroup barrier without a memory fence: this wave's LDS accesses are
// complete when it arrives, and the vector-memory waits before it are the
// caller's (a fence would also wait for every global load in flight); the empty asm
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Occupancy: at least three waves per SIMD (at most 168 VGPRs; 48 KiB of
// LDS per workgroup): the loop is latency-bound, and a third workgroup per
// CU hides more of it than the registers the compiler gives up cost.  (fp8
// pools with blocks shorter than a tile, whose raw loads span several
// blocks, and fp16 with 4-token blocks at head size 128 would spill at that
// bound and keep two.)
// kPrefix: the shared-prefix partials of pa_decode_shared_prefix -- query
// rows are the batch's decode queries (row r = sequence r), keys are one
// chunk of the shared prefix (sequence 0's table), no causal mask, and the
// workgroup writes (max, sum, unnormalised output) per row to the decode
// workspace instead of the normalised output.
// QT: the 16-bit type of q and of the Q K^T MFMAs (the pool's type for
// 16-bit pools; f16 or bf16 for fp8 pools).
// K/V tiles travel through registers: each wave loads its part of tile t+2
// (global_load_dwordx4, one tile ahead of the LDS ring) while the workgroup
// computes on tile t+1's predecessor, converts it in registers -- bf16 V to
// fp16; fp8 E4M3 codes to 16 bits (exactly: every E4M3 value is a bf16 and
// an fp16 value), K to QT and V to fp16 -- and stores it into the next LDS
// stage (ds_write_b128) in the swizzled row layout the fragment reads use.
// fp8 pools: the per-(block, head) scales are applied to the scores (K) and
// to the weights before the P V product (V), so the only added rounding is
// that of the scaled weights to fp16.
template <int KV, int QT, int D, int BS, bool kPrefix = false>
__global__ __launch_bounds__(kWaves * 64)
__attribute__((amdgpu_waves_per_eu((KV == PA_FP8_E4M3 && BS < 8) ? 2 : 3)))
void prefill_kernel(PrefillArgs a, int num_qtiles, int num_pairs, int lpt_by_seq) {
  constexpr bool kFp8 = KV == PA_FP8_E4M3;
  constexpr int kRowBytes = D * 2;
  constexpr int kChunks = D / 8;                       // 16-byte chunks per row
  constexpr int kTileBytes = kBN * kRowBytes;
  constexpr int kLoadsPerWave = kTileBytes / 1024 / kWaves;  // 1 KiB wave-loads per wave
  constexpr int kRowsPerLoad = 1024 / kRowBytes;
  constexpr int kBlocksPerLoad = kRowsPerLoad > BS ? kRowsPerLoad / BS : 1;
  // fp8 pools: raw tiles of kBN rows of D bytes, kRawLoads wave-loads each
  // for K and for V; wave w issues loads w, w + 4, ... of the 2 kRawLoads
  // (K first), so every wave issues kRawLoadsPerWave per tile.
  constexpr int kRawTileBytes = kBN * D;
  constexpr int kRawLoads = kRawTileBytes / 1024;
  constexpr int kRawLoadsPerWave = 2 * kRawLoads / kWaves;
  constexpr int kRawRowsPerLoad = 1024 / D;
  constexpr int kRawPieces = D / 16;                   // 16-byte pieces per raw row
  constexpr int kRawBlocksPerLoad = kRawRowsPerLoad > BS ? kRawRowsPerLoad / BS : 1;
  static_assert(!kFp8 || (kRawLoadsPerWave >= 1 && kRawBlocksPerLoad <= 4), "fp8 tile geometry");
  // 16-byte staging registers per lane (the wave's part of one tile)
  constexpr int kStage = kFp8 ? kRawLoadsPerWave : 2 * kLoadsPerWave;
  constexpr int kKSteps = D / 16;
  constexpr int kDBlocks = D / 32;
  static_assert(kLoadsPerWave >= 1 && kBlocksPerLoad <= 2, "tile geometry");

  // Three-stage ring of K and V tiles (the one consumed, the next one, the
  // one being filled), each stage its own array so that every access names
  // a compile-time stage (the loop is unrolled by three).  Rows are 16-byte-chunk
  // XOR-swizzled so that fragment reads do not collide on banks: K row r
  // keeps chunk c at c ^ swz_k(r), V at c ^ swz_v(r).  A transposing V read
  // touches 4 chunks of each of 4 consecutive rows per half-wave: swz_v
  // moves those rows to distinct aligned groups of 4 chunks.
  __shared__ __attribute__((aligned(1024))) char lds_k0[kTileBytes], lds_k1[kTileBytes],
      lds_k2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v0[kTileBytes], lds_v1[kTileBytes],
      lds_v2[kTileBytes];
  auto stage_k = [&](auto st) -> char* {
    if constexpr (decltype(st)::value == 0) return lds_k0;
    else if constexpr (decltype(st)::value == 1) return lds_k1;
    else return lds_k2;
  };
  auto stage_v = [&](auto st) -> char* {
    if constexpr (decltype(st)::value == 0) return lds_v0;
    else if constexpr (decltype(st)::value == 1) return lds_v1;
    else return lds_v2;
  };
  auto swz_k = [](int r) { return (r * kChunks / 16) % kChunks; };
  auto swz_v = [](int r) { return 4 * ((r * kChunks / 16) % (kChunks / 4)); };

  // Work item: (pair = seq * H + head, query tile); pairs are dealt to XCDs
  // round robin by pair (pair % 8), so all query tiles of a pair share an
  // XCD and its L2.  In a batch of few (sequence, query tile) classes, each
  // XCD takes its items in order of decreasing work (heads in order within
  // a class), so the longest items start first and the short ones fill the
  // end of the launch:
  // - lpt_by_seq = 0 (the grid is resident at once): classes ranked by key
  //   tiles, ties by class index;
  // - lpt_by_seq = 1 (several rounds of workgroups): classes ranked by the
  //   largest key-tile count of their sequence, ties by class index, so a
  //   sequence's query tiles stay together (last tile first) and the query
  //   tiles of a head, which read the same K/V tiles, run side by side and
  //   share them in the L2.
  // Otherwise pairs go in order, the query tiles of a pair last tile first.
  const int lin = blockIdx.x;
  const int xcd = lin % kXcds;
  const int g = lin / kXcds;
  const int H = a.num_heads;
  int pair, qtile;
  if (!kPrefix && lpt_order(a.num_seqs, num_qtiles)) {
    int* cost = (int*)lds_v2;          // [n] key tiles of class u (0: no rows)
    int* order = cost + kMaxLptClasses;  // [n] class at sorted position r
    int* sel = order + kMaxLptClasses;   // this workgroup's class and index in it
    int* scost = sel + 2;                // [n] largest key-tile count of u's sequence
    static_assert((3 * kMaxLptClasses + 2) * sizeof(int) <= kTileBytes, "LPT scratch");
    const int n = a.num_seqs * num_qtiles;
    const int tid = threadIdx.x;
    if (tid == 0) sel[0] = -1;
    if (tid < n) {
      const int sq = tid / num_qtiles, qt = num_qtiles - 1 - tid % num_qtiles;
      const int q0 = a.query_start_loc[sq];
      const int Sq = a.query_start_loc[sq + 1] - q0;
      const int keys = a.context_lens[sq] - Sq + min((qt + 1) * kBM, Sq);
      cost[tid] = qt * kBM < Sq ? (keys + kBN - 1) / kBN : 0;
    }
    __syncthreads();
    if (lpt_by_seq) {  // (uniform)
      if (tid < n) {
        const int s0 = (tid / num_qtiles) * num_qtiles;
        int mc = 0;
        for (int j = 0; j < num_qtiles; ++j) mc = max(mc, cost[s0 + j]);
        scost[tid] = mc;
      }
      __syncthreads();
    }
    const int* key = lpt_by_seq ? scost : cost;
    if (tid < n) {
      const int c = key[tid];
      int r = 0;
      for (int u = 0; u < n; ++u) {
        const int cu = key[u];
        r += (cu > c) || (cu == c && u < tid);
      }
      order[r] = tid;
    }
    __syncthreads();
    if (tid < n) {
      // items on this XCD before sorted position tid, and at it
      int before = 0;
      for (int r = 0; r < tid; ++r) before += heads_on(xcd, order[r] / num_qtiles, H);
      const int here = heads_on(xcd, order[tid] / num_qtiles, H);
      if (g >= before && g < before + here) {
        sel[0] = order[tid];
        sel[1] = g - before;
      }
    }
    __syncthreads();
    const int c = sel[0];
    const int j = sel[1];
    __syncthreads();  // the scratch is LDS the ring uses later
    if (c < 0) return;
    const int sq = c / num_qtiles;
    qtile = num_qtiles - 1 - c % num_qtiles;
    pair = sq * H + first_head_on(xcd, sq, H) + kXcds * j;
  } else {
    pair = xcd + kXcds * (g / num_qtiles);
    if (pair >= num_pairs) return;
    qtile = num_qtiles - 1 - (g % num_qtiles);
  }
  const int head = pair % H;
  // kPrefix: pair = (chunk, head); keys [k0, L) of the prefix
  const int chunk = kPrefix ? pair / H : 0;
  const int seq = kPrefix ? 0 : pair / H;
  const int qs = kPrefix ? 0 : a.query_start_loc[seq];
  const int S = kPrefix ? a.num_seqs : a.query_start_loc[seq + 1] - qs;
  const int q_begin = qtile * kBM;
  if (q_begin >= S) return;
  const int k0 = kPrefix ? chunk * a.chunk_keys : 0;
  const int L = kPrefix ? min(k0 + a.chunk_keys, a.prefix_len) : a.context_lens[seq];
  const int ctx = kPrefix ? 0 : L - S;  // tokens before the chunk
  const int t0 = k0 / kBN;              // first tile (chunks are whole tiles)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < kWaves);  // (fp8 pools: which raw loads are V)
  const int half = lane >> 5;
  const int col = lane & 31;

  // This wave's query rows and the last key any of the workgroup's rows sees.
  const int wq0 = q_begin + wave * kQW;
  const int wg_last_row = min(q_begin + kBM, S) - 1;
  const int n_keys = kPrefix ? L : ctx + wg_last_row + 1;
  const int n_tiles = (n_keys + kBN - 1) / kBN - t0;
  const int wave_last_key = wq0 < S ? (kPrefix ? L - 1 : ctx + min(wq0 + kQW, S) - 1) : -1;

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

  // The block table is read-only during the kernel: read it through the
  // constant address space so that the uniform lookups below are scalar
  // loads (a vector load here would make the wait for it also wait for every
  // global load issued before it).
  // Entries are read as unsigned (block ids are never negative): widening
  // one to 64 bits is then free, and the compiler waits for a scalar load
  // only where the entry is used, not right after issuing it.
  typedef const __attribute__((address_space(4))) uint32_t const_u32;
  const_u32* table = (const_u32*)(a.block_tables + int64_t(seq) * a.max_blocks_per_seq);
  const int last_idx = int(unsigned(L - 1) / BS);
  const int64_t last_blk = table[last_idx];
  // fp8 pools: scales through the constant address space (scalar reads);
  // register v of a lane holds key 8 (v / 4) + 4 half + v % 4 of a tile, in
  // its block (key / BS) of the tile's kScaleBlocks.
  typedef const __attribute__((address_space(4))) float const_f32;
  const_f32* kscale_c = (const_f32*)a.k_scale;
  const_f32* vscale_c = (const_f32*)a.v_scale;
  constexpr int kScaleBlocks = BS >= kBN ? 1 : kBN / BS;
  auto scale_of = [&](const float (&sc)[kScaleBlocks], int v) {
    const int k0 = 8 * (v / 4) + (v % 4);
    return half ? sc[BS >= kBN ? 0 : (k0 + 4) / BS] : sc[BS >= kBN ? 0 : k0 / BS];
  };
  const int64_t head_off = int64_t(head) * BS * D;      // elements
  const int64_t blk_stride = int64_t(H) * BS * D;
  const uint16_t* kpool = (const uint16_t*)a.k_cache;
  const uint16_t* vpool = (const uint16_t*)a.v_cache;

  const int64_t tile_stride = int64_t(H) * BS * D * 2;   // bytes between blocks
  const char* kbase0 = (const char*)a.k_cache + int64_t(head) * BS * D * 2;
  const char* vbase0 = (const char*)a.v_cache + int64_t(head) * BS * D * 2;

  // 16-bit pools: wave-load li = wave * kLoadsPerWave + i of a tile covers
  // rows li * kRowsPerLoad + lane / kChunks; the lane loads 16-byte chunk
  // lane % kChunks of its row (the same offset from the (block, head) base
  // in every tile) and stores it at its swizzled place in the stage.
  const int ld_pos = lane % kChunks;
  uint32_t ld_off[kLoadsPerWave], st_k[kLoadsPerWave], st_v[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int row = (wave * kLoadsPerWave + i) * kRowsPerLoad + lane / kChunks;
    ld_off[i] = uint32_t(((row % BS) * D + ld_pos * 8) * 2);
    st_k[i] = uint32_t(row * kRowBytes + (ld_pos ^ swz_k(row)) * 16);
    st_v[i] = uint32_t(row * kRowBytes + (ld_pos ^ swz_v(row)) * 16);
  }

  // fp8 pools: this wave's raw wave-loads (K or V, which wave-load of the
  // tile, the lane's row and 16-byte piece).
  bool raw_v[kRawLoadsPerWave];
  int raw_li[kRawLoadsPerWave], raw_row[kRawLoadsPerWave];
#pragma unroll
  for (int j = 0; j < kRawLoadsPerWave; ++j) {
    const int l = wave + kWaves * j;
    raw_v[j] = l >= kRawLoads;
    raw_li[j] = l % kRawLoads;
    raw_row[j] = raw_li[j] * kRawRowsPerLoad + lane / kRawPieces;
  }
  const int raw_piece = lane % kRawPieces;

  // The wave-loads of one wave cover kWaveRows consecutive rows of a tile.
  // When a block holds at least that many, they all fall in one block: the
  // wave reads one table entry per tile, and reads it an iteration ahead
  // (blk_hint), so that its latency hides behind the tile in between.
  constexpr int kWaveRows = kLoadsPerWave * kRowsPerLoad;
  constexpr bool kOneBlockPerWave = !kFp8 && kBlocksPerLoad == 1 && kWaveRows <= BS;
  auto wave_blk = [&](int t) -> uint32_t {
    return table[__builtin_amdgcn_readfirstlane(
        min(int(unsigned((t0 + t) * kBN + wave * kWaveRows) / BS), last_idx))];
  };

  // Loads of this wave's part of tile t into the staging registers.
  // blk_hint: wave_blk(t) where kOneBlockPerWave.
  u32x4_t stg[kStage];
  // fp8 pools: a tile's K and V scales, one pair per block, are vector
  // loads issued with its codes (in order with them, so no scalar read
  // waits inside the Q K^T chain), moved to scalar registers of the tile's
  // stage when the codes are stored.  (The prefix pass at head size 64
  // with 4-token blocks reads them at the tile instead: the staging
  // registers would cost it a wave per SIMD.)
  constexpr bool kScaleStaged = kFp8 && (kScaleBlocks <= 4 || D == 128 || !kPrefix);
  constexpr int kSc = 2 * kScaleBlocks;
  const __amdgpu_buffer_rsrc_t ksc_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.k_scale, 0, 0x7fffffff, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vsc_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.v_scale, 0, 0x7fffffff, kBufferFlags);
  uint32_t stg_sc[kSc];
  float sc0[kSc], sc1[kSc], sc2[kSc];
  auto stage_sc = [&](auto st) -> float (&)[kSc] {
    if constexpr (decltype(st)::value == 0) return sc0;
    else if constexpr (decltype(st)::value == 1) return sc1;
    else return sc2;
  };
  // The K and V scales of the kScaleBlocks blocks of the tile at key kb
  // into the staging registers.
  auto load_scales = [&](int kb) {
#pragma unroll
    for (int j = 0; j < kScaleBlocks; ++j) {
      const uint32_t blk =
          table[__builtin_amdgcn_readfirstlane(min(int(unsigned(kb) / BS) + j, last_idx))];
      const int32_t sc_off = int32_t((int64_t(blk) * H + head) * 4);
      stg_sc[2 * j] = __builtin_amdgcn_raw_buffer_load_b32(ksc_rsrc, 0, sc_off, 0);
      stg_sc[2 * j + 1] = __builtin_amdgcn_raw_buffer_load_b32(vsc_rsrc, 0, sc_off, 0);
    }
  };
  auto load_tile = [&](u32x4_t (&dst)[kStage], int t, uint32_t blk_hint) {
    const int kb = (t0 + t) * kBN;
    if constexpr (kFp8 && BS >= kBN) {
      // The tile lies in one block (tiles start at multiples of kBN, blocks
      // are multiples of it) and starts before L, so its block is the table
      // entry of kb, which holds L - 1 whenever the tile reaches past it:
      // a uniform base, and keys past the end re-read the last key (finite
      // data; those keys are masked).
      // (the min never clamps; it makes this the entry load_scales reads)
      const uint32_t blk =
          table[__builtin_amdgcn_readfirstlane(min(int(unsigned(kb) / BS), last_idx))];
      const int64_t base = int64_t(blk) * blk_stride + head_off;
      load_scales(kb);
#pragma unroll
      for (int j = 0; j < kRawLoadsPerWave; ++j) {
        const int keyc = min(kb + raw_row[j], L - 1);
        const uint32_t off = uint32_t(unsigned(keyc) % BS) * D + raw_piece * 16;
        dst[j] = *(const u32x4_t*)((const char*)(raw_v[j] ? a.v_cache : a.k_cache) + base + off);
      }
      return;
    }
    if constexpr (kFp8 && kRawBlocksPerLoad == 1) {
      // Each raw load lies in one block: the load's own block when its
      // first row is a key (that block then holds L - 1 if the rows reach
      // past it), else the last block.  A uniform base per load, and keys
      // past the end re-read the last key (finite data; those keys are
      // masked) through a clamped 32-bit lane offset.
      if constexpr (kScaleStaged) load_scales(kb);
#pragma unroll
      for (int j = 0; j < kRawLoadsPerWave; ++j) {
        const int row0 = raw_li[j] * kRawRowsPerLoad;
        const uint32_t blk =
            table[__builtin_amdgcn_readfirstlane(min(int(unsigned(kb + row0) / BS), last_idx))];
        const int keyc = min(kb + raw_row[j], L - 1);
        const uint32_t off = uint32_t(unsigned(keyc) % BS) * D + raw_piece * 16;
        const int64_t base = int64_t(blk) * blk_stride + head_off;
        dst[j] = *(const u32x4_t*)((const char*)(raw_v[j] ? a.v_cache : a.k_cache) + base + off);
      }
      return;
    }
    if constexpr (kFp8) {
      // The tile's scales (one pair per block), then per-lane addresses
      // over at most kRawBlocksPerLoad blocks (scalar table reads); keys
      // past the end re-read the last key (finite data; those keys are
      // masked).
      if constexpr (kScaleStaged) load_scales(kb);
#pragma unroll
      for (int j = 0; j < kRawLoadsPerWave; ++j) {
        const int row0 = raw_li[j] * kRawRowsPerLoad;
        const int b0 = __builtin_amdgcn_readfirstlane(int(unsigned(kb + row0) / BS));
        int64_t blks[kRawBlocksPerLoad];
#pragma unroll
        for (int b = 0; b < kRawBlocksPerLoad; ++b)
          blks[b] = table[__builtin_amdgcn_readfirstlane(min(b0 + b, last_idx))];
        const int key = kb + raw_row[j];
        const bool in = key < L;
        const int keyc = in ? key : L - 1;
        int64_t blk = last_blk;
        if (in) {
#pragma unroll
          for (int b = 0; b < kRawBlocksPerLoad; ++b)
            if (int(unsigned(key) / BS) == b0 + b) blk = blks[b];
        }
        const int64_t e =
            (blk * blk_stride + head_off + int64_t(unsigned(keyc) % BS) * D) + raw_piece * 16;
        dst[j] = *(const u32x4_t*)((const char*)(raw_v[j] ? a.v_cache : a.k_cache) + e);
      }
      return;
    }
    if (kBlocksPerLoad == 1 && kb + kBN <= L) {
      // Whole tile inside the sequence: one block per wave-load, uniform base.
      const int64_t in_blk = BS > kBN ? int64_t(kb % BS) * kRowBytes : 0;
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        const int li = wave * kLoadsPerWave + i;
        const int64_t blk =
            kOneBlockPerWave
                ? blk_hint
                : table[__builtin_amdgcn_readfirstlane(int(unsigned(kb + li * kRowsPerLoad) / BS))];
        dst[i] = *(const u32x4_t*)(kbase0 + blk * tile_stride + in_blk + ld_off[i]);
        dst[kLoadsPerWave + i] = *(const u32x4_t*)(vbase0 + blk * tile_stride + in_blk + ld_off[i]);
      }
      return;
    }
    // The tile reaches past the sequence end (or spans two blocks per
    // wave-load): per-lane addresses; keys past the end re-read the last key
    // (finite data; those keys are masked).
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int li = wave * kLoadsPerWave + i;
      const int row0 = li * kRowsPerLoad;
      const int b0 = __builtin_amdgcn_readfirstlane(int(unsigned(kb + row0) / BS));
      const int64_t blk_a = table[__builtin_amdgcn_readfirstlane(min(b0, last_idx))];
      const int64_t blk_b =
          kBlocksPerLoad > 1 ? table[__builtin_amdgcn_readfirstlane(min(b0 + 1, last_idx))] : blk_a;
      const int key = kb + row0 + lane / kChunks;
      const bool in = key < L;
      const int keyc = in ? key : L - 1;
      const int64_t blk = in ? (int(unsigned(key) / BS) == b0 ? blk_a : blk_b) : last_blk;
      const int64_t e =
          blk * blk_stride + head_off + int64_t(unsigned(keyc) % BS) * D + ld_pos * 8;
      dst[i] = *(const u32x4_t*)(kpool + e);
      dst[kLoadsPerWave + i] = *(const u32x4_t*)(vpool + e);
    }
  };

  // The staging registers (tile t+1) into stage st: bf16 V converted to
  // fp16 (RNE); fp8 codes, 16 per lane, to 16 bits (K: QT, V: fp16) as two
  // 16-byte chunks, 2 piece and 2 piece + 1, of the row.
  auto store_tile = [&](auto st, const u32x4_t (&src)[kStage]) {
    if constexpr (kFp8) {
#pragma unroll
      for (int j = 0; j < kRawLoadsPerWave; ++j) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // two codes per conversion, exact (scale 1): every E4M3 value is
          // a bf16 and an fp16 value
          if (QT == PA_BF16 && !raw_v[j]) {
            h[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[j][i], 1.0f, false));
            h[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[j][i], 1.0f, true));
          } else {
            h[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src[j][i], 1.0f, false));
            h[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src[j][i], 1.0f, true));
          }
        }
        const int row = raw_row[j];
        char* dst = (raw_v[j] ? stage_v(st) : stage_k(st)) + row * kRowBytes;
        const int sw = raw_v[j] ? swz_v(row) : swz_k(row);
        *(u32x4_t*)(dst + ((2 * raw_piece) ^ sw) * 16) = u32x4_t{h[0], h[1], h[2], h[3]};
        *(u32x4_t*)(dst + ((2 * raw_piece + 1) ^ sw) * 16) = u32x4_t{h[4], h[5], h[6], h[7]};
      }
      if constexpr (kScaleStaged) {
        float (&d)[kSc] = stage_sc(st);
#pragma unroll
        for (int j = 0; j < kSc; ++j)
          d[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(stg_sc[j]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        *(u32x4_t*)(stage_k(st) + st_k[i]) = src[i];
        u32x4_t v = src[kLoadsPerWave + i];
        if constexpr (KV == PA_BF16) v = bf16x8_to_f16x8(v);
        *(u32x4_t*)(stage_v(st) + st_v[i]) = v;
      }
    }
  };

  // Lane offsets of the transposing V reads: for k-step tt and half p of
  // the A operand's 8 keys, lane l reads dimensions d0 + 4 (j % 4) .. + 4 of
  // tile row 16 tt + 8 p + rl, with rl = 4 (l / 32) + j / 4, j = l % 16,
  // d0 = 32 db + 16 ((l / 16) % 2); it then holds keys 16 tt + 8 p + 4 (l / 32)
  // + 0..3 of dimension 32 db + l % 32 -- the order of P's registers.  The
  // row's swizzle depends on rl only, so each offset is a lane constant plus
  // a compile-time part.
  const int vt_rl = 4 * half + (lane % 16) / 4;
  const int vt_cl = 2 * ((lane / 16) % 2) + (lane % 4) / 2;   // chunk within the group of 4
  // K fragment reads: chunk (2 kk + half) ^ swz_k(col) of row col, i.e. the
  // lane's offset for kk = 0 XOR 32 kk (the chunk index's bit 0 is half).
  const uint32_t k_lane0 = uint32_t(col * kRowBytes + ((half ^ swz_k(col)) << 4));
  // Dimension block db adds 64 (db ^ vt_sq) bytes to the lane's offset;
  // the lane part below bit 6 is zero there, so the offset is vt_lane0 ^ 64 db.
  const int vt_sq = swz_v(vt_rl) / 4;
  const uint32_t vt_lane0 =
      uint32_t(vt_rl * kRowBytes + 16 * vt_cl + 8 * (lane % 2) + 64 * vt_sq);

  f32x16_t o[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[db][v] = 0.f;
  float m = kNoMax, l = 0.f;
  const int my_row = wq0 + col;           // query row of this lane's column
  const int my_lim = kPrefix ? L - 1 : ctx + my_row;   // last key it sees
  const int tile_lim = kPrefix ? L - 1 : ctx + wq0;    // last key every row of the wave sees

  // Prologue: tiles 0 and 1 into stages 0 and 1, tile 2 into the registers.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  if constexpr (!kFp8) {
    // tiles 0 and 1 in flight together (fp8 pools: one after the other, the
    // second set of registers would spill there)
    u32x4_t stg1[kStage];
    load_tile(stg, 0, kOneBlockPerWave ? wave_blk(0) : 0);
    if (n_tiles > 1) load_tile(stg1, 1, kOneBlockPerWave ? wave_blk(1) : 0);
    store_tile(S0{}, stg);
    if (n_tiles > 1) store_tile(S1{}, stg1);
  } else {
    load_tile(stg, 0, 0);
    store_tile(S0{}, stg);
    if (n_tiles > 1) {
      load_tile(stg, 1, 0);
      store_tile(S1{}, stg);
    }
  }
  if (n_tiles > 2) load_tile(stg, 2, kOneBlockPerWave ? wave_blk(2) : 0);
  // the table entry of the tile the next load is for
  uint32_t blk_next = kOneBlockPerWave ? wave_blk(min(3, n_tiles - 1)) : 0;
  wg_barrier();

  // One tile: consume tile t (stage st).  Once its Q K^T products are
  // issued, store tile t+2 from the registers into stage st+2 (nobody reads
  // it: its tile t-1 was consumed before the last barrier) and load tile t+3
  // into the registers; the barrier at the end publishes tile t+1's stage
  // (stored an iteration ago) and retires stage st.
  auto stage_next = [&](auto st, int t) {
    using Snn = std::integral_constant<int, (decltype(st)::value + 2) % 3>;
    if (t + 2 < n_tiles) {
      store_tile(Snn{}, stg);
      if (t + 3 < n_tiles) {
        load_tile(stg, t + 3, blk_next);
        if constexpr (kOneBlockPerWave) blk_next = wave_blk(min(t + 4, n_tiles - 1));
      }
    }
  };
  auto iter = [&](auto st, int t) {
    const int kb = (t0 + t) * kBN;
    const bool active = kb <= wave_last_key;
    uint32_t k_lane = k_lane0, vt_lane = vt_lane0;
    redefine(k_lane);
    redefine(vt_lane);
    const char* kl = stage_k(st);
    // chunk (2 kk + half) ^ swz_k(col) of row col: the lane's offset for
    // kk = 0, XOR 32 kk
    auto kfrag = [&](int kk) {
      return *(const uint4*)(kl + xor_here(k_lane, uint32_t(kk) << 5));
    };
    stage_next(st, t);
    if (active) {
      const uint4 kf0 = kfrag(0);
      const char* vl = stage_v(st);
      // fp8 pools: the K and V scales of the tile's blocks (staged with its
      // codes, else scalar reads issued before the MFMAs that wait for them).
      float sk[kScaleBlocks], sv[kScaleBlocks];
      if constexpr (kScaleStaged) {
#pragma unroll
        for (int j = 0; j < kScaleBlocks; ++j) {
          sk[j] = stage_sc(st)[2 * j];
          sv[j] = stage_sc(st)[2 * j + 1];
        }
      } else if constexpr (kFp8) {
#pragma unroll
        for (int j = 0; j < kScaleBlocks; ++j) {
          const int64_t blk =
              table[__builtin_amdgcn_readfirstlane(min(int(unsigned(kb) / BS) + j, last_idx))];
          sk[j] = kscale_c[blk * H + head];
          sv[j] = vscale_c[blk * H + head];
        }
      }
      // S^T = K Q^T : rows = keys of the tile, columns = this wave's queries.
      f32x16_t s;
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = 0.f;
      s = mfma_qk<QT>(kf0, qf[0], s);
#pragma unroll
      for (int kk = 1; kk < kKSteps; ++kk) s = mfma_qk<QT>(kfrag(kk), qf[kk], s);
      // K fragment reads two ahead of the MFMAs that use them
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int kk = 0; kk < kKSteps - 2; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      // Register v of this lane holds key 8*(v/4) + 4*half + v%4 of the tile.
      // Scores stay unscaled here; c = scale*log2(e) > 0 is folded into the
      // exponent below.
      // The scores are copied out of the accumulator once and never written
      // back (edits in place would make the compiler move the accumulator
      // between register files on every tile).
      const float c = a.scale_log2;
      float x[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) x[v] = kFp8 ? s[v] * scale_of(sk, v) : s[v];
      if (kb + kBN - 1 > tile_lim) {  // the tile crosses the causal diagonal (or the chunk end)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb + 8 * (v / 4) + 4 * half + (v % 4);
          x[v] = key <= my_lim ? x[v] : -INFINITY;
        }
      }
      float mx = x[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, x[v]);
      // (fp16 pools: the exchange through LDS; the VALU one needs two more
      // registers there and made the compiler spill inside the loop.)
      if constexpr (KV == PA_BF16) {
        const float2 mp = half_pair(mx);
        mx = fmaxf(mp.x, mp.y) * c;
      } else {
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * c;
      }
      // Rows whose maximum grew past the slack move their reference maximum.
      // The branch is taken for the whole wave (a vote), so the accumulators
      // are touched only on the rare tiles where some row needs it.
      const bool moves = mx > m + kRescaleSlack;
      if (__any(moves)) {
        const float m_new = moves ? mx : m;
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
        m = m_new;
      }
      float psum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        x[v] = __builtin_amdgcn_exp2f(fmaf(x[v], c, -m));
        if constexpr (kFp8) psum += x[v];
      }
      if constexpr (kFp8) l += psum;
      // P^T as B operands: k-step tt takes accumulator registers 8tt .. 8tt+7,
      // i.e. keys 16tt + 8*(e/4) + 4*half + e%4 for e = 0..7.
      uint4 pf[2];
      if constexpr (kFp8) {
        // the V scales go with the weights (the row sum above is unscaled)
#pragma unroll
        for (int v = 0; v < 16; ++v) x[v] *= scale_of(sv, v);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        pf[tt] = make_uint4(pack_f16(x[8 * tt + 0], x[8 * tt + 1]),
                            pack_f16(x[8 * tt + 2], x[8 * tt + 3]),
                            pack_f16(x[8 * tt + 4], x[8 * tt + 5]),
                            pack_f16(x[8 * tt + 6], x[8 * tt + 7]));
      if constexpr (!kFp8) {
        // 16-bit pools: the row sum of the fp16 weights the P V product
        // uses (two per v_dot2_f32_f16, float32 accumulation), so the
        // normaliser matches the rounded weights
        const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
        float ps = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pf[tt].x), one, ps, false);
          ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pf[tt].y), one, ps, false);
          ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pf[tt].z), one, ps, false);
          ps = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pf[tt].w), one, ps, false);
        }
        l += ps;
      }
      // O^T += V^T P^T : A = V^T from the V rows by transposing reads, in
      // the same key order as P; two dimension blocks' operands per wait.
      const uint32_t vbase =
          uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)vl));
      // Groups g = (tt, pair of dimension blocks) of four transposing
      // reads; group g + 1's reads are in flight while group g's MFMAs
      // issue (LDS operations complete in order: at most four outstanding
      // means group g has landed).
      constexpr int kGroups = 2 * (kDBlocks / 2);
      auto read_grp = [&](auto g_c, uint2 (&v)[4]) {
        constexpr int g = decltype(g_c)::value;
        constexpr int tt = g / (kDBlocks / 2);
        constexpr int db0 = 2 * (g % (kDBlocks / 2));
        v[0] = lds_read_tr16<(16 * tt) * kRowBytes>(vbase + xor_here(vt_lane, uint32_t(db0) << 6));
        v[1] = lds_read_tr16<(16 * tt + 8) * kRowBytes>(vbase + xor_here(vt_lane, uint32_t(db0) << 6));
        v[2] = lds_read_tr16<(16 * tt) * kRowBytes>(vbase + xor_here(vt_lane, uint32_t(db0 + 1) << 6));
        v[3] = lds_read_tr16<(16 * tt + 8) * kRowBytes>(vbase + xor_here(vt_lane, uint32_t(db0 + 1) << 6));
      };
      auto mfma_grp = [&](auto g_c, const uint2 (&v)[4]) {
        constexpr int g = decltype(g_c)::value;
        constexpr int tt = g / (kDBlocks / 2);
        constexpr int db0 = 2 * (g % (kDBlocks / 2));
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint4 va = make_uint4(v[2 * k].x, v[2 * k].y, v[2 * k + 1].x, v[2 * k + 1].y);
          o[db0 + k] = mfma_pv(va, pf[tt], o[db0 + k]);
        }
      };
      auto wait4 = [](uint2 (&v)[4]) {
        asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
      };
      using G0 = std::integral_constant<int, 0>;
      using G1 = std::integral_constant<int, 1>;
      uint2 va[4], vb[4];
      read_grp(G0{}, va);
      read_grp(G1{}, vb);
      wait4(va);
      mfma_grp(G0{}, va);
      if constexpr (kGroups == 4) {
        using G2 = std::integral_constant<int, 2>;
        using G3 = std::integral_constant<int, 3>;
        read_grp(G2{}, va);
        wait4(vb);
        mfma_grp(G1{}, vb);
        read_grp(G3{}, vb);
        wait4(va);
        mfma_grp(G2{}, va);
        lds_wait_tr(vb);
        mfma_grp(G3{}, vb);
      } else {
        lds_wait_tr(vb);
        mfma_grp(G1{}, vb);
      }
    }
    wg_barrier();
  };
  iter(S0{}, 0);
  for (int t = 1; t < n_tiles;) {
    iter(S1{}, t);
    if (++t >= n_tiles) break;
    iter(S2{}, t);
    if (++t >= n_tiles) break;
    iter(S0{}, t);
    ++t;
  }

  // Normalise and store: lane holds query my_row, dims 8*(v/4) + 4*half + v%4.
  const float2 lp = half_pair(l);
  l = lp.x + lp.y;
  if constexpr (kPrefix) {
    // (max, sum, unnormalised output) of this chunk for sequence my_row
    if (my_row < S && wq0 < S) {
      const int64_t pidx = (int64_t(my_row) * H + head) * a.max_parts + chunk;
      if (half == 0) {
        a.ws_ml[2 * pidx] = m;
        a.ws_ml[2 * pidx + 1] = l;
      }
      float* acc = a.ws_acc + pidx * D;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db * 32 + 8 * (v / 4) + 4 * half + (v % 4)] = o[db][v];
    }
    return;
  }
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

// Workgroups of prefill_kernel<KV, QT, D, BS> resident on the GPU at once
// (per CU by its registers and LDS, times the CUs), looked up once per
// instantiation on the first launch's device; 0 if the runtime cannot say
// (its error is then cleared, so that the launch's own status is reported).
template <int KV, int QT, int D, int BS>
int64_t resident_workgroups() {
  static const int64_t n = [] {
    int dev = 0, per_cu = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prefill_kernel<KV, QT, D, BS>,
                                                     kWaves * 64, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return int64_t(0);
    }
    return int64_t(per_cu) * cus;
  }();
  return n;
}

template <int KV, int QT, int D, int BS>
hipError_t launch_t(const PrefillArgs& a, int max_query_len, hipStream_t stream) {
  const int num_qtiles = (max_query_len + kBM - 1) / kBM;
  const int num_pairs = a.num_seqs * a.num_heads;
  const int padded_pairs = (num_pairs + kXcds - 1) / kXcds * kXcds;
  // longest-first order: at most ceil(H / 8) items of each class per XCD
  const bool lpt = lpt_order(a.num_seqs, num_qtiles);
  const int64_t blocks =
      lpt ? int64_t(kXcds) * a.num_seqs * num_qtiles * ((a.num_heads + kXcds - 1) / kXcds)
          : int64_t(padded_pairs) * num_qtiles;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  // Rank by sequence when the workgroups come in several rounds (a class
  // ranking would then start a head's query tiles rounds apart and read its
  // K/V several times); a grid resident at once keeps the class ranking,
  // whose placement balances the work per CU.
  const int by_seq = lpt && blocks > resident_workgroups<KV, QT, D, BS>() ? 1 : 0;
  hipLaunchKernelGGL((prefill_kernel<KV, QT, D, BS>), dim3(unsigned(blocks)), dim3(kWaves * 64), 0,
                     stream, a, num_qtiles, num_pairs, by_seq);
  return hipGetLastError();
}

template <int KV, int QT, int D>
hipError_t launch_bs(const PrefillArgs& a, int bs, int mq, hipStream_t stream) {
  switch (bs) {
    case 4: return launch_t<KV, QT, D, 4>(a, mq, stream);
    case 8: return launch_t<KV, QT, D, 8>(a, mq, stream);
    case 16: return launch_t<KV, QT, D, 16>(a, mq, stream);
    case 32: return launch_t<KV, QT, D, 32>(a, mq, stream);
    case 64: return launch_t<KV, QT, D, 64>(a, mq, stream);
  }
  return hipErrorInvalidValue;
}

template <int KV, int QT, int D, int BS>
hipError_t launch_prefix_t(const PrefillArgs& a, hipStream_t stream) {
  const int num_qtiles = (a.num_seqs + kBM - 1) / kBM;
  const int chunks = (a.prefix_len + a.chunk_keys - 1) / a.chunk_keys;
  const int num_pairs = chunks * a.num_heads;
  const int padded_pairs = (num_pairs + kXcds - 1) / kXcds * kXcds;
  const int64_t blocks = int64_t(padded_pairs) * num_qtiles;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<KV, QT, D, BS, true>), dim3(unsigned(blocks)),
                     dim3(kWaves * 64), 0, stream, a, num_qtiles, num_pairs, 0);
  return hipGetLastError();
}

template <int KV, int QT, int D>
hipError_t launch_prefix_bs(const PrefillArgs& a, int bs, hipStream_t stream) {
  switch (bs) {
    case 4: return launch_prefix_t<KV, QT, D, 4>(a, stream);
    case 8: return launch_prefix_t<KV, QT, D, 8>(a, stream);
    case 16: return launch_prefix_t<KV, QT, D, 16>(a, stream);
    case 32: return launch_prefix_t<KV, QT, D, 32>(a, stream);
    case 64: return launch_prefix_t<KV, QT, D, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <int KV, int QT>
hipError_t launch_prefix_d(const PrefillArgs& a, int d, int bs, hipStream_t stream) {
  if (d == 64) return launch_prefix_bs<KV, QT, 64>(a, bs, stream);
  if (d == 128) return launch_prefix_bs<KV, QT, 128>(a, bs, stream);
  return hipErrorInvalidValue;
}

template <int KV, int QT>
hipError_t launch_d(const PrefillArgs& a, int d, int bs, int mq, hipStream_t stream) {
  if (d == 64) return launch_bs<KV, QT, 64>(a, bs, mq, stream);
  if (d == 128) return launch_bs<KV, QT, 128>(a, bs, mq, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, int q_dtype, int head_dim,
                          int block_size, int max_query_len, hipStream_t stream) {
  const int mq = max_query_len;
  if (kv_dtype == PA_BF16) return launch_d<PA_BF16, PA_BF16>(a, head_dim, block_size, mq, stream);
  if (kv_dtype == PA_F16) return launch_d<PA_F16, PA_F16>(a, head_dim, block_size, mq, stream);
  if (kv_dtype == PA_FP8_E4M3 && q_dtype == PA_BF16)
    return launch_d<PA_FP8_E4M3, PA_BF16>(a, head_dim, block_size, mq, stream);
  if (kv_dtype == PA_FP8_E4M3 && q_dtype == PA_F16)
    return launch_d<PA_FP8_E4M3, PA_F16>(a, head_dim, block_size, mq, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefix_partials(const PrefillArgs& a, int kv_dtype, int q_dtype, int head_dim,
                                  int block_size, hipStream_t stream) {
  if (kv_dtype == PA_BF16) return launch_prefix_d<PA_BF16, PA_BF16>(a, head_dim, block_size, stream);
  if (kv_dtype == PA_F16) return launch_prefix_d<PA_F16, PA_F16>(a, head_dim, block_size, stream);
  if (kv_dtype == PA_FP8_E4M3 && q_dtype == PA_BF16)
    return launch_prefix_d<PA_FP8_E4M3, PA_BF16>(a, head_dim, block_size, stream);
  if (kv_dtype == PA_FP8_E4M3 && q_dtype == PA_F16)
    return launch_prefix_d<PA_FP8_E4M3, PA_F16>(a, head_dim, block_size, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
