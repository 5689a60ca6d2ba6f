// Paged single-query decode attention for gfx950 (CDNA4).  Included by
// decode_<dtype>.hip, one translation unit per storage type so the
// instantiations compile in parallel.
//
// What is computed ([P2] "PagedAttention：操作系统级 KV 缓存虚拟内存管理"):
//   §1.1   out = softmax(q·Kᵀ·scale)·V, one query row per head;
//   §3.2.2 step 4, §4.1: visit every logical block through the block table and
//          gather its K/V from a scattered physical block;
//   §4.1   reduce the softmax progressively (running max and sum, rescaled as
//          new tokens arrive), FlashAttention style;
//   §4.2   each block is contiguous, so it is read with wide vector loads.
//
// Mapping onto gfx950:
//   * The G = q_heads/kv_heads query rows of one kv-head are processed
//     together and stay in registers, so K and V are read from HBM once per
//     kv-head.
//   * Vector path (fp32, or G < 4, or blocks under 16 tokens): a token row
//     (head_dim elements) is spread over LPT lanes with 16 bytes per lane, so
//     one wave-wide global_load_dwordx4 moves 1 KiB: TPL = 64/LPT consecutive
//     tokens of one contiguous (block, kv-head) tile.  Each LPT-lane group
//     keeps its own running max/sum/output for the tokens it loads; scores
//     are reduced inside the group with DPP row rotations fused into v_add
//     (v_dot2 for fp16/bf16 products); groups and waves are merged once per
//     piece of work at the end.
//   * Matrix-core path (16-bit K/V, G ≥ 4, blocks of ≥ 16 tokens): 16-token
//     tiles go through MFMA, S = K·Qᵀ and Oᵀ += Vᵀ·Pᵀ (attend_range_mfma).
//   * Loads of the next chunk are issued before the current chunk is consumed
//     (two register buffers).
//   * Softmax runs in base 2: scores carry scale·log2(e) and v_exp_f32 does 2^x.
//
// Four ways of dealing out the work (all exact up to fp32 rounding order):
//   * Whole sequences: one workgroup per (sequence, kv-head), started in
//     batch order; the automatic choice when the batch has at least as many
//     units as the device holds workgroups at once.
//   * Uniform (the automatic choice for smaller batches): one fully resident
//     grid; every workgroup derives from the lengths the shortest partition
//     length whose partitions of all units fit the grid, numbers the
//     partitions densely and runs one; decode_reduce_kernel merges units of
//     more than one partition.
//   * Balanced (on request): the (sequence,
//     kv-head) units are laid end to end on one axis of CT-token chunks and
//     every workgroup of a single, fully resident grid takes an equal slice
//     of that axis.  Units cut by a slice boundary produce partial (max, sum,
//     output) records that the last arriving piece merges, through a
//     fan-in-16 tree for long units, so no second kernel runs and every CU
//     finishes at the same time whatever the length mix.
//   * Fixed partitions (an explicit partition length): one workgroup per
//     (sequence, kv-head, partition of P tokens) and a second kernel,
//     decode_reduce_kernel, merges the partitions of longer sequences.
//     Partitions of at most 512 tokens that hold whole chunks are taken one
//     per wave, NW consecutive ones to a workgroup, which merges them in LDS
//     before it writes one record (wave_tokens).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <type_traits>

#include "launch.h"

namespace pa {
namespace dec {

constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so 2^(m - m') never sees inf - inf
constexpr int kWaves = kDecodeWaves;
constexpr int kThreads = kWaves * 64;
constexpr int kFanIn = 16;      // records merged per node of the balanced kernel's merge tree
constexpr int kMaxLevels = 3;   // kFanIn^3 = 4096 ≥ pieces of any unit (≤ grid + 1)
static_assert(kMaxBalancedGrid + 1 <= kFanIn * kFanIn * kFanIn, "merge tree too shallow for the largest grid");
constexpr int kSeqsPerThread = 8;

template <int DT>
struct Elem;
template <>
struct Elem<kF32> {
  static constexpr int bytes = 4;
};
template <>
struct Elem<kF16> {
  static constexpr int bytes = 2;
};
template <>
struct Elem<kBF16> {
  static constexpr int bytes = 2;
};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

// Dot product of the 16-byte slices q and k (4 fp32 or 8 fp16/bf16), in fp32.
template <int DT>
__device__ __forceinline__ float dot16(const uint4& q, const uint4& k) {
  if constexpr (DT == kF32) {
    float acc = __uint_as_float(q.x) * __uint_as_float(k.x);
    acc = __builtin_fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = __builtin_fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = __builtin_fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    return acc;
  } else if constexpr (DT == kF16) {
    float acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.x), __builtin_bit_cast(half2_t, k.x), 0.f, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.y), __builtin_bit_cast(half2_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.z), __builtin_bit_cast(half2_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.w), __builtin_bit_cast(half2_t, k.w), acc, false);
    return acc;
  } else {
    float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.x), __builtin_bit_cast(bf162_t, k.x), 0.f, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.y), __builtin_bit_cast(bf162_t, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.z), __builtin_bit_cast(bf162_t, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.w), __builtin_bit_cast(bf162_t, k.w), acc, false);
    return acc;
  }
}

// Widen the elements of a 16-byte slice to fp32 (exact for every storage type).
template <int DT>
__device__ __forceinline__ void unpack(const uint4& u, float* f) {
  if constexpr (DT == kF32) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  } else if constexpr (DT == kF16) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t h = __builtin_bit_cast(half2_t, w[i]);
      f[2 * i] = static_cast<float>(h.x);
      f[2 * i + 1] = static_cast<float>(h.y);
    }
  } else {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over each aligned group of LPT lanes; every lane of the group gets it.
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (LPT == 8) {
    v += dpp<0x141>(v);  // row_half_mirror: lane i ↔ 7 - i within 8
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  } else if constexpr (LPT == 16) {
    v += dpp<0x128>(v);  // row_ror:8
    v += dpp<0x124>(v);  // row_ror:4
    v += dpp<0x122>(v);  // row_ror:2
    v += dpp<0x121>(v);  // row_ror:1
  } else {
    static_assert(LPT == 32, "lane groups of 8, 16 or 32");
    v = group_sum<16>(v);
    v += __shfl_xor(v, 16, 64);
  }
  return v;
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float qnan() { return __uint_as_float(0x7fc00000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ void store_out(void* out, int32_t out_dtype, int64_t idx, float x) {
  if (out_dtype == kF32) {
    static_cast<float*>(out)[idx] = x;
  } else if (out_dtype == kF16) {
    static_cast<_Float16*>(out)[idx] = static_cast<_Float16>(x);
  } else {
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(x);
  }
}

template <int DT, int D>
struct Shape {
  static constexpr int EB = Elem<DT>::bytes;
  static constexpr int ELEMS = 16 / EB;      // elements per lane per 16-byte load
  static constexpr int LPT = D / ELEMS;      // lanes per token row
  static constexpr int TPL = 64 / LPT;       // tokens per wave-wide load
  static constexpr int ROW = D * EB;         // bytes per token row
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "unsupported head_dim / dtype pair");
};

// A chunk is NLC wave-wide loads per tensor.  Blocks of ≥ TPL tokens: four
// loads (TPL-token groups never straddle a block, as both are powers of two).
// Smaller blocks: one load whose lane groups find their own blocks.
template <int DT, int D, int BS>
struct Chunk {
  static constexpr bool kSmallBlocks = BS < Shape<DT, D>::TPL;
  static constexpr int NLC = kSmallBlocks ? 1 : 4;
  static constexpr int CT = NLC * Shape<DT, D>::TPL;   // tokens per chunk
};

// LDS of one workgroup: the block ids of the range being read, staged once
// per batch (kTableBatch of them, a multiple of every CT / BS), and the
// buffers through which the NW waves merge their results.

// The matrix-core path: 16-bit K/V, blocks of at least 16 tokens (one 16-token
// MFMA tile never straddles a block) and at least 4 query rows per kv-head
// (below that the contraction is too thin to beat v_dot2).
template <int DT, int BS, int G>
constexpr bool kUseMfma = DT != kF32 && BS >= 16 && G >= 4;

// Waves per SIMD the decode kernels are compiled for, where that costs no
// spills: four (≤ 128 VGPRs) for the vector loop with one or two query rows
// (the balanced kernel, whose merge code also needs registers, with one);
// three (≤ 168) for the matrix-core loop of the partition kernel, whose MFMA
// accumulators then stay in VGPRs; otherwise what the register file allows.
template <int DT, int BS, int G, bool BALANCED>
constexpr int kMinWavesPerEU = kUseMfma<DT, BS, G> ? (BALANCED ? 1 : 3) : (G <= (BALANCED ? 1 : 2) ? 4 : 1);
// Kernels that keep more state live around the loop (the append kernels'
// new-token row, the uniform kernel's task): with two query rows the vector
// loop then spills at 4 waves, so it is compiled for 3.
template <int DT, int BS, int G, bool EXTRA>
constexpr int kMinWavesExtra = (EXTRA && !kUseMfma<DT, BS, G> && G == 2) ? 3 : kMinWavesPerEU<DT, BS, G, false>;

template <int NW, int G, int D, bool MFMA>
struct WaveMerge {
  // matrix-core path: each wave's K and V tiles, 16 tokens × D, rows
  // 16-byte aligned so each lane stores its 16-byte piece of a token row with
  // one write.  The row lengths were chosen by counting SQ_LDS_BANK_CONFLICT
  // on gfx950 (70B-layer GQA batch, per decode call): kt of D + 16 and vt of
  // D + 8 elements leave no conflicts in the row writes, the A-layout
  // read-back of K or the transposed read of V.  Rows of D + 4 elements
  // (8-byte aligned, two 8-byte writes per piece) cost 5.4 M conflict cycles
  // in each tile's writes; kt of D + 8, D + 24 … D + 40 cost 2.7 M in its
  // read-back, D + 64 8.1 M.
  struct Tiles {
    alignas(16) uint16_t vt[MFMA ? NW : 1][16][MFMA ? D + 8 : 1];
    alignas(16) uint16_t kt[MFMA ? NW : 1][16][MFMA ? D + 16 : 1];
  };
  union {             // the tiles live during the token loop, o after it
    float o[NW][G][D];  // matrix-core path: 4-float groups XOR-swizzled by row (wave_out)
    Tiles t;
  };
  float m[NW][G];
  float l[NW][G];
  int bad[NW];
  int32_t tbl[kTableBatch];   // physical block ids, -1 for an id outside the pool
  uint4 newrow[2][D / 4];     // pa_decode_append: the new token's K and V rows (≤ 4-byte elements)
};

// A 16-byte K/V load.  STREAM selects the non-temporal (streaming) cache
// policy, for tiles that no other workgroup of the call reads: it keeps them
// from displacing other lines and measured faster on the vector path.  Tiles
// shared by several sequences of the batch take the default policy, so the
// siblings that read them next find them in L2.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool STREAM>
__device__ __forceinline__ uint4 load_kv(const char* p) {
  if constexpr (STREAM) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core inner loop (16-bit K/V, G ≥ 4 query rows per kv-head).
//
// Per wave and 16-token chunk:
//   S  = K·Qᵀ        16 tokens × 16 rows (rows ≥ G are zero), D/32 MFMA
//                    16x16x32 steps; lane l loads token l%16, dims
//                    [32i + 8(l/16), +8) of the K tile, which is exactly the
//                    A operand, and holds S[tokens 4(l/16)..+3][row l%16].
//   softmax per row  the four lanes of a row (l, l±16, l±32) share the max;
//                    each keeps a partial sum.
//   Oᵀ += Vᵀ·Pᵀ      D/16 MFMA 16x16x16 tiles; Pᵀ is the lane's own four
//                    probabilities (the B operand layout), split into a
//                    16-bit head and a 16-bit remainder so the product keeps
//                    ~16 bits of each weight; Vᵀ is read transposed from the
//                    wave's V tile in LDS.  Lane l then owns
//                    O[row l%16][dims 16b + 4(l/16)..+3], so the per-row
//                    rescale by 2^(m_old − m_new) is lane-local.
//   Loads            K and V are loaded in whole token rows (1 KiB
//                    contiguous per wave instruction, so they may stream) and
//                    pass through the wave's LDS tiles: K is read back in the
//                    A layout (lane l: token l%16, dims 32i + 8(l/16)..+7),
//                    V transposed.  Loading K straight into the A layout
//                    would split every 128-byte line over two instructions.
// ---------------------------------------------------------------------------
// Column of output element (row, col) in a wave's merge buffer of the
// matrix-core path: its 4-float groups are XOR-swizzled by row, so the
// lanes of one row group (4 consecutive floats each, rows 8 apart in banks
// otherwise) write distinct banks; readers take consecutive columns of one
// row, which the swizzle keeps distinct too.
__device__ __forceinline__ int wave_out(int row, int col) { return col ^ (4 * (row & 7)); }

// The chunks of a table batch (tokens [tb, te), chunks of CT tokens from tb)
// that this wave takes: [first, limit).  Each wave takes one contiguous run of
// the workgroup's range [t_begin, t_end): wave w the tokens [t_begin +
// w·wt, +wt), where wt is wave_tokens when given (> 0: one caller partition
// per wave) or else the range split in NW runs, rounded up to whole chunks (so
// the runs meet on chunk bounds).
struct ChunkDeal {
  int32_t first, limit;
};
template <int CT, int NW>
__device__ __forceinline__ ChunkDeal deal_chunks(int32_t wave, int32_t wave_tokens, int32_t t_begin, int32_t t_end,
                                                 int32_t tb, int32_t te) {
  const int32_t wt = wave_tokens > 0 ? wave_tokens : ((t_end - t_begin + NW * CT - 1) / (NW * CT)) * CT;
  const int32_t lo = max(t_begin + wave * wt, tb);
  const int32_t hi = min(t_begin + (wave + 1) * wt, te);
  if (lo >= hi) return {0, 0};
  return {(lo - tb) / CT, (hi - tb + CT - 1) / CT};
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4_t mfma_k32(const uint4& a, const uint4& b, f32x4_t c) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                  0, 0);
  }
}

template <int DT>
__device__ __forceinline__ f32x4_t mfma_k16(const uint2& a, const uint2& b, f32x4_t c) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a), __builtin_bit_cast(i16x4_t, b), c,
                                                     0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c, 0,
                                                 0, 0);
  }
}

// x rounded to the 16-bit type (nearest-even) and back, as bits and value.
template <int DT>
__device__ __forceinline__ uint16_t round16(float x, float* back) {
  if constexpr (DT == kBF16) {
    const uint16_t h = f32_to_bf16_rne(x);
    *back = __uint_as_float(static_cast<uint32_t>(h) << 16);
    return h;
  } else {
    const _Float16 h = static_cast<_Float16>(x);
    *back = static_cast<float>(h);
    return __builtin_bit_cast(uint16_t, h);
  }
}

// The new token of pa_decode_append, as the workgroup that attends over it
// sees it: t is its index in the sequence (-1: none here), k and v the starts
// of its K and V rows for this kv-head in k_new / v_new.  The workgroup copies
// the two rows into LDS with its first block ids and uses them in place of
// what its chunk loads fetched from the slot, which it writes only after its
// token loop (the same bytes, so the result is the same).
struct NewToken {
  const char* k = nullptr;
  const char* v = nullptr;
  int32_t t = -1;
};

// Copy the new token's K and V rows (ROW bytes each) into LDS; called by every
// thread of the workgroup before the barrier that publishes the block ids, so
// the loads overlap the table loads.
template <int ROW, int N>
__device__ __forceinline__ void stage_new_token(const NewToken& nt, uint4 (&newrow)[2][N]) {
  constexpr int L16 = ROW / 16;
  static_assert(L16 <= N, "row buffer too small");
  if (nt.t >= 0 && threadIdx.x < 2 * L16) {
    const bool is_v = threadIdx.x >= L16;
    const int piece = threadIdx.x % L16;
    newrow[is_v ? 1 : 0][piece] = *reinterpret_cast<const uint4*>((is_v ? nt.v : nt.k) + piece * 16);
  }
}

// Whether sequence s shares its first physical block with a batch neighbour
// (s − 1 or s + 1), i.e. reads a prefix that a sibling scheduled next to it
// also reads.  Rows of empty sequences may hold anything; a false match only
// selects the default cache policy.
__device__ __forceinline__ bool shares_first_block(const int32_t* __restrict__ block_tables, int32_t table_stride,
                                                   int32_t s, int32_t num_seqs) {
  const int32_t first = block_tables[static_cast<int64_t>(s) * table_stride];
  bool shared = false;
  if (s > 0) shared = shared || block_tables[static_cast<int64_t>(s - 1) * table_stride] == first;
  if (s + 1 < num_seqs) shared = shared || block_tables[static_cast<int64_t>(s + 1) * table_stride] == first;
  return shared;
}

// R query rows (R ≤ 16) against kv-head g's tiles over tokens [t_begin,
// t_end).  q_lane: the start of this lane's query row (row lane % 16), or
// nullptr for a row past R or unused (it contributes zeros); q_dummy: any
// valid, cache-resident address (read by the loads of chunks past the end).
template <int DT, int D, int BS, int R, int NW, bool STREAM, bool NEWTOK, typename Emit>
__device__ __forceinline__ void attend_range_mfma(const char* __restrict__ k_pool, const char* __restrict__ v_pool,
                                                  const char* q_lane, const char* __restrict__ q_dummy,
                                                  const int32_t* __restrict__ table, int32_t g, int32_t kv_heads,
                                                  int32_t num_blocks, int32_t t_begin, int32_t t_end,
                                                  float scale_log2, NewToken nt, int32_t wave_tokens,
                                                  WaveMerge<NW, R, D, true>& sh, Emit&& emit) {
  constexpr int EB = 2;
  constexpr int ROW = D * EB;          // bytes per token row
  constexpr int CT = 16;               // tokens per chunk (the MFMA M dimension)
  constexpr int NKL = D / 32;          // 16-byte loads per lane per tensor per chunk
  constexpr int NB = D / 16;           // output tiles of 16 dims
  constexpr int64_t TILE = static_cast<int64_t>(BS) * ROW;
  constexpr int LPR = ROW / 16;        // lanes per V row in a contiguous load
  constexpr int RPI = 64 / LPR;        // V rows per load instruction
  static_assert(BS % CT == 0 && R <= 16, "matrix-core path needs 16-token tiles and ≤ 16 rows");
  static_assert(RPI * NKL == CT, "NKL contiguous loads cover the 16-row V tile");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tl = lane & 15;   // token (K/V loads, S/P columns) or row (Q, O) of this lane
  const int qd = lane >> 4;   // quarter: dim slice of the loads, token group of S/P

  // Qᵀ operand: row tl (zero where q_lane is null), dims [32i + 8qd, +8)
  const char* q_src = (q_lane ? q_lane : q_dummy) + qd * 16;
  // dead loads read here: the same 16 bytes for every lane with the new-token
  // path (one pointer fewer), this lane's slice of q otherwise (either fits
  // the 3-wave register budget only that way)
  const char* q_dead = NEWTOK ? q_dummy : q_src;
  uint4 qop[NKL];
#pragma unroll
  for (int i = 0; i < NKL; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(q_src + i * 64);
    qop[i] = q_lane ? v : make_uint4(0u, 0u, 0u, 0u);
  }
  float m = kNegBig, l = 0.f;
  f32x4_t ob[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) ob[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool bad_block = false;
  const int32_t vrow = lane / LPR;                                  // K/V: row within a load
  const int32_t v_off = vrow * ROW + (lane % LPR) * 16;

  const int32_t blk_first = t_begin / BS;
  const int32_t blk_last = (t_end - 1) / BS;
  for (int32_t bb = blk_first; bb <= blk_last; bb += kTableBatch) {
    const int32_t nb = min(kTableBatch, blk_last - bb + 1);
    __syncthreads();   // the previous batch's ids are no longer read
    for (int i = threadIdx.x; i < nb; i += NW * 64) {
      const int32_t phys = table[bb + i];
      sh.tbl[i] = static_cast<uint32_t>(phys) < static_cast<uint32_t>(num_blocks) ? phys : -1;
    }
    if constexpr (NEWTOK) {
      if (bb == blk_first) stage_new_token<ROW>(nt, sh.newrow);
    }
    __syncthreads();
    const int32_t tb = max(t_begin, bb * BS);
    const int32_t te = min(t_end, (bb + nb) * BS);

    // Issue chunk c's K and V loads (live = false: read q_dead, valid and
    // cache-resident).  Rows past te inside the block may be read; they are
    // masked before use.
    auto load_chunk = [&](int32_t c, bool live, uint4 (&kb)[NKL], uint4 (&vb)[NKL]) {
      const int32_t tok0 = tb + (live ? c : 0) * CT;
      int32_t phys = sh.tbl[tok0 / BS - bb];
      if (phys < 0) {
        bad_block = true;
        phys = 0;
      }
      const int64_t tile = (static_cast<int64_t>(phys) * kv_heads + g) * TILE + (tok0 % BS) * ROW;
#pragma unroll
      for (int i = 0; i < NKL; ++i) {
        kb[i] = load_kv<STREAM>(live ? k_pool + tile + v_off + i * RPI * ROW : q_dead);
        vb[i] = load_kv<STREAM>(live ? v_pool + tile + v_off + i * RPI * ROW : q_dead);
      }
    };

    auto consume_chunk = [&](int32_t c, uint4 (&kb)[NKL], uint4 (&vb)[NKL]) {
      const int32_t tok0 = tb + c * CT;
      if constexpr (NEWTOK) {
        // the new token's row (its slot is written after the loop) from LDS
        if (nt.t >= tok0 && nt.t < tok0 + CT) {   // wave-uniform
#pragma unroll
          for (int i = 0; i < NKL; ++i) {
            if (tok0 + i * RPI + vrow == nt.t) {
              kb[i] = sh.newrow[0][lane % LPR];
              vb[i] = sh.newrow[1][lane % LPR];
            }
          }
        }
      }
      // K rows into the wave's K tile, then read back in the A layout
#pragma unroll
      for (int i = 0; i < NKL; ++i) {
        const int row = i * RPI + vrow;
        *reinterpret_cast<uint4*>(&sh.t.kt[wave][row][(lane % LPR) * 8]) = kb[i];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      uint4 ka_op[NKL];
#pragma unroll
      for (int i = 0; i < NKL; ++i) {
        ka_op[i] = *reinterpret_cast<const uint4*>(&sh.t.kt[wave][tl][32 * i + 8 * qd]);
      }
      // S = K·Qᵀ
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NKL; ++i) sacc = mfma_k32<DT>(ka_op[i], qop[i], sacc);
      // this lane's V pieces into the wave's tile; padding rows become zero
      // (they may hold NaN, and 0·NaN would poison the product)
#pragma unroll
      for (int i = 0; i < NKL; ++i) {
        const int row = i * RPI + vrow;
        const uint4 v = tok0 + row < te ? vb[i] : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(&sh.t.vt[wave][row][(lane % LPR) * 8]) = v;
      }
      // online softmax of row tl over tokens 4qd..4qd+3
      float sc[4];
      bool valid[4];
      float mx = kNegBig;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        valid[r] = tok0 + 4 * qd + r < te;
        sc[r] = sacc[r] * scale_log2;
        if (valid[r]) mx = fmaxf(mx, sc[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m, mx);
      const float alpha = exp2f_fast(m - m_new);
      float p[4];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = valid[r] ? exp2f_fast(sc[r] - m_new) : 0.f;
        psum += p[r];
      }
      l = l * alpha + psum;
      m = m_new;
#pragma unroll
      for (int b = 0; b < NB; ++b) ob[b] *= alpha;
      // Pᵀ operand as 16-bit head + remainder
      uint16_t ph[4], pl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float back, back2;
        ph[r] = round16<DT>(p[r], &back);
        pl[r] = round16<DT>(p[r] - back, &back2);
      }
      const uint2 phi = make_uint2(ph[0] | (static_cast<uint32_t>(ph[1]) << 16), ph[2] | (static_cast<uint32_t>(ph[3]) << 16));
      const uint2 plo = make_uint2(pl[0] | (static_cast<uint32_t>(pl[1]) << 16), pl[2] | (static_cast<uint32_t>(pl[3]) << 16));
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // the V tile is written …
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");   // … before any lane reads it back
      // Oᵀ += Vᵀ·Pᵀ: lane reads dim 16b + tl of tokens 4qd..4qd+3
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint32_t v0 = sh.t.vt[wave][4 * qd + 0][16 * b + tl];
        const uint32_t v1 = sh.t.vt[wave][4 * qd + 1][16 * b + tl];
        const uint32_t v2 = sh.t.vt[wave][4 * qd + 2][16 * b + tl];
        const uint32_t v3 = sh.t.vt[wave][4 * qd + 3][16 * b + tl];
        const uint2 a = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
        ob[b] = mfma_k16<DT>(a, phi, ob[b]);
        ob[b] = mfma_k16<DT>(a, plo, ob[b]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // reads done before the next chunk's writes
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // This wave's run of chunks, as in the vector loop: two per iteration
    // through two named buffers, the next chunk's loads in flight.
    uint4 ka[NKL], va[NKL], kb2[NKL], vb2[NKL];
    const ChunkDeal dl = deal_chunks<CT, NW>(wave, wave_tokens, t_begin, t_end, tb, te);
    const int32_t lim = dl.limit;
    int32_t c = dl.first;
    load_chunk(c, c < lim, ka, va);
    for (; c < lim; c += 2) {
      load_chunk(c + 1, c + 1 < lim, kb2, vb2);
      __builtin_amdgcn_sched_barrier(0);
      consume_chunk(c, ka, va);
      if (c + 1 >= lim) break;
      load_chunk(c + 2, c + 2 < lim, ka, va);
      __builtin_amdgcn_sched_barrier(0);
      consume_chunk(c + 1, kb2, vb2);
    }
  }

  // The four quarters of a row hold partial sums over their tokens.
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);

  // Merge the NW waves through LDS and hand each output to emit.  o shares
  // its LDS with the tiles, so every wave must be done with them first.
  __syncthreads();
  if (tl < R) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      *reinterpret_cast<float4*>(&sh.o[wave][tl][wave_out(tl, 16 * b + 4 * qd)]) =
          make_float4(ob[b][0], ob[b][1], ob[b][2], ob[b][3]);
    if (qd == 0) {
      sh.m[wave][tl] = m;
      sh.l[wave][tl] = l;
    }
  }
  const bool wave_bad = __any(bad_block);
  if (lane == 0) sh.bad[wave] = wave_bad ? 1 : 0;
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) bad = bad || sh.bad[w] != 0;
  for (int idx = threadIdx.x; idx < R * D; idx += NW * 64) {
    const int r = idx / D;
    const int d = idx - r * D;
    float mm = kNegBig;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, sh.m[w][r]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = exp2f_fast(sh.m[w][r] - mm);
      L += sh.l[w][r] * a;
      O += sh.o[w][r][wave_out(r, d)] * a;
    }
    emit(r, d, mm, L, O, bad);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// attend_range: the G query rows of kv-head g of sequence s over tokens
// [t_begin, t_end), t_begin < t_end, t_begin a multiple of CT or (fixed
// partitions) of block_size.  Each of the NW waves takes one contiguous run of
// CT-token chunks (deal_chunks).  Every thread then calls emit(r, d, M, L, O, bad) for its share
// of the G×D outputs: M is the running max (base 2), L = Σ 2^(score−M),
// O = Σ 2^(score−M)·v[d] for query row r, and bad reports a block id outside
// the pool (then the values are meaningless).  Ends with a barrier, so the
// caller may call it again.
//
// Memory-level parallelism: every wave keeps the next chunk's 2·NLC loads in
// flight while it consumes the current one.  The loads are issued
// unconditionally (a load past the range reads this lane's 16 bytes of q,
// which are valid and cache-resident) and padding values are masked after
// unpacking, never by writing to the load registers, so the wait before each
// chunk is a fixed "all but the last 2·NLC loads" rather than a full drain.
// Block ids come from LDS, staged kTableBatch at a time, so no global load of
// the table sits between two chunks.
// ---------------------------------------------------------------------------
template <int DT, int D, int BS, int G, int NW, bool STREAM, bool NEWTOK, typename Emit>
__device__ __forceinline__ void attend_range(const char* __restrict__ k_pool, const char* __restrict__ v_pool,
                                             const char* __restrict__ q, const int32_t* __restrict__ table,
                                             int32_t s, int32_t g, int32_t kv_heads, int32_t num_blocks,
                                             int32_t t_begin, int32_t t_end, float scale_log2, NewToken nt,
                                             int32_t wave_tokens, WaveMerge<NW, G, D, kUseMfma<DT, BS, G>>& sh,
                                             Emit&& emit) {
  if constexpr (kUseMfma<DT, BS, G>) {
    constexpr int EB = 2;
    const int tl = threadIdx.x & 15;
    const char* q_head0 = q + ((static_cast<int64_t>(s) * kv_heads * G + g * G) * D) * EB;   // row g·G of sequence s
    attend_range_mfma<DT, D, BS, G, NW, STREAM, NEWTOK>(k_pool, v_pool, tl < G ? q_head0 + tl * D * EB : nullptr,
                                                        q_head0, table, g, kv_heads, num_blocks, t_begin, t_end,
                                                        scale_log2, nt, wave_tokens, sh, emit);
    return;
  } else {
  using S = Shape<DT, D>;
  using CK = Chunk<DT, D, BS>;
  constexpr int ELEMS = S::ELEMS, LPT = S::LPT, TPL = S::TPL, ROW = S::ROW;
  constexpr bool kSmallBlocks = CK::kSmallBlocks;
  constexpr int NLC = CK::NLC, CT = CK::CT;
  constexpr int64_t TILE = static_cast<int64_t>(BS) * ROW;
  static_assert(kTableBatch % (CT > BS ? CT / BS : 1) == 0, "table batches must hold whole chunks");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int q_heads = kv_heads * G;

  const int grp = lane / LPT;     // which token of a wave-wide load this lane reads
  const int sub = lane % LPT;     // which 16-byte slice of the row
  const int32_t lane_off = grp * ROW + sub * 16;

  // query rows of this kv-head: 16 bytes per lane per row
  const char* q_lane = q + ((static_cast<int64_t>(s) * q_heads + g * G) * D) * S::EB + sub * 16;
  uint4 qv[G];
#pragma unroll
  for (int r = 0; r < G; ++r) qv[r] = *reinterpret_cast<const uint4*>(q_lane + r * D * S::EB);

  float m[G], l[G], o[G][ELEMS];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    m[r] = kNegBig;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < ELEMS; ++e) o[r][e] = 0.f;
  }
  bool bad_block = false;

  const int32_t blk_first = t_begin / BS;
  const int32_t blk_last = (t_end - 1) / BS;
  for (int32_t bb = blk_first; bb <= blk_last; bb += kTableBatch) {
    const int32_t nb = min(kTableBatch, blk_last - bb + 1);
    __syncthreads();   // the previous batch's ids are no longer read
    for (int i = threadIdx.x; i < nb; i += NW * 64) {
      const int32_t phys = table[bb + i];
      sh.tbl[i] = static_cast<uint32_t>(phys) < static_cast<uint32_t>(num_blocks) ? phys : -1;
    }
    if constexpr (NEWTOK) {
      if (bb == blk_first) stage_new_token<ROW>(nt, sh.newrow);
    }
    __syncthreads();
    const int32_t tb = max(t_begin, bb * BS);
    const int32_t te = min(t_end, (bb + nb) * BS);

    // Byte offset of token t's row in its (block, kv-head) tile; t lies in this batch.
    auto tile_of = [&](int32_t t) {
      int32_t phys = sh.tbl[t / BS - bb];
      if (phys < 0) {
        bad_block = true;
        phys = 0;
      }
      return (static_cast<int64_t>(phys) * kv_heads + g) * TILE + (t % BS) * ROW;
    };

    // Issue the loads of chunk c (K and V, NLC wave-wide 16-byte loads each).
    // live = false: the chunk lies past the range; read q instead.  Padding
    // slots past t_end inside an allocated block may be read; their lanes are
    // masked before use.
    auto load_chunk = [&](int32_t c, bool live, uint4 (&kb)[NLC], uint4 (&vb)[NLC]) {
      const int32_t tok0 = tb + (live ? c : 0) * CT;
      if constexpr (!kSmallBlocks) {
        if constexpr (BS >= CT) {
          // a chunk never straddles a block: tb is a multiple of CT here
          const int64_t tile = tile_of(tok0) + lane_off;
#pragma unroll
          for (int i = 0; i < NLC; ++i) {
            kb[i] = load_kv<STREAM>(live ? k_pool + tile + i * TPL * ROW : q_lane);
            vb[i] = load_kv<STREAM>(live ? v_pool + tile + i * TPL * ROW : q_lane);
          }
        } else {
#pragma unroll
          for (int i = 0; i < NLC; ++i) {
            // a load starting past the range end re-reads the chunk's first
            // group (always inside an allocated block); its lanes are masked
            const int32_t t = tok0 + i * TPL < te ? tok0 + i * TPL : tok0;
            const int64_t tile = tile_of(t) + lane_off;
            kb[i] = load_kv<STREAM>(live ? k_pool + tile : q_lane);
            vb[i] = load_kv<STREAM>(live ? v_pool + tile : q_lane);
          }
        }
      } else {
        int32_t t = tok0 + grp;
        if (t >= te) t = te - 1;
        const int64_t off = tile_of(t) + sub * 16;
        kb[0] = load_kv<STREAM>(live ? k_pool + off : q_lane);
        vb[0] = load_kv<STREAM>(live ? v_pool + off : q_lane);
      }
    };

    // Fold chunk c into the running (m, l, o) of this lane group.
    auto consume_chunk = [&](int32_t c, uint4 (&kb)[NLC], uint4 (&vb)[NLC]) {
      const int32_t tok0 = tb + c * CT;
      const bool full = tok0 + CT <= te;   // wave-uniform
      if constexpr (NEWTOK) {
        // the new token's row (its slot is written after the loop) from LDS:
        // it sits in load i_new (wave-uniform), in the lanes of group g_new
        if (nt.t >= tok0 && nt.t < tok0 + CT) {   // wave-uniform
          const int32_t i_new = (nt.t - tok0) / TPL, g_new = (nt.t - tok0) % TPL;
#pragma unroll
          for (int i = 0; i < NLC; ++i) {
            if (i == i_new && grp == g_new) {
              kb[i] = sh.newrow[0][sub];
              vb[i] = sh.newrow[1][sub];
            }
          }
        }
      }
      bool valid[NLC];
#pragma unroll
      for (int i = 0; i < NLC; ++i) valid[i] = full || (tok0 + grp + i * TPL < te);
      float vf[NLC][ELEMS];
#pragma unroll
      for (int i = 0; i < NLC; ++i) unpack<DT>(vb[i], vf[i]);
      if (!full) {
        // padding may hold NaN or Inf: zero it, since 0·NaN would poison the sum
#pragma unroll
        for (int i = 0; i < NLC; ++i) {
#pragma unroll
          for (int e = 0; e < ELEMS; ++e) vf[i][e] = valid[i] ? vf[i][e] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < G; ++r) {
        float sc[NLC];
        float mx = kNegBig;
#pragma unroll
        for (int i = 0; i < NLC; ++i) {
          sc[i] = group_sum<LPT>(dot16<DT>(qv[r], kb[i])) * scale_log2;
          if (valid[i]) mx = fmaxf(mx, sc[i]);
        }
        const float m_new = fmaxf(m[r], mx);
        const float alpha = exp2f_fast(m[r] - m_new);
        float psum = 0.f;
        float pi[NLC];
#pragma unroll
        for (int i = 0; i < NLC; ++i) {
          pi[i] = valid[i] ? exp2f_fast(sc[i] - m_new) : 0.f;
          psum += pi[i];
        }
        l[r] = l[r] * alpha + psum;
#pragma unroll
        for (int e = 0; e < ELEMS; ++e) {
          float acc = o[r][e] * alpha;
#pragma unroll
          for (int i = 0; i < NLC; ++i) acc = __builtin_fmaf(pi[i], vf[i][e], acc);
          o[r][e] = acc;
        }
        m[r] = m_new;
      }
    };

    // This wave's run of chunks [first, limit) (deal_chunks), two per
    // iteration through two named buffers, with the next chunk's loads in
    // flight while the current one is consumed.  (The scheduling barriers keep
    // the compiler from hoisting the current chunk's arithmetic above the next
    // chunk's load issue, which would make the wave wait for its data before
    // the prefetch leaves.)
    uint4 ka[NLC], va[NLC], kb2[NLC], vb2[NLC];
    const ChunkDeal dl = deal_chunks<CT, NW>(wave, wave_tokens, t_begin, t_end, tb, te);
    const int32_t lim = dl.limit;
    int32_t c = dl.first;
    load_chunk(c, c < lim, ka, va);
    for (; c < lim; c += 2) {
      load_chunk(c + 1, c + 1 < lim, kb2, vb2);
      __builtin_amdgcn_sched_barrier(0);
      consume_chunk(c, ka, va);
      if (c + 1 >= lim) break;
      load_chunk(c + 2, c + 2 < lim, ka, va);
      __builtin_amdgcn_sched_barrier(0);
      consume_chunk(c + 1, kb2, vb2);
    }
  }

  // Merge the TPL lane groups of this wave (lanes differing above log2(LPT)).
#pragma unroll
  for (int mask = LPT; mask < 64; mask <<= 1) {
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const float m_o = __shfl_xor(m[r], mask, 64);
      const float l_o = __shfl_xor(l[r], mask, 64);
      const float mm = fmaxf(m[r], m_o);
      const float a = exp2f_fast(m[r] - mm);
      const float b = exp2f_fast(m_o - mm);
      l[r] = l[r] * a + l_o * b;
#pragma unroll
      for (int e = 0; e < ELEMS; ++e) {
        const float oo = __shfl_xor(o[r][e], mask, 64);
        o[r][e] = o[r][e] * a + oo * b;
      }
      m[r] = mm;
    }
  }

  // Merge the NW waves through LDS and hand each output to emit.
  if (lane < LPT) {
#pragma unroll
    for (int r = 0; r < G; ++r) {
#pragma unroll
      for (int e = 0; e < ELEMS; ++e) sh.o[wave][r][sub * ELEMS + e] = o[r][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < G; ++r) {
      sh.m[wave][r] = m[r];
      sh.l[wave][r] = l[r];
    }
  }
  const bool wave_bad = __any(bad_block);
  if (lane == 0) sh.bad[wave] = wave_bad ? 1 : 0;
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) bad = bad || sh.bad[w] != 0;
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int r = idx / D;
    const int d = idx - r * D;
    float mm = kNegBig;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, sh.m[w][r]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = exp2f_fast(sh.m[w][r] - mm);
      L += sh.l[w][r] * a;
      O += sh.o[w][r][d] * a;
    }
    emit(r, d, mm, L, O, bad);
  }
  __syncthreads();
  }
}

// Tokens at the start of sequence s that a shared-prefix call computes in its
// group's prefix pass: seq_prefix[s] clamped to [0, min(len, max_prefix)]
// and rounded down to a whole number of blocks (0 without seq_prefix).  The
// partition, prefix and reduce kernels all derive it this way, so they agree
// on every row's partial records.
template <int BS>
__device__ __forceinline__ int32_t prefix_of(const int32_t* __restrict__ seq_prefix, int32_t s, int32_t len,
                                             int32_t max_prefix) {
  if (!seq_prefix) return 0;
  const int32_t p = min(max(seq_prefix[s], 0), min(len, max_prefix));
  return p - p % BS;
}

// Partitions of part_tokens covering n ≥ 0 tokens.
__device__ __forceinline__ int32_t parts_of(int32_t n, int32_t part_tokens) {
  return n <= 0 ? 0 : (n + part_tokens - 1) / part_tokens;
}

// Fold n partial records (rows prow0 … prow0 + n − 1) of output element d into
// the running (M, L, O): the online-softmax merge by running max and sum.
template <int D>
__device__ __forceinline__ void fold_parts(const float* __restrict__ part_ml, const float* __restrict__ part_o,
                                           int64_t prow0, int32_t n, int d, float& M, float& L, float& O) {
  for (int32_t i = 0; i < n; ++i) {
    const float m_i = part_ml[2 * (prow0 + i)];
    const float mt = fmaxf(M, m_i);
    const float a = exp2f_fast(M - mt), b = exp2f_fast(m_i - mt);
    L = L * a + part_ml[2 * (prow0 + i) + 1] * b;
    O = O * a + part_o[(prow0 + i) * D + d] * b;
    M = mt;
  }
}

// Write zero rows (an empty context) or NaN rows (an invalid length) for all
// query heads of kv-head range [g0, g1) of sequence s.
template <int D, int G>
__device__ __forceinline__ void fill_rows(void* out, int32_t out_dtype, int32_t s, int32_t q_heads, int32_t g0,
                                          int32_t g1, float value) {
  const int64_t first = (static_cast<int64_t>(s) * q_heads + g0 * G) * D;
  const int32_t n = (g1 - g0) * G * D;
  for (int32_t i = threadIdx.x; i < n; i += blockDim.x) store_out(out, out_dtype, first + i, value);
}

// The KV write of pa_decode_append ([P2] §3.2.2 step 3, then step 4 in the
// same launch): the workgroup whose range ends at the context's last token
// stores that token's K and V rows of kv-head g, k_new/v_new[s][g][:], into
// slot kv_slots[s] (skipped when the slot is −1 or outside the pool), exactly
// as write_kv_kernel would.  It stores them after its token loop and waits for
// nothing: its own loads of that token read k_new/v_new (new_token_of), and no
// other workgroup reads the slot, because partitions start on block
// boundaries and the slot must hold token len−1 of sequence s.
template <int DT, int D, int BS>
__device__ __forceinline__ void append_token(const char* k_pool, const char* v_pool, const char* __restrict__ k_new,
                                             const char* __restrict__ v_new, const int32_t* __restrict__ kv_slots,
                                             int32_t s, int32_t g, int32_t kv_heads, int32_t num_blocks) {
  constexpr int ROW = D * Elem<DT>::bytes;   // bytes of one token's row
  constexpr int L16 = ROW / 16;              // 16-byte pieces per row
  static_assert(2 * L16 <= 64, "one wave stores both rows");
  if (threadIdx.x >= 2 * L16) return;
  const int32_t slot = kv_slots[s];
  if (slot < 0 || static_cast<int64_t>(slot) >= static_cast<int64_t>(num_blocks) * BS) return;
  const bool is_v = threadIdx.x >= L16;
  const int piece = threadIdx.x % L16;
  const int64_t dst = ((static_cast<int64_t>(slot / BS) * kv_heads + g) * BS + slot % BS) * ROW + piece * 16;
  const int64_t src = (static_cast<int64_t>(s) * kv_heads + g) * ROW + piece * 16;
  const uint4 v = *reinterpret_cast<const uint4*>((is_v ? v_new : k_new) + src);
  *reinterpret_cast<uint4*>(const_cast<char*>(is_v ? v_pool : k_pool) + dst) = v;
}

// The new token as the workgroup that owns token len−1 of (s, g) reads it:
// from k_new/v_new when append_token will write it into the pool (a valid
// slot), else none (then the pool already holds it).
template <int DT, int D, int BS>
__device__ __forceinline__ NewToken new_token_of(const char* __restrict__ k_new, const char* __restrict__ v_new,
                                                 const int32_t* __restrict__ kv_slots, int32_t s, int32_t g,
                                                 int32_t kv_heads, int32_t num_blocks, int32_t len) {
  NewToken nt;
  if (!kv_slots || len <= 0) return nt;
  const int32_t slot = kv_slots[s];
  if (slot < 0 || static_cast<int64_t>(slot) >= static_cast<int64_t>(num_blocks) * BS) return nt;
  constexpr int ROW = D * Elem<DT>::bytes;
  const int64_t off = (static_cast<int64_t>(s) * kv_heads + g) * ROW;
  nt.k = k_new + off;
  nt.v = v_new + off;
  nt.t = len - 1;
  return nt;
}

// attend_range with the cache policy chosen at run time (wave-uniform): the
// streaming policy unless the tiles are shared with a neighbouring sequence.
template <int DT, int D, int BS, int G, int NW, bool NEWTOK, typename Emit>
__device__ __forceinline__ void attend_range_policy(bool shared, const char* __restrict__ k_pool,
                                                    const char* __restrict__ v_pool, const char* __restrict__ q,
                                                    const int32_t* __restrict__ table, int32_t s, int32_t g,
                                                    int32_t kv_heads, int32_t num_blocks, int32_t t_begin,
                                                    int32_t t_end, float scale_log2, NewToken nt, int32_t wave_tokens,
                                                    WaveMerge<NW, G, D, kUseMfma<DT, BS, G>>& sh, Emit&& emit) {
  if (shared) {
    attend_range<DT, D, BS, G, NW, false, NEWTOK>(k_pool, v_pool, q, table, s, g, kv_heads, num_blocks, t_begin,
                                                  t_end, scale_log2, nt, wave_tokens, sh, emit);
  } else {
    attend_range<DT, D, BS, G, NW, true, NEWTOK>(k_pool, v_pool, q, table, s, g, kv_heads, num_blocks, t_begin,
                                                 t_end, scale_log2, nt, wave_tokens, sh, emit);
  }
}

// ---------------------------------------------------------------------------
// decode_partition_kernel (fixed partitions)
//   grid  = (max_parts, kv_heads, num_seqs), block = NW × 64 threads
//   Unit (s, g, p) covers tokens [p·P, min((p+1)·P, len_s)) of sequence s,
//   kv-head g, and the G query heads g·G … g·G+G-1.  Workgroups start in
//   linear order (x fastest), so the batch order is the dispatch order: the
//   host scheduler puts long sequences first and prefix-sharing ones side by
//   side (pa_bm_dispatch_order); which workgroup computes a unit changes
//   nothing in its result.  Workgroup w runs on XCD w mod 8, so with one
//   partition and kv_heads a multiple of 8, kv-head g of every sequence lands
//   on XCD g mod 8 and adjacent siblings find their shared tiles in its L2.
// ---------------------------------------------------------------------------
template <int DT, int D, int BS, int G, int NW, bool APPEND>
__global__ __launch_bounds__(NW * 64, (kMinWavesExtra<DT, BS, G, APPEND>)) void decode_partition_kernel(
    const char* __restrict__ k_pool, const char* __restrict__ v_pool, const char* __restrict__ q,
    void* __restrict__ out, int32_t out_dtype, float* __restrict__ part_ml, float* __restrict__ part_o,
    const int32_t* __restrict__ block_tables, int32_t table_stride, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ seq_prefix, int32_t max_prefix, int32_t num_seqs, int32_t num_blocks,
    int32_t kv_heads, int32_t max_ctx, int32_t max_parts, int32_t part_tokens, int32_t wave_tokens, float scale_log2,
    const char* __restrict__ k_new, const char* __restrict__ v_new, const int32_t* __restrict__ kv_slots) {
  const int p = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int q_heads = kv_heads * G;

  const int32_t len = context_lens[s];
  const bool bad_len = len < 0 || len > max_ctx;
  const int32_t len_c = bad_len ? 0 : len;
  // pa_decode_append (no shared prefix there): the last partition owns the
  // new token.  An empty or invalid context's only workgroup writes it at
  // once; otherwise the owner reads it from k_new/v_new and writes it into
  // the pool after its token loop.
  const bool owner = APPEND && p == max(parts_of(len_c, part_tokens), 1) - 1;
  if (len_c == 0) {
    if (owner) append_token<DT, D, BS>(k_pool, v_pool, k_new, v_new, kv_slots, s, g, kv_heads, num_blocks);
    if (p == 0) fill_rows<D, G>(out, out_dtype, s, q_heads, g, g + 1, bad_len ? qnan() : 0.f);
    return;
  }
  // With a shared prefix this workgroup covers part p of the suffix; the
  // prefix's npp partials were written by decode_prefix_kernel, which ran
  // before this kernel on the stream.  A suffix of one part folds them in
  // here; longer ones leave it to decode_reduce_kernel.
  const int32_t pre = prefix_of<BS>(seq_prefix, s, len_c, max_prefix);
  const int32_t npp = parts_of(pre, part_tokens);
  const int32_t nsp = parts_of(len_c - pre, part_tokens);
  if (p >= max(nsp, 1)) return;
  if (nsp == 0) {   // the context is all prefix: finish from its partials
    for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
      const int r = idx / D, d = idx - r * D;
      const int64_t row = static_cast<int64_t>(s) * q_heads + g * G + r;
      float M = kNegBig, L = 0.f, O = 0.f;
      fold_parts<D>(part_ml, part_o, row * max_parts, npp, d, M, L, O);
      store_out(out, out_dtype, row * D + d, L > 0.f ? O / L : (L != L ? qnan() : 0.f));
    }
    return;
  }
  const int32_t t_begin = pre + p * part_tokens;
  const int32_t t_end = min(t_begin + part_tokens, len_c);
  const int32_t* table = block_tables + static_cast<int64_t>(s) * table_stride;
  __shared__ WaveMerge<NW, G, D, kUseMfma<DT, BS, G>> sh;
  // after a prefix pass the tiles read here are this sequence's own
  const bool shared = pre == 0 && shares_first_block(block_tables, table_stride, s, num_seqs);
  const NewToken nt =
      owner ? new_token_of<DT, D, BS>(k_new, v_new, kv_slots, s, g, kv_heads, num_blocks, len_c) : NewToken{};
  attend_range_policy<DT, D, BS, G, NW, APPEND>(
      shared, k_pool, v_pool, q, table, s, g, kv_heads, num_blocks, t_begin, t_end, scale_log2, nt, wave_tokens, sh,
      [&](int r, int d, float M, float L, float O, bool bad) {
        const int64_t row = static_cast<int64_t>(s) * q_heads + g * G + r;
        if (nsp == 1) {
          if (npp > 0) fold_parts<D>(part_ml, part_o, row * max_parts, npp, d, M, L, O);
          store_out(out, out_dtype, row * D + d, bad ? qnan() : (L > 0.f ? O / L : (L != L ? qnan() : 0.f)));
        } else {
          const int64_t prow = row * max_parts + npp + p;
          part_o[prow * D + d] = bad ? qnan() : O;
          if (d == 0) {
            part_ml[2 * prow] = M;
            part_ml[2 * prow + 1] = L;
          }
        }
      });
  if (owner) append_token<DT, D, BS>(k_pool, v_pool, k_new, v_new, kv_slots, s, g, kv_heads, num_blocks);
}

// ---------------------------------------------------------------------------
// decode_prefix_kernel: the shared prefix of a group of sequences, read once
// per kv-head for every member ([P2] §3.4; [P1] "跨请求的内存共享": the
// members' tables point at the same physical blocks, so the tokens there
// are the same for all of them).
//   grid = (prefix partitions, kv_heads × member tiles, groups).
//   Group k is batch positions [group_start[k], group_start[k+1]); its
//   prefix is prefix_of(first member of the tile).  A member tile is 16/G
//   members, whose G query rows per kv-head fill the 16 rows of the
//   matrix-core tile, so K·Qᵀ and P·V serve all of them at once.  Each
//   writes the (max, sum, output) partial of prefix partition pp of every
//   row it holds as that row's part pp; the partition kernel adds the
//   suffix's parts after them and decode_reduce_kernel merges.
//   Tiles of one (group, kv-head) are kv_heads workgroups apart, so with
//   kv_heads a multiple of 8 they run on one XCD and share its L2; a group
//   held in one tile streams its prefix.
// ---------------------------------------------------------------------------
template <int DT, int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * 64, 3) void decode_prefix_kernel(
    const char* __restrict__ k_pool, const char* __restrict__ v_pool, const char* __restrict__ q,
    float* __restrict__ part_ml, float* __restrict__ part_o, const int32_t* __restrict__ block_tables,
    int32_t table_stride, const int32_t* __restrict__ context_lens, const int32_t* __restrict__ group_start,
    const int32_t* __restrict__ seq_prefix, int32_t max_prefix, int32_t num_seqs, int32_t num_blocks,
    int32_t kv_heads, int32_t max_ctx, int32_t max_parts, int32_t part_tokens, float scale_log2) {
  constexpr int MT = 16 / G;   // members per tile
  constexpr int EB = 2;
  const int pp = blockIdx.x;
  const int g = blockIdx.y % kv_heads;
  const int mt = blockIdx.y / kv_heads;
  // clamped, so a malformed group list yields wrong rows, never a stray access
  const int32_t m_begin = min(max(group_start[blockIdx.z], 0), num_seqs);
  const int32_t m_end = min(max(group_start[blockIdx.z + 1], m_begin), num_seqs);
  const int32_t m0 = m_begin + mt * MT;
  if (m0 >= m_end) return;
  const int32_t m1 = min(m0 + MT, m_end);
  const int32_t len0 = context_lens[m0];
  const int32_t pre = prefix_of<BS>(seq_prefix, m0, (len0 < 0 || len0 > max_ctx) ? 0 : len0, max_prefix);
  if (pp >= parts_of(pre, part_tokens)) return;
  const int32_t t_begin = pp * part_tokens;
  const int32_t t_end = min(t_begin + part_tokens, pre);
  const int q_heads = kv_heads * G;

  const int tl = threadIdx.x & 15;
  const int32_t member = m0 + tl / G;
  const char* q_dummy = q + ((static_cast<int64_t>(m0) * q_heads + g * G) * D) * EB;
  const char* q_lane =
      member < m1 ? q + ((static_cast<int64_t>(member) * q_heads + g * G + tl % G) * D) * EB : nullptr;
  const int32_t* table = block_tables + static_cast<int64_t>(m0) * table_stride;
  __shared__ WaveMerge<NW, 16, D, true> sh;
  auto emit = [&](int r, int d, float M, float L, float O, bool bad) {
    const int32_t mem = m0 + r / G;
    if (mem >= m1) return;
    const int64_t prow = (static_cast<int64_t>(mem) * q_heads + g * G + r % G) * max_parts + pp;
    part_o[prow * D + d] = bad ? qnan() : O;
    if (d == 0) {
      part_ml[2 * prow] = M;
      part_ml[2 * prow + 1] = L;
    }
  };
  if (m_end - m_begin <= MT) {
    attend_range_mfma<DT, D, BS, 16, NW, true, false>(k_pool, v_pool, q_lane, q_dummy, table, g, kv_heads, num_blocks,
                                               t_begin, t_end, scale_log2, NewToken{}, 0, sh, emit);
  } else {
    attend_range_mfma<DT, D, BS, 16, NW, false, false>(k_pool, v_pool, q_lane, q_dummy, table, g, kv_heads, num_blocks,
                                                t_begin, t_end, scale_log2, NewToken{}, 0, sh, emit);
  }
}

// ---------------------------------------------------------------------------
// decode_reduce_kernel: merge the partitions of sequences longer than one.
//   grid = (q_heads, num_seqs, D/DC), block = kReduceThreads; one workgroup
//   per DC output dims of a row.  With a shared prefix a row's parts are the
//   prefix's partials followed by the suffix's; rows whose suffix is one
//   part were finished by the partition kernel.  After the uniform split
//   (unit_desc set) a row's records are the G-row records of its unit's
//   tasks t0 … t0+n−1, found in unit_desc.
//   out = Σ_p 2^(m_p − M) o_p / Σ_p 2^(m_p − M) l_p with M = max_p m_p.
//   Each workgroup computes the per-partition weights 2^(m_p − M) into LDS
//   (up to kReduceLds partitions; beyond that they are recomputed on the
//   fly), then kReduceThreads/DC partition lanes per output element
//   accumulate its DC dims.  Few rows (a long-context batch) take DC = 16, so
//   a row's partitions are walked by 32 lanes in 8 workgroups instead of by
//   4 lanes in one.
// ---------------------------------------------------------------------------
constexpr int kReduceThreads = 512;
constexpr int kReduceLds = 4096;
constexpr int kReduceSplitRows = 256;   // below this many rows the dims are split

__device__ __forceinline__ float block_reduce_max(float v, float* sh /*[8]*/) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int w = 1; w < kReduceThreads / 64; ++w) r = fmaxf(r, sh[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float v, float* sh /*[8]*/) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < kReduceThreads / 64; ++w) r += sh[w];
  __syncthreads();
  return r;
}

template <int D, int DC, int BS>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(void* __restrict__ out, int32_t out_dtype,
                                                                       const float* __restrict__ part_ml,
                                                                       const float* __restrict__ part_o,
                                                                       const int32_t* __restrict__ context_lens,
                                                                       const int32_t* __restrict__ seq_prefix,
                                                                       int32_t max_prefix, int32_t q_heads,
                                                                       int32_t max_parts, int32_t part_tokens,
                                                                       int32_t max_ctx,
                                                                       const int32_t* __restrict__ unit_desc,
                                                                       int32_t group) {
  constexpr int LANES = kReduceThreads / DC;   // partition lanes per output element
  static_assert(D % DC == 0 && kReduceThreads % DC == 0, "dims split");
  const int s = blockIdx.y;
  const int h = blockIdx.x;
  const int d0 = blockIdx.z * DC;
  const int tid = threadIdx.x;
  const int32_t len = context_lens[s];
  const bool bad_len = len < 0 || len > max_ctx;
  const int32_t len_c = bad_len ? 0 : len;
  const int64_t row = static_cast<int64_t>(s) * q_heads + h;
  // Record p of this row sits at rec0 + p·ps.
  int32_t nparts;
  int64_t rec0, ps;
  if (unit_desc) {   // uniform split: the unit's records, G rows per task
    const int64_t u = row / group;
    nparts = unit_desc[2 * u + 1];
    if (nparts <= 1) return;   // written by the partition's own workgroup
    rec0 = static_cast<int64_t>(unit_desc[2 * u]) * group + h % group;
    ps = group;
  } else {
    const int32_t pre = prefix_of<BS>(seq_prefix, s, len_c, max_prefix);
    const int32_t nsp = parts_of(len_c - pre, part_tokens);
    if (nsp <= 1) return;  // finished by the partition kernel (empty, NaN and single-part rows)
    nparts = parts_of(pre, part_tokens) + nsp;
    rec0 = row * max_parts;
    ps = 1;
  }
  const float* ml = part_ml + rec0 * 2;
  const float* po = part_o + rec0 * D;
  const int64_t mls = 2 * ps, pos = ps * D;

  __shared__ float sh_red[kReduceThreads / 64];
  __shared__ float sh_w[kReduceLds];
  __shared__ float sh_acc[LANES][DC];
  const int dl = tid % DC;
  const int d = d0 + dl;
  const int pl = tid / DC;
  // This thread's first kPre output values do not depend on the weights:
  // their loads leave before the reductions below and overlap them.
  constexpr int kPre = 8;
  float pre_o[kPre];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int pp = pl + k * LANES;
    pre_o[k] = pp < nparts ? po[pp * pos + d] : 0.f;
  }
  // (max, sum) of partition tid, kept for the weight pass
  const bool own = tid < nparts;
  const float m0 = own ? ml[tid * mls] : kNegBig;
  const float l0 = own ? ml[tid * mls + 1] : 0.f;
  float mm = m0;
  for (int p = tid + kReduceThreads; p < nparts; p += kReduceThreads) mm = fmaxf(mm, ml[p * mls]);
  const float M = block_reduce_max(mm, sh_red);
  float part = 0.f;
  if (own) {
    const float wgt = exp2f_fast(m0 - M);
    if (tid < kReduceLds) sh_w[tid] = wgt;
    part += l0 * wgt;   // a NaN sum marks a partition that met a bad block id
  }
  for (int p = tid + kReduceThreads; p < nparts; p += kReduceThreads) {
    const float wgt = exp2f_fast(ml[p * mls] - M);
    if (p < kReduceLds) sh_w[p] = wgt;
    part += ml[p * mls + 1] * wgt;
  }
  const float L = block_reduce_sum(part, sh_red);   // its barriers also publish sh_w
  // four independent accumulators keep four loads in flight per thread; the
  // k-th partition of this lane goes to accumulator k mod 4 throughout
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int pp = pl + k * LANES;
    if (pp < nparts) {
      const float wgt = pp < kReduceLds ? sh_w[pp] : exp2f_fast(ml[pp * mls] - M);
      acc[k & 3] = __builtin_fmaf(wgt, pre_o[k], acc[k & 3]);
    }
  }
  static_assert(kPre % 4 == 0, "the loop below continues the accumulator rotation");
  int p = pl + kPre * LANES;
  for (; p + 3 * LANES < nparts; p += 4 * LANES) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int pp = p + k * LANES;
      const float wgt = pp < kReduceLds ? sh_w[pp] : exp2f_fast(ml[pp * mls] - M);
      acc[k] = __builtin_fmaf(wgt, po[pp * pos + d], acc[k]);
    }
  }
  for (; p < nparts; p += LANES) {
    const float wgt = p < kReduceLds ? sh_w[p] : exp2f_fast(ml[p * mls] - M);
    acc[0] = __builtin_fmaf(wgt, po[p * pos + d], acc[0]);
  }
  sh_acc[pl][dl] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (pl == 0) {
    float O = 0.f;
#pragma unroll
    for (int k = 0; k < LANES; ++k) O += sh_acc[k][dl];
    const float x = bad_len ? qnan() : (L > 0.f ? O / L : (L != L ? qnan() : 0.f));
    store_out(out, out_dtype, row * D + d, x);
  }
}

// ---------------------------------------------------------------------------
// Balanced split (the automatic choice when the batch does not fill the device)
// ---------------------------------------------------------------------------

// A value every lane of the wave holds alike, moved to scalar registers (the
// compiler cannot know that a value read back from LDS is uniform).
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Chunks of CT tokens a sequence of length len contributes per kv-head
// (0 for an empty or invalid length).
template <int CT>
__device__ __forceinline__ int64_t seq_chunks(int32_t len, int32_t max_ctx) {
  return (len <= 0 || len > max_ctx) ? 0 : (static_cast<int64_t>(len) + CT - 1) / CT;
}

// Exclusive prefix sum of v over the block's threads; *total gets the sum.
template <int NW>
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* total, int64_t* sh /*[NW]*/) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int64_t before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int64_t t = sh[w];
    if (w < wave) before += t;
    sum += t;
  }
  __syncthreads();
  *total = sum;
  return before + x - v;
}

// Slice boundary of workgroup w when C chunks are split over W workgroups:
// floor(w·C / W), computed without overflow for C < 2^40.
__device__ __forceinline__ int64_t slice_start(int64_t w, int64_t C, int64_t W) {
  return w * (C / W) + (w * (C % W)) / W;
}

// The workgroup whose slice holds chunk x: the largest w with slice_start(w) ≤ x.
__device__ __forceinline__ int64_t slice_owner(int64_t x, int64_t C, int64_t W) {
  return ((x + 1) * W - 1) / C;
}

// Partial records pass between workgroups that may sit on different XCDs,
// whose L2 caches are not kept coherent with each other.  They are stored and
// loaded as device-scope relaxed atomics, which go to the coherent level of
// the memory hierarchy, so no device-wide fence (an L2 write-back or
// invalidate) is needed.  A writer waits until its own stores have completed
// (wait_vmem) before the counter increment that publishes them, and a reader
// issues its loads only after the increment that tells it it is last.  (A
// workgroup-scope fence or barrier does not wait for global stores on this
// target, so the wait is explicit.)
//
// This ordering rests on gfx950 hardware behaviour, not on the C++/HIP memory
// model, which would ask for a release increment and an acquire read of the
// counter (each compiles to a device-wide cache write-back or invalidate here,
// and a fence per cut piece made the kernel 2.8x slower).  The assumptions:
//  * a store with device scope (sc1) is counted complete by vmcnt only once
//    it has reached the level that every XCD reads through, so after
//    wait_vmem no XCD can observe the record's old value;
//  * a load with device scope is served from that level, never from a stale
//    line in the reader's own L2, and a load issued after the counter's
//    atomic has returned (the reader branches on the returned value) cannot
//    be satisfied before the atomic.
// The balanced split is opt-in (PA_PARTITION_BALANCED); its results are tested
// on grids of 1 to 4000 workgroups (three-level merge trees).
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt and lgkmcnt not waited on
}
__device__ __forceinline__ void st_rec(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_rec(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge records child 0 … nchild-1 (slots slot0 + c·span) into either the
// final output rows of unit (s, g) or a record at slot0.  All threads call it.
template <int D, int G, int NW>
__device__ __forceinline__ void merge_records(float* __restrict__ rec_ml, float* __restrict__ rec_o, int64_t slot0,
                                              int64_t span, int32_t nchild, bool final_out, void* __restrict__ out,
                                              int32_t out_dtype, int32_t s, int32_t g, int32_t q_heads) {
  __shared__ float sh_scale[G][kFanIn];
  __shared__ float sh_ML[G][2];
  const int tid = threadIdx.x;
  if (tid < G) {
    const int r = tid;
    float M = kNegBig;
    float mc[kFanIn], lc[kFanIn];
    for (int c = 0; c < nchild; ++c) {
      const int64_t rr = (slot0 + c * span) * G + r;
      mc[c] = ld_rec(rec_ml + rr * 2);
      lc[c] = ld_rec(rec_ml + rr * 2 + 1);
      M = fmaxf(M, mc[c]);
    }
    float L = 0.f;
    for (int c = 0; c < nchild; ++c) {
      const float a = exp2f_fast(mc[c] - M);
      sh_scale[r][c] = a;
      L += lc[c] * a;   // a NaN sum marks a piece that met a bad block id
    }
    sh_ML[r][0] = M;
    sh_ML[r][1] = L;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += NW * 64) {
    const int r = idx / D;
    const int d = idx - r * D;
    float O = 0.f;
    for (int c = 0; c < nchild; ++c) O += sh_scale[r][c] * ld_rec(rec_o + ((slot0 + c * span) * G + r) * D + d);
    if (final_out) {
      const float L = sh_ML[r][1];
      const int64_t row = static_cast<int64_t>(s) * q_heads + g * G + r;
      store_out(out, out_dtype, row * D + d, L > 0.f ? O / L : (L != L ? qnan() : 0.f));
    } else {
      st_rec(rec_o + (slot0 * G + r) * D + d, O);   // same thread read this element of child 0 above
    }
  }
  __syncthreads();   // every read of child 0's (max, sum) is done
  if (!final_out && tid < G) {
    st_rec(rec_ml + (slot0 * G + tid) * 2, sh_ML[tid][0]);
    st_rec(rec_ml + (slot0 * G + tid) * 2 + 1, sh_ML[tid][1]);
  }
}

// ---------------------------------------------------------------------------
// decode_balanced_kernel
//   grid = W workgroups (all resident at once), block = NW × 64 threads.
//   Unit u = s·kv_heads + g owns c_s = ceil(len_s / CT) consecutive chunks of
//   a global axis of C = kv_heads·Σ c_s chunks; workgroup w processes chunks
//   [floor(wC/W), floor((w+1)C/W)).  A unit cut by slice boundaries yields
//   one piece per workgroup it touches; piece k of unit u writes a record at
//   slot u + first_owner(u) + k (slots are distinct because both u and w only
//   grow along the axis).  Records merge up a fan-in-kFanIn tree: node k of a
//   level counts its finished children in ctr[level][first_owner(u) + 1 + k],
//   the last child to arrive merges them (or writes the output at the root)
//   and resets the counter to zero for the next call.  A unit cut into n
//   pieces holds the n − 1 slice boundaries first_owner + 1 … first_owner +
//   n − 1 strictly inside it, no other unit holds them, and no level has more
//   than n − 1 nodes, so the counters of different units are distinct.
// ---------------------------------------------------------------------------
template <int DT, int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * 64, (kMinWavesPerEU<DT, BS, G, true>)) void decode_balanced_kernel(
    const char* __restrict__ k_pool, const char* __restrict__ v_pool, const char* __restrict__ q,
    void* __restrict__ out, int32_t out_dtype, int32_t* __restrict__ ctr, float* __restrict__ rec_ml,
    float* __restrict__ rec_o, const int32_t* __restrict__ block_tables, int32_t table_stride,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_blocks, int32_t kv_heads,
    int32_t max_ctx, float scale_log2) {
  constexpr int NT = NW * 64;
  constexpr int CT = Chunk<DT, D, BS>::CT;
  // slices are cut at multiples of CT; the matrix-core loop reads 16-token tiles
  static_assert(!kUseMfma<DT, BS, G> || CT % 16 == 0, "balanced slices must hold whole matrix-core tiles");
  const int64_t w = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t q_heads = kv_heads * G;

  // Rows of empty or invalid sequences, spread over the grid.
  for (int64_t s = w; s < num_seqs; s += gridDim.x) {
    const int32_t len = context_lens[s];
    if (len <= 0 || len > max_ctx) {
      fill_rows<D, G>(out, out_dtype, static_cast<int32_t>(s), q_heads, 0, kv_heads, len == 0 ? 0.f : qnan());
    }
  }

  // Total chunks.  Each thread covers kSeqsPerThread consecutive sequences per
  // round; their lengths are loaded together (clamped indices, no branches),
  // so the loads overlap instead of waiting one by one.
  __shared__ int64_t sh_scan[NW];
  __shared__ int64_t sh_found[2];
  constexpr int64_t kPerRound = static_cast<int64_t>(NT) * kSeqsPerThread;
  auto thread_chunks = [&](int64_t round_base, int64_t (&ck)[kSeqsPerThread]) {
    int32_t lk[kSeqsPerThread];
#pragma unroll
    for (int k = 0; k < kSeqsPerThread; ++k) {
      const int64_t sq = round_base + static_cast<int64_t>(tid) * kSeqsPerThread + k;
      lk[k] = context_lens[sq < num_seqs ? sq : num_seqs - 1];
    }
    int64_t mine = 0;
#pragma unroll
    for (int k = 0; k < kSeqsPerThread; ++k) {
      const int64_t sq = round_base + static_cast<int64_t>(tid) * kSeqsPerThread + k;
      ck[k] = sq < num_seqs ? seq_chunks<CT>(lk[k], max_ctx) : 0;
      mine += ck[k];
    }
    return mine;
  };
  int64_t total = 0;
  for (int64_t base = 0; base < num_seqs; base += kPerRound) {
    int64_t ck[kSeqsPerThread];
    int64_t round_total;
    block_exclusive_scan<NW>(thread_chunks(base, ck), &round_total, sh_scan);
    total += round_total;
  }
  const int64_t C = uniform(total) * kv_heads;
  // Workgroups past the chunk count sit out, so every slice holds at least one
  // chunk and a unit's pieces are exactly the workgroups its chunks span.
  const int64_t W = min(static_cast<int64_t>(gridDim.x), C);
  if (w >= W) return;
  const int64_t start = slice_start(w, C, W);
  const int64_t end = slice_start(w + 1, C, W);
  if (start >= end) return;

  // Locate the sequence holding chunk `start` and the chunks before it.
  if (tid == 0) sh_found[0] = -1;
  __syncthreads();
  int64_t run = 0;
  for (int64_t base = 0; base < num_seqs; base += kPerRound) {
    int64_t ck[kSeqsPerThread];
    const int64_t mine = thread_chunks(base, ck);
    int64_t round_total;
    const int64_t excl = block_exclusive_scan<NW>(mine, &round_total, sh_scan);
    const int64_t lo = (run + excl) * kv_heads;
    const int64_t hi = (run + excl + mine) * kv_heads;
    if (lo <= start && start < hi) {   // exactly one thread
      int64_t P = run + excl;
      for (int k = 0; k < kSeqsPerThread; ++k) {
        if ((P + ck[k]) * kv_heads > start) {
          sh_found[0] = base + static_cast<int64_t>(tid) * kSeqsPerThread + k;
          sh_found[1] = P;
          break;
        }
        P += ck[k];
      }
    }
    run += round_total;
    __syncthreads();
    if (sh_found[0] >= 0) break;
  }

  // Walk the units that meet [start, end).
  int32_t s = static_cast<int32_t>(uniform(sh_found[0]));
  int64_t P = uniform(sh_found[1]);
  __shared__ int sh_last;
  __shared__ WaveMerge<NW, G, D, kUseMfma<DT, BS, G>> sh;
  for (; s < num_seqs; ++s) {
    const int32_t len = context_lens[s];
    const int64_t c = seq_chunks<CT>(len, max_ctx);
    const int64_t base = P * kv_heads;
    if (base >= end) break;
    P += c;
    if (c == 0) continue;
    const int32_t* table = block_tables + static_cast<int64_t>(s) * table_stride;
    const bool shared = shares_first_block(block_tables, table_stride, s, num_seqs);
    for (int32_t g = start > base ? static_cast<int32_t>((start - base) / c) : 0; g < kv_heads; ++g) {
      const int64_t off = base + g * c;
      if (off >= end) break;
      const int64_t a = max(start, off) - off;
      const int64_t b = min(end, off + c) - off;
      const int32_t t0 = static_cast<int32_t>(a * CT);
      const int32_t t1 = static_cast<int32_t>(min(b * CT, static_cast<int64_t>(len)));
      // A whole unit writes its output; a piece writes a record and climbs the
      // merge tree.  One call site for both keeps a single copy of the loop.
      const bool whole = a == 0 && b == c;
      const int64_t u = static_cast<int64_t>(s) * kv_heads + g;
      const int64_t first_w = slice_owner(off, C, W);
      const int64_t slot0 = u + first_w;
      int32_t n = static_cast<int32_t>(slice_owner(off + c - 1, C, W) - first_w + 1);   // pieces
      int32_t idx = static_cast<int32_t>(w - first_w);
      const int64_t my_slot = slot0 + idx;
      attend_range_policy<DT, D, BS, G, NW, false>(
          shared, k_pool, v_pool, q, table, s, g, kv_heads, num_blocks, t0, t1, scale_log2, NewToken{}, 0, sh,
          [&](int r, int d, float M, float L, float O, bool bad) {
            if (whole) {
              const int64_t row = static_cast<int64_t>(s) * q_heads + g * G + r;
              store_out(out, out_dtype, row * D + d, bad ? qnan() : (L > 0.f ? O / L : 0.f));
              return;
            }
            const int64_t rr = my_slot * G + r;
            st_rec(rec_o + rr * D + d, O);
            if (d == 0) {
              st_rec(rec_ml + rr * 2, M);
              st_rec(rec_ml + rr * 2 + 1, bad ? qnan() : L);
            }
          });
      if (whole) continue;
      // Climb the merge tree while this workgroup is the last child to finish.
      int64_t span = 1;
      for (int level = 0; level < kMaxLevels; ++level) {
        const int32_t parent = idx / kFanIn;
        const int32_t nchild = min(kFanIn, n - parent * kFanIn);
        const int64_t pslot = slot0 + static_cast<int64_t>(parent) * kFanIn * span;
        int32_t* counter = ctr + static_cast<int64_t>(level) * kCounterSlots + first_w + 1 + parent;
        wait_vmem();       // this wave's record stores have completed …
        __syncthreads();   // … and so have every other wave's
        if (tid == 0) sh_last = atomicAdd(counter, 1) == nchild - 1;
        __syncthreads();
        if (!sh_last) break;
        if (tid == 0) atomicExch(counter, 0);
        const int32_t n_up = (n + kFanIn - 1) / kFanIn;
        merge_records<D, G, NW>(rec_ml, rec_o, pslot, span, nchild, n_up == 1, out, out_dtype, s, g, q_heads);
        if (n_up == 1) break;
        idx = parent;
        n = n_up;
        span *= kFanIn;
      }
      __syncthreads();   // sh_last is read by every thread before the next piece rewrites it
    }
  }
}

// ---------------------------------------------------------------------------
// Uniform split: every (sequence, kv-head) unit is cut into partitions of one
// length P, chosen on the device from the lengths so that all of the batch's
// partitions fit in one grid of `budget` workgroups that are resident at
// once.  Tasks are numbered densely, so workgroup t (on XCD t mod 8) always
// has work and each XCD gets an equal count, with no idle workgroups mixed
// in.
// ---------------------------------------------------------------------------
constexpr int kUniformLaneLens = 4;   // lengths a lane keeps in registers (the batch's first 256)

// A length as the split counts it: a valid length as it is, an empty or
// invalid one as 0 (its unit still takes one workgroup, which writes its zero
// or NaN rows), -1 past the end of the batch.
__device__ __forceinline__ int32_t split_len(const int32_t* __restrict__ lens, int32_t s, int32_t num_seqs,
                                             int32_t max_ctx) {
  if (s >= num_seqs) return -1;
  const int32_t l = lens[s];
  return (l < 0 || l > max_ctx) ? 0 : l;
}

// Partitions of P tokens that a unit of split length l takes.
__device__ __forceinline__ int64_t unit_parts(int32_t l, int64_t P) {
  return l < 0 ? 0 : (l == 0 ? 1 : (l + P - 1) / P);
}

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

struct UniformTask {
  int32_t s, g, p;   // sequence, kv-head, partition
  int32_t n;         // partitions of this unit
  int32_t t0;        // task index of its partition 0
  int64_t P;         // partition length in tokens
};

// Task t of the uniform split.  Every wave computes it on its own (registers
// and cross-lane operations only).  Returns false past the last task.
template <int BS>
__device__ bool uniform_task(const int32_t* __restrict__ lens, int32_t num_seqs, int32_t kv_heads, int32_t max_ctx,
                             int64_t t, int64_t budget, UniformTask* out) {
  const int lane = threadIdx.x & 63;
  const int64_t kmax = max<int64_t>(1, (static_cast<int64_t>(max_ctx) + BS - 1) / BS);
  const int64_t per_head = budget / kv_heads;   // partitions one kv-head may take over the whole batch
  if (per_head <= num_seqs) {                   // no room to split: one workgroup per unit
    if (t >= static_cast<int64_t>(num_seqs) * kv_heads) return false;
    out->s = static_cast<int32_t>(t / kv_heads);
    out->g = static_cast<int32_t>(t % kv_heads);
    out->p = 0;
    out->n = 1;
    out->t0 = static_cast<int32_t>(t);
    out->P = kmax * BS;
    return true;
  }
  constexpr int kCached = 64 * kUniformLaneLens;
  int32_t lc[kUniformLaneLens];
  int64_t sum = 0;
#pragma unroll
  for (int k = 0; k < kUniformLaneLens; ++k) {
    lc[k] = split_len(lens, 64 * k + lane, num_seqs, max_ctx);
    sum += max(lc[k], 0);
  }
  for (int32_t s = kCached + lane; s < num_seqs; s += 64) sum += max(split_len(lens, s, num_seqs, max_ctx), 0);
  sum = uniform(wave_sum(sum));
  auto count = [&](int64_t P) -> int64_t {
    int64_t c = 0;
#pragma unroll
    for (int k = 0; k < kUniformLaneLens; ++k) c += unit_parts(lc[k], P);
    for (int32_t s = kCached + lane; s < num_seqs; s += 64) c += unit_parts(split_len(lens, s, num_seqs, max_ctx), P);
    return uniform(wave_sum(c));
  };
  // Smallest k with count(k·BS) ≤ per_head.  Σ⌈l/P⌉ ≥ Σl/P bounds k from
  // below; Σ⌈l/P⌉ ≤ Σl/P + num_seqs gives a k that fits; kmax (one partition
  // per unit) always fits.
  int64_t lo = max<int64_t>(1, (sum + per_head * BS - 1) / (per_head * BS));
  const int64_t room = (per_head - num_seqs) * BS;
  int64_t hi = max(lo, min(kmax, (sum + room - 1) / room));
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (count(mid * BS) <= per_head) hi = mid;
    else lo = mid + 1;
  }
  const int64_t P = hi * BS;
  // Tasks in batch order: sequence s holds kv_heads × n_s consecutive tasks,
  // kv-head by kv-head.  Scan 64 sequences at a time for the one holding t.
  int64_t base = 0;
  auto visit = [&](int32_t l, int32_t s0) -> bool {
    const int64_t n = unit_parts(l, P);
    const int64_t c = n * kv_heads;
    int64_t incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int64_t total = uniform(__shfl(incl, 63, 64));
    if (t >= base + total) {
      base += total;
      return false;
    }
    const int w = __builtin_ctzll(__ballot(base + incl > t));
    const int64_t before = uniform(__shfl(incl - c, w, 64));
    const int64_t nn = uniform(__shfl(n, w, 64));
    const int64_t local = t - base - before;
    out->s = s0 + w;
    out->g = static_cast<int32_t>(local / nn);
    out->p = static_cast<int32_t>(local % nn);
    out->n = static_cast<int32_t>(nn);
    out->t0 = static_cast<int32_t>(t - out->p);
    out->P = P;
    return true;
  };
#pragma unroll
  for (int k = 0; k < kUniformLaneLens; ++k)
    if (visit(lc[k], 64 * k)) return true;
  for (int32_t s0 = kCached; s0 < num_seqs; s0 += 64)
    if (visit(split_len(lens, s0 + lane, num_seqs, max_ctx), s0)) return true;
  return false;
}

// ---------------------------------------------------------------------------
// decode_uniform_kernel
//   grid = budget workgroups (1-D, all resident at once), block = NW × 64.
//   Workgroup t runs task t of uniform_task: tokens [p·P, min((p+1)·P, len))
//   of unit (s, g).  A unit of one partition writes its output rows; a unit
//   of n > 1 writes one record per partition at its task index (rows
//   t·G … t·G+G−1) and, from partition 0, (t0, n) into unit_desc[unit] for
//   decode_reduce_kernel.
// ---------------------------------------------------------------------------
template <int DT, int D, int BS, int G, int NW, bool APPEND>
__global__ __launch_bounds__(NW * 64, (kMinWavesExtra<DT, BS, G, true>)) void decode_uniform_kernel(
    const char* __restrict__ k_pool, const char* __restrict__ v_pool, const char* __restrict__ q,
    void* __restrict__ out, int32_t out_dtype, float* __restrict__ part_ml, float* __restrict__ part_o,
    int32_t* __restrict__ unit_desc, const int32_t* __restrict__ block_tables, int32_t table_stride,
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_blocks, int32_t kv_heads,
    int32_t max_ctx, float scale_log2, const char* __restrict__ k_new, const char* __restrict__ v_new,
    const int32_t* __restrict__ kv_slots) {
  const int64_t t = blockIdx.x;
  UniformTask tk;
  if (!uniform_task<BS>(context_lens, num_seqs, kv_heads, max_ctx, t, gridDim.x, &tk)) return;
  const int32_t s = tk.s, g = tk.g;
  const int q_heads = kv_heads * G;
  const bool owner = APPEND && tk.p == tk.n - 1;   // the unit's last partition owns the new token
  if (tk.p == 0 && threadIdx.x == 0) {
    const int64_t u = static_cast<int64_t>(s) * kv_heads + g;
    unit_desc[2 * u] = tk.t0;
    unit_desc[2 * u + 1] = tk.n;
  }
  const int32_t len = context_lens[s];
  const bool bad_len = len < 0 || len > max_ctx;
  if (bad_len || len == 0) {
    if (owner) append_token<DT, D, BS>(k_pool, v_pool, k_new, v_new, kv_slots, s, g, kv_heads, num_blocks);
    fill_rows<D, G>(out, out_dtype, s, q_heads, g, g + 1, bad_len ? qnan() : 0.f);
    return;
  }
  const int32_t t_begin = static_cast<int32_t>(tk.p * tk.P);
  const int32_t t_end = static_cast<int32_t>(min<int64_t>(t_begin + tk.P, len));
  const bool single = tk.n == 1;
  const int32_t* table = block_tables + static_cast<int64_t>(s) * table_stride;
  __shared__ WaveMerge<NW, G, D, kUseMfma<DT, BS, G>> sh;
  const bool shared = shares_first_block(block_tables, table_stride, s, num_seqs);
  const NewToken nt =
      owner ? new_token_of<DT, D, BS>(k_new, v_new, kv_slots, s, g, kv_heads, num_blocks, len) : NewToken{};
  attend_range_policy<DT, D, BS, G, NW, APPEND>(
      shared, k_pool, v_pool, q, table, s, g, kv_heads, num_blocks, t_begin, t_end, scale_log2, nt, 0, sh,
      [&](int r, int d, float M, float L, float O, bool bad) {
        if (single) {
          const int64_t row = static_cast<int64_t>(s) * q_heads + g * G + r;
          store_out(out, out_dtype, row * D + d, bad ? qnan() : (L > 0.f ? O / L : (L != L ? qnan() : 0.f)));
          return;
        }
        const int64_t rec = t * G + r;
        part_o[rec * D + d] = bad ? qnan() : O;
        if (d == 0) {
          part_ml[2 * rec] = M;
          part_ml[2 * rec + 1] = L;
        }
      });
  if (owner) append_token<DT, D, BS>(k_pool, v_pool, k_new, v_new, kv_slots, s, g, kv_heads, num_blocks);
}

// ---------------------------------------------------------------------------
// Host-side launch
// ---------------------------------------------------------------------------

// Workgroups of `kernel` (kThreads threads, static LDS only) that the current
// device holds at once; cached per device in `cache` (atomics: host threads
// may ask at once, and all compute the same value).
template <typename Kernel>
hipError_t resident_workgroups(Kernel kernel, std::atomic<int> (&cache)[64], int32_t* resident_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int resident = dev >= 0 && dev < 64 ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (resident == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    resident = per_cu * cus;
    if (resident <= 0) resident = cus > 0 ? cus : 1;
    if (dev >= 0 && dev < 64) cache[dev].store(resident, std::memory_order_relaxed);
  }
  *resident_out = resident;
  return hipSuccess;
}

// Workgroups of the balanced kernel: every one resident at once (occupancy ×
// CUs), at most one per chunk the batch can hold, or PA_DECODE_GRID.
template <int DT, int D, int BS, int G>
hipError_t balanced_grid(const PoolDesc& p, int32_t num_seqs, int32_t max_ctx, int32_t* grid) {
  constexpr int CT = Chunk<DT, D, BS>::CT;
  static std::atomic<int> cache[64];
  int32_t resident = 0;
  hipError_t e = resident_workgroups(decode_balanced_kernel<DT, D, BS, G, kWaves>, cache, &resident);
  if (e != hipSuccess) return e;
  int64_t W = resident;
  if (const char* v = std::getenv("PA_DECODE_GRID")) {
    const long x = std::strtol(v, nullptr, 10);
    if (x > 0) W = x;
  }
  const int64_t bound = static_cast<int64_t>(num_seqs) * p.kv_heads * ((static_cast<int64_t>(max_ctx) + CT - 1) / CT);
  if (W > bound) W = bound;
  if (W > kMaxBalancedGrid) W = kMaxBalancedGrid;
  if (W < 1) W = 1;
  *grid = static_cast<int32_t>(W);
  return hipSuccess;
}

// The merge of partial records; fewer rows than CUs split each row's dims
// over D/16 workgroups.
template <int D, int BS, int G>
void launch_reduce(const DecodeArgs& a, const int32_t* seq_prefix, const int32_t* unit_desc, hipStream_t stream) {
  if (static_cast<int64_t>(a.q_heads) * a.num_seqs < kReduceSplitRows) {
    hipLaunchKernelGGL((decode_reduce_kernel<D, 16, BS>), dim3(a.q_heads, a.num_seqs, D / 16), dim3(kReduceThreads),
                       0, stream, a.out, a.out_dtype, a.part_ml, a.part_o, a.context_lens, seq_prefix, a.max_prefix,
                       a.q_heads, a.max_parts, a.partition_tokens, a.max_context_len, unit_desc, G);
  } else {
    hipLaunchKernelGGL((decode_reduce_kernel<D, D, BS>), dim3(a.q_heads, a.num_seqs, 1), dim3(kReduceThreads), 0,
                       stream, a.out, a.out_dtype, a.part_ml, a.part_o, a.context_lens, seq_prefix, a.max_prefix,
                       a.q_heads, a.max_parts, a.partition_tokens, a.max_context_len, unit_desc, G);
  }
}

template <int DT, int D, int BS, int G>
hipError_t launch_typed(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
  static_assert(decode_chunk_tokens(DT, D, BS, G) == (kUseMfma<DT, BS, G> ? 16 : Chunk<DT, D, BS>::CT),
                "the host's chunk length differs from the kernels'");
  if (a.kv_slots && (a.balanced || a.group_start)) return hipErrorInvalidValue;   // the host writes first there
  if (a.balanced) {
    hipLaunchKernelGGL((decode_balanced_kernel<DT, D, BS, G, kWaves>), dim3(a.grid), dim3(kThreads), 0, stream,
                       static_cast<const char*>(p.k), static_cast<const char*>(p.v), static_cast<const char*>(a.q),
                       a.out, a.out_dtype, a.counters, a.part_ml, a.part_o, a.block_tables, a.table_stride,
                       a.context_lens, a.num_seqs, p.num_blocks, p.kv_heads, a.max_context_len, a.scale_log2);
    return hipGetLastError();
  }
  if (a.uniform) {
    auto kernel = a.kv_slots ? decode_uniform_kernel<DT, D, BS, G, kWaves, true>
                             : decode_uniform_kernel<DT, D, BS, G, kWaves, false>;
    hipLaunchKernelGGL(kernel, dim3(a.grid), dim3(kThreads), 0, stream, static_cast<const char*>(p.k),
                       static_cast<const char*>(p.v), static_cast<const char*>(a.q), a.out, a.out_dtype, a.part_ml,
                       a.part_o, a.unit_desc, a.block_tables, a.table_stride, a.context_lens, a.num_seqs,
                       p.num_blocks, p.kv_heads, a.max_context_len, a.scale_log2, static_cast<const char*>(a.k_new),
                       static_cast<const char*>(a.v_new), a.kv_slots);
    hipError_t e = hipGetLastError();
    // with no more than one workgroup per unit and kv-head nothing splits (uniform_task)
    if (e != hipSuccess || a.grid / p.kv_heads <= a.num_seqs) return e;
    launch_reduce<D, BS, G>(a, nullptr, a.unit_desc, stream);
    return hipGetLastError();
  }
  const bool shared_prefix = a.group_start != nullptr && a.num_groups > 0 && a.max_prefix > 0;
  if (shared_prefix) {
    if constexpr (DT != kF32 && BS >= 16) {
      const int32_t tiles = (a.max_group_size + 16 / G - 1) / (16 / G);
      const int32_t prefix_parts = (a.max_prefix + a.partition_tokens - 1) / a.partition_tokens;
      // an odd count of prefix partitions, for the reason given at the
      // partition kernel's launch below (parts past a prefix return at once)
      hipLaunchKernelGGL((decode_prefix_kernel<DT, D, BS, G, kWaves>),
                         dim3(prefix_parts | 1, p.kv_heads * tiles, a.num_groups), dim3(kThreads), 0, stream,
                         static_cast<const char*>(p.k), static_cast<const char*>(p.v), static_cast<const char*>(a.q),
                         a.part_ml, a.part_o, a.block_tables, a.table_stride, a.context_lens, a.group_start,
                         a.seq_prefix, a.max_prefix, a.num_seqs, p.num_blocks, p.kv_heads, a.max_context_len,
                         a.max_parts, a.partition_tokens, a.scale_log2);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else {
      return hipErrorInvalidValue;   // the host takes the plain path for these pools
    }
  }
  const int32_t* seq_prefix = shared_prefix ? a.seq_prefix : nullptr;
  // partitions of the longest suffix (the whole context without a prefix)
  const int32_t suffix_parts =
      static_cast<int32_t>(std::max<int64_t>(1, (static_cast<int64_t>(a.max_context_len) + a.partition_tokens - 1) /
                                                    a.partition_tokens));
  // Workgroup w runs on XCD w mod 8 and the partition index varies fastest, so
  // with an even count the first partitions of all (sequence, kv-head) units
  // (often the only ones a short context has) would gather on half, a quarter
  // or an eighth of the XCDs.  An odd count spreads them over all eight; the
  // extra column's workgroups return at once, like any partition past a
  // context's end.
  dim3 grid(suffix_parts | 1, p.kv_heads, a.num_seqs);
  auto kernel = a.kv_slots ? decode_partition_kernel<DT, D, BS, G, kWaves, true>
                           : decode_partition_kernel<DT, D, BS, G, kWaves, false>;
  hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, static_cast<const char*>(p.k),
                     static_cast<const char*>(p.v), static_cast<const char*>(a.q), a.out, a.out_dtype, a.part_ml,
                     a.part_o, a.block_tables, a.table_stride, a.context_lens, seq_prefix, a.max_prefix, a.num_seqs,
                     p.num_blocks, p.kv_heads, a.max_context_len, a.max_parts, a.partition_tokens, a.wave_tokens,
                     a.scale_log2, static_cast<const char*>(a.k_new), static_cast<const char*>(a.v_new), a.kv_slots);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || suffix_parts <= 1) return e;
  launch_reduce<D, BS, G>(a, seq_prefix, nullptr, stream);
  return hipGetLastError();
}

// Dispatch on (head_dim, block_size, group) to Fn<DT, D, BS, G>::run(args...).
template <int DT, template <int, int, int, int> class Fn, typename... Args>
hipError_t dispatch(const PoolDesc& p, int32_t group, Args&&... args) {
  auto by_group = [&](auto d_tag, auto bs_tag) -> hipError_t {
    constexpr int D = decltype(d_tag)::value;
    constexpr int BS = decltype(bs_tag)::value;
    switch (group) {
      case 1: return Fn<DT, D, BS, 1>::run(p, args...);
      case 2: return Fn<DT, D, BS, 2>::run(p, args...);
      case 4: return Fn<DT, D, BS, 4>::run(p, args...);
      case 8: return Fn<DT, D, BS, 8>::run(p, args...);
      default: return hipErrorInvalidValue;
    }
  };
  auto by_bs = [&](auto d_tag) -> hipError_t {
    switch (p.block_size) {
      case 4: return by_group(d_tag, std::integral_constant<int, 4>{});
      case 8: return by_group(d_tag, std::integral_constant<int, 8>{});
      case 16: return by_group(d_tag, std::integral_constant<int, 16>{});
      case 32: return by_group(d_tag, std::integral_constant<int, 32>{});
      case 64: return by_group(d_tag, std::integral_constant<int, 64>{});
      default: return hipErrorInvalidValue;
    }
  };
  switch (p.head_dim) {
    case 64: return by_bs(std::integral_constant<int, 64>{});
    case 128: return by_bs(std::integral_constant<int, 128>{});
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D, int BS, int G>
struct LaunchFn {
  static hipError_t run(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
    return launch_typed<DT, D, BS, G>(p, a, stream);
  }
};

template <int DT, int D, int BS, int G>
struct CapacityFn {
  static hipError_t run(const PoolDesc& p, int32_t num_seqs, int32_t max_ctx, DecodeCapacity* cap) {
    static std::atomic<int> partition_cache[64], uniform_cache[64];
    hipError_t e = balanced_grid<DT, D, BS, G>(p, num_seqs, max_ctx, &cap->balanced_grid);
    if (e != hipSuccess) return e;
    e = resident_workgroups(decode_partition_kernel<DT, D, BS, G, kWaves, false>, partition_cache, &cap->partition);
    if (e != hipSuccess) return e;
    return resident_workgroups(decode_uniform_kernel<DT, D, BS, G, kWaves, false>, uniform_cache, &cap->uniform);
  }
};

template <int DT>
hipError_t launch_dtype(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
  return dispatch<DT, LaunchFn>(p, a.q_heads / p.kv_heads, a, stream);
}

template <int DT>
hipError_t capacity_dtype(const PoolDesc& p, int32_t group, int32_t num_seqs, int32_t max_ctx, DecodeCapacity* cap) {
  return dispatch<DT, CapacityFn>(p, group, num_seqs, max_ctx, cap);
}

}  // namespace dec
}  // namespace pa
