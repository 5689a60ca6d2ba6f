// Paged single-query decode attention for gfx950 (CDNA4), split-K over the
// context.  Included by decode_<dtype>.hip, one translation unit per storage
// type so the instantiations compile in parallel.
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
//   * Work unit = (sequence, kv-head, partition of P tokens).  One workgroup of
//     NW wave64s per unit; the G = q_heads/kv_heads query rows of the kv-head
//     stay in registers, so K and V of the unit are read from HBM exactly once.
//   * A token row (head_dim elements) is spread over LPT lanes with 16 bytes
//     per lane, so one wave-wide global_load_dwordx4 moves 1 KiB: TPL = 64/LPT
//     consecutive tokens of one contiguous (block, kv-head) tile.
//   * Each LPT-lane group keeps its own running max/sum/output for the tokens
//     it loads, so the hot loop needs no cross-group traffic: scores are
//     reduced inside the group with DPP row rotations fused into v_add
//     (v_dot2 for fp16/bf16 products), groups and waves are merged once per
//     unit at the end.
//   * Loads of the next block are issued before the current block is consumed
//     (two register buffers), keeping ~2 KiB per lane-group of K/V in flight.
//   * Softmax runs in base 2: scores carry scale·log2(e) and v_exp_f32 does
//     2^x.
//   * A unit that holds a whole sequence writes the normalised output; longer
//     sequences write fp32 (max, sum, unnormalised output) per partition and
//     decode_reduce_kernel merges them.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace pa {
namespace dec {

constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so 2^(m - m') never sees inf - inf

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

// ---------------------------------------------------------------------------
// decode_partition_kernel
//   grid  = (max_parts, kv_heads, num_seqs), block = NW × 64 threads
//   Unit (s, g, p) covers tokens [p·P, min((p+1)·P, len_s)) of sequence s,
//   kv-head g, and the G query heads g·G … g·G+G-1.
// ---------------------------------------------------------------------------
template <int DT, int D, int BS, int G, int NW>
__global__ __launch_bounds__(NW * 64) void decode_partition_kernel(
    const char* __restrict__ k_pool, const char* __restrict__ v_pool, const char* __restrict__ q,
    void* __restrict__ out, int32_t out_dtype, float* __restrict__ part_ml, float* __restrict__ part_o,
    const int32_t* __restrict__ block_tables, int32_t table_stride, const int32_t* __restrict__ context_lens,
    int32_t num_blocks, int32_t kv_heads, int32_t max_ctx, int32_t max_parts, int32_t part_tokens,
    float scale_log2) {
  using S = Shape<DT, D>;
  constexpr int ELEMS = S::ELEMS, LPT = S::LPT, TPL = S::TPL, ROW = S::ROW;
  // A chunk is NLC wave-wide loads per tensor.  Blocks of ≥ TPL tokens: four
  // loads (TPL-token groups never straddle a block, as both are powers of
  // two).  Smaller blocks: one load whose lane groups find their own blocks.
  constexpr bool kSmallBlocks = BS < TPL;
  constexpr int NLC = kSmallBlocks ? 1 : 4;
  constexpr int CT = NLC * TPL;              // tokens per chunk
  constexpr int64_t TILE = static_cast<int64_t>(BS) * ROW;

  const int p = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int q_heads = kv_heads * G;

  const int32_t len = context_lens[s];
  const bool bad_len = len < 0 || len > max_ctx;
  const int32_t len_c = bad_len ? 0 : len;
  const int32_t nparts = len_c <= part_tokens ? 1 : (len_c + part_tokens - 1) / part_tokens;
  if (p >= nparts) return;

  const int32_t t_begin = p * part_tokens;
  const int32_t t_end = min(t_begin + part_tokens, len_c);
  const int32_t nchunks = (t_end - t_begin + CT - 1) / CT;
  const int32_t* table = block_tables + static_cast<int64_t>(s) * table_stride;

  const int grp = lane / LPT;     // which token of a wave-wide load this lane reads
  const int sub = lane % LPT;     // which 16-byte slice of the row
  const int32_t lane_off = grp * ROW + sub * 16;

  // query rows of this kv-head: 16 bytes per lane per row
  uint4 qv[G];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const int h = g * G + r;
    qv[r] = *reinterpret_cast<const uint4*>(q + ((static_cast<int64_t>(s) * q_heads + h) * D) * S::EB + sub * 16);
  }

  float m[G], l[G], o[G][ELEMS];
#pragma unroll
  for (int r = 0; r < G; ++r) {
    m[r] = kNegBig;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < ELEMS; ++e) o[r][e] = 0.f;
  }
  bool bad_block = false;

  auto lookup = [&](int32_t t) {
    int32_t phys = table[t / BS];
    if (static_cast<uint32_t>(phys) >= static_cast<uint32_t>(num_blocks)) {
      bad_block = true;
      phys = 0;
    }
    return (static_cast<int64_t>(phys) * kv_heads + g) * TILE;
  };

  // Issue the loads of chunk c (K and V, NLC wave-wide 16-byte loads each).
  // Every address stays inside an allocated block; padding slots past the
  // context may be read but their lanes are masked before use.
  auto load_chunk = [&](int32_t c, uint4 (&kb)[NLC], uint4 (&vb)[NLC]) {
    const int32_t tok0 = t_begin + c * CT;
    if constexpr (!kSmallBlocks) {
      if constexpr (BS >= CT) {
        const int64_t tile = lookup(tok0) + (tok0 % BS) * ROW;
        const char* kt = k_pool + tile;
        const char* vt = v_pool + tile;
#pragma unroll
        for (int i = 0; i < NLC; ++i) {
          kb[i] = *reinterpret_cast<const uint4*>(kt + lane_off + i * TPL * ROW);
          vb[i] = *reinterpret_cast<const uint4*>(vt + lane_off + i * TPL * ROW);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NLC; ++i) {
          // a load starting past the partition end re-reads the chunk's first
          // group (always inside an allocated block); its lanes are masked
          const int32_t t = tok0 + i * TPL < t_end ? tok0 + i * TPL : tok0;
          const int64_t tile = lookup(t) + (t % BS) * ROW;
          kb[i] = *reinterpret_cast<const uint4*>(k_pool + tile + lane_off);
          vb[i] = *reinterpret_cast<const uint4*>(v_pool + tile + lane_off);
        }
      }
    } else {
      int32_t t = tok0 + grp;
      if (t >= t_end) t = t_end - 1;
      const int64_t off = lookup(t) + (t % BS) * ROW + sub * 16;
      kb[0] = *reinterpret_cast<const uint4*>(k_pool + off);
      vb[0] = *reinterpret_cast<const uint4*>(v_pool + off);
    }
  };

  // Fold chunk c into the running (m, l, o) of this lane group.
  auto consume_chunk = [&](int32_t c, uint4 (&kb)[NLC], uint4 (&vb)[NLC]) {
    const int32_t tok0 = t_begin + c * CT;
    const bool full = tok0 + CT <= t_end;
    bool valid[NLC];
#pragma unroll
    for (int i = 0; i < NLC; ++i) {
      valid[i] = full || (tok0 + grp + i * TPL < t_end);
      if (!valid[i]) vb[i] = make_uint4(0u, 0u, 0u, 0u);  // padding may hold NaN: never multiply it
    }
    float vf[NLC][ELEMS];
#pragma unroll
    for (int i = 0; i < NLC; ++i) unpack<DT>(vb[i], vf[i]);
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

  // Chunks wave, wave+NW, wave+2NW, … with the next chunk's loads in flight.
  {
    uint4 ka[NLC], va[NLC], kb2[NLC], vb2[NLC];
    int32_t c = wave;
    if (c < nchunks) load_chunk(c, ka, va);
    for (; c < nchunks; c += 2 * NW) {
      if (c + NW < nchunks) load_chunk(c + NW, kb2, vb2);
      consume_chunk(c, ka, va);
      if (c + NW >= nchunks) break;
      if (c + 2 * NW < nchunks) load_chunk(c + 2 * NW, ka, va);
      consume_chunk(c + NW, kb2, vb2);
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

  // Merge the NW waves through LDS and write the unit's result.
  __shared__ float sh_o[NW][G][D];
  __shared__ float sh_m[NW][G];
  __shared__ float sh_l[NW][G];
  __shared__ int sh_bad[NW];
  if (lane < LPT) {
#pragma unroll
    for (int r = 0; r < G; ++r) {
#pragma unroll
      for (int e = 0; e < ELEMS; ++e) sh_o[wave][r][sub * ELEMS + e] = o[r][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < G; ++r) {
      sh_m[wave][r] = m[r];
      sh_l[wave][r] = l[r];
    }
  }
  const bool wave_bad = __any(bad_block);
  if (lane == 0) sh_bad[wave] = wave_bad ? 1 : 0;
  __syncthreads();
  bool bad = bad_len;
#pragma unroll
  for (int w = 0; w < NW; ++w) bad = bad || sh_bad[w] != 0;
  const float nan = __uint_as_float(0x7fc00000u);
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int r = idx / D;
    const int d = idx - r * D;
    float mm = kNegBig;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, sh_m[w][r]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = exp2f_fast(sh_m[w][r] - mm);
      L += sh_l[w][r] * a;
      O += sh_o[w][r][d] * a;
    }
    const int h = g * G + r;
    const int64_t row = static_cast<int64_t>(s) * q_heads + h;
    if (nparts == 1) {
      const float x = bad ? nan : (L > 0.f ? O / L : 0.f);
      store_out(out, out_dtype, row * D + d, x);
    } else {
      const int64_t prow = row * max_parts + p;
      part_o[prow * D + d] = bad ? nan : O;
      if (d == 0) {
        part_ml[2 * prow] = mm;
        part_ml[2 * prow + 1] = L;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode_reduce_kernel: merge the partitions of sequences longer than one.
//   grid = (D / 32, q_heads, num_seqs), block = 256 = 32 dims × 8 partition lanes
//   out = Σ_p 2^(m_p − M) o_p / Σ_p 2^(m_p − M) l_p with M = max_p m_p.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(void* __restrict__ out, int32_t out_dtype,
                                                            const float* __restrict__ part_ml,
                                                            const float* __restrict__ part_o,
                                                            const int32_t* __restrict__ context_lens,
                                                            int32_t q_heads, int32_t max_parts,
                                                            int32_t part_tokens, int32_t max_ctx) {
  const int s = blockIdx.z;
  const int h = blockIdx.y;
  const int32_t len = context_lens[s];
  const bool bad_len = len < 0 || len > max_ctx;
  const int32_t len_c = bad_len ? 0 : len;
  const int32_t nparts = len_c <= part_tokens ? 1 : (len_c + part_tokens - 1) / part_tokens;
  if (nparts == 1) return;  // written by the partition kernel (NaN rows included)
  const int64_t row = static_cast<int64_t>(s) * q_heads + h;
  const float* ml = part_ml + row * max_parts * 2;
  const float* po = part_o + row * max_parts * D;

  __shared__ float sh_red[256];
  // M = max over partitions
  float mm = kNegBig;
  for (int pp = threadIdx.x; pp < nparts; pp += 256) mm = fmaxf(mm, ml[2 * pp]);
  sh_red[threadIdx.x] = mm;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh_red[threadIdx.x] = fmaxf(sh_red[threadIdx.x], sh_red[threadIdx.x + w]);
    __syncthreads();
  }
  mm = sh_red[0];
  __syncthreads();
  // L = Σ l_p 2^(m_p - M)
  float L = 0.f;
  for (int pp = threadIdx.x; pp < nparts; pp += 256) L += ml[2 * pp + 1] * exp2f_fast(ml[2 * pp] - mm);
  sh_red[threadIdx.x] = L;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh_red[threadIdx.x] += sh_red[threadIdx.x + w];
    __syncthreads();
  }
  L = sh_red[0];
  __syncthreads();
  // O[d] = Σ_p 2^(m_p - M) o_p[d], partitions strided over 8 lanes groups
  const int dl = threadIdx.x & 31;
  const int pl = threadIdx.x >> 5;
  const int d = blockIdx.x * 32 + dl;
  float acc = 0.f;
  for (int pp = pl; pp < nparts; pp += 8) acc += po[static_cast<int64_t>(pp) * D + d] * exp2f_fast(ml[2 * pp] - mm);
  sh_red[threadIdx.x] = acc;
  __syncthreads();
  if (pl == 0) {
    float O = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) O += sh_red[k * 32 + dl];
    const float x = bad_len ? __uint_as_float(0x7fc00000u) : (L > 0.f ? O / L : 0.f);
    store_out(out, out_dtype, row * D + d, x);
  }
}

constexpr int kWaves = 4;

template <int DT, int D, int BS, int G>
hipError_t launch_typed(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.max_parts, p.kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<DT, D, BS, G, kWaves>), grid, dim3(kWaves * 64), 0, stream,
                     static_cast<const char*>(p.k), static_cast<const char*>(p.v),
                     static_cast<const char*>(a.q), a.out, a.out_dtype, a.part_ml, a.part_o, a.block_tables,
                     a.table_stride, a.context_lens, p.num_blocks, p.kv_heads, a.max_context_len, a.max_parts,
                     a.partition_tokens, a.scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(D / 32, a.q_heads, a.num_seqs), dim3(256), 0, stream, a.out,
                     a.out_dtype, a.part_ml, a.part_o, a.context_lens, a.q_heads, a.max_parts,
                     a.partition_tokens, a.max_context_len);
  return hipGetLastError();
}

template <int DT, int D, int BS>
hipError_t launch_group(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
  switch (a.q_heads / p.kv_heads) {
    case 1: return launch_typed<DT, D, BS, 1>(p, a, stream);
    case 2: return launch_typed<DT, D, BS, 2>(p, a, stream);
    case 4: return launch_typed<DT, D, BS, 4>(p, a, stream);
    case 8: return launch_typed<DT, D, BS, 8>(p, a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT, int D>
hipError_t launch_bs(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
  switch (p.block_size) {
    case 4: return launch_group<DT, D, 4>(p, a, stream);
    case 8: return launch_group<DT, D, 8>(p, a, stream);
    case 16: return launch_group<DT, D, 16>(p, a, stream);
    case 32: return launch_group<DT, D, 32>(p, a, stream);
    case 64: return launch_group<DT, D, 64>(p, a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_dtype(const PoolDesc& p, const DecodeArgs& a, hipStream_t stream) {
  switch (p.head_dim) {
    case 64: return launch_bs<DT, 64>(p, a, stream);
    case 128: return launch_bs<DT, 128>(p, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dec
}  // namespace pa
