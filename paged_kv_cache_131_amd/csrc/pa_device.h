// Device helpers shared by the HIP kernels of libpagedattn (decode, write,
// copy, swap, prefill): element types and their MFMA operands, 16-byte
// loads, output rounding and the block-table lookups of one 32-token chunk.
// Included by each .hip source into its own anonymous namespace.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ u32x4 load16(const void* ptr) {
  return *reinterpret_cast<const u32x4*>(ptr);
}

// K/V tiles are read exactly once per launch: stream them past the caches.
__device__ __forceinline__ u32x4 load16_stream(const void* ptr) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max and sum of x over lanes l, l^16, l^32, l^48 (the four lanes holding
// one MFMA column), by lane-swap instructions (no LDS round trip).
__device__ __forceinline__ float max_over_column(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_column(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// x of the lane picked by a DPP control within the lane's row of 16.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// x combined (sum, or max when MAX) over aligned groups of N consecutive
// lanes, N = 4, 8, 16, 32 or 64; every lane of a group gets the group's value,
// bit-identical across the group (each step adds the two halves in either
// order). Within a row of 16: quad_perm [1,0,3,2] and [2,3,0,1] (lane ^ 1,
// lane ^ 2), row_half_mirror (the other quad of the eight) and row_mirror
// (the other eight); across rows the lane-swap instructions. No LDS.
template <int N, bool MAX = false>
__device__ __forceinline__ float reduce_lanes(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group of 4 to 64 lanes");
  const auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  x = op(x, dpp_f<0xB1>(x));
  x = op(x, dpp_f<0x4E>(x));
  if constexpr (N >= 8) x = op(x, dpp_f<0x141>(x));
  if constexpr (N >= 16) x = op(x, dpp_f<0x140>(x));
  if constexpr (N >= 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  }
  if constexpr (N >= 64) {
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
  return x;
}

// V tiles are stored as sub-tiles [block_size/Bs][head_dim][Bs]: Bs = 32 for
// a block_size that is a multiple of 32 above 32, else Bs = block_size (a
// plain [head_dim][block_size] tile). The element of channel c and in-block
// token t of (block, KV head) lies at the offset v_elem(...) below; channel
// c + 1 of the same token is Bs elements further.
__device__ __forceinline__ int v_subtile(int block_size) {
  return (block_size > 32 && (block_size & 31) == 0) ? 32 : block_size;
}

__device__ __forceinline__ size_t v_elem(int block, int num_kv_heads, int kv_head, int head_dim, int block_size,
                                         int Bs, int c, int t) {
  return ((size_t)block * num_kv_heads + kv_head) * head_dim * block_size + ((size_t)(t / Bs) * head_dim + c) * Bs +
         (t % Bs);
}

// ---------------------------------------------------------------------------
// Element types
// ---------------------------------------------------------------------------
template <int E>
struct ElemT;

template <>
struct ElemT<kF32> {
  using raw = uint32_t;
  static constexpr int kVec = 4;  // elements per 16 bytes
  __device__ static void widen(u32x4 w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
  // zero the elements of tokens >= nvalid (one token per element)
  __device__ static u32x4 keep_first(u32x4 w, int nvalid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = i < nvalid ? w[i] : 0u;
    return w;
  }
};

template <>
struct ElemT<kF16> {
  using raw = uint16_t;
  using op8 = f16x8;
  using scalar = _Float16;
  static constexpr int kVec = 8;
  __device__ static void widen(u32x4 w, float* f) {
    const f16x8 h = __builtin_bit_cast(f16x8, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(h[i]);
  }
  __device__ static u32x4 keep_first(u32x4 w, int nvalid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t m = 2 * i + 1 < nvalid ? 0xffffffffu : (2 * i < nvalid ? 0x0000ffffu : 0u);
      w[i] &= m;
    }
    return w;
  }
  // c + the dot product of the 8 elements of a and b: four two-element dot
  // instructions (16-bit products are exact in fp32, accumulated in fp32).
  // Each pair is copied out of the vector before the bit cast: a bit cast
  // of the subscripted element itself was compiled as a cast of element 0
  // for every i (hipcc of ROCm 7.2).
  __device__ static float dot8(u32x4 a, u32x4 b, float c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = a[i], y = b[i];
      c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), c, false);
    }
    return c;
  }
  // p = hi + lo: hi the nearest 16-bit values, lo the residuals rounded
  __device__ static void split(const float* p, op8& hi, op8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const _Float16 h = static_cast<_Float16>(p[e]);
      hi[e] = h;
      lo[e] = static_cast<_Float16>(p[e] - static_cast<float>(h));
    }
  }
};

template <>
struct ElemT<kBF16> {
  using raw = uint16_t;
  using op8 = bf16x8;
  using scalar = __bf16;
  static constexpr int kVec = 8;
  __device__ static void widen(u32x4 w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static u32x4 keep_first(u32x4 w, int nvalid) { return ElemT<kF16>::keep_first(w, nvalid); }
  // as ElemT<kF16>::dot8
  __device__ static float dot8(u32x4 a, u32x4 b, float c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = a[i], y = b[i];
      c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), c, false);
    }
    return c;
  }
  // p = hi + lo: hi the nearest bf16 values (one packed conversion per pair,
  // unpacked by shifts), lo the residuals rounded
  __device__ static void split(const float* p, op8& hi, op8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t hh = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{p[2 * i], p[2 * i + 1]}), bf16x2));
      const float r0 = p[2 * i] - __uint_as_float(hh << 16);
      const float r1 = p[2 * i + 1] - __uint_as_float(hh & 0xffff0000u);
      h[i] = hh;
      l[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r0, r1}), bf16x2));
    }
    hi = __builtin_bit_cast(op8, h);
    lo = __builtin_bit_cast(op8, l);
  }
};

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void store_out(void* out, size_t idx, float v, int out_dtype) {
  if (out_dtype == kF32) {
    static_cast<float*>(out)[idx] = v;
  } else if (out_dtype == kF16) {
    static_cast<_Float16*>(out)[idx] = static_cast<_Float16>(v);
  } else {
    static_cast<__bf16*>(out)[idx] = static_cast<__bf16>(v);
  }
}

// Four consecutive outputs (idx a multiple of 4) converted one by one as
// store_out does; `vec`: `out` is aligned for one 16-byte (fp32) or 8-byte
// (16-bit) store of the four.
__device__ __forceinline__ void store_out4(void* out, size_t idx, f32x4 v, int out_dtype, bool vec) {
  if (!vec) {
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(out, idx + e, v[e], out_dtype);
  } else if (out_dtype == kF32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = v;
  } else {
    uint16_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      h[e] = out_dtype == kF16 ? __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[e]))
                               : __builtin_bit_cast(uint16_t, static_cast<__bf16>(v[e]));
    uint2 w;
    w.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    w.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = w;
  }
}

// ---------------------------------------------------------------------------
// Block-table lookups for one 32-token chunk. A chunk spans at most four
// blocks (block_size >= 8); ids are read with wave-uniform addresses and the
// logical block is clamped to the segment's last block, so tokens past the
// context never index past the table's valid entries. Ids are clamped into
// the pool.
// ---------------------------------------------------------------------------
struct ChunkIds {
  int lb0;
  int id0, id1, id2, id3;
};

// The block table is read-only for the whole launch; reading it through the
// constant address space lets wave-uniform reads use scalar loads, which are
// counted apart from the K/V vector loads in flight.
typedef const __attribute__((address_space(4))) int32_t const_i32;

__device__ __forceinline__ int table_entry(const int32_t* tbl, int lb, int lbl) {
  const const_i32* t = (const const_i32*)tbl;
  return t[min(lb, lbl)];
}

// Raw entries of the (up to four) blocks of the chunk starting at `cs`,
// loaded unconditionally and used (clamped) only when picked, so the loads
// stay in flight until then.
__device__ __forceinline__ ChunkIds load_chunk_ids(const int32_t* tbl, int cs, int lbl, int log2_block) {
  ChunkIds c;
  c.lb0 = cs >> log2_block;
  c.id0 = table_entry(tbl, c.lb0, lbl);
  c.id1 = table_entry(tbl, c.lb0 + 1, lbl);
  c.id2 = table_entry(tbl, c.lb0 + 2, lbl);
  c.id3 = table_entry(tbl, c.lb0 + 3, lbl);
  return c;
}

// The table entry of token tok's block, as stored.
__device__ __forceinline__ int pick_entry(ChunkIds c, int tok, int log2_block, int lbl) {
  const int k = min(tok >> log2_block, lbl) - c.lb0;
  int id = c.id0;
  id = k >= 1 ? c.id1 : id;
  id = k >= 2 ? c.id2 : id;
  id = k >= 3 ? c.id3 : id;
  return id;
}

__device__ __forceinline__ int pick_block(ChunkIds c, int tok, int log2_block, int lbl, int num_blocks) {
  return min(max(pick_entry(c, tok, log2_block, lbl), 0), num_blocks - 1);
}

}  // namespace
}  // namespace pa
