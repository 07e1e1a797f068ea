// HIP kernel for gfx950 (CDNA4): prompt-phase attention over the paged KV
// cache. Every query of a prompt attends to the cached tokens up to its own
// position ("PagedAttention 论文精读笔记" §2.1 attention equation, §2.2 prompt
// phase: all prompt tokens at once, a matrix-matrix product), K and V found
// through the sequence's block table.
//
// One wave per (tile, KV head): a tile is qt consecutive queries of one
// sequence, and the 16 columns of the MFMA tiles hold its (query, head) pairs
// of the KV head's group. The wave walks the context in 32-token chunks up to
// the tile's last position with an fp32 online softmax; a chunk's K rows and
// V columns are 16-byte loads straight from the pool, as in decode, and the
// causal limit is a per-column mask. P enters PV as a rounded 16-bit part plus
// its rounding residual (two MFMAs), which keeps the products fp32-accurate.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// Tiles of sequence s; a sequence whose rows do not lie inside
// [0, total_q) in order gets none.
__device__ __forceinline__ int seq_tiles(const PrefillParams& p, int s) {
  const int a = p.q_start[s], b = p.q_start[s + 1];
  return (a >= 0 && b > a && b <= p.total_q) ? (b - a + p.qt - 1) / p.qt : 0;
}

template <int E, int D>
__global__ __launch_bounds__(64) void prefill_kernel(PrefillParams p) {
  using Tr = ElemT<E>;
  using op8 = typename Tr::op8;
  using scalar = typename Tr::scalar;
  using raw = typename Tr::raw;
  constexpr int MQ = D / 32;  // QK k-steps
  constexpr int NT = D / 16;  // PV column tiles
  const int lane = threadIdx.x, col = lane & 15, grp = lane >> 4;
  const int kvh = blockIdx.y, g = p.group, qt = p.qt, Hq = p.num_heads, Hkv = p.num_kv_heads;

  // tile map: every wave scans the query counts (the longest tiles, the last
  // of each sequence, are handed out first)
  const int S = p.num_seqs;
  const int per = (S + 63) >> 6;
  const int s_lo = min(lane * per, S), s_hi = min(s_lo + per, S);
  int mine = 0;
  for (int s = s_lo; s < s_hi; ++s) mine += seq_tiles(p, s);
  int incl = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  const int T = __shfl(incl, 63);
  const int excl = incl - mine;
  const int x = blockIdx.x;
  if (x >= T) return;
  const int tile = T - 1 - x;
  const unsigned long long ball = __ballot(tile >= excl && tile < incl);
  if (ball == 0) return;  // counts past int range only
  const int owner = __builtin_ctzll(ball);
  int s_found = 0, k_found = 0;
  if (lane == owner) {
    int c = excl;
    for (int s = s_lo; s < s_hi; ++s) {
      const int nt = seq_tiles(p, s);
      if (tile < c + nt) {
        s_found = s;
        k_found = tile - c;
        break;
      }
      c += nt;
    }
  }
  const int s = __builtin_amdgcn_readfirstlane(__shfl(s_found, owner));
  const int k = __builtin_amdgcn_readfirstlane(__shfl(k_found, owner));
  if (k >= seq_tiles(p, s)) return;
  const int q0 = p.q_start[s], n = p.q_start[s + 1] - q0, L = p.context_lens[s];
  if (n > L || L > (p.max_blocks_per_seq << p.log2_block)) return;  // precondition violated
  const int j0 = k * qt, nq = min(qt, n - j0);
  const int pos0 = L - n + j0, p_max = pos0 + nq - 1;

  // column (query qi, head hh); columns past the tile read q = 0 at p_max
  const int qi = col / g, hh = col - qi * g;
  const bool cvalid = qi < nq;
  const int pcol = cvalid ? pos0 + qi : p_max;
  op8 qop[MQ];
  {
    const raw* qrow = static_cast<const raw*>(p.q) + ((size_t)(q0 + j0 + (cvalid ? qi : 0)) * Hq + kvh * g + hh) * D;
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (cvalid) w = load16(qrow + 32 * m + 8 * grp);
      qop[m] = __builtin_bit_cast(op8, w);
    }
  }

  const int lg = p.log2_block, B = p.block_size;
  const int32_t* tbl = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  const int lbl = p_max >> lg;
  const int nch = p_max / kChunk + 1;
  const raw* __restrict__ kc = static_cast<const raw*>(p.k_cache);
  const raw* __restrict__ vc = static_cast<const raw*>(p.v_cache);

  u32x4 ka[2][MQ], vr[NT];
  auto load_k = [&](int cs, const ChunkIds& ids) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int tok = cs + 8 * (col >> 2) + 4 * c + (col & 3);
      const int phys = pick_block(ids, tok, lg, lbl, p.num_blocks);
      const raw* row = kc + (((size_t)phys * Hkv + kvh) * B + (tok & (B - 1))) * D + 8 * grp;
#pragma unroll
      for (int m = 0; m < MQ; ++m) ka[c][m] = load16(row + 32 * m);
    }
  };
  auto load_v = [&](int cs, const ChunkIds& ids) {
    const int tv = cs + 8 * grp;
    const int physv = pick_block(ids, tv, lg, lbl, p.num_blocks);
    const raw* vb = vc + (((size_t)physv * Hkv + kvh) * D + col) * B + (tv & (B - 1));
#pragma unroll
    for (int j = 0; j < NT; ++j) vr[j] = load16(vb + (size_t)16 * j * B);
  };

  ChunkIds ids1 = load_chunk_ids(tbl, min(1, nch - 1) * kChunk, lbl, lg);
  {
    const ChunkIds ids0 = load_chunk_ids(tbl, 0, lbl, lg);
    load_k(0, ids0);
    load_v(0, ids0);
  }
  f32x4 o[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  for (int ci = 0; ci < nch; ++ci) {
    const int cs = ci * kChunk;
    const int cs_next = min(ci + 1, nch - 1) * kChunk;
    const ChunkIds ids2 = load_chunk_ids(tbl, min(ci + 2, nch - 1) * kChunk, lbl, lg);
    // scores: the lane holds tokens cs + 8*grp + 0..7 of column `col`
    f32x4 sc0 = f32x4{0.f, 0.f, 0.f, 0.f}, sc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      sc0 = mfma_16x16x32(__builtin_bit_cast(op8, ka[0][m]), qop[m], sc0);
      sc1 = mfma_16x16x32(__builtin_bit_cast(op8, ka[1][m]), qop[m], sc1);
    }
    load_k(cs_next, ids1);  // unconditional: the last chunk re-reads itself
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = sc0[i] * p.scale_log2;
      sv[4 + i] = sc1[i] * p.scale_log2;
    }
    if (cs + kChunk - 1 > pos0) {  // causal limit inside this chunk
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = (cs + 8 * grp + e <= pcol) ? sv[e] : kNegInf;
    }
    float cmax = kNegInf;
#pragma unroll
    for (int e = 0; e < 8; ++e) cmax = fmaxf(cmax, sv[e]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = fast_exp2(m_run - m_new);
    float pe[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = fast_exp2(sv[e] - m_new);
      psum += pe[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
      // output rows of this lane are columns 4*grp+i; their factor lives in lane 4*grp+i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * grp + i);
#pragma unroll
        for (int j = 0; j < NT; ++j) o[j][i] *= ai;
      }
    }
    op8 phi, plo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const scalar hi = static_cast<scalar>(pe[e]);
      phi[e] = hi;
      plo[e] = static_cast<scalar>(pe[e] - static_cast<float>(hi));
    }
    if (cs + kChunk - 1 > p_max) {  // tokens past the tile's last position: no V
      const int nvalid = p_max + 1 - (cs + 8 * grp);
#pragma unroll
      for (int j = 0; j < NT; ++j) vr[j] = Tr::keep_first(vr[j], nvalid);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      o[j] = mfma_16x16x32(phi, __builtin_bit_cast(op8, vr[j]), o[j]);
      o[j] = mfma_16x16x32(plo, __builtin_bit_cast(op8, vr[j]), o[j]);
    }
    load_v(cs_next, ids1);
    ids1 = ids2;
  }

  // rows of this lane: columns r = 4*grp + i, i.e. query r / g, head r % g
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * grp + i;
    const float lr = __shfl(l_tot, r);
    const int qr = r / g;
    if (qr < nq) {
      const size_t base = ((size_t)(q0 + j0 + qr) * Hq + kvh * g + (r - qr * g)) * D + col;
#pragma unroll
      for (int j = 0; j < NT; ++j) store_out(p.out, base + 16 * j, o[j][i] / lr, p.out_dtype);
    }
  }
}

const void* prefill_fn(int elem, int head_dim) {
  if (elem == kBF16) return head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<kBF16, 64>)
                                           : reinterpret_cast<const void*>(&prefill_kernel<kBF16, 128>);
  if (elem == kF16) return head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<kF16, 64>)
                                          : reinterpret_cast<const void*>(&prefill_kernel<kF16, 128>);
  return nullptr;
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int elem, int head_dim, unsigned tiles, hipStream_t stream) {
  const void* fn = prefill_fn(elem, head_dim);
  if (!fn) return hipErrorInvalidDeviceFunction;
  PrefillParams args = p;
  void* kargs[] = {&args};
  return hipLaunchKernel(fn, dim3(tiles, (unsigned)p.num_kv_heads, 1), dim3(64, 1, 1), kargs, 0, stream);
}

}  // namespace pa
