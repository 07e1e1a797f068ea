// HIP kernel for gfx950 (CDNA4): prompt-phase attention over the paged KV
// cache. Every query of a prompt attends to the cached tokens up to its own
// position ("PagedAttention 论文精读笔记" §2.1 attention equation, §2.2 prompt
// phase: all prompt tokens at once, a matrix-matrix product), K and V found
// through the sequence's block table.
//
// A workgroup of four waves takes a tile of consecutive queries of one
// sequence and one KV head. The context is walked in 32-token chunks up to the
// tile's last position; each chunk's K rows and V columns are brought into a
// three-stage LDS ring by direct global-to-LDS loads, a quarter per wave, two
// chunks ahead of use, so the four waves share one copy of every K/V byte.
// Each wave owns NG groups of 16 MFMA columns, a column being one (query, head)
// pair of the KV head's group; QK^T and PV are 16x16x32 MFMAs whose operands
// come from the ring, with an fp32 online softmax between them and the causal
// limit as a per-column mask. P enters PV as a rounded 16-bit part plus its
// rounding residual (two MFMAs), which keeps the products fp32-accurate.
//
// LDS layout of one stage, in 16-byte units, swizzled for conflict-free
// operand reads. A 16-byte LDS read of 64 lanes is served in four passes of
// 16 lanes, grouped by lane bit 5 and the parity of lane bits 2-4 (measured on
// gfx950 with SQ_LDS_BANK_CONFLICT over patterns that tell the groupings
// apart); a pass costs one cycle when its 16 lanes fall in distinct 16-byte
// bank groups (64 four-byte banks), one more per extra lane in a group.
//   K: token t of the chunk, head-dim segment s (8 elements) at unit
//      t * D/8 + (s ^ fk(t));
//   V, after K's 32*D/8 units: channel c, token group u (8 tokens) at unit
//      c * 4 + (u ^ fv(c)). (In the pool a chunk's V is one 32-token
//      sub-tile [head_dim][32] of its block, or several whole blocks.)

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPrefillWaves = 4;
// 16-column groups per wave: two at head_dim 128 (the K and V operands read
// from LDS serve twice the columns; 190 VGPRs, two waves per SIMD; +17% at 32
// query / 8 KV heads, +1 to +11% at groups 1, 2, 3, 8), one at head_dim 64
// (two lost 6% at 32/8 heads).
template <int D>
constexpr int prefill_groups() { return D == 128 ? 2 : 1; }
constexpr float kRescaleSlack = 8.f;  // log2 units

typedef __attribute__((address_space(3))) const void lds_void;

// One LDS array per ring stage.
template <int S, int D>
__device__ __forceinline__ uint16_t* stage_buf() {
  __shared__ __attribute__((aligned(16))) uint16_t buf[2 * kChunk * D];
  return buf;
}

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes bytes [16 l, 16 l + 16) from LDS byte address `lds` on (M0 holds the
// wave's base). Issued as inline assembly so that the compiler does not track
// it: its own waits would otherwise drain every ring load before any LDS
// read. The ring's explicit waits (wait_and_barrier) cover these loads.
// M0 is reserved to the compiler, which warns that it may not honour the
// clobber (the build silences that warning for this file); no code it
// generates for this kernel reads M0, and each load sets it itself.
__device__ __forceinline__ void load_lds16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}
// The same from a wave-uniform base plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void load_lds16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)p);
}

__device__ __forceinline__ int k_swizzle(int t, int D) { return ((t & 3) | ((t >> 1) & 12)) & (D / 8 - 1); }
// V: the four 8-token groups of channel c are permuted by bit 2 of c. With the
// previous (c >> 2) & 3, two lanes of every pass shared a bank group (57M
// conflict cycles per launch of the 32-prompt batch; 5M now, all in the
// output staging, which has since been fixed too).
__device__ __forceinline__ int v_swizzle(int c) { return (c >> 1) & 2; }

// Wait until at most N of this wave's vector memory operations are in flight,
// then meet the other waves; LDS accesses are not moved across it.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Tiles of sequence s; a sequence whose rows do not lie inside
// [0, total_q) in order gets none.
__device__ __forceinline__ int seq_tiles(const PrefillParams& p, int s, int qb) {
  const int a = p.q_start[s], b = p.q_start[s + 1];
  return (a >= 0 && b > a && b <= p.total_q) ? (b - a + qb - 1) / qb : 0;
}

template <int E, int D, int NG>
struct PrefillTile {
  using Tr = ElemT<E>;
  using op8 = typename Tr::op8;
  using scalar = typename Tr::scalar;
  using raw = typename Tr::raw;
  static constexpr int MQ = D / 32;                        // QK k-steps
  static constexpr int NT = D / 16;                        // PV column tiles
  static constexpr int KU = kChunk * D / 8;                // 16-byte units of K (and of V) per chunk
  static constexpr int LPW = 2 * KU / 64 / kPrefillWaves;  // direct loads per wave per chunk

  const PrefillParams& p;
  int lane, col, grp, wave, kvh;
  const int32_t* tbl;
  int lbl, p_last, nch;
  // ring loads: this wave's instructions, per lane the byte offset inside the
  // block (without the chunk's offset) and, for V, which of the chunk's blocks
  uint32_t block_bytes;
  uint32_t k_off[LPW / 2];
  int k_blk[LPW / 2];
  const char* v_src[LPW / 2];  // V: the lane's address in block 0 of the pool
  bool v_ge1[LPW / 2], v_ge2[LPW / 2], v_ge3[LPW / 2];  // V: block index >= 1, 2, 3
  int pos_w, last_w;  // first position and last chunk of this wave's queries (-1: none)
  op8 qop[NG][MQ];
  int pcol[NG];
  f32x4 o[NG][NT];
  float m_run[NG], l_run[NG];

  __device__ explicit PrefillTile(const PrefillParams& pp) : p(pp) {}

  // Loop-invariant parts of the ring loads. K instruction i covers whole
  // tokens (64 units, 4 or 8 tokens), so it reads one block; a V instruction
  // spans the chunk's 32 tokens, so each lane finds its own block.
  __device__ void init_loads() {
    const int lg = p.log2_block, B = p.block_size;
    block_bytes = (uint32_t)p.num_kv_heads * (uint32_t)B * D * 2u;
#pragma unroll
    for (int ii = 0; ii < LPW / 2; ++ii) {
      const int i = wave * (LPW / 2) + ii;
      const int u = i * 64 + lane;
      const int t = u / (D / 8);
      const int seg = (u % (D / 8)) ^ k_swizzle(t, D);
      k_off[ii] = (uint32_t)(((kvh * B + (t & (B - 1))) * D + 8 * seg) * 2);
      k_blk[ii] = __builtin_amdgcn_readfirstlane((i * 64 / (D / 8)) >> lg);
      const int c = u >> 2;
      const int tg = (u & 3) ^ v_swizzle(c);
      const int Bs = v_subtile(B);  // V sub-tiles: channel stride Bs
      v_src[ii] = static_cast<const char*>(p.v_cache) + ((size_t)kvh * D * B + c * Bs + ((8 * tg) & (Bs - 1))) * 2;
      const int vb = (8 * tg) >> lg;
      v_ge1[ii] = vb >= 1;
      v_ge2[ii] = vb >= 2;
      v_ge3[ii] = vb >= 3;
    }
  }

  // Direct loads of the chunk starting at `cs` into stage S: this wave's
  // instructions i write units i*64 + lane.
  template <int S>
  __device__ void issue(int cs, const ChunkIds& c) {
    const int last = p.num_blocks - 1;
    const int id0 = min(max(c.id0, 0), last), id1 = min(max(c.id1, 0), last);
    const int id2 = min(max(c.id2, 0), last), id3 = min(max(c.id3, 0), last);
    const uint32_t in_block = (uint32_t)(cs & (p.block_size - 1));  // chunk's first token inside its block
    // the chunk's V sub-tile inside the block (blocks larger than the chunk)
    const uint64_t v_sub = (uint64_t)(in_block / (uint32_t)v_subtile(p.block_size)) * D * v_subtile(p.block_size) * 2;
    const char* kc = static_cast<const char*>(p.k_cache) + (size_t)in_block * (D * 2);
    const uint16_t* st = stage_buf<S, D>();
#pragma unroll
    for (int ii = 0; ii < LPW / 2; ++ii) {
      const int i = wave * (LPW / 2) + ii;
      const int kb = k_blk[ii];
      const int id = kb == 0 ? id0 : (kb == 1 ? id1 : (kb == 2 ? id2 : id3));
      load_lds16(kc + (size_t)id * block_bytes, k_off[ii], lds_address(st + i * 512));
    }
#pragma unroll
    for (int ii = 0; ii < LPW / 2; ++ii) {
      const int i = wave * (LPW / 2) + ii;
      const uint32_t id = (uint32_t)(v_ge3[ii] ? id3 : (v_ge2[ii] ? id2 : (v_ge1[ii] ? id1 : id0)));
      load_lds16(v_src[ii] + ((uint64_t)id * block_bytes + v_sub), lds_address(st + kChunk * D + i * 512));
    }
  }

  template <int S>
  __device__ void compute(int cs) {
    const uint16_t* st = stage_buf<S, D>();
    // K operand: row `col` of the MFMA is token 8*(col/4) + 4c + col%4, so the
    // scores land where PV wants its P operand
    u32x4 ka[2][MQ];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int t = 8 * (col >> 2) + 4 * c + (col & 3);
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        const int seg = (4 * m + grp) ^ k_swizzle(t, D);
        ka[c][m] = *reinterpret_cast<const u32x4*>(st + (t * (D / 8) + seg) * 8);
      }
    }
    float sv[NG][8];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      f32x4 sc0 = f32x4{0.f, 0.f, 0.f, 0.f}, sc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        sc0 = mfma_16x16x32(__builtin_bit_cast(op8, ka[0][m]), qop[gi][m], sc0);
        sc1 = mfma_16x16x32(__builtin_bit_cast(op8, ka[1][m]), qop[gi][m], sc1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // raw scores; the positive scale is applied in the exponent
        sv[gi][i] = sc0[i];
        sv[gi][4 + i] = sc1[i];
      }
    }
    // V operand: tokens cs + 8*grp .. +7 of channel col + 16 j
    u32x4 vr[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int c = col + 16 * j;
      vr[j] = *reinterpret_cast<const u32x4*>(st + kChunk * D + (c * 4 + (grp ^ v_swizzle(c))) * 8);
    }
    if (cs + kChunk - 1 > p_last) {  // tokens past the tile's last position: no V
      const int nvalid = p_last + 1 - (cs + 8 * grp);
#pragma unroll
      for (int j = 0; j < NT; ++j) vr[j] = Tr::keep_first(vr[j], nvalid);
    }
    const bool masked = cs + kChunk - 1 > pos_w;
    if (masked) {  // causal limit inside this chunk
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[gi][e] = (cs + 8 * grp + e <= pcol[gi]) ? sv[gi][e] : kNegInf;
    }
    // column maxima of every group first, one (rare) rescale branch for all,
    // then a branch-free run of exponentials, splits and PV products in which
    // one group's MFMAs can overlap the next group's vector work
    bool grow[NG];
    float cmax[NG];
    bool any_grow = false;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      float c = kNegInf;
#pragma unroll
      for (int e = 0; e < 8; ++e) c = fmaxf(c, sv[gi][e]);
      cmax[gi] = max_over_column(c) * p.scale_log2;
      // The reference maximum moves only when a score exceeds it by more than
      // 2^8: exponentials stay <= 256 and the output is rescaled rarely. The
      // result does not depend on the reference (it cancels in o / l).
      grow[gi] = cmax[gi] > m_run[gi] + kRescaleSlack;
      any_grow |= grow[gi];
    }
    if (__any(any_grow)) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const float m_new = grow[gi] ? cmax[gi] : m_run[gi];
        const float alpha = fast_exp2(m_run[gi] - m_new);
        l_run[gi] *= alpha;
        m_run[gi] = m_new;
        // output rows of this lane are columns 4*grp+i; their factor lives in lane 4*grp+i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * grp + i);
#pragma unroll
          for (int j = 0; j < NT; ++j) o[gi][j][i] *= ai;
        }
      }
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      float pe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(__builtin_fmaf(sv[gi][e], p.scale_log2, -m_run[gi]));
      float psum = pe[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) psum += pe[e];
      l_run[gi] += psum;
      op8 phi, plo;
      Tr::split(pe, phi, plo);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        o[gi][j] = mfma_16x16x32(phi, __builtin_bit_cast(op8, vr[j]), o[gi][j]);
        o[gi][j] = mfma_16x16x32(plo, __builtin_bit_cast(op8, vr[j]), o[gi][j]);
      }
    }
    // scheduling hint for the region above: alternate one MFMA (mask 0x008)
    // with three vector-ALU instructions (0x002), so that a group's PV
    // products issue between the next group's exponentials and splits
    // (+1% to +3% over the plain order on every head shape measured)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
  }

  // One chunk of the ring: stage S holds chunk ci. False past the last chunk.
  template <int S>
  __device__ bool step(int ci, ChunkIds& ids_next) {
    if (ci >= nch) return false;
    if (ci + 1 < nch) {
      wait_and_barrier<LPW>();  // this wave's loads of chunk ci landed; chunk ci+1's may fly
    } else {
      wait_and_barrier<0>();
    }
    // every wave is past chunk ci-1, whose stage takes chunk ci+2
    if (ci + 2 < nch) {
      const ChunkIds ids = ids_next;
      ids_next = load_chunk_ids(tbl, min(ci + 3, nch - 1) * kChunk, lbl, p.log2_block);
      this->template issue<(S + 2) % 3>((ci + 2) * kChunk, ids);
    }
    if (ci <= last_w) this->template compute<S>(ci * kChunk);
    return true;
  }
};

template <int E, int D, int NG>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_kernel(PrefillParams p) {
  using Tile = PrefillTile<E, D, NG>;
  using op8 = typename Tile::op8;
  using raw = typename Tile::raw;
  constexpr int MQ = Tile::MQ, NT = Tile::NT;
  Tile T(p);
  T.lane = threadIdx.x & 63;
  T.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  T.col = T.lane & 15;
  T.grp = T.lane >> 4;
  // XCD-aware order: the hardware hands workgroup L = x + y * X to XCD L % 8.
  // Each XCD takes a contiguous range of work items w = kvh * X + x, so the
  // tiles it runs together (consecutive tiles of one sequence and KV head)
  // share their K/V in that XCD's L2.
  const unsigned X = gridDim.x, N = X * gridDim.y;
  const unsigned lin = blockIdx.x + blockIdx.y * X;
  const unsigned xcd = lin % 8, q8 = N / 8, rem = N % 8;
  const unsigned w = xcd * q8 + min(xcd, rem) + lin / 8;
  T.kvh = (int)(w / X);
  const int lane = T.lane, col = T.col, grp = T.grp, wave = T.wave;
  const int g = p.group, qt = p.qt, Hq = p.num_heads;
  const int qw = NG * qt, qb = kPrefillWaves * qw;  // queries per wave, per tile

  // tile map: every wave scans the query counts (the longest tiles, the last
  // of each sequence, are handed out first)
  const int S = p.num_seqs;
  const int per = (S + 63) >> 6;
  const int s_lo = min(lane * per, S), s_hi = min(s_lo + per, S);
  int mine = 0;
  for (int s = s_lo; s < s_hi; ++s) mine += seq_tiles(p, s, qb);
  int incl = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  const int ntiles = __shfl(incl, 63);
  const int excl = incl - mine;
  const int x = (int)(w % X);
  if (x >= ntiles) return;
  const int tile = ntiles - 1 - x;
  const unsigned long long ball = __ballot(tile >= excl && tile < incl);
  if (ball == 0) return;  // counts past int range only
  const int owner = __builtin_ctzll(ball);
  int s_found = 0, k_found = 0;
  if (lane == owner) {
    int c = excl;
    for (int s = s_lo; s < s_hi; ++s) {
      const int nt = seq_tiles(p, s, qb);
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
  if (k >= seq_tiles(p, s, qb)) return;
  const int q0 = p.q_start[s], n = p.q_start[s + 1] - q0, L = p.context_lens[s];
  // precondition violated: the whole workgroup leaves together
  if (n > L || L > (p.max_blocks_per_seq << p.log2_block)) return;
  const int j0 = k * qb, nq = min(qb, n - j0);
  const int pos0 = L - n + j0;
  T.p_last = pos0 + nq - 1;
  T.nch = T.p_last / kChunk + 1;
  T.tbl = p.block_tables + (size_t)s * p.max_blocks_per_seq;
  T.lbl = T.p_last >> p.log2_block;
  const int nq_w = min(max(nq - wave * qw, 0), qw);
  T.pos_w = pos0 + wave * qw;
  T.last_w = nq_w > 0 ? (T.pos_w + nq_w - 1) / kChunk : -1;
  T.init_loads();

  // columns (query qi, head hh) of each group; columns past the tile read q = 0
  const int qi = col / g, hh = col - qi * g;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int jq = gi * qt + qi;  // query within the wave
    const bool cvalid = qi < qt && jq < nq_w;
    T.pcol[gi] = cvalid ? T.pos_w + jq : T.pos_w + nq_w - 1;
    const raw* qrow = static_cast<const raw*>(p.q) +
                      ((size_t)(q0 + j0 + wave * qw + (cvalid ? jq : 0)) * Hq + T.kvh * g + hh) * D;
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (cvalid && p.q_sign != 0) w = load16(qrow + 32 * m + 8 * grp);
      if (p.q_sign < 0) w ^= 0x80008000u;  // -q, exactly: the scale enters as |scale|
      T.qop[gi][m] = __builtin_bit_cast(op8, w);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) T.o[gi][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    T.m_run[gi] = kNegInf;
    T.l_run[gi] = 0.f;
  }
  // chunk 0's ring loads fly together with the q loads; both complete here,
  // so the ring's later waits count ring loads only (the builtin form tells
  // the compiler that q is done)
  const int nch = T.nch;
  {
    const ChunkIds ids0 = load_chunk_ids(T.tbl, 0, T.lbl, p.log2_block);
    T.template issue<0>(0, ids0);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  ChunkIds ids_next = load_chunk_ids(T.tbl, min(2, nch - 1) * kChunk, T.lbl, p.log2_block);
  if (nch > 1) {
    const ChunkIds ids1 = load_chunk_ids(T.tbl, kChunk, T.lbl, p.log2_block);
    T.template issue<1>(kChunk, ids1);
  }
  for (int ci = 0;; ci += 3) {
    if (!T.template step<0>(ci, ids_next)) break;
    if (!T.template step<1>(ci + 1, ids_next)) break;
    if (!T.template step<2>(ci + 2, ids_next)) break;
  }

  // Rows of this lane: columns r = 4*grp + i, i.e. query r / g, head r % g;
  // a row is normalised with one reciprocal. A query's g heads are g*D
  // contiguous outputs, so each wave stages its rows, group by group, in its
  // own half of a ring stage (free once every wave is past the last chunk's
  // reads) and stores them 16 bytes per lane; element dd of row r sits at
  // r*D + (dd ^ ((r >> 2) << 4)): the 64 lanes of a write instruction (rows
  // 4*grp + i, elements 16j + col) then fall in 64 distinct banks, and a
  // 16-byte unit of the read-back stays contiguous. An output not 16-byte
  // aligned takes the per-element stores.
  __syncthreads();
  const bool vec_out = (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
  const int es = p.out_dtype == kF32 ? 4 : 2;
  char* stg = reinterpret_cast<char*>(wave < 2 ? stage_buf<0, D>() : stage_buf<1, D>()) + (wave & 1) * (16 * D * 4);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float l_tot = sum_over_column(T.l_run[gi]);
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv[i] = 1.f / __shfl(l_tot, 4 * grp + i);
    if (vec_out) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int e = r * D + ((16 * j + col) ^ ((r >> 2) << 4));
          const float v = T.o[gi][j][i] * inv[i];
          if (es == 4) reinterpret_cast<float*>(stg)[e] = v;
          else
            reinterpret_cast<uint16_t*>(stg)[e] =
                p.out_dtype == kF16 ? __builtin_bit_cast(uint16_t, static_cast<_Float16>(v))
                                    : __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
        }
      }
      // this wave's own writes, then its reads, in order
      const int upr = D * es / 16;  // 16-byte units per row
      for (int u = lane; u < qt * g * upr; u += 64) {
        const int r = u / upr, c = u - r * upr;
        const int qr = r / g, jq = gi * qt + qr;
        if (jq < nq_w) {
          const int e0 = (c * 16 / es) ^ ((r >> 2) << 4);  // the unit's first element, as staged
          const u32x4 val = *reinterpret_cast<const u32x4*>(stg + (size_t)(r * D + e0) * es);
          const size_t base = ((size_t)(q0 + j0 + wave * qw + jq) * Hq + T.kvh * g + (r - qr * g)) * D;
          *reinterpret_cast<u32x4*>(static_cast<char*>(p.out) + (base + (size_t)c * 16 / es) * es) = val;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        const int qr = r / g;
        const int jq = gi * qt + qr;
        if (qr < qt && jq < nq_w) {
          const size_t base = ((size_t)(q0 + j0 + wave * qw + jq) * Hq + T.kvh * g + (r - qr * g)) * D + col;
#pragma unroll
          for (int j = 0; j < NT; ++j) store_out(p.out, base + 16 * j, T.o[gi][j][i] * inv[i], p.out_dtype);
        }
      }
    }
  }
}

const void* prefill_fn(int elem, int head_dim) {
  constexpr int G64 = prefill_groups<64>(), G128 = prefill_groups<128>();
  if (elem == kBF16) return head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<kBF16, 64, G64>)
                                           : reinterpret_cast<const void*>(&prefill_kernel<kBF16, 128, G128>);
  if (elem == kF16) return head_dim == 64 ? reinterpret_cast<const void*>(&prefill_kernel<kF16, 64, G64>)
                                          : reinterpret_cast<const void*>(&prefill_kernel<kF16, 128, G128>);
  return nullptr;
}

}  // namespace

int prefill_queries_per_tile(int group, int head_dim) {
  const int ng = head_dim == 128 ? prefill_groups<128>() : prefill_groups<64>();
  return kPrefillWaves * ng * (16 / group);
}

hipError_t launch_prefill(const PrefillParams& p, int elem, int head_dim, unsigned tiles, hipStream_t stream) {
  const void* fn = prefill_fn(elem, head_dim);
  if (!fn) return hipErrorInvalidDeviceFunction;
  PrefillParams args = p;
  void* kargs[] = {&args};
  return hipLaunchKernel(fn, dim3(tiles, (unsigned)p.num_kv_heads, 1), dim3(64 * kPrefillWaves, 1, 1), kargs, 0,
                         stream);
}

}  // namespace pa
