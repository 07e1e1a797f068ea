// HIP kernels for gfx950 (CDNA4): paged decode attention, slot-mapped KV
// write, copy-on-write block copy, workspace fill.
//
// Method: exact single-query attention over a KV cache cut into fixed-size
// physical blocks that a per-sequence block table maps from logical order
// ("PagedAttention 论文精读笔记" §2.1 attention equation, §4.2 block-wise
// form; "paged-attention은 도대체 뭘 최적화 하는 것일까" §14 address
// translation). Blocks are consumed 32 tokens at a time with an fp32 online
// softmax, partial results of split contexts are combined by their maxima and
// exponential sums ("PagedAttention paper review", "How does this work?").
//
// Pool layout (per physical block and KV head, one contiguous tile):
//   K tile [block_size][head_dim]  -- token rows
//   V tile [block_size/Bs][head_dim][Bs], Bs = min(block_size, 32)  -- token
//          columns of 32-token sub-tiles ([head_dim][block_size] up to 32)
// so that both MFMA operands of the two contractions (QK over head_dim, PV
// over tokens) are 16-byte contiguous loads straight from HBM, and a 32-token
// chunk's V is whole cache lines at every block size.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pa_device.h"
#include "pa_internal.h"

// Decode workspace of pa_decode_noalloc: a fixed array per device, so that
// callers that cannot allocate still get the split path. Host code never
// passes this name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address static_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[pa::kStaticScratchBytes];

namespace pa {

hipError_t static_scratch(void** ptr) {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static void* addr[kDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {

// The length a decode works on: the stored one, cut to what the block
// table can address and, with fixed partitions, to max_parts partitions (a
// context longer than the host's bound is cut there rather than left
// without a merging piece).
__device__ __forceinline__ int capped_len(const DecodeParams& p, int L_raw) {
  int L = min(L_raw, p.max_blocks_per_seq << p.log2_block);
  if (p.mode != kModeBalanced) L = (int)min((long long)L, (long long)p.max_parts * p.part_chunks * kChunk);
  return L;
}

// Stored length of sequence s (wave-uniform), read with a scalar load so
// that it never waits behind the K/V vector loads in flight.
__device__ __forceinline__ int len_uniform(const DecodeParams& p, int s) {
  const const_i32* lens = (const const_i32*)p.context_lens;
  return lens[__builtin_amdgcn_readfirstlane(s)];
}

// Dynamic shared memory of a decode workgroup: the stored lengths
// (lens_pad ints; the balanced split and the partition stream copy every
// length there at their start and walk their sequences from it), then the
// result buffer of res_slots finished segments.
extern __shared__ __align__(16) int32_t g_lens[];

__device__ __forceinline__ int lds_len(int s) { return __builtin_amdgcn_readfirstlane(g_lens[s]); }

// Position of the token the fused write stores for a piece ending at t1 of
// a sequence of stored length L_raw, cut to L: its last, when the piece holds
// it and the length was not cut; else -1.
__device__ __forceinline__ int new_token_pos(const DecodeParams& p, int t1, int L, int L_raw) {
  return (p.k_new != nullptr && L == L_raw && t1 == L && L > 0) ? L - 1 : -1;
}

__device__ __forceinline__ u32x4 put_elem16(u32x4 w, int e, uint32_t v) {
  const int wi = e >> 1, sh = (e & 1) * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = i == wi ? ((w[i] & ~(0xffffu << sh)) | ((v & 0xffffu) << sh)) : w[i];
  return w;
}

__device__ __forceinline__ u32x4 put_elem32(u32x4 w, int e, uint32_t v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = i == e ? v : w[i];
  return w;
}

// element e (< 16 / sizeof(U)) of a 16-byte register group set to v; e < 0: unchanged
template <typename U>
__device__ __forceinline__ u32x4 put_elem(u32x4 w, int e, uint32_t v) {
  return sizeof(U) == 4 ? put_elem32(w, e, v) : put_elem16(w, e, v);
}

// One sequence's share of a worker's work: tokens [t0, t1) of sequence s,
// whose last logical block is lbl; tnew is the position of the token the
// fused write stores (the sequence's last, when this piece holds it and the
// call brings one), else -1.
struct Segment {
  int s, t0, t1, lbl, npieces, slot, first_slot;
  int tnew;
  int valid;
};

__device__ __forceinline__ Segment invalid_segment() {
  Segment g;
  g.s = g.t0 = g.t1 = g.lbl = g.npieces = g.slot = g.first_slot = 0;
  g.tnew = -1;
  g.valid = 0;
  return g;
}

__device__ __forceinline__ Segment uniform(Segment g) {
  g.s = __builtin_amdgcn_readfirstlane(g.s);
  g.t0 = __builtin_amdgcn_readfirstlane(g.t0);
  g.t1 = __builtin_amdgcn_readfirstlane(g.t1);
  g.lbl = __builtin_amdgcn_readfirstlane(g.lbl);
  g.npieces = __builtin_amdgcn_readfirstlane(g.npieces);
  g.slot = __builtin_amdgcn_readfirstlane(g.slot);
  g.first_slot = __builtin_amdgcn_readfirstlane(g.first_slot);
  g.tnew = __builtin_amdgcn_readfirstlane(g.tnew);
  g.valid = __builtin_amdgcn_readfirstlane(g.valid);
  return g;
}

__device__ __forceinline__ int num_chunks(int L) { return L > 0 ? (L + kChunk - 1) / kChunk : 0; }

// ---------------------------------------------------------------------------
// MFMA engine (16-bit elements, group g in [1, 8]).
//
// One wave runs v_mfma_f32_16x16x32 on each chunk of 32 tokens:
//   QK: D[token slot][head slot] = K rows (A, 16 x 32) x q^T (B, 32 x 16),
//       two row groups of 16 tokens, head_dim/32 k-steps each;
//   PV: D[head slot][dd] = P (A, 16 x 32 tokens) x V (B, 32 tokens x 16),
//       head_dim/16 column tiles.
// Lane l feeds A row / B column l%16 and k-slots 8*(l/16)..+7; D[4*(l/16)+i]
// [l%16] comes back in register i. Token slots are arranged so that the QK
// result of lane l (tokens 8*(l/16)+0..7 of its head slot) is exactly the P
// operand lane l must supply, and V's token-minor tile makes each lane's
// eight tokens at one dd a single 16-byte load.
// Head slots: c < g carry head c with P rounded to 16 bits ("hi"), g <= c <
// 2g carry head c-g with the rounding residual ("lo"), the rest are zero; the
// two PV results are added at the end, so P enters the product with ~16
// significant bits instead of 8.
// ---------------------------------------------------------------------------
template <int E, int D, int SUB>
struct MfmaEngine {
  using Tr = ElemT<E>;
  using op8 = typename Tr::op8;
  using scalar = typename Tr::scalar;
  using raw = typename Tr::raw;
  static constexpr int kSub = SUB;   // 32-token sub-chunks per step
  static constexpr int MQ = D / 32;  // QK k-steps
  static constexpr int NT = D / 16;  // PV column tiles
  static constexpr int kPad = 4;
  struct Smem {
    float o[16][D + kPad];
    float ml[16][2];
  };

  op8 qop[MQ];
  f32x4 o[NT];
  float m_run;
  float l_run;
  uint32_t vn[NT];  // the segment's new token's V at this lane's output columns 16j + col

  // q of one sequence as the QK B operand (columns = head slots), and the
  // new token's V values this lane's B operands carry (fused write)
  struct Q {
    u32x4 w[MQ];
    uint32_t vn[NT];
  };

  __device__ void load_q(Q& q, const DecodeParams& p, int s, int kvh, int lane) const {
    const int col = lane & 15, grp = lane >> 4, g = p.group;
    const int hs = col < g ? col : (col < 2 * g ? col - g : -1);
    const raw* qb = static_cast<const raw*>(p.q) + ((size_t)s * p.num_heads + (size_t)kvh * g) * D;
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (hs >= 0) w = load16(qb + (size_t)hs * D + 32 * m + 8 * grp);
      q.w[m] = w;
    }
    // read unconditionally (from q when the call brings no new token: an
    // in-bounds row, never used) so every segment issues the same loads
    const raw* vb = static_cast<const raw*>(p.v_new ? p.v_new : p.q) + ((size_t)s * p.num_kv_heads + kvh) * D + col;
#pragma unroll
    for (int j = 0; j < NT; ++j) q.vn[j] = vb[16 * j];
  }

  __device__ void reset(const Q& q) {
#pragma unroll
    for (int m = 0; m < MQ; ++m) qop[m] = __builtin_bit_cast(op8, q.w[m]);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      vn[j] = q.vn[j];
    }
    m_run = kNegInf;
    l_run = 0.f;
  }

  // registers of one step: K rows (A operands) and V columns (B operands)
  // of SUB sub-chunks
  struct Frag {
    u32x4 ka[SUB][2][MQ];
    u32x4 vr[SUB][NT];
  };

  // The row of the segment's new token (g.tnew) comes from the caller's
  // k_new, not from the cache slot the same launch writes.
  __device__ void load_k(Frag& f, const DecodeParams& p, int kvh, int lane, int cs, const ChunkIds* ids,
                         const Segment& g) const {
    const int col = lane & 15, grp = lane >> 4;
    const int B = p.block_size, lg = p.log2_block, Hkv = p.num_kv_heads;
    const raw* __restrict__ kc = static_cast<const raw*>(p.k_cache);
    const raw* kn = static_cast<const raw*>(p.k_new) + ((size_t)g.s * Hkv + kvh) * D + 8 * grp;
    // K rows: A-operand row `col` of row group c holds token 8*(col/4)+4c+col%4
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int tok = cs + kChunk * u + 8 * (col >> 2) + 4 * c + (col & 3);
        const int phys = pick_block(ids[u], tok, lg, g.lbl, p.num_blocks);
        const raw* row = kc + (((size_t)phys * Hkv + kvh) * B + (tok & (B - 1))) * D + 8 * grp;
        row = tok == g.tnew ? kn : row;
#pragma unroll
        for (int m = 0; m < MQ; ++m) f.ka[u][c][m] = load16_stream(row + 32 * m);
      }
  }

  __device__ void load_v(Frag& f, const DecodeParams& p, int kvh, int lane, int cs, const ChunkIds* ids,
                         const Segment& g) const {
    const int lbl = g.lbl;
    const int col = lane & 15, grp = lane >> 4;
    const int B = p.block_size, lg = p.log2_block, Hkv = p.num_kv_heads;
    const raw* __restrict__ vc = static_cast<const raw*>(p.v_cache);
    const int Bs = v_subtile(B);
    // V: B operand, tokens 8*grp..+7 of each sub-chunk at dd = 16j + col
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const int tv = cs + kChunk * u + 8 * grp;
      const int physv = pick_block(ids[u], tv, lg, lbl, p.num_blocks);
      const raw* vb = vc + v_elem(physv, Hkv, kvh, D, B, Bs, col, tv & (B - 1));
#pragma unroll
      for (int j = 0; j < NT; ++j) f.vr[u][j] = load16_stream(vb + (size_t)16 * j * Bs);
    }
  }

  // Compute the step at `cs` from `f`; as soon as a register set is
  // consumed it is refilled with the next step (K after QK, V after PV), so
  // one step's loads are always in flight behind the math.
  __device__ void step(Frag& f, const DecodeParams& p, Smem&, int kvh, int lane, int cs, const Segment& cur,
                       int cs_next, const ChunkIds* ids_next, const Segment& nxt) {
    const int col = lane & 15, grp = lane >> 4, g = p.group;
    const int t1 = cur.t1;
    const bool has_new = cur.tnew >= cs && cur.tnew < cs + SUB * kChunk;
    // scores: in sub-chunk u the lane holds tokens cs+32u+8*grp+0..7 of head slot `col`
    f32x4 sc[SUB][2];
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      sc[u][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      sc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        sc[u][0] = mfma_16x16x32(__builtin_bit_cast(op8, f.ka[u][0][m]), qop[m], sc[u][0]);
        sc[u][1] = mfma_16x16x32(__builtin_bit_cast(op8, f.ka[u][1][m]), qop[m], sc[u][1]);
      }
    }
    // unconditional refill (at the end of the stream the last step re-reads
    // itself from L2) keeps the count of loads in flight the same on every
    // path, so the PV wait below never has to drain the next step's K loads
    load_k(f, p, kvh, lane, cs_next, ids_next, nxt);
    float sv[SUB][8];
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[u][i] = sc[u][0][i] * p.scale_log2;
        sv[u][4 + i] = sc[u][1][i] * p.scale_log2;
      }
    const bool partial = cs + SUB * kChunk > t1;
    if (partial) {
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[u][e] = (cs + kChunk * u + 8 * grp + e < t1) ? sv[u][e] : kNegInf;
    }

    // online softmax (base 2), per head slot
    float cmax = kNegInf;
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) cmax = fmaxf(cmax, sv[u][e]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = fast_exp2(m_run - m_new);
    float pe[SUB][8];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pe[u][e] = fast_exp2(sv[u][e] - m_new);
        psum += pe[u][e];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
      // output rows of this lane are head slots 4*grp+i; their factor lives in lane 4*grp+i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * grp + i);
#pragma unroll
        for (int j = 0; j < NT; ++j) o[j][i] *= ai;
      }
    }

    // P operands: hi part, lo residual or zero depending on the head slot
    const int part = col < g ? 0 : (col < 2 * g ? 1 : 2);
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      op8 pa;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const scalar hi = static_cast<scalar>(pe[u][e]);
        const scalar lo = static_cast<scalar>(pe[u][e] - static_cast<float>(hi));
        pa[e] = part == 0 ? hi : (part == 1 ? lo : static_cast<scalar>(0.f));
      }
      if (partial) {
        const int nvalid = t1 - (cs + kChunk * u + 8 * grp);
#pragma unroll
        for (int j = 0; j < NT; ++j) f.vr[u][j] = Tr::keep_first(f.vr[u][j], nvalid);
      }
      if (has_new) {
        // the new token's V replaces what its slot held before this launch
        const int e = cur.tnew - (cs + kChunk * u + 8 * grp);
        const int en = e >= 0 && e < 8 ? e : -1;
#pragma unroll
        for (int j = 0; j < NT; ++j) f.vr[u][j] = put_elem<raw>(f.vr[u][j], en, vn[j]);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) o[j] = mfma_16x16x32(pa, __builtin_bit_cast(op8, f.vr[u][j]), o[j]);
    }
    load_v(f, p, kvh, lane, cs_next, ids_next, nxt);
  }

  __device__ void finish(Smem& sm, int lane) {
    const int col = lane & 15, grp = lane >> 4;
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.o[4 * grp + i][16 * j + col] = o[j][i];
    if (grp == 0) {
      sm.ml[col][0] = m_run;
      sm.ml[col][1] = l_tot;
    }
    __syncthreads();
  }

  __device__ static float o_val(const Smem& sm, int h, int dd, int g) { return sm.o[h][dd] + sm.o[h + g][dd]; }
  __device__ static float m_val(const Smem& sm, int h) { return sm.ml[h][0]; }
  __device__ static float l_val(const Smem& sm, int h) { return sm.ml[h][1]; }
};

// ---------------------------------------------------------------------------
// Vector engine (any element type, group bucket G >= g).
//
// QK: 16-byte coalesced loads of token rows, LPR lanes per row, partial dot
// products reduced across those lanes. Softmax over the chunk's 32 scores
// through LDS. PV: 16-byte loads of VEC consecutive tokens at one dd from the
// token-minor V tile, fp32 FMAs, accumulators reduced across lanes at the end.
// ---------------------------------------------------------------------------
template <int E, int D, int G>
struct VecEngine {
  using Tr = ElemT<E>;
  using raw = typename Tr::raw;
  static constexpr int VEC = Tr::kVec;
  static constexpr int LPR = D / VEC;           // lanes per K row
  static constexpr int RPS = 64 / LPR;          // K rows per load step
  static constexpr int KSTEPS = kChunk / RPS;   // K load steps per chunk
  static constexpr int LPD = kChunk / VEC;      // lanes per V dd-row of a chunk
  static constexpr int DPS = 64 / LPD;          // dd rows per V load step
  static constexpr int VSTEPS = D / DPS;        // V load steps per chunk
  static constexpr int kSub = 1;
  struct Smem {
    float sc[G][kChunk];
    float pl[G][kChunk];
    float o[G][D];
    float ml[G][2];
  };

  float qv[G][VEC];
  float acc[G][VSTEPS];
  float m_run[G];
  float l_run[G];
  uint32_t vn[VSTEPS];  // the segment's new token's V at this lane's rows st*DPS + lane/LPD

  struct Q {
    u32x4 w[G];
    uint32_t vn[VSTEPS];
  };

  __device__ void load_q(Q& q, const DecodeParams& p, int s, int kvh, int lane) const {
    const int piece = lane % LPR, g = p.group;
    const raw* qb = static_cast<const raw*>(p.q) + ((size_t)s * p.num_heads + (size_t)kvh * g) * D;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (h < g) w = load16(qb + (size_t)h * D + piece * VEC);
      q.w[h] = w;
    }
    // read unconditionally (from q when the call brings no new token: an
    // in-bounds row, never used) so every segment issues the same loads
    const raw* vb = static_cast<const raw*>(p.v_new ? p.v_new : p.q) + ((size_t)s * p.num_kv_heads + kvh) * D +
                    lane / LPD;
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st) q.vn[st] = vb[st * DPS];
  }

  __device__ void reset(const Q& q) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      Tr::widen(q.w[h], qv[h]);
#pragma unroll
      for (int st = 0; st < VSTEPS; ++st) acc[h][st] = 0.f;
      m_run[h] = kNegInf;
      l_run[h] = 0.f;
    }
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st) vn[st] = q.vn[st];
  }

  struct Frag {
    u32x4 kr[KSTEPS];
    u32x4 vr[VSTEPS];
  };

  // The row of the segment's new token (g.tnew) comes from the caller's
  // k_new, not from the cache slot the same launch writes.
  __device__ void load_k(Frag& f, const DecodeParams& p, int kvh, int lane, int cs, const ChunkIds* idp,
                         const Segment& g) const {
    const ChunkIds ids = idp[0];
    const int B = p.block_size, lg = p.log2_block, Hkv = p.num_kv_heads;
    const raw* __restrict__ kc = static_cast<const raw*>(p.k_cache);
    const int piece = lane % LPR;
    const raw* kn = static_cast<const raw*>(p.k_new) + ((size_t)g.s * Hkv + kvh) * D + piece * VEC;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      const int tok = cs + st * RPS + lane / LPR;
      const int phys = pick_block(ids, tok, lg, g.lbl, p.num_blocks);
      const raw* row = kc + (((size_t)phys * Hkv + kvh) * B + (tok & (B - 1))) * D + piece * VEC;
      f.kr[st] = load16_stream(tok == g.tnew ? kn : row);
    }
  }

  __device__ void load_v(Frag& f, const DecodeParams& p, int kvh, int lane, int cs, const ChunkIds* idp,
                         const Segment& g) const {
    const int lbl = g.lbl;
    const ChunkIds ids = idp[0];
    const int B = p.block_size, lg = p.log2_block, Hkv = p.num_kv_heads;
    const raw* __restrict__ vc = static_cast<const raw*>(p.v_cache);
    const int tg = lane % LPD, ddl = lane / LPD;
    const int tv = cs + tg * VEC;
    const int physv = pick_block(ids, tv, lg, lbl, p.num_blocks);
    const int Bs = v_subtile(B);
    const raw* vb = vc + v_elem(physv, Hkv, kvh, D, B, Bs, ddl, tv & (B - 1));
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st) f.vr[st] = load16_stream(vb + (size_t)st * DPS * Bs);
  }

  __device__ void step(Frag& f, const DecodeParams& p, Smem& sm, int kvh, int lane, int cs, const Segment& cur,
                       int cs_next, const ChunkIds* ids_next, const Segment& nxt) {
    const int t1 = cur.t1;
    const bool has_new = cur.tnew >= cs && cur.tnew < cs + kChunk;
    const int piece = lane % LPR;
    const int tg = lane % LPD;
    const int tv = cs + tg * VEC;

    // QK
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      float kf[VEC];
      Tr::widen(f.kr[st], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) d = fmaf(qv[h][e], kf[e], d);
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) d += __shfl_xor(d, off);
        if (piece == 0) sm.sc[h][st * RPS + lane / LPR] = d;
      }
    }
    load_k(f, p, kvh, lane, cs_next, ids_next, nxt);
    __syncthreads();

    // softmax over the chunk's 32 tokens
    const bool partial = cs + kChunk > t1;
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bool valid = lane < kChunk && cs + lane < t1;
      const float sv = valid ? sm.sc[h][lane] * p.scale_log2 : kNegInf;
      float cmax = sv;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
      const float m_new = fmaxf(m_run[h], cmax);
      alpha[h] = fast_exp2(m_run[h] - m_new);
      const float pv = fast_exp2(sv - m_new);
      l_run[h] = l_run[h] * alpha[h] + pv;
      m_run[h] = m_new;
      if (lane < kChunk) sm.pl[h][lane] = pv;
    }
    __syncthreads();

    // PV
    const int enew = has_new && cur.tnew >= tv && cur.tnew < tv + VEC ? cur.tnew - tv : -1;
    float pw[G][VEC];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) pw[h][e] = sm.pl[h][tg * VEC + e];
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st) {
      u32x4 w = f.vr[st];
      if (partial) w = Tr::keep_first(w, t1 - tv);
      if (has_new) w = put_elem<raw>(w, enew, vn[st]);  // the new token's V, not its slot's old value
      float vf[VEC];
      Tr::widen(w, vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = acc[h][st] * alpha[h];
#pragma unroll
        for (int e = 0; e < VEC; ++e) a = fmaf(pw[h][e], vf[e], a);
        acc[h][st] = a;
      }
    }
    load_v(f, p, kvh, lane, cs_next, ids_next, nxt);
    __syncthreads();  // sc/pl are rewritten by the next chunk
  }

  __device__ void finish(Smem& sm, int lane) {
    const int tg = lane % LPD, ddl = lane / LPD;
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int st = 0; st < VSTEPS; ++st) {
        float v = acc[h][st];
#pragma unroll
        for (int off = LPD / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (tg == 0) sm.o[h][st * DPS + ddl] = v;
      }
      float l = l_run[h];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
      if (lane == 0) {
        sm.ml[h][0] = m_run[h];
        sm.ml[h][1] = l;
      }
    }
    __syncthreads();
  }

  __device__ static float o_val(const Smem& sm, int h, int dd, int) { return sm.o[h][dd]; }
  __device__ static float m_val(const Smem& sm, int h) { return sm.ml[h][0]; }
  __device__ static float l_val(const Smem& sm, int h) { return sm.ml[h][1]; }
};

// ---------------------------------------------------------------------------
// Segment driver, epilogue and merge (shared by both engines)
// ---------------------------------------------------------------------------
template <class Eng, int D>
__device__ void write_zero_rows(const DecodeParams& p, int s, int kvh, int lane) {
  const int g = p.group;
  const size_t base = ((size_t)s * p.num_heads + (size_t)kvh * g) * D;
  for (int idx = lane; idx < g * D; idx += 64) store_out(p.out, base + idx, 0.f, p.out_dtype);
}

__device__ __forceinline__ long long owner_of(long long c, long long W, long long T) {
  return ((c + 1) * W - 1) / T;
}

// Yields a worker's segments in order. Balanced mode: the chunks of all
// sequences (per KV head) are laid end to end and worker w owns chunks
// [start, end); fixed mode: a single partition.
struct SegmentSource {
  int mode;
  int s;          // next sequence to look at
  long long c;    // first chunk of sequence s in the laid-out order
  int k;          // fixed-partition stream: next partition of sequence s
  long long start, end, W, T;
  int w;
  Segment fixed;  // one-partition-per-workgroup mode's only segment

  __device__ Segment next(const DecodeParams& p) {
    if (mode == kModeFixed) {
      const Segment g = fixed;
      fixed.valid = 0;
      return g;
    }
    if (mode == kModeFixedStream) return next_partition(p);
    while (s < p.num_seqs && c < end) {
      const int L_raw = lds_len(s);
      const int L = capped_len(p, L_raw);
      const int n = num_chunks(L);
      if (n == 0) {
        ++s;
        continue;
      }
      const long long c0 = start > c ? start : c;
      const long long c1 = end < c + n ? end : c + n;
      Segment g;
      g.s = s;
      g.t0 = (int)(c0 - c) * kChunk;
      g.t1 = min((int)(c1 - c) * kChunk, L);
      g.lbl = (g.t1 - 1) >> p.log2_block;
      g.tnew = new_token_pos(p, g.t1, L, L_raw);
      const int first = (int)owner_of(c, W, T);
      const int last = (int)owner_of(c + n - 1, W, T);
      g.npieces = last - first + 1;
      g.slot = w + s;
      g.first_slot = first + s;
      g.valid = 1;
      c += n;
      ++s;
      return uniform(g);
    }
    return invalid_segment();
  }

  // Fixed partitions of part_chunks chunks, laid end to end like the chunks:
  // the worker takes every partition whose first chunk lies in [start, end).
  __device__ Segment next_partition(const DecodeParams& p) {
    const int pc = p.part_chunks;
    while (s < p.num_seqs && c < end) {
      const int L_raw = lds_len(s);
      const int L = capped_len(p, L_raw);
      const int n = num_chunks(L);
      const int np = (n + pc - 1) / pc;
      if (c + (long long)k * pc < start) k = (int)((start - c + pc - 1) / pc);
      if (k < np) {
        if (c + (long long)k * pc >= end) break;
        Segment g;
        g.s = s;
        g.t0 = k * pc * kChunk;
        g.t1 = (int)min((long long)g.t0 + (long long)pc * kChunk, (long long)L);
        g.lbl = (g.t1 - 1) >> p.log2_block;
        g.tnew = new_token_pos(p, g.t1, L, L_raw);
        g.npieces = np;
        g.slot = s * p.max_parts + k;
        g.first_slot = s * p.max_parts;
        g.valid = 1;
        ++k;
        return uniform(g);
      }
      c += n;
      ++s;
      k = 0;
    }
    return invalid_segment();
  }
};

// A position in the worker's chunk stream: segment rel (0 = current, 1 =
// next, 2 = the one after) and the chunk's first token.
struct Pos {
  int rel;
  int cs;
};

__device__ __forceinline__ Segment seg_at(int rel, const Segment& a, const Segment& b, const Segment& c) {
  return rel == 0 ? a : (rel == 1 ? b : c);
}

// The chunk after x; at the end of the stream x itself (its refill then
// re-reads data already in L2).
__device__ __forceinline__ Pos advance(Pos x, const Segment& a, const Segment& b, const Segment& c) {
  const Segment g = seg_at(x.rel, a, b, c);
  if (x.cs + kChunk < g.t1) return Pos{x.rel, x.cs + kChunk};
  if (x.rel < 2) {
    const Segment n = seg_at(x.rel + 1, a, b, c);
    if (n.valid) return Pos{x.rel + 1, n.t0};
  }
  return x;
}

__device__ __forceinline__ ChunkIds ids_at(const DecodeParams& p, Pos x, const Segment& a, const Segment& b,
                                           const Segment& c) {
  const Segment g = seg_at(x.rel, a, b, c);
  return load_chunk_ids(p.block_tables + (size_t)g.s * p.max_blocks_per_seq, x.cs, g.lbl, p.log2_block);
}

// Finished segments wait in LDS and are stored to memory when the worker's
// stream ends (or when the buffer is full). A store issued in the middle of
// the stream is counted with the K/V loads in flight, so the wait for the
// next load issued after it also waits for the store, which under the
// stream's load takes several microseconds: stored at every segment end, a
// step of 512-token partitions spent a fifth of its time there.
// Slot k: values [g][D] (normalised outputs of a whole sequence, or the
// unnormalised partial of a piece), (m, l) of each head, and a record
// {sequence, pieces, partial-result slot, first slot, 1 if the split record
// is written}.
constexpr int kResRec = 5;

template <bool NT>
__device__ __forceinline__ void store16(f32x4* dst, f32x4 v) {
  if (NT) {
    __builtin_nontemporal_store(v, dst);
  } else {
    *dst = v;
  }
}

struct ResultBuf {
  float* vals;
  float* ml;
  int* rec;
  int n;
};

__device__ __forceinline__ ResultBuf result_buffer(const DecodeParams& p, int D) {
  ResultBuf rb;
  rb.vals = reinterpret_cast<float*>(g_lens + p.lens_pad);
  rb.ml = rb.vals + (size_t)p.res_slots * p.group * D;
  rb.rec = reinterpret_cast<int*>(rb.ml + (size_t)p.res_slots * p.group * 2);
  rb.n = 0;
  return rb;
}

// Store every buffered result: whole sequences to `out`, pieces of split
// ones to the workspace, and the split records. NT: non-temporal stores, for
// a buffer that filled up mid-stream (they complete sooner under the
// stream's load, so the load waits behind them are shorter: 512-token
// partitions at the long-context shape 939 -> 913 us); at the stream's end
// ordinary stores.
template <int D, bool NT>
__device__ void flush_results(const DecodeParams& p, ResultBuf& rb, int kvh, int lane) {
  const int gq = p.group, Hq = p.num_heads, n4 = gq * D / 4;
  const size_t head0 = (size_t)kvh * gq;
  const bool out_vec = p.out_dtype == kF32 && (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
  for (int k = 0; k < rb.n; ++k) {
    const int* r = rb.rec + kResRec * k;
    const int s = __builtin_amdgcn_readfirstlane(r[0]), np = __builtin_amdgcn_readfirstlane(r[1]);
    const int slot = __builtin_amdgcn_readfirstlane(r[2]);
    const float* v = rb.vals + (size_t)k * gq * D;
    if (r[4] && lane == 0) {
      p.ws_meta[2 * s] = r[3];
      p.ws_meta[2 * s + 1] = np;
    }
    if (np == 1) {
      const size_t base = ((size_t)s * Hq + head0) * D;
      if (out_vec) {
        for (int i = lane; i < n4; i += 64)
          store16<NT>(reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + base) + i, reinterpret_cast<const f32x4*>(v)[i]);
      } else {
        for (int idx = lane; idx < gq * D; idx += 64) store_out(p.out, base + idx, v[idx], p.out_dtype);
      }
    } else {
      const size_t row0 = (size_t)slot * Hq + head0;
      for (int i = lane; i < n4; i += 64)
        store16<NT>(reinterpret_cast<f32x4*>(p.ws_acc + row0 * D) + i, reinterpret_cast<const f32x4*>(v)[i]);
      for (int i = lane; i < 2 * gq; i += 64) p.ws_ml[row0 * 2 + i] = rb.ml[(size_t)k * gq * 2 + i];
    }
  }
  rb.n = 0;
}

template <class Eng, int D>
__device__ void segment_epilogue(const DecodeParams& p, const typename Eng::Smem& sm, const Segment& g, int kvh,
                                 int lane, ResultBuf& rb) {
  if (rb.n == p.res_slots) flush_results<D, true>(p, rb, kvh, lane);
  const int gq = p.group;
  const int k = rb.n;
  float* v = rb.vals + (size_t)k * gq * D;
  if (g.npieces == 1) {
    for (int idx = lane; idx < gq * D; idx += 64) {
      const int h = idx / D, dd = idx % D;
      v[idx] = Eng::o_val(sm, h, dd, gq) / Eng::l_val(sm, h);
    }
  } else {
    for (int idx = lane; idx < gq * D; idx += 64) {
      const int h = idx / D, dd = idx % D;
      v[idx] = Eng::o_val(sm, h, dd, gq);
    }
    for (int h = lane; h < gq; h += 64) {
      rb.ml[((size_t)k * gq + h) * 2] = Eng::m_val(sm, h);
      rb.ml[((size_t)k * gq + h) * 2 + 1] = Eng::l_val(sm, h);
    }
  }
  if (lane == 0) {
    int* r = rb.rec + kResRec * k;
    r[0] = g.s;
    r[1] = g.npieces;
    r[2] = g.slot;
    r[3] = g.first_slot;
    // the piece holding a sequence's first token records where its pieces
    // are (single pieces too, so the merge kernel never reads a stale record)
    r[4] = p.mode == kModeBalanced && g.t0 == 0 && kvh == 0;
  }
  rb.n = k + 1;
  __syncthreads();
}

// Runs all of a worker's segments as one stream of 32-token chunks: the
// register set of a chunk is refilled with the next chunk of the stream,
// which may already belong to the next segment, whose q is fetched at the
// same time; block ids are read two chunks ahead. A segment's epilogue
// therefore overlaps the next segment's first loads.
template <class Eng, int D>
__device__ void run_stream(const DecodeParams& p, typename Eng::Smem& sm, SegmentSource& src, int kvh, int lane) {
  static_assert(Eng::kSub == 1, "the chunk stream assumes one 32-token chunk per step");
  Segment A = src.next(p);
  if (!A.valid) return;
  // the first chunk's block ids and q are requested before the next
  // segments are walked
  Pos p0{0, A.t0};
  const ChunkIds ids0 = ids_at(p, p0, A, A, A);
  Eng eng;
  typename Eng::Q q, qn;
  eng.load_q(q, p, A.s, kvh, lane);
  ResultBuf rb = result_buffer(p, D);
  Segment B = src.next(p);
  Segment C = B.valid ? src.next(p) : invalid_segment();
  Pos p1 = advance(p0, A, B, C);
  Pos p2 = advance(p1, A, B, C);
  ChunkIds ids1 = ids_at(p, p1, A, B, C);
  typename Eng::Frag f;
  eng.load_k(f, p, kvh, lane, p0.cs, &ids0, A);
  eng.load_v(f, p, kvh, lane, p0.cs, &ids0, A);
  eng.reset(q);  // after the first K/V loads are issued: only the first QK needs q
  for (;;) {
    const ChunkIds ids2 = ids_at(p, p2, A, B, C);
    const bool leaving = p1.rel != 0;                       // p0 is the current segment's last chunk
    const bool at_end = !leaving && p1.cs == p0.cs;         // and there is no next segment
    const Segment n1 = seg_at(p1.rel, A, B, C);
    if (leaving) eng.load_q(qn, p, n1.s, kvh, lane);
    eng.step(f, p, sm, kvh, lane, p0.cs, A, p1.cs, &ids1, n1);
    if (leaving || at_end) {
      eng.finish(sm, lane);
      segment_epilogue<Eng, D>(p, sm, A, kvh, lane, rb);
      if (at_end) break;
      A = B;
      B = C;
      C = B.valid ? src.next(p) : invalid_segment();
      p1.rel -= 1;
      p2.rel -= 1;
      eng.reset(qn);
    }
    p0 = p1;
    p1 = p2;
    p2 = advance(p2, A, B, C);
    ids1 = ids2;
  }
  flush_results<D, false>(p, rb, kvh, lane);
}

// Workgroups are handed to the 8 XCDs (each with its own L2) in turn by
// linear id; with W a multiple of 8 that is blockIdx.x % 8 for every KV
// head. Numbering the persistent workers XCD-major puts neighbouring chunk
// ranges -- the same or adjacent sequences, e.g. samples sharing a prompt's
// blocks -- on one XCD, so blocks several of them read are fetched once into
// that L2. The one-workgroup-per-partition mode keeps its own numbering.
__device__ __forceinline__ int worker_index(int bx, int W, int mode) {
  if (mode == kModeFixed || (W & 7)) return bx;
  return (bx & 7) * (W >> 3) + (bx >> 3);
}

template <class Eng, int D>
__global__ __launch_bounds__(64) void decode_kernel(DecodeParams p) {
  __shared__ typename Eng::Smem sm;
  const int lane = threadIdx.x;
  const int kvh = blockIdx.y;
  const int W = gridDim.x;
  const int w = worker_index(blockIdx.x, W, p.mode);
  SegmentSource src;
  src.mode = p.mode;
  src.w = w;

  if (p.mode == kModeFixed) {
    const int s = w / p.max_parts, part = w % p.max_parts;
    const int P = p.part_chunks * kChunk;
    const int L_raw = len_uniform(p, s);
    const int L = capped_len(p, L_raw);
    if (L <= 0) {
      if (part == 0) write_zero_rows<Eng, D>(p, s, kvh, lane);
      return;
    }
    const int t0 = part * P;
    if (t0 >= L) return;
    Segment g;
    g.s = s;
    g.t0 = t0;
    g.t1 = min(t0 + P, L);
    g.lbl = (g.t1 - 1) >> p.log2_block;
    g.npieces = (L + P - 1) / P;
    g.slot = s * p.max_parts + part;
    g.first_slot = s * p.max_parts;
    g.tnew = new_token_pos(p, g.t1, L, L_raw);
    g.valid = 1;
    src.fixed = uniform(g);
    run_stream<Eng, D>(p, sm, src, kvh, lane);
    return;
  }

  // Balanced split or fixed-partition stream: every worker scans the lengths
  // itself (S <= kMaxBalancedSeqs), so no planning launch is needed.
  const int S = p.num_seqs;
  // lengths to LDS, four coalesced loads in flight per lane at a time
  for (int s0 = 0; s0 < S; s0 += 256) {
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = s0 + 64 * i + lane;
      v[i] = s < S ? p.context_lens[s] : 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = s0 + 64 * i + lane;
      if (s < S) g_lens[s] = v[i];
    }
  }
  __syncthreads();
  const int per = (S + 63) >> 6;
  const int s_lo = min(lane * per, S), s_hi = min(s_lo + per, S);
  long long mine = 0;
  for (int s = s_lo; s < s_hi; ++s) mine += num_chunks(capped_len(p, g_lens[s]));
  long long incl = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  const long long T = __shfl(incl, 63);
  const long long excl = incl - mine;

  for (int s = w; s < S; s += W)
    if (capped_len(p, lds_len(s)) <= 0) write_zero_rows<Eng, D>(p, s, kvh, lane);
  if (T == 0) return;
  // with no more workers than chunks every range is non-empty, so the pieces
  // of a sequence are exactly the workers owner_of(first chunk)..owner_of(last)
  const long long Wn = (long long)W < T ? (long long)W : T;
  if (w >= Wn) return;
  const long long start = (long long)w * T / Wn, end = (long long)(w + 1) * T / Wn;

  const unsigned long long ball = __ballot(start >= excl && start < incl);
  if (ball == 0ull) return;  // unreachable while 0 <= start < T
  const int owner = __builtin_ctzll(ball);
  int s_first = 0;
  long long c_first = 0;
  if (lane == owner) {
    long long c = excl;
    for (int s = s_lo; s < s_hi; ++s) {
      const int n = num_chunks(capped_len(p, g_lens[s]));
      if (start < c + n) {
        s_first = s;
        c_first = c;
        break;
      }
      c += n;
    }
  }
  src.s = __builtin_amdgcn_readfirstlane(__shfl(s_first, owner));
  src.c = __shfl(c_first, owner);
  src.k = 0;
  src.start = start;
  src.end = end;
  src.W = Wn;
  src.T = T;
  src.fixed = invalid_segment();
  run_stream<Eng, D>(p, sm, src, kvh, lane);
}

// Combine the partial results of every split (sequence, KV head): the
// pieces' maxima and exponential sums give piece k of head h the weight
// w_k = 2^(m_k - M) / sum_j 2^(m_j - M) l_j with M = max_j m_j (base-2 units),
// and out = sum_k w_k acc_k. The (m, l) pairs are staged in LDS up to
// kMergeTile pieces; longer piece lists take a plain per-output loop. The
// balanced split leaves few pieces per sequence: one wave per (sequence, KV
// head), its first pieces requested together with the (m, l) pairs. Fixed
// partitions, or a balanced split of few sequences over many workers, leave
// many: four waves per (sequence, query head), reading 16 bytes per lane.
constexpr int kMergeTile = 256;

template <int W>
struct MergeSmem {
  float wgt[kMaxGroup][kMergeTile];
  float ls[kMaxGroup][kMergeTile];
  float part[W][kMaxGroup][128];
};

template <int D, int W>
__device__ void merge_long(const DecodeParams& p, int s, int head0, int nh, int tid, int first_slot, int npieces) {
  const int Hq = p.num_heads;
  for (int idx = tid; idx < nh * D; idx += 64 * W) {
    const int head = head0 + idx / D, dd = idx % D;
    float M = kNegInf;
    for (int k = 0; k < npieces; ++k) M = fmaxf(M, p.ws_ml[((size_t)(first_slot + k) * Hq + head) * 2]);
    float num = 0.f, den = 0.f;
    for (int k = 0; k < npieces; ++k) {
      const size_t r = (size_t)(first_slot + k) * Hq + head;
      const float wgt = fast_exp2(p.ws_ml[r * 2] - M);
      den = fmaf(wgt, p.ws_ml[r * 2 + 1], den);
      num = fmaf(wgt, p.ws_acc[r * D + dd], num);
    }
    store_out(p.out, ((size_t)s * Hq + head) * D + dd, num / den, p.out_dtype);
  }
}

// The W-wave form with one query head per workgroup (its only use): every
// lane reads 16 bytes, D/4 lanes per piece, so one wave instruction covers
// 64/(D/4) pieces and the first kIn instructions (all pieces up to
// kIn * W * 64/(D/4)) are in flight before the weights are formed. Piece k
// of wave v's instruction t is (t W + v) 64/(D/4) + lane / (D/4). The lane
// groups of a wave are then added by lane swaps and the W waves in wave order.
template <int D, int W>
__device__ void merge_one_head(const DecodeParams& p, MergeSmem<W>& sm, int s, int head, int tid, int first_slot,
                               int npieces) {
  constexpr int LPP = D / 4;     // lanes per piece
  constexpr int PPW = 64 / LPP;  // pieces per wave instruction
  constexpr int kIn = 16;
  const int Hq = p.num_heads;
  const int wave = tid >> 6, lane = tid & 63;
  const int po = lane / LPP, d4 = (lane % LPP) * 4;
  const size_t step = (size_t)Hq * D;
  const float* base = p.ws_acc + ((size_t)first_slot * Hq + head) * D + d4;
  f32x4 x[kIn];
#pragma unroll
  for (int t = 0; t < kIn; ++t) {
    const int k = (t * W + wave) * PPW + po;
    x[t] = k < npieces ? *reinterpret_cast<const f32x4*>(base + (size_t)k * step) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int i = tid; i < npieces; i += 64 * W) {
    const size_t r = ((size_t)(first_slot + i) * Hq + head) * 2;
    sm.wgt[0][i] = p.ws_ml[r];
    sm.ls[0][i] = p.ws_ml[r + 1];
  }
  __syncthreads();
  if (wave == 0) {
    float M = kNegInf;
    for (int k = lane; k < npieces; k += 64) M = fmaxf(M, sm.wgt[0][k]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float den = 0.f;
    for (int k = lane; k < npieces; k += 64) {
      const float e = fast_exp2(sm.wgt[0][k] - M);
      sm.wgt[0][k] = e;
      den = fmaf(e, sm.ls[0][k], den);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
    const float inv = 1.f / den;
    for (int k = lane; k < npieces; k += 64) sm.wgt[0][k] *= inv;
  }
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < kIn; ++t) {
    const int k = (t * W + wave) * PPW + po;
    if (k < npieces) acc += sm.wgt[0][k] * x[t];
  }
#pragma unroll 4
  for (int k = (kIn * W + wave) * PPW + po; k < npieces; k += W * PPW)
    acc += sm.wgt[0][k] * *reinterpret_cast<const f32x4*>(base + (size_t)k * step);
#pragma unroll
  for (int off = LPP; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  if (po == 0) {
    sm.part[wave][0][d4] = acc.x;
    sm.part[wave][0][d4 + 1] = acc.y;
    sm.part[wave][0][d4 + 2] = acc.z;
    sm.part[wave][0][d4 + 3] = acc.w;
  }
  __syncthreads();
  for (int d = tid; d < D; d += 64 * W) {
    float o = sm.part[0][0][d];
#pragma unroll
    for (int v = 1; v < W; ++v) o += sm.part[v][0][d];
    store_out(p.out, ((size_t)s * Hq + head) * D + d, o, p.out_dtype);
  }
}

// The one-wave form (few pieces per sequence): lane l holds output elements
// l, l + 64, ... of every head; each lane's first kPre pieces are requested
// together with the (m, l) pairs.
template <int D>
__device__ void merge_heads_one_wave(const DecodeParams& p, MergeSmem<1>& sm, int s, int head0, int nh, int tid,
                                     int first_slot, int npieces) {
  constexpr int kPre = 4;
  const int Hq = p.num_heads;
  const int lane = tid;
  constexpr int PER = D / 64;
  const size_t step = (size_t)Hq * D;
  const float* acc0 = p.ws_acc + ((size_t)first_slot * Hq + head0) * D + lane;
  float pre[kPre][kMaxGroup][PER];
#pragma unroll
  for (int j = 0; j < kPre; ++j)
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        pre[j][h][i] = (h < nh && j < npieces) ? acc0[(size_t)h * D + j * step + 64 * i] : 0.f;
  // (m, l) of every (head, piece): m into wgt, l kept in the same slot's pair
  for (int i = tid; i < nh * npieces; i += 64) {
    const int h = i / npieces, k = i % npieces;
    const size_t r = ((size_t)(first_slot + k) * Hq + head0 + h) * 2;
    sm.wgt[h][k] = p.ws_ml[r];
    sm.ls[h][k] = p.ws_ml[r + 1];
  }
  __syncthreads();
  // weights: lane h walks head h's pieces
  if (tid < nh) {
    float M = kNegInf;
    for (int k = 0; k < npieces; ++k) M = fmaxf(M, sm.wgt[tid][k]);
    float den = 0.f;
    for (int k = 0; k < npieces; ++k) {
      const float e = fast_exp2(sm.wgt[tid][k] - M);
      sm.wgt[tid][k] = e;
      den = fmaf(e, sm.ls[tid][k], den);
    }
    const float inv = 1.f / den;
    for (int k = 0; k < npieces; ++k) sm.wgt[tid][k] *= inv;
  }
  __syncthreads();
  float acc[kMaxGroup][PER];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[h][i] = 0.f;
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    if (j < npieces) {
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h < nh) {
          const float w = sm.wgt[h][j];
#pragma unroll
          for (int i = 0; i < PER; ++i) acc[h][i] = fmaf(w, pre[j][h][i], acc[h][i]);
        }
      }
    }
  }
#pragma unroll 2
  for (int k = kPre; k < npieces; ++k) {
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < nh) {
        const float w = sm.wgt[h][k];
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[h][i] = fmaf(w, acc0[(size_t)h * D + k * step + 64 * i], acc[h][i]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h)
    if (h < nh)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        store_out(p.out, ((size_t)s * Hq + head0 + h) * D + lane + 64 * i, acc[h][i], p.out_dtype);
}

// Combines the pieces of query heads head0 .. head0+nh-1 of sequence s when
// it was split; called by the whole workgroup. L_raw and the split record
// (meta_first, meta_n; balanced mode) were loaded by the caller.
template <int D, int W>
__device__ void merge_sequence(const DecodeParams& p, MergeSmem<W>& sm, int s, int head0, int nh, int tid, int L_raw,
                               int meta_first, int meta_n) {
  static_assert(D <= 128, "partial-sum tile");
  const int L = capped_len(p, L_raw);
  if (L <= 0) return;
  int first_slot, npieces;
  if (p.mode != kModeBalanced) {
    const int P = p.part_chunks * kChunk;
    npieces = (L + P - 1) / P;
    first_slot = s * p.max_parts;
  } else {
    first_slot = meta_first;
    npieces = meta_n;
  }
  if (npieces <= 1) return;
  if (npieces > kMergeTile) {
    merge_long<D, W>(p, s, head0, nh, tid, first_slot, npieces);
  } else if constexpr (W > 1) {
    // the W-wave launch gives each workgroup one query head
    if (nh == 1) merge_one_head<D, W>(p, sm, s, head0, tid, first_slot, npieces);
    else merge_long<D, W>(p, s, head0, nh, tid, first_slot, npieces);
  } else {
    merge_heads_one_wave<D>(p, sm, s, head0, nh, tid, first_slot, npieces);
  }
}

// Position-L-1 slot of sequence s for the fused write, or -1 when no write is
// made: the conditions under which the attention kernel took that position
// from k_new/v_new (new_token_pos), and a table entry inside the pool.
__device__ __forceinline__ int new_token_slot(const DecodeParams& p, int s, int L) {
  if (L <= 0 || capped_len(p, L) != L) return -1;
  const int t = L - 1;
  const int phys = p.block_tables[(size_t)s * p.max_blocks_per_seq + (t >> p.log2_block)];
  if (phys < 0 || phys >= p.num_blocks) return -1;  // no such slot: nothing stored, as in the plain write
  return phys * p.block_size + (t & (p.block_size - 1));
}

// The launch after the attention kernel: workgroups of W waves, grid
// (sequences, KV heads, head split Z) with g / Z query heads each. It merges
// the sequence's pieces when it was split and, for pa_write_decode, the
// z = 0 workgroup stores the new token into the cache. That store follows
// every read of the cache by the attention kernel, which took the new token
// from k_new/v_new; its values are read first and stored last, so its round
// trips overlap the merge's.
template <int D, typename U, int W>
__global__ __launch_bounds__(64 * W) void merge_kernel(DecodeParams p) {
  __shared__ MergeSmem<W> sm;
  const int s = blockIdx.x, kvh = blockIdx.y, tid = threadIdx.x;
  const int Hkv = p.num_kv_heads;
  const int nh = p.group / gridDim.z, head0 = kvh * p.group + (int)blockIdx.z * nh;
  // every load that depends on nothing else is issued first
  const int L = p.context_lens[s];
  int meta_first = 0, meta_n = 0;
  if (p.merge && p.mode == kModeBalanced) {
    meta_first = p.ws_meta[2 * s];
    meta_n = p.ws_meta[2 * s + 1];
  }
  // the new token's elements e = tid, tid + 64W, ..., read unconditionally
  // (from q without one: an in-bounds row, never stored) and widened, so
  // nothing waits for them before the merge
  constexpr int NE = (D + 64 * W - 1) / (64 * W);
  uint32_t kn[NE], vn[NE];
  {
    const size_t src = ((size_t)s * Hkv + kvh) * D;
    const U* ks = static_cast<const U*>(p.k_new ? p.k_new : p.q) + src;
    const U* vs = static_cast<const U*>(p.v_new ? p.v_new : p.q) + src;
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int e = min(tid + 64 * W * j, D - 1);
      kn[j] = ks[e];
      vn[j] = vs[e];
    }
  }
  // the slot's block-table entry is requested before the merge's loads
  const int slot = (p.k_new && blockIdx.z == 0) ? new_token_slot(p, s, L) : -1;
  if (p.merge) merge_sequence<D, W>(p, sm, s, head0, nh, tid, L, meta_first, meta_n);
  if (slot >= 0) {
    const int B = p.block_size, phys = slot / B, off = slot % B, Bs = v_subtile(B);
    U* kd = const_cast<U*>(static_cast<const U*>(p.k_cache)) + (((size_t)phys * Hkv + kvh) * B + off) * D;
    U* vd = const_cast<U*>(static_cast<const U*>(p.v_cache)) + v_elem(phys, Hkv, kvh, D, B, Bs, 0, off);
    // non-temporal: the V column dirties one cache line per element, and
    // left in the cache those partial lines were written back during the
    // next decode's stream, slowing it by about 5%
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int e = tid + 64 * W * j;
      if (e < D) {
        __builtin_nontemporal_store(static_cast<U>(kn[j]), kd + e);
        __builtin_nontemporal_store(static_cast<U>(vn[j]), vd + (size_t)e * Bs);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// KV write, block copy, swap
// ---------------------------------------------------------------------------
template <typename U>
__global__ __launch_bounds__(64) void write_kv_kernel(const U* __restrict__ k_new, const U* __restrict__ v_new,
                                                      U* __restrict__ k_cache, U* __restrict__ v_cache,
                                                      const int32_t* __restrict__ slots, int Hkv, int D, int B,
                                                      long long total_slots) {
  const int n = blockIdx.x, h = blockIdx.y;
  const int slot = slots[n];
  if (slot < 0 || (long long)slot >= total_slots) return;
  const int phys = slot / B, off = slot % B, Bs = v_subtile(B);
  const U* kr = k_new + ((size_t)n * Hkv + h) * D;
  const U* vr = v_new + ((size_t)n * Hkv + h) * D;
  U* kd = k_cache + (((size_t)phys * Hkv + h) * B + off) * D;
  U* vd = v_cache + v_elem(phys, Hkv, h, D, B, Bs, 0, off);
  // non-temporal, like the fused write's store: the V column's partial lines
  // must not linger in the cache into the decode that reads the pool next
  for (int i = threadIdx.x; i < D; i += 64) {
    __builtin_nontemporal_store(kr[i], kd + i);
    __builtin_nontemporal_store(vr[i], vd + (size_t)i * Bs);
  }
}

template <typename U>
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* k_cache, uint8_t* v_cache,
                                                          const int32_t* __restrict__ mapping, int num_blocks,
                                                          size_t block_bytes) {
  const int pair = blockIdx.x;
  const int src = mapping[2 * pair], dst = mapping[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint8_t* base = blockIdx.y ? v_cache : k_cache;
  const U* s = reinterpret_cast<const U*>(base + (size_t)src * block_bytes);
  U* d = reinterpret_cast<U*>(base + (size_t)dst * block_bytes);
  const size_t n = block_bytes / sizeof(U);
  for (size_t i = (size_t)blockIdx.z * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.z * blockDim.x)
    d[i] = s[i];
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
// 32-token sub-chunks per MFMA step. Two (32 KiB of K/V in flight per wave)
// measured slower on MI355X than one: bytes in flight are not the limit.
constexpr int kMfmaSub = 1;

template <class Eng, int D>
const void* kernel_of() {
  return reinterpret_cast<const void*>(&decode_kernel<Eng, D>);
}

template <int E, int D>
const void* vec_kernel(int G) {
  switch (G) {
    case 1: return kernel_of<VecEngine<E, D, 1>, D>();
    case 2: return kernel_of<VecEngine<E, D, 2>, D>();
    case 4: return kernel_of<VecEngine<E, D, 4>, D>();
    case 8: return kernel_of<VecEngine<E, D, 8>, D>();
    default: return nullptr;
  }
}

template <int E>
const void* vec_kernel_d(int D, int G) {
  return D == 64 ? vec_kernel<E, 64>(G) : (D == 128 ? vec_kernel<E, 128>(G) : nullptr);
}

const void* decode_fn(int elem, int head_dim, int algo, int G) {
  if (algo == kAlgoMfma) {
    if (elem == kBF16) return head_dim == 64 ? kernel_of<MfmaEngine<kBF16, 64, kMfmaSub>, 64>()
                                             : (head_dim == 128 ? kernel_of<MfmaEngine<kBF16, 128, kMfmaSub>, 128>() : nullptr);
    if (elem == kF16) return head_dim == 64 ? kernel_of<MfmaEngine<kF16, 64, kMfmaSub>, 64>()
                                            : (head_dim == 128 ? kernel_of<MfmaEngine<kF16, 128, kMfmaSub>, 128>() : nullptr);
    return nullptr;
  }
  if (elem == kF32) return vec_kernel_d<kF32>(head_dim, G);
  if (elem == kF16) return vec_kernel_d<kF16>(head_dim, G);
  if (elem == kBF16) return vec_kernel_d<kBF16>(head_dim, G);
  return nullptr;
}

}  // namespace

size_t decode_static_lds(int elem, int head_dim, int algo, int G) {
  if (algo == kAlgoMfma) {
    if (elem == kF32) return 0;
    return head_dim == 64 ? sizeof(MfmaEngine<kBF16, 64, kMfmaSub>::Smem) : sizeof(MfmaEngine<kBF16, 128, kMfmaSub>::Smem);
  }
  const int D = head_dim;
  switch (G) {
    case 1: return D == 64 ? sizeof(VecEngine<kF32, 64, 1>::Smem) : sizeof(VecEngine<kF32, 128, 1>::Smem);
    case 2: return D == 64 ? sizeof(VecEngine<kF32, 64, 2>::Smem) : sizeof(VecEngine<kF32, 128, 2>::Smem);
    case 4: return D == 64 ? sizeof(VecEngine<kF32, 64, 4>::Smem) : sizeof(VecEngine<kF32, 128, 4>::Smem);
    default: return D == 64 ? sizeof(VecEngine<kF32, 64, 8>::Smem) : sizeof(VecEngine<kF32, 128, 8>::Smem);
  }
}

hipError_t launch_decode(const DecodeParams& p, int elem, int head_dim, int algo, int G, unsigned workers,
                         bool merge, size_t lds_per_workgroup, hipStream_t stream) {
  const void* fn = decode_fn(elem, head_dim, algo, G);
  if (!fn) return hipErrorInvalidDeviceFunction;
  DecodeParams args = p;
  args.merge = merge ? 1 : 0;
  // dynamic LDS: the lengths (balanced split and partition stream), then as
  // many result slots as the workgroup's share of the CU's LDS leaves room
  // for (at least one; one segment per workgroup needs no more)
  args.lens_pad = p.mode == kModeFixed ? 0 : (p.num_seqs + 3) / 4 * 4;
  const size_t lens_bytes = (size_t)args.lens_pad * sizeof(int32_t);
  const size_t slot_bytes = ((size_t)p.group * head_dim + 2 * (size_t)p.group + kResRec) * sizeof(float);
  const size_t fixed = decode_static_lds(elem, head_dim, algo, G) + lens_bytes;
  size_t slots = lds_per_workgroup > fixed ? (lds_per_workgroup - fixed) / slot_bytes : 0;
  if (p.mode == kModeFixed || slots < 1) slots = 1;
  if (slots > (size_t)kMaxResultSlots) slots = kMaxResultSlots;
  args.res_slots = (int)slots;
  void* kargs[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3(workers, (unsigned)p.num_kv_heads, 1), dim3(64, 1, 1), kargs,
                                 lens_bytes + slots * slot_bytes, stream);
  // the closing launch merges split sequences and stores the fused write
  if (e != hipSuccess || (!merge && !p.k_new)) return e;
  // few pieces per sequence: one wave per (sequence, KV head); many (fixed
  // partitions, or a balanced split of few sequences over many workers):
  // four waves per (sequence, query head)
  const bool wide = merge && (p.mode == kModeBalanced ? (long long)workers > 4LL * p.num_seqs : p.max_parts > 4);
  const void* mf;
  if (wide) {
    if (elem == kF32)
      mf = head_dim == 64 ? reinterpret_cast<const void*>(&merge_kernel<64, uint32_t, 4>)
                          : reinterpret_cast<const void*>(&merge_kernel<128, uint32_t, 4>);
    else
      mf = head_dim == 64 ? reinterpret_cast<const void*>(&merge_kernel<64, uint16_t, 4>)
                          : reinterpret_cast<const void*>(&merge_kernel<128, uint16_t, 4>);
  } else {
    if (elem == kF32)
      mf = head_dim == 64 ? reinterpret_cast<const void*>(&merge_kernel<64, uint32_t, 1>)
                          : reinterpret_cast<const void*>(&merge_kernel<128, uint32_t, 1>);
    else
      mf = head_dim == 64 ? reinterpret_cast<const void*>(&merge_kernel<64, uint16_t, 1>)
                          : reinterpret_cast<const void*>(&merge_kernel<128, uint16_t, 1>);
  }
  const unsigned z = wide ? (unsigned)p.group : 1u;
  return hipLaunchKernel(mf, dim3((unsigned)p.num_seqs, (unsigned)p.num_kv_heads, z), dim3(wide ? 256 : 64, 1, 1),
                         kargs, 0, stream);
}

int decode_waves_per_cu(int elem, int head_dim, int algo, int G) {
  const void* fn = decode_fn(elem, head_dim, algo, G);
  if (!fn) return 0;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, 64, 0) != hipSuccess) return 0;
  return blocks;
}

hipError_t launch_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache, const int32_t* slots,
                           int num_tokens, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           int elem_bytes, hipStream_t stream) {
  const dim3 grid((unsigned)num_tokens, (unsigned)num_kv_heads), block(64);
  const long long total = (long long)num_blocks * block_size;
  if (elem_bytes == 4) {
    hipLaunchKernelGGL(write_kv_kernel<uint32_t>, grid, block, 0, stream, static_cast<const uint32_t*>(k_new),
                       static_cast<const uint32_t*>(v_new), static_cast<uint32_t*>(k_cache),
                       static_cast<uint32_t*>(v_cache), slots, num_kv_heads, head_dim, block_size, total);
  } else {
    hipLaunchKernelGGL(write_kv_kernel<uint16_t>, grid, block, 0, stream, static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), static_cast<uint16_t*>(k_cache),
                       static_cast<uint16_t*>(v_cache), slots, num_kv_heads, head_dim, block_size, total);
  }
  return hipGetLastError();
}

// One workgroup slice per (pair, K/V): 16-byte (or byte) moves between a
// pool block and its host slot image.
template <typename U, bool OUT>
__global__ __launch_bounds__(256) void swap_kernel(uint8_t* k_cache, uint8_t* v_cache, uint8_t* host,
                                                   const int32_t* __restrict__ mapping, int num_blocks,
                                                   int host_slots, size_t block_bytes) {
  const int pair = blockIdx.x;
  const int blk = mapping[2 * pair], slot = mapping[2 * pair + 1];
  if (blk < 0 || blk >= num_blocks || slot < 0 || slot >= host_slots) return;
  uint8_t* pool = (blockIdx.y ? v_cache : k_cache) + (size_t)blk * block_bytes;
  uint8_t* img = host + ((size_t)slot * 2 + blockIdx.y) * block_bytes;
  const U* s = reinterpret_cast<const U*>(OUT ? pool : img);
  U* d = reinterpret_cast<U*>(OUT ? img : pool);
  const size_t n = block_bytes / sizeof(U);
  for (size_t i = (size_t)blockIdx.z * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.z * blockDim.x)
    d[i] = s[i];
}

hipError_t launch_swap(void* k_cache, void* v_cache, void* host, const int32_t* mapping, int num_pairs,
                       int num_blocks, int host_slots, size_t block_bytes, bool out, hipStream_t stream) {
  uint8_t* k = static_cast<uint8_t*>(k_cache);
  uint8_t* v = static_cast<uint8_t*>(v_cache);
  uint8_t* h = static_cast<uint8_t*>(host);
  const bool wide = block_bytes % 16 == 0;
  const size_t n = wide ? block_bytes / 16 : block_bytes;
  const unsigned slices = (unsigned)((n + 255) / 256 < 64 ? (n + 255) / 256 : 64);
  const dim3 grid((unsigned)num_pairs, 2, slices), block(256);
  if (wide && out)
    hipLaunchKernelGGL((swap_kernel<u32x4, true>), grid, block, 0, stream, k, v, h, mapping, num_blocks, host_slots,
                       block_bytes);
  else if (wide)
    hipLaunchKernelGGL((swap_kernel<u32x4, false>), grid, block, 0, stream, k, v, h, mapping, num_blocks,
                       host_slots, block_bytes);
  else if (out)
    hipLaunchKernelGGL((swap_kernel<uint8_t, true>), grid, block, 0, stream, k, v, h, mapping, num_blocks,
                       host_slots, block_bytes);
  else
    hipLaunchKernelGGL((swap_kernel<uint8_t, false>), grid, block, 0, stream, k, v, h, mapping, num_blocks,
                       host_slots, block_bytes);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* mapping, int num_pairs, int num_blocks,
                              size_t block_bytes, hipStream_t stream) {
  uint8_t* k = static_cast<uint8_t*>(k_cache);
  uint8_t* v = static_cast<uint8_t*>(v_cache);
  if (block_bytes % 16 == 0) {
    const size_t n = block_bytes / 16;
    const unsigned slices = (unsigned)((n + 255) / 256 < 64 ? (n + 255) / 256 : 64);
    hipLaunchKernelGGL(copy_blocks_kernel<u32x4>, dim3((unsigned)num_pairs, 2, slices), dim3(256), 0, stream, k, v,
                       mapping, num_blocks, block_bytes);
  } else {
    const unsigned slices = (unsigned)((block_bytes + 255) / 256 < 64 ? (block_bytes + 255) / 256 : 64);
    hipLaunchKernelGGL(copy_blocks_kernel<uint8_t>, dim3((unsigned)num_pairs, 2, slices), dim3(256), 0, stream, k, v,
                       mapping, num_blocks, block_bytes);
  }
  return hipGetLastError();
}

}  // namespace pa
