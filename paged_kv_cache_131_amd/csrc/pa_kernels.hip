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

#include <climits>
#include <mutex>

#include "pa_device.h"
#include "pa_internal.h"

// Decode workspace of pa_decode_noalloc: a fixed array per device, so that
// callers that cannot allocate still get the split path. Host code never
// passes this name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address static_scratch() looks up. Static
// storage: zero when the code object is loaded, as the arrival counters at
// the start of every decode workspace must be before their first use.
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
// table can address and to the host's bound max_context_len (in every split
// mode: the partitions and workspaces are sized from that bound).
__device__ __forceinline__ int capped_len(const DecodeParams& p, int L_raw) {
  return min(min(L_raw, p.max_blocks_per_seq << p.log2_block), p.max_len);
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

// What the piece holding an item's first chunk records for the merge
// (bits of Segment::kind): where the sequence's own pieces are, where its
// family's pieces are, or that it has no family (shared mode).
enum RecordKind : int { kRecOwn = 1, kRecFamily = 2, kRecNoFamily = 4 };

// One share of a worker's work: tokens [t0, t1) of sequences s .. s +
// members - 1 (more than one: the common prefix of a family, which maps the
// same blocks in every member), whose last logical block is lbl; tnew is
// the position of the token the fused write stores (the sequence's last,
// when this piece holds it and the call brings one), else -1. slot and
// first_slot are partial-result slots (of member 0 for a family: member m
// adds m); direct: the piece is a whole sequence and writes its output.
// flags (shared mode only; the other modes derive the same from t0 and
// npieces): members in bits 0-15, RecordKind bits the piece records when it
// holds the item's first chunk in bits 16-18, direct in bit 19.
struct Segment {
  int s, t0, t1, lbl, npieces, slot, first_slot;
  int tnew;
  int valid;
  int flags;
};

__device__ __forceinline__ int segment_flags(int members, int kind, int direct) {
  return members | (kind << 16) | (direct << 19);
}

__device__ __forceinline__ Segment invalid_segment() {
  Segment g;
  g.s = g.t0 = g.t1 = g.lbl = g.npieces = g.slot = g.first_slot = 0;
  g.tnew = -1;
  g.valid = 0;
  g.flags = segment_flags(1, 0, 0);
  return g;
}

// The family kernel (SHARED true) runs the shared mode only, the others
// never do.
template <bool SHARED>
__device__ __forceinline__ int seg_members(const Segment& g) {
  return SHARED ? (g.flags & 0xffff) : 1;
}
// Output of a whole sequence, written directly (no merge).
template <bool SHARED>
__device__ __forceinline__ int seg_direct(const Segment& g) {
  return SHARED ? (g.flags >> 19) & 1 : g.npieces == 1;
}
// Split record the piece writes: the piece holding a sequence's first token
// in the balanced split (single pieces too, so the merge never reads a stale
// record); the plan's choice in shared mode; none with fixed partitions.
template <bool SHARED>
__device__ __forceinline__ int seg_kind(const DecodeParams& p, const Segment& g) {
  if (SHARED) return (g.flags >> 16) & 7;
  return p.mode == kModeBalanced && g.t0 == 0 ? kRecOwn : 0;
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
  g.flags = __builtin_amdgcn_readfirstlane(g.flags);
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
// One column group (NCG = 1): a sequence takes 2g consecutive head slots:
// c < g carry head c with P rounded to 16 bits ("hi"), g <= c < 2g carry
// head c-g with the rounding residual ("lo"); the two PV results are added at
// the end, so P enters the product with ~16 significant bits instead of 8.
// Slots no sequence takes are zero.
// NCG 16-slot column groups (family kernel): every slot carries a distinct
// (member, head) pair, 16/g members per group, all against the same K and V
// registers, so the blocks a family shares are read once for all of them;
// P enters PV as two products into the same accumulator, the rounded part
// and its residual.
// ---------------------------------------------------------------------------
template <int E, int D, int SUB, int NCG>
struct MfmaEngine {
  using Tr = ElemT<E>;
  using op8 = typename Tr::op8;
  using scalar = typename Tr::scalar;
  using raw = typename Tr::raw;
  static constexpr int kSub = SUB;   // 32-token sub-chunks per step
  static constexpr int kGroups = NCG;
  static constexpr bool kDistinct = NCG > 1;  // distinct (member, head) slots, P's parts in two products
  static constexpr int MQ = D / 32;  // QK k-steps
  static constexpr int NT = D / 16;  // PV column tiles
  static constexpr int kPad = 4;
  static constexpr int kMaxGroup = pa::kMaxGroup;  // a sequence's heads per KV head (one result)
  struct alignas(16) Smem {
    float o[16][D + kPad];
    float ml[16][2];
  };

  op8 qop[NCG][MQ];
  f32x4 o[NCG][NT];
  float m_run[NCG];
  float l_run[NCG];
  uint32_t vn[NT];  // the segment's new token's V at this lane's output columns 16j + col
  int ncg;          // column groups the current segment uses

  // q of every column group as the QK B operand (columns = head slots), and
  // the new token's V values this lane's B operands carry (fused write)
  struct Q {
    u32x4 w[NCG][MQ];
    uint32_t vn[NT];
  };

  // Head of the segment's member `member` that this lane's column carries
  // in column group cg, or -1 (a slot no member takes).
  __device__ static int column_head(int g, int members, int cg, int col, int& member) {
    if (!kDistinct) {
      member = 0;
      return col < g ? col : (col < 2 * g ? col - g : -1);
    }
    const int per = 16 / g, mi = col / g;
    member = cg * per + mi;
    if (mi >= per || member >= members) return -1;
    return col - mi * g;
  }

  // Part of P this lane's column carries: 0 rounded, 1 residual, 2 none
  // (one column group; the family kernel uses both parts in every column).
  __device__ static int column_part(int g, int col) { return col < g ? 0 : (col < 2 * g ? 1 : 2); }

  __device__ __forceinline__ static void load_q_group(u32x4* w, const DecodeParams& p, int s, int members, int cg, int kvh,
                                      int lane) {
    const int col = lane & 15, grp = lane >> 4, g = p.group;
    int member;
    const int hs = column_head(g, members, cg, col, member);
    const raw* qb = static_cast<const raw*>(p.q) + ((size_t)(s + (hs >= 0 ? member : 0)) * p.num_heads +
                                                    (size_t)kvh * g) * D;
#pragma unroll
    for (int m = 0; m < MQ; ++m) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (hs >= 0) x = load16(qb + (size_t)hs * D + 32 * m + 8 * grp);
      w[m] = x;
    }
  }

  __device__ __forceinline__ void load_q(Q& q, const DecodeParams& p, const Segment& seg, int kvh, int lane) const {
    const int col = lane & 15;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) load_q_group(q.w[cg], p, seg.s, seg_members<kDistinct>(seg), cg, kvh, lane);
    // read unconditionally (from q when the call brings no new token: an
    // in-bounds row, never used) so every segment issues the same loads
    const raw* vb = static_cast<const raw*>(p.v_new ? p.v_new : p.q) + ((size_t)seg.s * p.num_kv_heads + kvh) * D + col;
#pragma unroll
    for (int j = 0; j < NT; ++j) q.vn[j] = vb[16 * j];
  }

  // Start a segment with its q (loaded during the previous segment's last
  // chunk, every column group for every segment, so the code path is the
  // same whether a segment is a family's or not).
  __device__ __forceinline__ void reset(const Q& q, const DecodeParams& p, const Segment& seg, int kvh, int lane, Smem& sm) {
    if (NCG == 1) {
      ncg = 1;
    } else {
      const int per = 16 / p.group;
      ncg = min((seg_members<kDistinct>(seg) + per - 1) / per, NCG);
    }
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int m = 0; m < MQ; ++m) qop[cg][m] = __builtin_bit_cast(op8, q.w[cg][m]);
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
#pragma unroll
      for (int j = 0; j < NT; ++j) o[cg][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run[cg] = kNegInf;
      l_run[cg] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) vn[j] = q.vn[j];
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

  // QK of column group cg: in sub-chunk u the lane holds tokens
  // cs+32u+8*grp+0..7 of head slot `col`, scaled to base-2 units and masked
  // past the segment's end.
  __device__ __forceinline__ void scores(const Frag& f, const DecodeParams& p, const op8 (&qg)[MQ], int grp, int cs, int t1,
                         bool partial, float (&sv)[SUB][8]) const {
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < MQ; ++m) {
        s0 = mfma_16x16x32(__builtin_bit_cast(op8, f.ka[u][0][m]), qg[m], s0);
        s1 = mfma_16x16x32(__builtin_bit_cast(op8, f.ka[u][1][m]), qg[m], s1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[u][i] = s0[i] * p.scale_log2;
        sv[u][4 + i] = s1[i] * p.scale_log2;
      }
    }
    if (partial) {
#pragma unroll
      for (int u = 0; u < SUB; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[u][e] = (cs + kChunk * u + 8 * grp + e < t1) ? sv[u][e] : kNegInf;
    }
  }

  // Online softmax (base 2) of column group cg's scores and its PV products
  // with the chunk's V (P as a rounded part or its residual, by head slot).
  __device__ __forceinline__ void softmax_pv(const Frag& f, int cg, int grp, int part, float (&sv)[SUB][8]) {
    float cmax = kNegInf;
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) cmax = fmaxf(cmax, sv[u][e]);
    cmax = max_over_column(cmax);
    const float m_new = fmaxf(m_run[cg], cmax);
    const float alpha = fast_exp2(m_run[cg] - m_new);
    float pe[SUB][8];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < SUB; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pe[u][e] = fast_exp2(sv[u][e] - m_new);
        psum += pe[u][e];
      }
    l_run[cg] = l_run[cg] * alpha + psum;
    m_run[cg] = m_new;
    if (__any(alpha != 1.f)) {
      // output rows of this lane are head slots 4*grp+i; their factor lives in lane 4*grp+i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * grp + i);
#pragma unroll
        for (int j = 0; j < NT; ++j) o[cg][j][i] *= ai;
      }
    }
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      if constexpr (kDistinct) {
        op8 phi, plo;
        Tr::split(pe[u], phi, plo);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          o[cg][j] = mfma_16x16x32(phi, __builtin_bit_cast(op8, f.vr[u][j]), o[cg][j]);
          o[cg][j] = mfma_16x16x32(plo, __builtin_bit_cast(op8, f.vr[u][j]), o[cg][j]);
        }
      } else {
        op8 pa;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const scalar hi = static_cast<scalar>(pe[u][e]);
          const scalar lo = static_cast<scalar>(pe[u][e] - static_cast<float>(hi));
          pa[e] = part == 0 ? hi : (part == 1 ? lo : static_cast<scalar>(0.f));
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) o[cg][j] = mfma_16x16x32(pa, __builtin_bit_cast(op8, f.vr[u][j]), o[cg][j]);
      }
    }
  }

  // Compute the step at `cs` from `f`; as soon as a register set is
  // consumed it is refilled with the next step (K after the last QK, V after
  // the last PV), so one step's loads are always in flight behind the math.
  // Column groups run one after the other: group cg's QK, softmax and PV
  // (the K refill waits for the last group's QK). The stream's last step
  // (REFILL false) loads nothing.
  template <bool REFILL>
  __device__ __forceinline__ void step(Frag& f, const DecodeParams& p, Smem& sm, int kvh, int lane, int cs, const Segment& cur,
                       int cs_next, const ChunkIds* ids_next, const Segment& nxt) {
    const int col = lane & 15, grp = lane >> 4, g = p.group;
    const int t1 = cur.t1;
    const int nact = NCG == 1 ? 1 : ncg;
    const bool has_new = cur.tnew >= cs && cur.tnew < cs + SUB * kChunk;
    const bool partial = cs + SUB * kChunk > t1;
    const int part = kDistinct ? 0 : column_part(g, col);
    float sv[SUB][8];
    scores(f, p, qop[0], grp, cs, t1, partial, sv);
    if (NCG == 1 && REFILL) {
      // the refill of every step but the last (a separate copy of the step)
      // is unconditional: the count of loads in flight is the same on every
      // path of this code, so the PV wait below never has to drain the next
      // step's K loads
      load_k(f, p, kvh, lane, cs_next, ids_next, nxt);
    }
    // V of tokens past the segment's end is selected out (never multiplied),
    // the new token's V replaces what its slot held before this launch
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      if (partial) {
        const int nvalid = t1 - (cs + kChunk * u + 8 * grp);
#pragma unroll
        for (int j = 0; j < NT; ++j) f.vr[u][j] = Tr::keep_first(f.vr[u][j], nvalid);
      }
      if (has_new) {
        const int e = cur.tnew - (cs + kChunk * u + 8 * grp);
        const int en = e >= 0 && e < 8 ? e : -1;
#pragma unroll
        for (int j = 0; j < NT; ++j) f.vr[u][j] = put_elem<raw>(f.vr[u][j], en, vn[j]);
      }
    }
    softmax_pv(f, 0, grp, part, sv);
    if constexpr (NCG > 1) {
#pragma unroll
      for (int cg = 1; cg < NCG; ++cg) {
        if (cg < nact) {
          scores(f, p, qop[cg], grp, cs, t1, partial, sv);
          softmax_pv(f, cg, grp, part, sv);
        }
      }
    }
    if (REFILL) {
      if (NCG > 1) load_k(f, p, kvh, lane, cs_next, ids_next, nxt);
      load_v(f, p, kvh, lane, cs_next, ids_next, nxt);
    }
  }

  // Column group cg's results into sm: o[head slot][dd], (m, l) per slot.
  __device__ __forceinline__ void finish(Smem& sm, int lane, int cg) {
    const int col = lane & 15, grp = lane >> 4;
    const float l_tot = sum_over_column(l_run[cg]);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.o[4 * grp + i][16 * j + col] = o[cg][j][i];
    if (grp == 0) {
      sm.ml[col][0] = m_run[cg];
      sm.ml[col][1] = l_tot;
    }
    __syncthreads();
  }

  // members whose results group cg holds, and the first head slot of member mi
  __device__ int members_in_group(const DecodeParams& p, const Segment& g, int cg) const {
    if (!kDistinct) return 1;
    const int per = 16 / p.group;
    return max(0, min(per, seg_members<kDistinct>(g) - cg * per));
  }
  __device__ static int member_row(const DecodeParams& p, int mi) { return kDistinct ? mi * p.group : 0; }
  __device__ static int member_of(const DecodeParams& p, int cg, int mi) {
    return kDistinct ? cg * (16 / p.group) + mi : 0;
  }

  // outputs dd..dd+3 of head h (dd a multiple of 4)
  __device__ static f32x4 o_val4(const Smem& sm, int row, int h, int dd, int g) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.o[row + h][dd]);
    if (kDistinct) return a;
    return a + *reinterpret_cast<const f32x4*>(&sm.o[row + h + g][dd]);
  }
  __device__ static float m_val(const Smem& sm, int row, int h) { return sm.ml[row + h][0]; }
  __device__ static float l_val(const Smem& sm, int row, int h) { return sm.ml[row + h][1]; }
};

// ---------------------------------------------------------------------------
// Vector engine (any element type, group bucket G >= g).
//
// QK: 16-byte coalesced loads of token rows, LPR lanes per row (a K group),
// partial dot products (two-element dot instructions on 16-bit elements, fp32
// FMAs on fp32 ones) reduced across those lanes by DPP moves, so that every
// lane of K group q holds the scores of its tokens q*KSTEPS .. +KSTEPS-1.
// PV: 8 consecutive tokens at one dd per lane (one 16-byte load of 16-bit
// elements, two of fp32) from the token-minor V tile, taken from the lane's
// own K group's tokens, so the lane forms their
// weights itself; the chunk maximum crosses the groups by lane swaps. No LDS
// inside the chunk loop; accumulators are reduced across lanes at the end.
// ---------------------------------------------------------------------------
template <int E, int D, int G>
struct VecEngine {
  using Tr = ElemT<E>;
  using raw = typename Tr::raw;
  static constexpr int VEC = Tr::kVec;
  static constexpr int LPR = D / VEC;           // lanes per K row (one K group)
  static constexpr int RPS = 64 / LPR;          // K groups: rows per load step
  static constexpr int KSTEPS = kChunk / RPS;   // K load steps per chunk = tokens per K group
  // A V lane takes TV = 8 consecutive tokens (VPL 16-byte loads per dd row;
  // always inside one row of the token-minor V tile) of its own K group (NTG
  // token groups per K group), or, when a K group holds fewer than TV tokens
  // (16-bit elements, head_dim 64), of two neighbouring K groups (kPair).
  // Eight tokens rather than one load's worth for fp32: half the partial
  // sums per lane (fp32, head_dim 128, four heads: 482 registers and no
  // spill, against 512 and 116 bytes of scratch).
  static constexpr int TV = 8;
  static constexpr int VPL = TV / VEC;
  static constexpr bool kPair = KSTEPS < TV;
  static constexpr int NTG = kPair ? 1 : KSTEPS / TV;
  static constexpr int VLANES = kPair ? 2 * LPR : LPR;  // lanes of one V group
  static constexpr int DPS = VLANES / NTG;      // dd rows per V load step
  static constexpr int VSTEPS = D / DPS;        // V load steps per chunk
  static_assert(kPair ? (VLANES == 16 && KSTEPS * 2 == TV) : (KSTEPS % TV == 0), "lane layout");
  // QK by two-element dot instructions (16-bit elements), except bf16 with
  // one query head per KV head, where widening is two bit operations per
  // pair and FMAs measured faster (OPT-13B shape 205.8 vs 209.8 us); fp16
  // widening takes a conversion per element (209.3 vs 211.1 us with dot2)
  static constexpr bool kDot = E == kF16 || (E == kBF16 && G > 1);
  // Scores of every head held at once (the K refill issued before the
  // softmax) unless they take more than 64 registers (fp32, head_dim 128,
  // eight heads: spilled 728 bytes per lane); then head by head.
  static constexpr bool kPerHead = G * KSTEPS > 64;
  static constexpr int kSub = 1;
  static constexpr int kGroups = 1;
  static constexpr int kMaxGroup = G;
  struct alignas(16) Smem {
    float o[G][D];
    float ml[G][2];
  };

  u32x4 qr[G];  // this lane's piece of q, as stored
  float acc[G][VSTEPS];
  float m_run[G];
  float l_run[G];
  uint32_t vn[VSTEPS];  // the segment's new token's V at this lane's dd rows

  // lane roles: K group kq (token rows kq * KSTEPS + st), piece of the row;
  // V group, its first token (relative to the chunk) and the lane's dd row
  __device__ static int kq(int lane) { return lane / LPR; }
  __device__ static int v_tok(int lane) {
    return kPair ? (lane / VLANES) * TV : kq(lane) * KSTEPS + (lane % LPR) % NTG * TV;
  }
  __device__ static int v_row(int lane) { return kPair ? lane % VLANES : (lane % LPR) / NTG; }

  struct Q {
    u32x4 w[G];
    uint32_t vn[VSTEPS];
  };

  __device__ void load_q(Q& q, const DecodeParams& p, const Segment& seg, int kvh, int lane) const {
    const int s = seg.s;
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
                    v_row(lane);
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st) q.vn[st] = vb[st * DPS];
  }

  __device__ void reset(const Q& q, const DecodeParams&, const Segment&, int, int, Smem&) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      qr[h] = q.w[h];
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
    u32x4 vr[VSTEPS][VPL];
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
      const int tok = cs + kq(lane) * KSTEPS + st;
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
    const int tv = cs + v_tok(lane);
    const int physv = pick_block(ids, tv, lg, lbl, p.num_blocks);
    const int Bs = v_subtile(B);
    const raw* vb = vc + v_elem(physv, Hkv, kvh, D, B, Bs, v_row(lane), tv & (B - 1));
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st)
#pragma unroll
      for (int u = 0; u < VPL; ++u) f.vr[st][u] = load16_stream(vb + (size_t)st * DPS * Bs + u * VEC);
  }

  // Scores (log2 units, -inf past t1) of head h for this lane's K group's
  // KSTEPS tokens, k0 the group's first.
  __device__ __forceinline__ void qk_head(const Frag& f, const DecodeParams& p, int h, int k0, int t1,
                                          float (&sv)[KSTEPS]) const {
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      float d = 0.f;
      if constexpr (kDot) {
        d = Tr::dot8(qr[h], f.kr[st], d);
      } else {
        float qf[VEC], kf[VEC];
        Tr::widen(qr[h], qf);
        Tr::widen(f.kr[st], kf);
#pragma unroll
        for (int e = 0; e < VEC; ++e) d = fmaf(qf[e], kf[e], d);
      }
      d = reduce_lanes<LPR>(d);
      sv[st] = k0 + st < t1 ? d * p.scale_log2 : kNegInf;
    }
  }

  // The chunk maximum of head h across the K groups, its rescale factor, and
  // P of the lane's TV V tokens; m and l of the head move on.
  __device__ __forceinline__ void softmax_head(int h, int lane, const float (&sv)[KSTEPS], float (&pw)[TV],
                                               float& alpha) {
    float cmax = sv[0];
#pragma unroll
    for (int st = 1; st < KSTEPS; ++st) cmax = fmaxf(cmax, sv[st]);
    cmax = reduce_groups<true>(cmax);
    const float m_new = fmaxf(m_run[h], cmax);
    alpha = fast_exp2(m_run[h] - m_new);
    m_run[h] = m_new;
    if constexpr (kPair) {
      // tokens 0..KSTEPS-1 of the pair are the even group's, the rest the
      // odd group's: the other group's scores come from lane ^ 8
      const bool odd = (lane & 8) != 0;
#pragma unroll
      for (int e = 0; e < KSTEPS; ++e) {
        const float other = dpp_f<0x128>(sv[e]);  // row_ror:8
        pw[e] = fast_exp2((odd ? other : sv[e]) - m_new);
        pw[KSTEPS + e] = fast_exp2((odd ? sv[e] : other) - m_new);
      }
    } else {
      const int base = (lane % LPR) % NTG * TV;
#pragma unroll
      for (int e = 0; e < TV; ++e) {
        float x = sv[e];
#pragma unroll
        for (int k = 1; k < NTG; ++k) x = base == k * TV ? sv[k * TV + e] : x;
        pw[e] = fast_exp2(x - m_new);
      }
    }
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < TV; ++e) psum += pw[e];
    l_run[h] = l_run[h] * alpha + psum;
  }

  // REFILL false: the stream's last step, which loads nothing.
  // Every lane of K group kq ends QK with the scores of that group's KSTEPS
  // tokens; the chunk maximum combines the groups by lane swaps, and the P of
  // a lane's own TV V tokens is formed where it is used: no LDS round trip.
  template <bool REFILL>
  __device__ __forceinline__ void step(Frag& f, const DecodeParams& p, Smem&, int kvh, int lane, int cs,
                                       const Segment& cur, int cs_next, const ChunkIds* ids_next, const Segment& nxt) {
    const int t1 = cur.t1;
    const bool has_new = cur.tnew >= cs && cur.tnew < cs + kChunk;
    const int k0 = cs + kq(lane) * KSTEPS;  // this lane's first K token
    const int tv = cs + v_tok(lane);        // this lane's first V token

    float pw[G][TV];
    float alpha[G];
    if constexpr (kPerHead) {
      // QK and P head by head, then the refill of K
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float sv[KSTEPS];
        qk_head(f, p, h, k0, t1, sv);
        softmax_head(h, lane, sv, pw[h], alpha[h]);
      }
      if (REFILL) load_k(f, p, kvh, lane, cs_next, ids_next, nxt);
    } else {
      // QK of every head; then the refill of K, whose registers are free;
      // then the chunk maximum and P of the lane's V tokens, head by head
      float sv[G][KSTEPS];
#pragma unroll
      for (int h = 0; h < G; ++h) qk_head(f, p, h, k0, t1, sv[h]);
      if (REFILL) load_k(f, p, kvh, lane, cs_next, ids_next, nxt);
#pragma unroll
      for (int h = 0; h < G; ++h) softmax_head(h, lane, sv[h], pw[h], alpha[h]);
    }

    // PV
    const bool partial = cs + kChunk > t1;
    const int enew = has_new && cur.tnew >= tv && cur.tnew < tv + TV ? cur.tnew - tv : -1;
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st) {
      float a[G];
#pragma unroll
      for (int h = 0; h < G; ++h) a[h] = acc[h][st] * alpha[h];
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        u32x4 w = f.vr[st][u];
        if (partial) w = Tr::keep_first(w, t1 - tv - u * VEC);
        if (has_new) {  // the new token's V, not its slot's old value
          const int en = enew >= u * VEC && enew < (u + 1) * VEC ? enew - u * VEC : -1;
          w = put_elem<raw>(w, en, vn[st]);
        }
        float vf[VEC];
        Tr::widen(w, vf);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < VEC; ++e) a[h] = fmaf(pw[h][u * VEC + e], vf[e], a[h]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h][st] = a[h];
    }
    if (REFILL) load_v(f, p, kvh, lane, cs_next, ids_next, nxt);
  }

  // x combined over the K groups (lanes l, l + LPR, ...): the two groups of a
  // row of 16 by a rotation of 8, then rows by lane swaps
  template <bool MAX>
  __device__ static float reduce_groups(float x) {
    const auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    if constexpr (LPR <= 8) x = op(x, dpp_f<0x128>(x));
    if constexpr (LPR <= 16) {
      const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
    }
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return op(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }

  // x summed over the lanes sharing this lane's dd row (all V groups and
  // token groups): every chunk token once
  __device__ static float sum_over_row(float x) {
    if constexpr (NTG >= 2) x += dpp_f<0xB1>(x);
    if constexpr (NTG >= 4) x += dpp_f<0x4E>(x);
    if constexpr (VLANES <= 16) {
      const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    }
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }

  __device__ void finish(Smem& sm, int lane, int) {
    const bool writer = lane < VLANES && (kPair || (lane % LPR) % NTG == 0);
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int st = 0; st < VSTEPS; ++st) {
        const float v = sum_over_row(acc[h][st]);
        if (writer) sm.o[h][st * DPS + v_row(lane)] = v;
      }
      const float l = sum_over_row(l_run[h]);
      if (lane == 0) {
        sm.ml[h][0] = m_run[h];
        sm.ml[h][1] = l;
      }
    }
    __syncthreads();
  }

  __device__ int members_in_group(const DecodeParams&, const Segment&, int) const { return 1; }
  __device__ static int member_row(const DecodeParams&, int) { return 0; }
  __device__ static int member_of(const DecodeParams&, int, int) { return 0; }
  __device__ static f32x4 o_val4(const Smem& sm, int, int h, int dd, int) {
    return *reinterpret_cast<const f32x4*>(&sm.o[h][dd]);
  }
  __device__ static float m_val(const Smem& sm, int, int h) { return sm.ml[h][0]; }
  __device__ static float l_val(const Smem& sm, int, int h) { return sm.ml[h][1]; }
};

// ---------------------------------------------------------------------------
// Segment driver, epilogue and merge (shared by both engines)
// ---------------------------------------------------------------------------
template <class Eng, int D>
__device__ __forceinline__ void write_zero_rows(const DecodeParams& p, int s, int kvh, int lane) {
  const int g = p.group;
  const size_t base = ((size_t)s * p.num_heads + (size_t)kvh * g) * D;
  for (int idx = lane; idx < g * D; idx += 64) store_out(p.out, base + idx, 0.f, p.out_dtype);
}

__device__ __forceinline__ long long owner_of(long long c, long long W, long long T) {
  return ((c + 1) * W - 1) / T;
}

// Work item i of a shared-mode plan: {sequence | members << 16, family
// index (members > 1) or first token, end token, first chunk in the
// laid-out order, the worker holding that chunk, the workers it spans, 0,
// 0}, read with scalar loads (the plan is read-only for the launch); a
// worker's first item comes with its worker record.
struct Item {
  int seq, members, fam, t0, t1, owner, npieces;
  long long c;
};

__device__ __forceinline__ Item make_item(const const_i32* r) {
  Item it;
  it.seq = r[0] & 0xffff;
  it.members = r[0] >> 16;
  it.fam = it.members > 1 ? r[1] : -1;
  it.t0 = it.members > 1 ? 0 : r[1];
  it.t1 = r[2];
  it.c = r[3];
  it.owner = r[4];
  it.npieces = r[5];
  return it;
}

__device__ __forceinline__ Item item_at(const DecodeParams& p, int i) {
  return make_item((const const_i32*)p.items + (size_t)i * kItemInts);
}

// Yields a worker's segments in order. Balanced mode: the chunks of all
// sequences (per KV head) are laid end to end and worker w owns chunks
// [start, end); shared mode: the same over the plan's work items; fixed
// mode: a single partition.
// Fields of the shared mode's walk (the family kernel's only); none for the
// other kernels.
template <bool SHARED>
struct ItemWalk {
  int num_items;  // items of the plan
  int first;      // the worker's first item, whose record is `first_item`
  Item first_item;
};
template <>
struct ItemWalk<false> {};

template <bool SHARED>
struct SegmentSource : ItemWalk<SHARED> {
  int mode;
  int s;          // next sequence (shared mode: next item) to look at
  long long c;    // first chunk of sequence (item) s in the laid-out order
  int k;          // fixed-partition stream: next partition of sequence s
  long long start, end, W, T;
  int w;
  Segment fixed;  // one-partition-per-workgroup mode's only segment

  __device__ Segment next(const DecodeParams& p) {
    if constexpr (SHARED) {
      return next_item(p);
    } else {
      if (mode == kModeFixed) {
        const Segment g = fixed;
        fixed.valid = 0;
        return g;
      }
      if (mode == kModeFixedStream) return next_partition(p);
      return next_sequence(p);
    }
  }

  __device__ Segment next_sequence(const DecodeParams& p) {
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
      g.flags = segment_flags(1, 0, 0);
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

  // Shared mode: items laid end to end like the sequences of the balanced
  // split. A family's common prefix (members > 1) always leaves partial
  // results, in the family region: piece slot (w + family) * fam_max +
  // member. A member's own rest (first token > 0) merges with them; a
  // sequence outside every family is treated as in the balanced split.
  __device__ Segment next_item(const DecodeParams& p) {
    while (s < this->num_items && c < end) {
      const Item it = s == this->first ? this->first_item : item_at(p, s);
      const int n = num_chunks(it.t1 - it.t0);
      c = it.c;
      if (n == 0) {
        ++s;
        continue;
      }
      const long long c0 = start > c ? start : c;
      const long long c1 = end < c + n ? end : c + n;
      Segment g;
      g.s = it.seq;
      g.t0 = it.t0 + (int)(c0 - c) * kChunk;
      g.t1 = min(it.t0 + (int)(c1 - c) * kChunk, it.t1);
      g.lbl = (g.t1 - 1) >> p.log2_block;
      const int first = it.owner;
      g.npieces = it.npieces;
      const bool head = c0 == c;
      if (it.members > 1) {
        g.tnew = -1;  // a family's common prefix ends before every member's last token
        g.slot = p.fam_base + (w + it.fam) * p.fam_max;
        g.first_slot = p.fam_base + (first + it.fam) * p.fam_max;
        g.flags = segment_flags(it.members, head ? kRecFamily : 0, 0);
      } else {
        const int L_raw = len_uniform(p, it.seq);
        g.tnew = new_token_pos(p, g.t1, it.t1, L_raw);
        g.slot = w + s;
        g.first_slot = first + s;
        g.flags = segment_flags(1, head ? (it.t0 == 0 ? (kRecOwn | kRecNoFamily) : kRecOwn) : 0,
                                it.t0 == 0 && g.npieces == 1);
      }
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
        g.flags = segment_flags(1, 0, 0);
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
// {sequence, pieces, partial-result slot, first slot, RecordKind bits of the
// split record to write, 1 if the values are the sequence's output}.
constexpr int kResRec = 6;

template <bool NT>
__device__ __forceinline__ void store16(f32x4* dst, f32x4 v) {
  if (NT) {
    __builtin_nontemporal_store(v, dst);
  } else {
    *dst = v;
  }
}

// The pieces of split sequences a worker of the in-kernel merge stored (at
// most two: only the first and the last segment of a worker's chunk range
// can be part of a sequence): sequence, pieces, worker holding the first.
struct Arrival {
  int s, np, first;
};

struct ResultBuf {
  float* vals;
  float* ml;
  int* rec;
  int n;
  int narr;
  Arrival arr0, arr1;
};

__device__ __forceinline__ ResultBuf result_buffer(const DecodeParams& p, int D) {
  ResultBuf rb;
  rb.vals = reinterpret_cast<float*>(g_lens + p.lens_pad);
  rb.ml = rb.vals + (size_t)p.res_slots * p.group * D;
  rb.rec = reinterpret_cast<int*>(rb.ml + (size_t)p.res_slots * p.group * 2);
  rb.n = 0;
  rb.narr = 0;
  rb.arr0 = rb.arr1 = Arrival{0, 0, 0};
  return rb;
}

// Partial results of the in-kernel merge are written and read by waves on
// different XCDs within one launch, and each XCD has its own L2: they go
// through agent-scope coherent (sc1) buffer accesses, which neither leave a
// line behind in this XCD's L2 nor read a stale one from it. Byte offsets
// from the region's base fit 31 bits (checked by the host).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, -1, 0x00020000);
}
constexpr int kCohSc1 = 16;  // cache-policy operand: sc1
__device__ __forceinline__ void coh_store16(__amdgpu_buffer_rsrc_t r, size_t off, f32x4 v) {
  const u32x4 u = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(u, r, (int)off, 0, kCohSc1);
}
__device__ __forceinline__ void coh_store4(__amdgpu_buffer_rsrc_t r, size_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, kCohSc1);
}
__device__ __forceinline__ f32x4 coh_load16(__amdgpu_buffer_rsrc_t r, size_t off) {
  const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCohSc1);
  return f32x4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
}
__device__ __forceinline__ f32x2 coh_load8(__amdgpu_buffer_rsrc_t r, size_t off) {
  const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kCohSc1);
  return f32x2{__uint_as_float(u[0]), __uint_as_float(u[1])};
}

// Store every buffered result: whole sequences to `out`, pieces of split
// ones to the workspace, and the split records. NT: non-temporal stores, for
// a buffer that filled up mid-stream (they complete sooner under the
// stream's load, so the load waits behind them are shorter: 512-token
// partitions at the long-context shape 939 -> 913 us); at the stream's end
// ordinary stores.
template <int D, int MAXG, bool NT, bool SHARED>
__device__ __forceinline__ void flush_results(const DecodeParams& p, ResultBuf& rb, int kvh, int lane) {
  constexpr int kStride = SHARED ? 4 : 2;  // ints per sequence in ws_meta
  constexpr int kV4 = (MAXG * D / 4 + 63) / 64;  // 16-byte pieces per lane and result
  const int gq = p.group, Hq = p.num_heads, n4 = gq * D / 4;
  const size_t head0 = (size_t)kvh * gq;
  const bool out_vec = (reinterpret_cast<uintptr_t>(p.out) & (p.out_dtype == kF32 ? 15 : 7)) == 0;
  const bool coh = !SHARED && p.ctr != nullptr;  // pieces merged in this launch
  for (int k = 0; k < rb.n; ++k) {
    const int* r = rb.rec + kResRec * k;
    const int s = __builtin_amdgcn_readfirstlane(r[0]), np = __builtin_amdgcn_readfirstlane(r[1]);
    const int slot = __builtin_amdgcn_readfirstlane(r[2]);
    const float* v = rb.vals + (size_t)k * gq * D;
    const int kind = coh ? 0 : r[4];
    if (kind && lane == 0) {
      // split record of sequence s: {own first slot, own pieces}, or in
      // shared mode {family first slot, family pieces, own first, own pieces}
      int* meta = p.ws_meta + (size_t)s * kStride;
      if (kind & kRecOwn) {
        meta[kStride - 2] = r[3];
        meta[kStride - 1] = np;
      }
      if (SHARED && (kind & kRecFamily)) {
        meta[0] = r[3];
        meta[1] = np;
      }
      if (SHARED && (kind & kRecNoFamily)) {
        meta[0] = 0;
        meta[1] = 0;
      }
    }
    // the result's LDS reads all issued before its first store
    f32x4 t[kV4];
#pragma unroll
    for (int u = 0; u < kV4; ++u) {
      const int i = lane + 64 * u;
      if (i < n4) t[u] = reinterpret_cast<const f32x4*>(v)[i];
    }
    if (r[5]) {
      const size_t base = ((size_t)s * Hq + head0) * D;
      // one loop per output form, the choice made once per result
      if (p.out_dtype == kF32 && out_vec) {
        f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + base);
#pragma unroll
        for (int u = 0; u < kV4; ++u)
          if (lane + 64 * u < n4) store16<NT>(o + lane + 64 * u, t[u]);
      } else if (out_vec) {
        const int dt = p.out_dtype;
#pragma unroll
        for (int u = 0; u < kV4; ++u)
          if (lane + 64 * u < n4) store_out4(p.out, base + 4 * (size_t)(lane + 64 * u), t[u], dt, true);
      } else {
        const int dt = p.out_dtype;
#pragma unroll
        for (int u = 0; u < kV4; ++u)
          if (lane + 64 * u < n4) store_out4(p.out, base + 4 * (size_t)(lane + 64 * u), t[u], dt, false);
      }
    } else if (coh) {
      const size_t row0 = (size_t)slot * Hq + head0;
      const __amdgpu_buffer_rsrc_t ra = ws_rsrc(p.ws_acc), rm = ws_rsrc(p.ws_ml);
#pragma unroll
      for (int u = 0; u < kV4; ++u) {
        const int i = lane + 64 * u;
        if (i < n4) coh_store16(ra, (row0 * D + 4 * (size_t)i) * 4, t[u]);
      }
      for (int i = lane; i < 2 * gq; i += 64) coh_store4(rm, (row0 * 2 + i) * 4, rb.ml[(size_t)k * gq * 2 + i]);
    } else {
      const size_t row0 = (size_t)slot * Hq + head0;
#pragma unroll
      for (int u = 0; u < kV4; ++u) {
        const int i = lane + 64 * u;
        if (i < n4) store16<NT>(reinterpret_cast<f32x4*>(p.ws_acc + row0 * D) + i, t[u]);
      }
      for (int i = lane; i < 2 * gq; i += 64) p.ws_ml[row0 * 2 + i] = rb.ml[(size_t)k * gq * 2 + i];
    }
  }
  rb.n = 0;
}

// Buffers the result of one sequence of a finished segment: member m
// (0 unless the segment is a family's common prefix), whose head slots start
// at row `row` of the engine's staging area.
template <class Eng, int D>
__device__ void segment_epilogue(const DecodeParams& p, const typename Eng::Smem& sm, const Segment& g, int m,
                                 int row, int kvh, int lane, ResultBuf& rb) {
  constexpr bool kShared = Eng::kGroups > 1;
  if (rb.n == p.res_slots) flush_results<D, Eng::kMaxGroup, true, kShared>(p, rb, kvh, lane);
  const int gq = p.group;
  const int k = rb.n;
  float* v = rb.vals + (size_t)k * gq * D;
  const int direct = seg_direct<kShared>(g);
  // 16 bytes per lane and access, every read issued before the first write
  // (one LDS round trip per result, not one per element)
  constexpr int kV4 = (Eng::kMaxGroup * D / 4 + 63) / 64;
  const int n4 = gq * D / 4;
  f32x4 t[kV4];
#pragma unroll
  for (int u = 0; u < kV4; ++u) {
    const int i = lane + 64 * u;
    if (i < n4) {
      const int h = 4 * i / D, dd = 4 * i % D;
      t[u] = Eng::o_val4(sm, row, h, dd, gq);
      if (direct) t[u] = t[u] / Eng::l_val(sm, row, h);
    }
  }
#pragma unroll
  for (int u = 0; u < kV4; ++u) {
    const int i = lane + 64 * u;
    if (i < n4) reinterpret_cast<f32x4*>(v)[i] = t[u];
  }
  if (!direct) {
    for (int h = lane; h < gq; h += 64) {
      rb.ml[((size_t)k * gq + h) * 2] = Eng::m_val(sm, row, h);
      rb.ml[((size_t)k * gq + h) * 2 + 1] = Eng::l_val(sm, row, h);
    }
  }
  if (lane == 0) {
    int* r = rb.rec + kResRec * k;
    r[0] = g.s + m;
    r[1] = g.npieces;
    r[2] = g.slot + m;
    r[3] = g.first_slot + m;
    r[4] = kvh == 0 ? seg_kind<kShared>(p, g) : 0;
    r[5] = direct;
  }
  if (!kShared && !direct && p.ctr != nullptr) {
    const Arrival a{g.s, g.npieces, g.first_slot - g.s};
    if (rb.narr == 0) rb.arr0 = a;
    else rb.arr1 = a;
    rb.narr = min(rb.narr + 1, 2);
  }
  rb.n = k + 1;
  __syncthreads();
}

// Every result of a finished segment: column group by column group, each
// member the group holds.
template <class Eng, int D>
__device__ void finish_segment(const DecodeParams& p, Eng& eng, typename Eng::Smem& sm, const Segment& g, int kvh,
                               int lane, ResultBuf& rb) {
#pragma unroll
  for (int cg = 0; cg < Eng::kGroups; ++cg) {
    const int nm = eng.members_in_group(p, g, cg);
    if (nm > 0) {
      eng.finish(sm, lane, cg);
      for (int mi = 0; mi < nm; ++mi)
        segment_epilogue<Eng, D>(p, sm, g, Eng::member_of(p, cg, mi), Eng::member_row(p, mi), kvh, lane, rb);
    }
  }
}

// Runs all of a worker's segments as one stream of 32-token chunks: the
// register set of a chunk is refilled with the next chunk of the stream,
// which may already belong to the next segment, whose q is fetched at the
// same time; block ids are read two chunks ahead. A segment's epilogue
// therefore overlaps the next segment's first loads.
template <class Eng, int D>
__device__ __forceinline__ void run_stream(const DecodeParams& p, typename Eng::Smem& sm, SegmentSource<(Eng::kGroups > 1)>& src,
                           int kvh, int lane, ResultBuf& rb) {
  static_assert(Eng::kSub == 1, "the chunk stream assumes one 32-token chunk per step");
  Segment A = src.next(p);
  if (!A.valid) return;
  // the first chunk's block ids and q are requested before the next
  // segments are walked
  Pos p0{0, A.t0};
  const ChunkIds ids0 = ids_at(p, p0, A, A, A);
  Eng eng;
  typename Eng::Q q, qn;
  eng.load_q(q, p, A, kvh, lane);
  Segment B = src.next(p);
  Segment C = B.valid ? src.next(p) : invalid_segment();
  Pos p1 = advance(p0, A, B, C);
  Pos p2 = advance(p1, A, B, C);
  ChunkIds ids1 = ids_at(p, p1, A, B, C);
  typename Eng::Frag f;
  eng.load_k(f, p, kvh, lane, p0.cs, &ids0, A);
  eng.load_v(f, p, kvh, lane, p0.cs, &ids0, A);
  eng.reset(q, p, A, kvh, lane, sm);  // after the first K/V loads are issued: only the first QK needs q
  for (;;) {
    const ChunkIds ids2 = ids_at(p, p2, A, B, C);
    const bool leaving = p1.rel != 0;                       // p0 is the current segment's last chunk
    const bool at_end = !leaving && p1.cs == p0.cs;         // and there is no next segment
    const Segment n1 = seg_at(p1.rel, A, B, C);
    if (leaving) eng.load_q(qn, p, n1, kvh, lane);
    if (at_end) {
      // the last step issues no refill: nothing of the stream is left in
      // flight behind its results
      eng.template step<false>(f, p, sm, kvh, lane, p0.cs, A, p1.cs, &ids1, n1);
      finish_segment<Eng, D>(p, eng, sm, A, kvh, lane, rb);
      break;
    }
    eng.template step<true>(f, p, sm, kvh, lane, p0.cs, A, p1.cs, &ids1, n1);
    if (leaving) {
      finish_segment<Eng, D>(p, eng, sm, A, kvh, lane, rb);
      A = B;
      B = C;
      C = B.valid ? src.next(p) : invalid_segment();
      p1.rel -= 1;
      p2.rel -= 1;
      eng.reset(qn, p, A, kvh, lane, sm);
    }
    p0 = p1;
    p1 = p2;
    p2 = advance(p2, A, B, C);
    ids1 = ids2;
  }
  // a launch that merges itself flushes in settle(), with the new tokens'
  // loads in flight
  if ((Eng::kGroups > 1) || p.ctr == nullptr) flush_results<D, Eng::kMaxGroup, false, (Eng::kGroups > 1)>(p, rb, kvh, lane);
}

// The in-kernel merge, run by the worker whose piece completed the count of
// a split sequence, for up to two sequences at once (a worker's first and
// last segment; their pieces' loads go out together): pieces first ..
// first + np - 1 of each, in piece order, folded with a running maximum.
// The weights are those of the closing launch's merge -- piece k of head h
// weighs 2^(m_k - M) over M = max_j m_j, and out = sum_k 2^(m_k - M) acc_k /
// sum_k 2^(m_k - M) l_k -- rescaled as M grows. Lane l covers 4 channels of
// every (64 / (D/4))-th head; each piece's (m, l) pair and 16-byte share of
// acc are read with agent-scope loads, kIn pieces in flight.
template <int D, int MAXG>
struct MergeAcc {
  static constexpr int RPI = 64 / (D / 4);         // head rows per wave instruction
  static constexpr int HPL = (MAXG + RPI - 1) / RPI;  // heads per lane
  float M[HPL], den[HPL];
  f32x4 num[HPL];
  __device__ void init() {
#pragma unroll
    for (int j = 0; j < HPL; ++j) {
      M[j] = kNegInf;
      den[j] = 0.f;
      num[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __device__ void fold(int j, f32x2 ml, f32x4 a) {
    const float m = ml.x, Mn = fmaxf(M[j], m);
    if (Mn != kNegInf) {
      const float c = fast_exp2(M[j] - Mn), e = fast_exp2(m - Mn);
      den[j] = fmaf(den[j], c, e * ml.y);
      num[j] = num[j] * c + e * a;
      M[j] = Mn;
    }
  }
};

template <int D, int MAXG>
__device__ __forceinline__ void merge_arrived(const DecodeParams& p, int kvh, int lane, const Arrival& a0, bool m0,
                                              const Arrival& a1, bool m1) {
  using Acc = MergeAcc<D, MAXG>;
  constexpr int LPR = D / 4, RPI = Acc::RPI, HPL = Acc::HPL;
  constexpr int kIn = 8;
  const int gq = p.group, Hq = p.num_heads;
  const int r = lane / LPR, d4 = (lane % LPR) * 4;
  const int head0 = kvh * gq;
  const __amdgpu_buffer_rsrc_t ra = ws_rsrc(p.ws_acc), rm = ws_rsrc(p.ws_ml);
  const int n0 = m0 ? a0.np : 0, total = n0 + (m1 ? a1.np : 0);
  Acc acc0, acc1;
  acc0.init();
  acc1.init();
  for (int k0 = 0; k0 < total; k0 += kIn) {
    // every load of the batch unconditional (past the last piece or head:
    // the last one again), so that they all go out before the first wait
    f32x2 ml[kIn][HPL];
    f32x4 v[kIn][HPL];
#pragma unroll
    for (int i = 0; i < kIn; ++i) {
      const int k = min(k0 + i, total - 1);
      const int slot = k < n0 ? a0.first + a0.s + k : a1.first + a1.s + (k - n0);
#pragma unroll
      for (int j = 0; j < HPL; ++j) {
        const int h = min(r + j * RPI, gq - 1);
        const size_t row = (size_t)slot * Hq + head0 + h;
        ml[i][j] = coh_load8(rm, row * 2 * 4);
        v[i][j] = coh_load16(ra, (row * D + d4) * 4);
      }
    }
#pragma unroll
    for (int i = 0; i < kIn; ++i) {
      const int k = k0 + i;
      if (k >= total) continue;
#pragma unroll
      for (int j = 0; j < HPL; ++j) {
        if (r + j * RPI >= gq) continue;
        if (k < n0) acc0.fold(j, ml[i][j], v[i][j]);
        else acc1.fold(j, ml[i][j], v[i][j]);
      }
    }
  }
  const bool out_vec = (reinterpret_cast<uintptr_t>(p.out) & (p.out_dtype == kF32 ? 15 : 7)) == 0;
#pragma unroll
  for (int j = 0; j < HPL; ++j) {
    const int h = r + j * RPI;
    if (h >= gq) continue;
    if (m0) store_out4(p.out, ((size_t)a0.s * Hq + head0 + h) * D + d4, acc0.num[j] * (1.f / acc0.den[j]),
                       p.out_dtype, out_vec);
    if (m1) store_out4(p.out, ((size_t)a1.s * Hq + head0 + h) * D + d4, acc1.num[j] * (1.f / acc1.den[j]),
                       p.out_dtype, out_vec);
  }
}

// The fused write of a launch that merges itself: worker w of W stores the
// new tokens of sequences w, w + W, ... for its KV head (the slot of
// position L-1, when the length was not cut and the table entry lies inside
// the pool). It may overlap the other workers' reads of the cache: the one
// worker that reads the slot's chunk takes that token's K row and V
// elements from k_new/v_new, never from the slot, and the store changes no
// other byte. Non-temporal: a V column dirties one cache line per element,
// which left in the cache is written back during the next decode's stream.
// kBatch sequences per round trip: loads, then stores.
template <typename U, int D>
struct NewTokens {
  static constexpr int kBatch = 8;
  static constexpr int NE = D / 64;
  int phys[kBatch], off[kBatch];
  U kv[kBatch][NE], vv[kBatch][NE];

  // s0 < num_seqs and max_blocks_per_seq >= 1. Every load unconditional
  // (for a sequence without a write: an in-bounds row, unused), so that they
  // all go out before the first wait. LDS_LENS: the lengths are in LDS (the
  // balanced split's copy), else read from memory.
  template <bool LDS_LENS = true>
  __device__ void load(const DecodeParams& p, int s0, int W, int kvh, int lane) {
    const int S = p.num_seqs, Hkv = p.num_kv_heads;
    const U* kn = static_cast<const U*>(p.k_new);
    const U* vn = static_cast<const U*>(p.v_new);
    const const_i32* tables = (const const_i32*)p.block_tables;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int s = s0 + i * W;
      const int sc = min(s, S - 1);
      const int L = LDS_LENS ? lds_len(sc) : len_uniform(p, sc);
      const bool ok = s < S && L > 0 && capped_len(p, L) == L;
      const int t = ok ? L - 1 : 0;
      const int ph = tables[(size_t)sc * p.max_blocks_per_seq + (t >> p.log2_block)];
      phys[i] = ok ? ph : -1;
      off[i] = t & (p.block_size - 1);
      const size_t src = ((size_t)sc * Hkv + kvh) * D;
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        kv[i][j] = kn[src + lane + 64 * j];
        vv[i][j] = vn[src + lane + 64 * j];
      }
    }
  }

  __device__ void store(const DecodeParams& p, int kvh, int lane) const {
    const int Hkv = p.num_kv_heads, B = p.block_size, Bs = v_subtile(B);
    U* kc = const_cast<U*>(static_cast<const U*>(p.k_cache));
    U* vc = const_cast<U*>(static_cast<const U*>(p.v_cache));
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (phys[i] < 0 || phys[i] >= p.num_blocks) continue;
      U* kd = kc + (((size_t)phys[i] * Hkv + kvh) * B + off[i]) * D;
      U* vd = vc + v_elem(phys[i], Hkv, kvh, D, B, Bs, 0, off[i]);
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        const int e = lane + 64 * j;
        __builtin_nontemporal_store(kv[i][j], kd + e);
        __builtin_nontemporal_store(vv[i][j], vd + (size_t)e * Bs);
      }
    }
  }
};

// The new tokens of sequences w, w + W, ... for KV head kvh, stored by
// worker w of the family kernel when its stream has ended (or at once when
// it has none). The attention takes position L-1 from k_new/v_new and never
// reads the slot, so the stores may overlap other workers' reads of the
// same blocks; they are the last thing a worker does, after its results.
template <class Eng, int D>
__device__ __forceinline__ void store_new_tokens(const DecodeParams& p, int w, int W, int kvh, int lane) {
  using NT = NewTokens<typename Eng::raw, D>;
  if (p.k_new == nullptr || p.max_blocks_per_seq <= 0) return;
  for (int s0 = w; s0 < p.num_seqs; s0 += NT::kBatch * W) {
    NT nt;
    nt.template load<false>(p, s0, W, kvh, lane);
    nt.store(p, kvh, lane);
  }
}

// End of a balanced-split worker whose launch merges itself. The buffered
// results are stored (the pieces with agent-scope stores, so nothing of them
// waits in this XCD's L2); once every store is acknowledged, each piece
// counts its arrival, and the worker whose add completes a sequence's count
// merges it, reading every piece with agent-scope loads, and sets the
// counter back to zero for the next launch. No worker waits for another.
// The new tokens' loads go out with the merge's, their stores last: issued
// before the flush, the scalar table loads would hold up its LDS reads (one
// counter covers both), and stores ahead of the merge's loads would hold
// those up in the in-order vector-memory count.
template <class Eng, int D>
__device__ __forceinline__ void settle(const DecodeParams& p, ResultBuf& rb, int w, int W, int kvh, int lane) {
  using NT = NewTokens<typename Eng::raw, D>;
  const bool writes = p.k_new != nullptr && w < p.num_seqs && p.max_blocks_per_seq > 0;
  flush_results<D, Eng::kMaxGroup, false, false>(p, rb, kvh, lane);
  int* c0 = p.ctr + (size_t)kvh * W + rb.arr0.first;
  int* c1 = p.ctr + (size_t)kvh * W + rb.arr1.first;
  int old0 = 0, old1 = 0;
  if (rb.narr > 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) {
      old0 = __hip_atomic_fetch_add(c0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (rb.narr > 1) old1 = __hip_atomic_fetch_add(c1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  NT nt;
  if (writes) nt.load(p, w, W, kvh, lane);
  if (rb.narr > 0) {
    old0 = __builtin_amdgcn_readfirstlane(old0);
    old1 = __builtin_amdgcn_readfirstlane(old1);
    asm volatile("" ::: "memory");
    const bool m0 = old0 == rb.arr0.np - 1, m1 = rb.narr > 1 && old1 == rb.arr1.np - 1;
    if (lane == 0) {
      if (m0) __hip_atomic_store(c0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (m1) __hip_atomic_store(c1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (m0 || m1) merge_arrived<D, Eng::kMaxGroup>(p, kvh, lane, rb.arr0, m0, rb.arr1, m1);
  }
  if (writes) {
    nt.store(p, kvh, lane);
    for (int s0 = w + NT::kBatch * W; s0 < p.num_seqs; s0 += NT::kBatch * W) {
      NT more;
      more.load(p, s0, W, kvh, lane);
      more.store(p, kvh, lane);
    }
  }
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
  SegmentSource<(Eng::kGroups > 1)> src;
  src.mode = p.mode;
  src.w = w;

  if constexpr (Eng::kGroups > 1) {
    // the family kernel runs the shared mode only; the plan launch wrote
    // this worker's chunk range and first item
    const int S = p.num_seqs;
    for (int s = w; s < S; s += W)
      if (capped_len(p, len_uniform(p, s)) <= 0) write_zero_rows<Eng, D>(p, s, kvh, lane);
    const const_i32* wr = (const const_i32*)p.wrec + (size_t)w * kWorkerInts;
    const int start = wr[0], end = wr[1], first = wr[2], T = wr[3];
    if (p.mode != kModeShared) return;
    if (start >= end) {
      store_new_tokens<Eng, D>(p, w, W, kvh, lane);
      return;
    }
    src.s = first;
    src.c = start;
    src.k = 0;
    src.start = start;
    src.end = end;
    src.W = min(W, T);
    src.T = T;
    src.num_items = wr[4];
    src.first = first;
    src.first_item = make_item(wr + 8);
    src.fixed = invalid_segment();
    ResultBuf rb = result_buffer(p, D);
    run_stream<Eng, D>(p, sm, src, kvh, lane, rb);
    store_new_tokens<Eng, D>(p, w, W, kvh, lane);
    return;
  } else {
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
    g.flags = segment_flags(1, 0, 0);
    g.t0 = t0;
    g.t1 = min(t0 + P, L);
    g.lbl = (g.t1 - 1) >> p.log2_block;
    g.npieces = (L + P - 1) / P;
    g.slot = s * p.max_parts + part;
    g.first_slot = s * p.max_parts;
    g.tnew = new_token_pos(p, g.t1, L, L_raw);
    g.valid = 1;
    src.fixed = uniform(g);
    ResultBuf rb = result_buffer(p, D);
    run_stream<Eng, D>(p, sm, src, kvh, lane, rb);
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
  ResultBuf rb = result_buffer(p, D);
  if (w < Wn) {
    const long long start = (long long)w * T / Wn, end = (long long)(w + 1) * T / Wn;
    // never empty while 0 <= start < T
    const unsigned long long ball = __ballot(start >= excl && start < incl);
    const int owner = ball ? __builtin_ctzll(ball) : 0;
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
    src.end = ball ? end : start;
    src.W = Wn;
    src.T = T;
    src.fixed = invalid_segment();
    run_stream<Eng, D>(p, sm, src, kvh, lane, rb);
  }
  if (p.ctr != nullptr) settle<Eng, D>(p, rb, w, W, kvh, lane);
  }
}

// ---------------------------------------------------------------------------
// Shared-mode plan (a link launch, then one workgroup, ahead of the decode
// launch).
//
// Sequences that map the same physical blocks at the same logical positions
// from position 0 on (forks of one prompt: parallel samples, beams, requests
// on a shared prefix; the kernels see only their block-id lists) hold the
// same K/V there. Adjacent sequences with at least kSharedMinChunks chunks of
// such a common prefix form families of up to fam_max members. Work items,
// laid end to end in 32-token chunks as the balanced split lays out
// sequences: a family's common prefix (tokens [0, Sf), Sf a multiple of 32
// and below every member's last token), then each member's rest [Sf, L); a
// sequence outside every family is one item [0, L). The W' = min(W, T)
// workers get contiguous chunk ranges of about equal estimated cost (a
// family's chunks, with more column groups, and every item's end cost more
// than a plain chunk), each at least one chunk.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

// floor(a / b) for 0 <= a < 2^53 and 0 < b < 2^53: the correctly rounded
// double quotient is within one of it, and one integer check on either
// side makes it exact (cheaper than a 64-bit integer division).
__device__ __forceinline__ long long floor_div(long long a, long long b) {
  long long q = (long long)((double)a / (double)b);
  if (q * b > a) --q;
  else if ((q + 1) * b <= a) ++q;
  return q;
}

// Inclusive scan of one int over the wave's 64 lanes with DPP moves: sums
// (or maxima of non-negative values) within rows of 16 lanes by shifts of
// 1, 2, 4, 8, then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then row 1's into rows 2 and 3 (row_bcast:31). Lanes
// shifted in from outside a row, and rows a broadcast skips, add 0.
template <bool MAX>
__device__ __forceinline__ int wave_scan(int x) {
  const auto op = [](int a, int b) { return MAX ? max(a, b) : a + b; };
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = op(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return x;
}

// Inclusive sums of three ints per thread over the workgroup, in one pass:
// wave scans, the waves' totals through LDS.
__device__ int3 plan_scan3(int3 x, int3* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x.x = wave_scan<false>(x.x);
  x.y = wave_scan<false>(x.y);
  x.z = wave_scan<false>(x.z);
  if (lane == 63) tot[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int3 v = lane < kPlanWaves ? tot[lane] : int3{0, 0, 0};
    v.x = wave_scan<false>(v.x);
    v.y = wave_scan<false>(v.y);
    v.z = wave_scan<false>(v.z);
    if (lane < kPlanWaves) tot[lane] = v;
  }
  __syncthreads();
  if (wave > 0) {
    x.x += tot[wave - 1].x;
    x.y += tot[wave - 1].y;
    x.z += tot[wave - 1].z;
  }
  __syncthreads();
  return x;
}

// Inclusive maximum of one non-negative int per thread over the workgroup.
__device__ int plan_scan_max(int x, int* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_scan<true>(x);
  if (lane == 63) tot[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int v = lane < kPlanWaves ? tot[lane] : 0;
    v = wave_scan<true>(v);
    if (lane < kPlanWaves) tot[lane] = v;
  }
  __syncthreads();
  if (wave > 0) x = max(x, tot[wave - 1]);
  __syncthreads();
  return x;
}

// Common prefix, in blocks, of sequence s's block-id list with sequence
// s - 1's (0 for s = 0), written to p.links[s]: one wave per sequence,
// kLinkSpan loads of 64 entries per lane and row in flight per round.
constexpr int kLinkWaves = 4;
constexpr int kLinkSpan = 4;

__global__ __launch_bounds__(64 * kLinkWaves) void link_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * kLinkWaves + (threadIdx.x >> 6);
  if (s >= p.num_seqs) return;  // whole waves
  int c = 0;
  if (s > 0) {
    const int lg = p.log2_block, B = p.block_size, mb = p.max_blocks_per_seq;
    const int32_t* a = p.block_tables + (size_t)s * mb;
    const int32_t* b = a - mb;
    // the first round's entries are requested with the lengths (clamped to
    // the rows' last entry: in bounds whatever the lengths), so the compare
    // waits for one round trip, not two
    int va[kLinkSpan], vb[kLinkSpan];
#pragma unroll
    for (int h = 0; h < kLinkSpan; ++h) {
      const int k = min(64 * h + lane, mb - 1);
      va[h] = a[k];
      vb[h] = b[k];
    }
    const int la = max(capped_len(p, p.context_lens[s]), 0);
    const int lb = max(capped_len(p, p.context_lens[s - 1]), 0);
    // both lengths are within their tables, so entries below n exist in both rows
    const int n = min((la + B - 1) >> lg, (lb + B - 1) >> lg);
    c = n;
    for (int k0 = 0; k0 < n; k0 += 64 * kLinkSpan) {
      if (k0 > 0) {
#pragma unroll
        for (int h = 0; h < kLinkSpan; ++h) {
          const int k = min(k0 + 64 * h + lane, n - 1);
          va[h] = a[k];
          vb[h] = b[k];
        }
      }
      int found = -1;
#pragma unroll
      for (int h = 0; h < kLinkSpan; ++h) {
        const int k = k0 + 64 * h + lane;
        const unsigned long long m = __ballot(k < n && va[h] != vb[h]);
        if (found < 0 && m) found = k0 + 64 * h + __builtin_ctzll(m);
      }
      if (found >= 0) {
        c = found;
        break;
      }
    }
  }
  if (lane == 0) p.links[s] = c;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(DecodeParams p, int W) {
  __shared__ int s_fam[kSharedMaxSeqs];     // per family leader: shared tokens (0: no family)
  __shared__ int s_cb[kSharedMaxSeqs];      // per leader: least common prefix (blocks) of its members
  __shared__ int s_ml[kSharedMaxSeqs];      // per leader: least last-token position of its group
  __shared__ int s_gn[kSharedMaxSeqs];      // per leader: sequences in its group
  __shared__ int s_item[2 * kSharedMaxSeqs + 1];  // first chunk of every item, then the total
  __shared__ int s_cost[2 * kSharedMaxSeqs + 1];  // cost before every item, then the total
  __shared__ int s_first[kSharedMaxWorkersTotal];  // every worker's first item
  __shared__ int s_bound[kSharedMaxWorkersTotal + 1];  // worker w's chunks: [s_bound[w], s_bound[w + 1])
  __shared__ int s_rec[2 * kSharedMaxSeqs][kItemInts];
  __shared__ int s_tot[kPlanWaves];
  __shared__ int3 s_tot3[kPlanWaves];
  __shared__ int s_misc[4];
  const int S = p.num_seqs, t = threadIdx.x;
  const int B = p.block_size, F = p.fam_max;
  // one sequence per thread (S <= kPlanThreads); loads of valid rows for
  // every thread, results used where they apply
  const int s = t;
  const bool has = s < S;
  const int sc = min(s, S - 1);
  const int L_raw = p.context_lens[sc];
  const int cpre = p.links[sc];
  const int L = has ? max(capped_len(p, L_raw), 0) : 0;
  // families: runs of linked sequences cut into groups of F from the run's start
  const bool link = has && s > 0 && cpre * B >= kSharedMinChunks * kChunk;
  const int run = plan_scan_max(has && !link ? s : 0, s_tot);
  const int leader = run + F * ((s - run) / F);
  if (has && leader == s) {
    s_cb[s] = INT_MAX;
    s_ml[s] = L - 1;
    s_gn[s] = 1;
  }
  __syncthreads();
  if (has && leader != s) {
    atomicMin(&s_cb[leader], cpre);
    atomicMin(&s_ml[leader], L - 1);
    atomicAdd(&s_gn[leader], 1);
  }
  __syncthreads();
  // the shared tokens: the members' least common prefix, below every
  // member's last token, in whole chunks; a group of one, or one sharing
  // fewer than kSharedMinChunks chunks, disbands (every member alone)
  int members = 0;
  if (has && leader == s) {
    const int gsize = s_gn[s];
    int sf = 0;
    if (gsize > 1) sf = (int)(min((long long)s_cb[s] * B, (long long)s_ml[s]) / kChunk * kChunk);
    members = gsize;
    if (gsize < 2 || sf < kSharedMinChunks * kChunk) {
      members = 1;
      sf = 0;
    }
    s_fam[s] = sf;
  }
  __syncthreads();
  const int my_sf = has ? s_fam[leader] : 0;
  const bool fam_leader = has && leader == s && members > 1;
  // items of this sequence (a family leader: the common prefix, then its
  // rest), their index, the family index, their chunks and costs
  const int nitems = has ? (fam_leader ? 2 : 1) : 0;
  const int pre_chunks = fam_leader ? my_sf / kChunk : 0;
  const int own_chunks = num_chunks(L - my_sf);
  const int chunks = pre_chunks + own_chunks;
  const int per = 16 / p.group;  // members a column group holds
  const int fam_rate = kCostChunk + kCostGroupChunk * ((members + per - 1) / per);
  const int fam_cost = fam_leader ? pre_chunks * fam_rate + kCostMemberEnd * members + kCostItemEnd : 0;
  const int own_cost = own_chunks > 0 ? own_chunks * kCostChunk + kCostItemEnd : 0;
  // one pass: items (< 2^15) in the low half and families in the high half
  // of the first sum, chunks in the second, costs in the third
  const int3 sums = plan_scan3(int3{nitems | ((fam_leader ? 1 : 0) << 16), chunks, fam_cost + own_cost}, s_tot3);
  const int item0 = (sums.x & 0xffff) - nitems;
  const int fam = (sums.x >> 16) - 1;
  const int c0 = sums.y - chunks;
  const int k0 = sums.z - fam_cost - own_cost;
  if (t == kPlanThreads - 1) {
    s_misc[1] = item0 + nitems;  // items
    s_misc[2] = c0 + chunks;     // chunks per KV head
    s_misc[3] = sums.z;          // total cost
    s_item[item0 + nitems] = c0 + chunks;
    s_cost[item0 + nitems] = sums.z;
  }
  if (fam_leader) {
    s_rec[item0][0] = s | (members << 16);
    s_rec[item0][1] = fam;
    s_rec[item0][2] = my_sf;
    s_rec[item0][3] = c0;
    s_item[item0] = c0;
    s_cost[item0] = k0;
  }
  if (has) {
    const int it = item0 + nitems - 1;
    s_rec[it][0] = s | (1 << 16);
    s_rec[it][1] = my_sf;
    s_rec[it][2] = L;
    s_rec[it][3] = c0 + pre_chunks;
    s_item[it] = c0 + pre_chunks;
    s_cost[it] = k0 + fam_cost;
  }
  __syncthreads();
  const int NI = s_misc[1], T = s_misc[2], C = s_misc[3];
  const int Wn = min(W, T);
  // worker boundaries: boundary b (0 < b < Wn) at the chunk x where the cost
  // reaches X = floor(b C / Wn), found by the item whose cost range
  // [s_cost[i], s_cost[i + 1]) holds X; then pulled towards the even split
  // so that every worker keeps at least one chunk: s_bound[b] =
  // x (T - Wn) / T + b is strictly increasing in b, with s_bound[0] = 0 and
  // s_bound[Wn] = T
  if (T > 0) {
    for (int i = t; i < NI; i += kPlanThreads) {
      const long long k = s_cost[i], k1 = s_cost[i + 1];
      if (k1 == k) continue;
      const int m = s_rec[i][0] >> 16;
      const int rate = m > 1 ? kCostChunk + kCostGroupChunk * ((m + per - 1) / per) : kCostChunk;
      const long long n = s_item[i + 1] - s_item[i];
      // X >= k  <=>  b C >= k Wn;  X < k1  <=>  b C < k1 Wn
      const int b0 = (int)floor_div(k * Wn + C - 1, C), b1 = (int)floor_div(k1 * Wn + C - 1, C);
      for (int b = max(b0, 1); b < min(b1, Wn); ++b) {
        const int off = (int)(floor_div((long long)b * C, Wn) - k) / rate;
        const long long x = s_item[i] + (off < n ? off : n);
        s_bound[b] = (int)floor_div(x * (T - Wn), T) + b;
        s_first[b] = i;  // the item x lies in: the start of the search for b's first item
      }
    }
    if (t == 0) {
      s_bound[0] = 0;
      s_bound[Wn] = T;
      s_first[0] = 0;
    }
  }
  __syncthreads();
  // every worker's range and first item; each item's first and last owner
  // marked by the workers holding its first and its last chunk
  for (int w = t; w < Wn; w += kPlanThreads) {
    const int start = s_bound[w], end = s_bound[w + 1];
    // the last item whose first chunk is at or before `start` (items
    // without chunks share their successor's first chunk), walked to from
    // the item the boundary's cost target fell in (the pull towards the
    // even split moves it by a few chunks)
    int lo = s_first[w], steps = 0;
    while (steps < 8 && lo > 0 && s_item[lo] > start) --lo, ++steps;
    while (steps < 8 && lo + 1 < NI && s_item[lo + 1] <= start) ++lo, ++steps;
    if (steps == 8) {  // far off (runs of items without chunks): binary search
      lo = 0;
      int hi = NI;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_item[mid] <= start) lo = mid;
        else hi = mid;
      }
    }
    s_first[w] = lo;
    for (int i = lo; i < NI && s_item[i] < end; ++i) {
      const int c = s_item[i], c1 = s_item[i + 1];
      if (c1 == c) continue;
      if (c >= start) s_rec[i][4] = w;
      if (c1 <= end) s_rec[i][5] = w;  // last chunk c1 - 1 in [start, end)
    }
  }
  __syncthreads();
  for (int i = t; i < NI; i += kPlanThreads) {
    const bool some = s_item[i + 1] > s_item[i];
    const int o0 = some ? s_rec[i][4] : 0;
    s_rec[i][4] = o0;
    s_rec[i][5] = some ? s_rec[i][5] - o0 + 1 : 0;
    s_rec[i][6] = 0;
    s_rec[i][7] = 0;
  }
  __syncthreads();
  for (int i = t; i < NI * kItemInts; i += kPlanThreads) p.items[i] = s_rec[i / kItemInts][i % kItemInts];
  for (int w = t; w < W; w += kPlanThreads) {
    int32_t* r = p.wrec + (size_t)w * kWorkerInts;
    const bool live = w < Wn;
    const int first = live ? s_first[w] : 0;
    r[0] = live ? s_bound[w] : 0;
    r[1] = live ? s_bound[w + 1] : 0;
    r[2] = first;
    r[3] = T;
    r[4] = NI;
    r[5] = r[6] = r[7] = 0;
#pragma unroll
    for (int j = 0; j < kItemInts; ++j) r[8 + j] = NI > 0 ? s_rec[first][j] : 0;
  }
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

// Where the k-th piece of a sequence's partial results lies: its family's
// pieces first (shared mode: slots fam_first + k * fam_stride), then its own
// (slots own_first + k - fam_n).
template <bool SHARED>
struct PieceMap {
  int fam_first, fam_n, fam_stride, own_first;
  __device__ int slot(int k) const {
    if (!SHARED) return own_first + k;
    return k < fam_n ? fam_first + k * fam_stride : own_first + (k - fam_n);
  }
};

template <int W>
struct MergeSmem {
  float wgt[kMaxGroup][kMergeTile];
  float ls[kMaxGroup][kMergeTile];
  float part[W][kMaxGroup][128];
};

template <int D, int W, bool SHARED>
__device__ void merge_long(const DecodeParams& p, int s, int head0, int nh, int tid, const PieceMap<SHARED>& pm,
                           int npieces) {
  const int Hq = p.num_heads;
  for (int idx = tid; idx < nh * D; idx += 64 * W) {
    const int head = head0 + idx / D, dd = idx % D;
    float M = kNegInf;
    for (int k = 0; k < npieces; ++k) M = fmaxf(M, p.ws_ml[((size_t)pm.slot(k) * Hq + head) * 2]);
    float num = 0.f, den = 0.f;
    for (int k = 0; k < npieces; ++k) {
      const size_t r = (size_t)pm.slot(k) * Hq + head;
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
template <int D, int W, bool SHARED>
__device__ void merge_one_head(const DecodeParams& p, MergeSmem<W>& sm, int s, int head, int tid,
                               const PieceMap<SHARED>& pm, int npieces) {
  constexpr int LPP = D / 4;     // lanes per piece
  constexpr int PPW = 64 / LPP;  // pieces per wave instruction
  constexpr int kIn = 16;
  const int Hq = p.num_heads;
  const int wave = tid >> 6, lane = tid & 63;
  const int po = lane / LPP, d4 = (lane % LPP) * 4;
  const size_t step = (size_t)Hq * D;
  const float* base = p.ws_acc + (size_t)head * D + d4;
  f32x4 x[kIn];
#pragma unroll
  for (int t = 0; t < kIn; ++t) {
    const int k = (t * W + wave) * PPW + po;
    x[t] = k < npieces ? *reinterpret_cast<const f32x4*>(base + (size_t)pm.slot(k) * step) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int i = tid; i < npieces; i += 64 * W) {
    const size_t r = ((size_t)pm.slot(i) * Hq + head) * 2;
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
    acc += sm.wgt[0][k] * *reinterpret_cast<const f32x4*>(base + (size_t)pm.slot(k) * step);
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
template <int D, bool SHARED>
__device__ void merge_heads_one_wave(const DecodeParams& p, MergeSmem<1>& sm, int s, int head0, int nh, int tid,
                                     const PieceMap<SHARED>& pm, int npieces) {
  constexpr int kPre = 4;
  const int Hq = p.num_heads;
  const int lane = tid;
  constexpr int PER = D / 64;
  const size_t step = (size_t)Hq * D;
  const float* acc0 = p.ws_acc + (size_t)head0 * D + lane;
  float pre[kPre][kMaxGroup][PER];
#pragma unroll
  for (int j = 0; j < kPre; ++j)
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        pre[j][h][i] = acc0[(size_t)min(h, nh - 1) * D + (size_t)pm.slot(min(j, npieces - 1)) * step + 64 * i];
  // (m, l) of every (head, piece): m into wgt, l kept in the same slot's pair
  for (int i = tid; i < nh * npieces; i += 64) {
    const int h = i / npieces, k = i % npieces;
    const size_t r = ((size_t)pm.slot(k) * Hq + head0 + h) * 2;
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
  // the remaining pieces kBatch at a time, every load of a batch
  // unconditional (past the last piece or head: the last one again) so that
  // they all go out before the first wait; loads under per-head conditions
  // were each put behind a vmcnt(0) wait, a round trip per (piece, head)
  constexpr int kBatch = 4;
  for (int k0 = kPre; k0 < npieces; k0 += kBatch) {
    float x[kBatch][kMaxGroup][PER];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const size_t off = (size_t)pm.slot(min(k0 + b, npieces - 1)) * step;
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
#pragma unroll
        for (int i = 0; i < PER; ++i) x[b][h][i] = acc0[(size_t)min(h, nh - 1) * D + off + 64 * i];
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      if (k0 + b < npieces) {
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h < nh) {
            const float w = sm.wgt[h][k0 + b];
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[h][i] = fmaf(w, x[b][h][i], acc[h][i]);
          }
        }
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
template <int D, int W, bool SHARED>
__device__ void merge_sequence(const DecodeParams& p, MergeSmem<W>& sm, int s, int head0, int nh, int tid, int L_raw,
                               const int* meta) {
  static_assert(D <= 128, "partial-sum tile");
  const int L = capped_len(p, L_raw);
  if (L <= 0) return;
  PieceMap<SHARED> pm{0, 0, 1, 0};
  int npieces;
  if (SHARED) {
    pm = PieceMap<SHARED>{meta[0], meta[1], p.fam_max, meta[2]};
    npieces = meta[1] + meta[3];
  } else if (p.mode == kModeFixed || p.mode == kModeFixedStream) {
    const int P = p.part_chunks * kChunk;
    npieces = (L + P - 1) / P;
    pm.own_first = s * p.max_parts;
  } else {
    pm.own_first = meta[0];
    npieces = meta[1];
  }
  if (npieces <= 1) return;
  if (npieces > kMergeTile) {
    merge_long<D, W, SHARED>(p, s, head0, nh, tid, pm, npieces);
  } else if constexpr (W > 1) {
    // the W-wave launch gives each workgroup one query head
    if (nh == 1) merge_one_head<D, W, SHARED>(p, sm, s, head0, tid, pm, npieces);
    else merge_long<D, W, SHARED>(p, s, head0, nh, tid, pm, npieces);
  } else {
    merge_heads_one_wave<D, SHARED>(p, sm, s, head0, nh, tid, pm, npieces);
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
// the sequence's pieces when it was split and, for pa_write_decode outside
// the shared mode (whose decode kernel stores them), the z = 0 workgroup
// stores the new token into the cache. The attention kernel took the new
// token from k_new/v_new; its values are read first and stored last, so
// their round trips overlap the merge's.
template <int D, typename U, int W, bool SHARED>
__global__ __launch_bounds__(64 * W) void merge_kernel(DecodeParams p) {
  __shared__ MergeSmem<W> sm;
  const int s = blockIdx.x, kvh = blockIdx.y, tid = threadIdx.x;
  const int Hkv = p.num_kv_heads;
  const int nh = p.group / gridDim.z, head0 = kvh * p.group + (int)blockIdx.z * nh;
  // every load that depends on nothing else is issued first
  const int L = p.context_lens[s];
  // split record: {own first slot, own pieces}, or in shared mode {family
  // first slot, family pieces, own first slot, own pieces}
  int meta[4] = {0, 0, 0, 0};
  if (SHARED) {
#pragma unroll
    for (int i = 0; i < 4; ++i) meta[i] = p.ws_meta[(size_t)s * 4 + i];
  } else if (p.merge && p.mode == kModeBalanced) {
    meta[0] = p.ws_meta[2 * s];
    meta[1] = p.ws_meta[2 * s + 1];
  }
  // the new token's elements e = tid, tid + 64W, ..., read unconditionally
  // (from q without one: an in-bounds row, never stored) and widened, so
  // nothing waits for them before the merge
  constexpr int NE = (D + 64 * W - 1) / (64 * W);
  uint32_t kn[NE] = {}, vn[NE] = {};
  if constexpr (!SHARED) {
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
  const int slot = (!SHARED && p.k_new && blockIdx.z == 0) ? new_token_slot(p, s, L) : -1;
  if (p.merge) merge_sequence<D, W, SHARED>(p, sm, s, head0, nh, tid, L, meta);
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

template <int NCG>
const void* mfma_kernel(int elem, int head_dim) {
  if (elem == kBF16) return head_dim == 64 ? kernel_of<MfmaEngine<kBF16, 64, kMfmaSub, NCG>, 64>()
                                           : (head_dim == 128 ? kernel_of<MfmaEngine<kBF16, 128, kMfmaSub, NCG>, 128>() : nullptr);
  if (elem == kF16) return head_dim == 64 ? kernel_of<MfmaEngine<kF16, 64, kMfmaSub, NCG>, 64>()
                                          : (head_dim == 128 ? kernel_of<MfmaEngine<kF16, 128, kMfmaSub, NCG>, 128>() : nullptr);
  return nullptr;
}

const void* decode_fn(int elem, int head_dim, int algo, int G) {
  if (algo == kAlgoMfma) return mfma_kernel<1>(elem, head_dim);
  if (algo == kAlgoMfmaShared) return mfma_kernel<kSharedColumnGroups>(elem, head_dim);
  if (elem == kF32) return vec_kernel_d<kF32>(head_dim, G);
  if (elem == kF16) return vec_kernel_d<kF16>(head_dim, G);
  if (elem == kBF16) return vec_kernel_d<kBF16>(head_dim, G);
  return nullptr;
}

}  // namespace

size_t decode_static_lds(int elem, int head_dim, int algo, int G) {
  if (algo == kAlgoMfma) {
    if (elem == kF32) return 0;
    return head_dim == 64 ? sizeof(MfmaEngine<kBF16, 64, kMfmaSub, 1>::Smem)
                          : sizeof(MfmaEngine<kBF16, 128, kMfmaSub, 1>::Smem);
  }
  if (algo == kAlgoMfmaShared) {
    if (elem == kF32) return 0;
    return head_dim == 64 ? sizeof(MfmaEngine<kBF16, 64, kMfmaSub, kSharedColumnGroups>::Smem)
                          : sizeof(MfmaEngine<kBF16, 128, kMfmaSub, kSharedColumnGroups>::Smem);
  }
  const int D = head_dim;
  switch (G) {
    case 1: return D == 64 ? sizeof(VecEngine<kF32, 64, 1>::Smem) : sizeof(VecEngine<kF32, 128, 1>::Smem);
    case 2: return D == 64 ? sizeof(VecEngine<kF32, 64, 2>::Smem) : sizeof(VecEngine<kF32, 128, 2>::Smem);
    case 4: return D == 64 ? sizeof(VecEngine<kF32, 64, 4>::Smem) : sizeof(VecEngine<kF32, 128, 4>::Smem);
    default: return D == 64 ? sizeof(VecEngine<kF32, 64, 8>::Smem) : sizeof(VecEngine<kF32, 128, 8>::Smem);
  }
}

template <int D, typename U, int W>
const void* merge_fn_w(bool shared) {
  return shared ? reinterpret_cast<const void*>(&merge_kernel<D, U, W, true>)
                : reinterpret_cast<const void*>(&merge_kernel<D, U, W, false>);
}

// The closing launch's kernel: element width, head_dim, one or four waves,
// and whether split records come from the shared mode (only 16-bit
// elements run it).
const void* merge_fn(int elem, int head_dim, bool wide, bool shared) {
  if (elem == kF32) {
    if (wide) return head_dim == 64 ? merge_fn_w<64, uint32_t, 4>(false) : merge_fn_w<128, uint32_t, 4>(false);
    return head_dim == 64 ? merge_fn_w<64, uint32_t, 1>(false) : merge_fn_w<128, uint32_t, 1>(false);
  }
  if (wide) return head_dim == 64 ? merge_fn_w<64, uint16_t, 4>(shared) : merge_fn_w<128, uint16_t, 4>(shared);
  return head_dim == 64 ? merge_fn_w<64, uint16_t, 1>(shared) : merge_fn_w<128, uint16_t, 1>(shared);
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
  args.lens_pad = (p.mode == kModeFixed || p.mode == kModeShared) ? 0 : (p.num_seqs + 3) / 4 * 4;
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
  // (both done by the decode kernel itself when it has arrival counters; in
  // the shared mode the decode kernel stores the new tokens and this launch
  // only merges)
  if (e != hipSuccess || p.ctr != nullptr || (!merge && !p.k_new)) return e;
  // few pieces per sequence: one wave per (sequence, KV head); many (fixed
  // partitions, or a balanced split of few sequences over many workers):
  // four waves per (sequence, query head)
  const bool few_seqs = p.mode == kModeBalanced || p.mode == kModeShared;
  const bool wide = merge && (few_seqs ? (long long)workers > 4LL * p.num_seqs : p.max_parts > 4);
  const bool shared = p.mode == kModeShared;
  const void* mf = merge_fn(elem, head_dim, wide, shared);
  const unsigned z = wide ? (unsigned)p.group : 1u;
  return hipLaunchKernel(mf, dim3((unsigned)p.num_seqs, (unsigned)p.num_kv_heads, z), dim3(wide ? 256 : 64, 1, 1),
                         kargs, 0, stream);
}

hipError_t launch_plan(const DecodeParams& p, unsigned workers, hipStream_t stream) {
  DecodeParams args = p;
  int W = (int)workers;
  void* largs[] = {&args};
  const unsigned groups = (unsigned)((p.num_seqs + kLinkWaves - 1) / kLinkWaves);
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&link_kernel), dim3(groups),
                                       dim3(64 * kLinkWaves), largs, 0, stream);
  if (e != hipSuccess) return e;
  void* kargs[] = {&args, &W};
  return hipLaunchKernel(reinterpret_cast<const void*>(&plan_kernel), dim3(1), dim3(kPlanThreads), kargs, 0, stream);
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
