// Internal interface between the C ABI (pa_api.cpp) and the HIP kernels
// (pa_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Tokens one wave consumes per step of the decode loop. Balanced splits and
// fixed partitions both fall on multiples of it.
constexpr int kChunk = 32;
// Upper bound on balanced-split workers summed over KV heads; sizes workspaces.
constexpr int kMaxWorkersTotal = 8192;
// Arrival counters of the balanced split's in-kernel merge: one per (KV
// head, worker), at the start of every decode workspace (a fixed region, so
// calls of any shape and mode leave each other's counters alone).
constexpr int kArrivalSlots = kMaxWorkersTotal;
// Largest query-head group (num_heads / num_kv_heads) any kernel handles.
constexpr int kMaxGroup = 8;
// Balanced splits scan every sequence length in every worker; above this
// many sequences the automatic mode falls back to one wave per sequence.
constexpr int kMaxBalancedSeqs = 4096;

enum Elem : int { kF32 = 0, kF16 = 1, kBF16 = 2 };
// Balanced: chunk ranges per persistent worker. Fixed: one workgroup per
// partition. FixedStream: fixed partitions taken in ranges by persistent
// workers.
enum Mode : int { kModeBalanced = 0, kModeFixed = 1, kModeFixedStream = 2, kModeShared = 3 };

// Shared mode (balanced split over work items, where adjacent sequences
// that map the same blocks from position 0 on form families whose common
// prefix is attended once for all members).
constexpr int kSharedMaxSeqs = 1024;      // sequences a shared-mode call takes (the plan's LDS)
constexpr int kSharedColumnGroups = 2;    // 16-column MFMA groups of a family segment
constexpr int kSharedMinChunks = 2;       // a shorter common prefix does not form a family
constexpr int kSharedMaxWorkersTotal = 2048;  // workers summed over KV heads (sizes the workspace)
constexpr int kItemInts = 8;              // ints per work item record
constexpr int kWorkerInts = 16;           // ints per worker record: range, first item, its record
// Estimated cost of the shared-mode work, in sixteenths of a one-group
// 32-token chunk (per-worker clock logs of the parallel-sampling step: a
// chunk 2.3 us, a two-group family chunk 2.5 us, a member's epilogue about
// 0.4 us, the end of an item and the start of the next about 0.6 us). The
// plan splits the total cost evenly over the workers.
constexpr int kCostChunk = 16;        // a chunk, one column group
constexpr int kCostGroupChunk = 0;    // more per chunk and column group of a family's prefix
constexpr int kCostMemberEnd = 8;     // a finished family prefix, per member
constexpr int kCostItemEnd = 4;       // a finished item
// Most members of a family: column groups times the members one 16-column
// group holds (a member takes g columns, one per query head).
inline int shared_family_max(int group) { return kSharedColumnGroups * (16 / group); }
// kAlgoMfmaShared: the MFMA engine with kSharedColumnGroups column groups
// (shared mode only).
enum Algo : int { kAlgoVector = 1, kAlgoMfma = 2, kAlgoMfmaShared = 3 };

struct DecodeParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* k_new;  // [num_seqs][num_kv_heads][head_dim] new token per sequence (fused write), or null
  const void* v_new;
  int32_t* ws_meta;   // [num_seqs][2] balanced split: (first slot, pieces) of each sequence
  float* ws_ml;       // [slots][num_heads][2]  (running max in log2 units, sum)
  float* ws_acc;      // [slots][num_heads][head_dim] (unnormalised output)
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;        // num_heads / num_kv_heads
  int32_t block_size;
  int32_t log2_block;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  float scale_log2;     // scale * log2(e): scores live in base-2 exponent units
  int32_t mode;         // Mode
  int32_t part_chunks;  // fixed mode: chunks per partition
  int32_t max_parts;    // fixed mode: partitions per sequence (grid.x = num_seqs*max_parts)
  int32_t out_dtype;    // Elem of `out`
  int32_t merge;        // set by launch_decode: some sequence is split and needs merging
  int32_t lens_pad;     // set by launch_decode: ints of dynamic LDS holding the lengths
  int32_t res_slots;    // set by launch_decode: finished segments the LDS result buffer holds
  int32_t max_len;      // host bound of the context lengths: longer ones are cut to it
  // shared mode: the plan written by plan_kernel, and where family partials go
  int32_t* items;       // [2 * num_seqs][kItemInts] work items
  int32_t* wrec;        // [workers][kWorkerInts] per-worker range and first item
  int32_t* links;       // [num_seqs] common prefix (blocks) with the previous sequence
  int32_t fam_base;     // first partial-result slot of the family region
  int32_t fam_max;      // most members of a family (sub-slots per family slot)
  int32_t meta_stride;  // ints per sequence in ws_meta: 2, or 4 in shared mode
  // balanced split merged inside the decode kernel (no closing launch): the
  // workspace's arrival counters, indexed kv_head * workers + the worker
  // holding a split sequence's first chunk; zero before the launch, and the
  // worker that completes a count sets it back to zero. Null: the closing
  // launch merges and stores the new tokens.
  int32_t* ctr;
};

// Most finished segments a decode workgroup keeps in LDS before storing them.
constexpr int kMaxResultSlots = 32;

// Size of the library's own decode workspace for callers that cannot
// allocate (one array per device, kept until the process ends).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
// Device address of that array on the current device, looked up once per
// device (hipGetSymbolAddress) and kept; an error leaves *ptr untouched.
hipError_t static_scratch(void** ptr);

// Launch the decode kernel for (elem, head_dim, algo, group bucket G),
// grid = (workers per KV head, num_kv_heads), 64 threads per workgroup, then,
// unless the decode kernel merges itself (ctr set), when `merge` is set or
// the call brings new tokens (k_new), the closing kernel (grid = (num_seqs,
// num_kv_heads)) that combines the partial results of split sequences and
// stores the new tokens into the cache.
// lds_per_workgroup: the share of a CU's LDS one decode workgroup may take
// (the CU's LDS over the resident workgroups per CU the worker count assumes).
hipError_t launch_decode(const DecodeParams& p, int elem, int head_dim, int algo, int G,
                         unsigned workers, bool merge, size_t lds_per_workgroup, hipStream_t stream);
// Shared mode: the planning launches ahead of launch_decode: one compares
// every sequence's block-id list with its predecessor's (a wave per
// sequence), the next (one workgroup) forms the families and lays out the
// work items and every worker's range.
hipError_t launch_plan(const DecodeParams& p, unsigned workers, hipStream_t stream);
// Resident waves per CU of that kernel (0 if unknown).
int decode_waves_per_cu(int elem, int head_dim, int algo, int G);

hipError_t launch_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* slots, int num_tokens, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int elem_bytes, hipStream_t stream);

struct PrefillParams {
  void* out;
  const void* q;               // [total_q][num_heads][head_dim]
  const int32_t* q_start;      // [num_seqs + 1]
  int32_t total_q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t block_size;
  int32_t log2_block;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t qt;                  // query tokens per tile: the 16 MFMA columns hold qt x group (query, head) pairs
  float scale_log2;             // |scale| * log2(e), > 0
  int32_t q_sign;               // sign of the scale: q enters as q, -q, or 0
  int32_t out_dtype;
};

// Prompt-phase attention: grid (tiles, num_kv_heads), tiles an upper bound of
// sum over sequences of ceil(queries / prefill_queries_per_tile(group, head_dim)).
int prefill_queries_per_tile(int group, int head_dim);
hipError_t launch_prefill(const PrefillParams& p, int elem, int head_dim, unsigned tiles, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* mapping, int num_pairs,
                              int num_blocks, size_t block_bytes, hipStream_t stream);

// Whole-block moves between the pool and a device-mapped host swap space of
// host_slots slots ([K image][V image] of block_bytes each); `out` selects
// pool -> host.
hipError_t launch_swap(void* k_cache, void* v_cache, void* host, const int32_t* mapping, int num_pairs,
                       int num_blocks, int host_slots, size_t block_bytes, bool out, hipStream_t stream);


}  // namespace pa
