// extern "C" entry points of libpagedattn.so: argument checks, choice of
// kernel family and split mode, workspace layout, launch. Declarations and
// the contract of every call are in include/pagedattn.h.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "pa_internal.h"
#include "pagedattn.h"

namespace {

constexpr int kAbiVersion = 7;
constexpr size_t kAlign = 256;
constexpr size_t kCounterBytes = (size_t)pa::kArrivalSlots * sizeof(int32_t);
static_assert(kCounterBytes == PA_WORKSPACE_COUNTER_BYTES, "counter region of the header");

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool valid_dtype(int d) { return d == PA_F32 || d == PA_F16 || d == PA_BF16; }
int elem_bytes(int d) { return d == PA_F32 ? 4 : 2; }
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}

// How a decode call splits its work.
struct Plan {
  int mode;         // pa::Mode
  int part_chunks;  // fixed: chunks per partition
  int max_parts;    // fixed: partitions per sequence
  int max_workers;  // balanced: upper bound of workers per KV head
  size_t slots;     // partial-result slots (0 = never split)
};

// Shared mode takes at most kSharedMaxSeqs sequences and keeps chunk
// counts in int; otherwise the call runs the balanced split.
bool shared_ok(int num_seqs, int max_context_len) {
  const long long max_chunks = ((long long)max_context_len + pa::kChunk - 1) / pa::kChunk;
  // chunk counts and the plan's costs (at most 2 * kCostChunk per chunk
  // plus the item ends) in int
  return num_seqs <= pa::kSharedMaxSeqs && (long long)num_seqs * max_chunks < (1LL << 26);
}

Plan make_plan(int num_seqs, int num_kv_heads, int max_context_len, int partition_size) {
  Plan pl{pa::kModeFixed, 1, 1, 0, 0};
  const long long max_chunks = ((long long)max_context_len + pa::kChunk - 1) / pa::kChunk;
  if (partition_size == PA_PARTITION_SHARED && shared_ok(num_seqs, max_context_len)) {
    pl.mode = pa::kModeShared;
    const long long wmax = (pa::kSharedMaxWorkersTotal + num_kv_heads - 1) / num_kv_heads;
    const long long cap = (long long)num_seqs * max_chunks;
    pl.max_workers = (int)(wmax < cap ? wmax : cap);
    if (pl.max_workers < 1) pl.max_workers = 1;
    pl.slots = (size_t)pl.max_workers + 2 * (size_t)num_seqs;  // ordinary pieces: worker + item
    return pl;
  }
  if ((partition_size == PA_PARTITION_AUTO || partition_size == PA_PARTITION_SHARED) &&
      num_seqs <= pa::kMaxBalancedSeqs) {
    pl.mode = pa::kModeBalanced;
    const long long wmax = (pa::kMaxWorkersTotal + num_kv_heads - 1) / num_kv_heads;
    const long long cap = (long long)num_seqs * max_chunks;
    pl.max_workers = (int)(wmax < cap ? wmax : cap);
    if (pl.max_workers < 1) pl.max_workers = 1;
    pl.slots = (size_t)pl.max_workers + (size_t)num_seqs;
    return pl;
  }
  if (partition_size > 0) {
    pl.part_chunks = partition_size / pa::kChunk;
    pl.max_parts = (int)((max_chunks + pl.part_chunks - 1) / pl.part_chunks);
  } else {  // NONE, or AUTO with too many sequences: every sequence in one piece
    pl.part_chunks = (int)(max_chunks < INT_MAX ? max_chunks : INT_MAX);
    pl.max_parts = 1;
  }
  if (pl.max_parts < 1) pl.max_parts = 1;
  // persistent workers take real partitions in ranges when the per-worker
  // length scan is affordable; else (and without partitions, where whole
  // sequences would be dealt out unevenly) one workgroup per partition
  if (num_seqs <= pa::kMaxBalancedSeqs && pl.max_parts > 1) pl.mode = pa::kModeFixedStream;
  pl.slots = pl.max_parts > 1 ? (size_t)num_seqs * pl.max_parts : 0;
  return pl;
}

struct WorkspaceLayout {
  size_t ctr, meta, items, wrec, links, ml, acc, total;
  int fam_base, fam_max;  // shared mode: first family slot, sub-slots per family slot
};

// Workspace: the arrival counters (the same fixed region in every mode, so
// that no call's other regions ever overlap them; they hold zeros between
// calls), split records, then (shared mode) the plan's items, worker records
// and prefix links, then (m, l) and the partial outputs of every slot.
// Shared mode adds a family region after the ordinary slots: family slot
// (worker + family index) holds fam_max sub-slots, one per member.
WorkspaceLayout layout(const Plan& pl, int num_seqs, int num_heads, int num_kv_heads, int head_dim) {
  WorkspaceLayout w{0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (pl.slots == 0) return w;
  const bool shared = pl.mode == pa::kModeShared;
  size_t slots = pl.slots;
  if (shared) {
    w.fam_base = (int)pl.slots;
    w.fam_max = pa::shared_family_max(num_heads / num_kv_heads);
    slots += ((size_t)pl.max_workers + (size_t)num_seqs / 2 + 1) * (size_t)w.fam_max;
  }
  const size_t meta = round_up((size_t)num_seqs * (shared ? 4 : 2) * sizeof(int32_t));
  const size_t items = shared ? round_up((size_t)num_seqs * 2 * pa::kItemInts * sizeof(int32_t)) : 0;
  const size_t wrec = shared ? round_up((size_t)pl.max_workers * pa::kWorkerInts * sizeof(int32_t)) : 0;
  const size_t links = shared ? round_up((size_t)num_seqs * sizeof(int32_t)) : 0;
  const size_t ml = round_up(slots * (size_t)num_heads * 2 * sizeof(float));
  const size_t acc = round_up(slots * (size_t)num_heads * head_dim * sizeof(float));
  w.ctr = 0;
  w.meta = kCounterBytes;
  w.items = w.meta + meta;
  w.wrec = w.items + items;
  w.links = w.wrec + wrec;
  w.ml = w.links + links;
  w.acc = w.ml + ml;
  w.total = w.acc + acc;
  return w;
}

// Bytes a call with these sizes needs: shared mode also covers the
// balanced split it falls back to for fp32 elements or the vector engine.
size_t workspace_need(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int max_context_len,
                      int partition_size) {
  const Plan pl = make_plan(num_seqs, num_kv_heads, max_context_len, partition_size);
  size_t need = layout(pl, num_seqs, num_heads, num_kv_heads, head_dim).total;
  if (pl.mode == pa::kModeShared) {
    const Plan bal = make_plan(num_seqs, num_kv_heads, max_context_len, PA_PARTITION_AUTO);
    const size_t b = layout(bal, num_seqs, num_heads, num_kv_heads, head_dim).total;
    if (b > need) need = b;
  }
  return need;
}

bool decode_shape_ok(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int max_context_len,
                     int partition_size) {
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads) return false;
  if (head_dim != 64 && head_dim != 128) return false;
  if (max_context_len < 1) return false;
  if (partition_size < PA_PARTITION_SHARED) return false;
  if (partition_size > 0 && partition_size % pa::kChunk) return false;
  return true;
}

// Resident 64-thread waves per CU for each kernel, and CU counts, per device.
constexpr int kMaxDevices = 64;
constexpr int kMfmaWavesPerCu = 4;
std::mutex g_mutex;
int g_cus[kMaxDevices];
int g_lds_per_cu[kMaxDevices];
int g_waves[kMaxDevices][3][2][4][9];  // [device][elem][head_dim 64/128][algo][G]

// Balanced-split workers for one launch (all KV heads). The MFMA engine runs
// one wave per SIMD: measured on MI355X, more resident waves of it split the
// same bytes-in-flight over more pieces and lose bandwidth; the vector engine,
// with more VALU work per byte, wants every resident wave.
// Also sets *lds_per_workgroup: the CU's LDS over its resident workgroups.
int workers_target(int elem, int head_dim, int algo, int G, size_t* lds_per_workgroup) {
  int dev = 0;
  *lds_per_workgroup = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 2048;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_cus[dev] == 0) {
    int cus = 0, lds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess || lds < 1)
      lds = 65536;
    g_cus[dev] = cus;
    g_lds_per_cu[dev] = lds;
  }
  int& waves = g_waves[dev][elem][head_dim == 128][algo][G];
  if (waves == 0) {
    waves = pa::decode_waves_per_cu(elem, head_dim, algo, G);
    if (waves < 1) waves = 8;
    if ((algo == pa::kAlgoMfma || algo == pa::kAlgoMfmaShared) && waves > kMfmaWavesPerCu) waves = kMfmaWavesPerCu;
  }
  *lds_per_workgroup = (size_t)g_lds_per_cu[dev] / (size_t)waves;
  return g_cus[dev] * waves;
}

// Device address of a host swap space that is pinned, mapped for the device
// and holds `bytes` from `host` on; null otherwise (any error the queries
// leave is cleared).
void* mapped_host(const void* host, size_t bytes) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, host) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) return nullptr;
  void* start = nullptr;
  size_t size = 0;
  if (hipPointerGetAttribute(&start, HIP_POINTER_ATTRIBUTE_RANGE_START_ADDR, const_cast<void*>(host)) != hipSuccess ||
      hipPointerGetAttribute(&size, HIP_POINTER_ATTRIBUTE_RANGE_SIZE, const_cast<void*>(host)) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  const uintptr_t h = reinterpret_cast<uintptr_t>(host), s0 = reinterpret_cast<uintptr_t>(start);
  if (h < s0 || h - s0 > size || bytes > size - (h - s0)) return nullptr;
  return attr.devicePointer;
}

pa_status swap_impl(void* k_cache, void* v_cache, const void* host, int32_t host_slots, const int32_t* mapping,
                    int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                    pa_dtype dtype, bool out, void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_INVALID_ARG;
  if (num_pairs < 0 || host_slots < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
    return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !host || !mapping || host_slots == 0) return PA_ERR_INVALID_ARG;
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);
  const uintptr_t a = block_bytes % 16 == 0 ? 16 : 1;
  if (!aligned(k_cache, a) || !aligned(v_cache, a) || !aligned(host, a) || !aligned(mapping, 4))
    return PA_ERR_INVALID_ARG;
  void* dev_host = mapped_host(host, (size_t)host_slots * 2 * block_bytes);
  if (!dev_host) return PA_ERR_INVALID_ARG;
  const hipError_t e = pa::launch_swap(k_cache, v_cache, dev_host, mapping, num_pairs, num_blocks, host_slots,
                                       block_bytes, out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int32_t pa_abi_version(void) { return kAbiVersion; }

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  if (!decode_shape_ok(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size)) return 0;
  return workspace_need(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size);
}

pa_status pa_write_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_INVALID_ARG;
  if (num_tokens < 0 || num_kv_heads < 1 || num_kv_heads > 65535 || head_dim < 1 || block_size < 1 ||
      num_blocks < 1)
    return PA_ERR_INVALID_ARG;
  if ((long long)num_blocks * block_size > INT_MAX) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  const uintptr_t a = (uintptr_t)elem_bytes(dtype);
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k_new, a) || !aligned(v_new, a) || !aligned(k_cache, a) || !aligned(v_cache, a) ||
      !aligned(slot_mapping, 4))
    return PA_ERR_INVALID_ARG;
  const hipError_t e = pa::launch_write_kv(k_new, v_new, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,
                                           head_dim, block_size, num_blocks, elem_bytes(dtype),
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_prefill(void* out, const void* q, const int32_t* q_start, int32_t total_q, const void* k_cache,
                     const void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t num_blocks, int32_t max_blocks_per_seq, float scale, pa_dtype dtype, pa_dtype out_dtype,
                     void* stream) {
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || total_q < 0 || num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads)
    return PA_ERR_INVALID_ARG;
  if (num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  if (num_blocks < 1 || max_blocks_per_seq < 1 || !std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  const int log2b = log2_exact(block_size);
  if (block_size < 8 || block_size > 128 || log2b < 0) return PA_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size > INT_MAX) return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (dtype == PA_F32) return PA_ERR_UNSUPPORTED;
  const int group = num_heads / num_kv_heads;
  if (group > pa::kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (num_seqs > pa::kMaxBalancedSeqs) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (!out || !q || !q_start || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 4) ||
      !aligned(q_start, 4) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PA_ERR_INVALID_ARG;
  pa::PrefillParams p{};
  p.out = out;
  p.q = q;
  p.q_start = q_start;
  p.total_q = total_q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.block_size = block_size;
  p.log2_block = log2b;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.qt = 16 / group;
  // the kernel scales by a positive factor: the sign goes onto q (exact), and
  // a zero scale becomes q = 0 (every score 0) with factor 1
  p.q_sign = scale > 0.f ? 1 : (scale < 0.f ? -1 : 0);
  p.scale_log2 = (scale != 0.f ? std::fabs(scale) : 1.f) * 1.4426950408889634f;
  p.out_dtype = out_dtype;
  const int qb = pa::prefill_queries_per_tile(group, head_dim);
  const long long tiles = ((long long)total_q + qb - 1) / qb + num_seqs;
  if (tiles > INT_MAX) return PA_ERR_UNSUPPORTED;
  const int elem = dtype == PA_F16 ? pa::kF16 : pa::kBF16;
  const hipError_t e = pa::launch_prefill(p, elem, head_dim, (unsigned)tiles, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_swap_out(void* host, int32_t host_slots, const void* k_cache, const void* v_cache,
                      const int32_t* block_mapping, int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream) {
  return swap_impl(const_cast<void*>(k_cache), const_cast<void*>(v_cache), host, host_slots, block_mapping,
                   num_pairs, num_kv_heads, head_dim, block_size, num_blocks, dtype, true, stream);
}

pa_status pa_swap_in(void* k_cache, void* v_cache, const void* host, int32_t host_slots,
                     const int32_t* block_mapping, int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream) {
  return swap_impl(k_cache, v_cache, host, host_slots, block_mapping, num_pairs, num_kv_heads, head_dim, block_size,
                   num_blocks, dtype, false, stream);
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping, int32_t num_pairs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         pa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_INVALID_ARG;
  if (num_pairs < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
    return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_ERR_INVALID_ARG;
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype);
  const uintptr_t a = block_bytes % 16 == 0 ? 16 : 1;
  if (!aligned(k_cache, a) || !aligned(v_cache, a) || !aligned(block_mapping, 4)) return PA_ERR_INVALID_ARG;
  const hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, block_mapping, num_pairs, num_blocks, block_bytes,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"

// What a decode call with these sizes runs: kernel family and group bucket,
// split plan, workspace layout, workers per KV head (the grid's x), and
// whether the balanced split merges inside the decode kernel. Shared by the
// call and pa_decode_launches.
struct DecodeChoice {
  int kernel_algo, G, elem;
  Plan pl;
  WorkspaceLayout wl;
  long long workers;
  size_t lds_per_workgroup;
  bool in_kernel;
};

static pa_status choose_decode(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t max_context_len, int32_t partition_size, pa_dtype dtype, pa_algo algo,
                               DecodeChoice* c) {
  const int group = num_heads / num_kv_heads;
  if (algo == PA_ALGO_MFMA) {
    if (dtype == PA_F32) return PA_ERR_UNSUPPORTED;
    c->kernel_algo = pa::kAlgoMfma;
  } else if (algo == PA_ALGO_VECTOR) {
    c->kernel_algo = pa::kAlgoVector;
  } else {
    // measured on MI355X: the MFMA engine leads at every group size (the
    // vector engine takes 0.4% longer in bf16 and 3% in fp16 at the OPT-13B
    // shape, g = 1; 293 against 204 us at the Llama-3-8B shape, g = 4)
    c->kernel_algo = dtype != PA_F32 ? pa::kAlgoMfma : pa::kAlgoVector;
  }
  c->G = c->kernel_algo == pa::kAlgoMfma ? 0 : (group <= 1 ? 1 : group <= 2 ? 2 : group <= 4 ? 4 : 8);
  c->pl = make_plan(num_seqs, num_kv_heads, max_context_len, partition_size);
  if (c->pl.mode == pa::kModeShared) {
    if (c->kernel_algo == pa::kAlgoMfma) c->kernel_algo = pa::kAlgoMfmaShared;
    else c->pl = make_plan(num_seqs, num_kv_heads, max_context_len, PA_PARTITION_AUTO);  // vector engine: balanced
  }
  const Plan& pl = c->pl;
  c->wl = layout(pl, num_seqs, num_heads, num_kv_heads, head_dim);
  c->elem = dtype == PA_F32 ? pa::kF32 : (dtype == PA_F16 ? pa::kF16 : pa::kBF16);
  c->lds_per_workgroup = 0;
  const int target = workers_target(c->elem, head_dim, c->kernel_algo, c->G, &c->lds_per_workgroup);
  if (pl.mode == pa::kModeBalanced || pl.mode == pa::kModeFixedStream || pl.mode == pa::kModeShared) {
    // rounded down: every worker of the grid must be resident at once, or
    // the ones left over start only when others finish
    c->workers = target / num_kv_heads;
    const long long cap = pl.mode == pa::kModeFixedStream ? (long long)num_seqs * pl.max_parts : pl.max_workers;
    if (c->workers > cap) c->workers = cap;
    if (c->workers < 1) c->workers = 1;
  } else {
    c->workers = (long long)num_seqs * pl.max_parts;
    if (c->workers > INT_MAX) return PA_ERR_UNSUPPORTED;
  }
  // The balanced split merges inside the decode kernel when there are at
  // least a quarter as many sequences as workers per KV head, so that a
  // split sequence has few pieces (one wave merges them, a round trip per
  // eight); fewer sequences spread over many workers leave up to one piece
  // per worker, which the closing launch merges with many waves per sequence
  // (measured on MI355X, graph replay: 32 x 2,048 tokens 51.3 -> 50.5 us
  // merged in-kernel; 16 x 256 12.9 -> 15.5 us, 16 sequences of the long-
  // context shape 815 -> 822 us, so those keep the closing launch).
  // Every counter index and partial-result byte offset must fit (always, at
  // the sizes the workspace is laid out for).
  const WorkspaceLayout& wl = c->wl;
  c->in_kernel = pl.mode == pa::kModeBalanced && wl.total > 0 && 4LL * num_seqs >= c->workers &&
                 c->workers * num_kv_heads <= pa::kArrivalSlots && wl.total - wl.ml < ((size_t)1 << 31);
  return PA_OK;
}

static pa_status decode_impl(void* out, const void* q, const void* k_new, const void* v_new, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                             float scale, int32_t partition_size, void* workspace, size_t workspace_bytes, pa_dtype dtype,
                             pa_dtype out_dtype, pa_algo algo, void* stream, bool static_workspace = false) {
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return PA_ERR_INVALID_ARG;
  if (algo != PA_ALGO_AUTO && algo != PA_ALGO_VECTOR && algo != PA_ALGO_MFMA) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads) return PA_ERR_INVALID_ARG;
  if (num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  if (max_context_len < 1 || num_blocks < 1 || max_blocks_per_seq < 1) return PA_ERR_INVALID_ARG;
  if (partition_size < PA_PARTITION_SHARED || (partition_size > 0 && partition_size % pa::kChunk))
    return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  const int log2b = log2_exact(block_size);
  if (block_size < 8 || block_size > 128 || log2b < 0) return PA_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size > INT_MAX) return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  const int group = num_heads / num_kv_heads;
  if (group > pa::kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_INVALID_ARG;
  if (k_new && (!aligned(k_new, 16) || !aligned(v_new, 16))) return PA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 4) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PA_ERR_INVALID_ARG;

  DecodeChoice dc;
  const pa_status st = choose_decode(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size,
                                     dtype, algo, &dc);
  if (st != PA_OK) return st;
  const Plan& pl = dc.pl;
  const WorkspaceLayout& wl = dc.wl;
  if (static_workspace) {
    // the library's fixed per-device array; looked up after every argument
    // check, so a rejected call touches no device
    if (wl.total > pa::kStaticScratchBytes) return PA_ERR_WORKSPACE;
    if (pa::static_scratch(&workspace) != hipSuccess) return PA_ERR_LAUNCH;
    workspace_bytes = pa::kStaticScratchBytes;
  }
  if (wl.total > 0) {
    if (!workspace || workspace_bytes < wl.total) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PA_ERR_INVALID_ARG;
  }

  pa::DecodeParams p{};
  p.out = out;
  p.q = q;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  char* ws = static_cast<char*>(workspace);
  p.ws_meta = wl.total ? reinterpret_cast<int32_t*>(ws + wl.meta) : nullptr;
  p.ws_ml = wl.total ? reinterpret_cast<float*>(ws + wl.ml) : nullptr;
  p.ws_acc = wl.total ? reinterpret_cast<float*>(ws + wl.acc) : nullptr;
  const bool shared = pl.mode == pa::kModeShared;
  p.items = shared ? reinterpret_cast<int32_t*>(ws + wl.items) : nullptr;
  p.wrec = shared ? reinterpret_cast<int32_t*>(ws + wl.wrec) : nullptr;
  p.links = shared ? reinterpret_cast<int32_t*>(ws + wl.links) : nullptr;
  p.fam_base = wl.fam_base;
  p.fam_max = wl.fam_max;
  p.meta_stride = shared ? 4 : 2;
  p.ctr = dc.in_kernel ? reinterpret_cast<int32_t*>(ws + wl.ctr) : nullptr;
  p.max_len = max_context_len;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.block_size = block_size;
  p.log2_block = log2b;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.mode = pl.mode;
  p.part_chunks = pl.part_chunks;
  p.max_parts = pl.max_parts;
  p.out_dtype = out_dtype;

  if (shared) {
    const hipError_t e = pa::launch_plan(p, (unsigned)dc.workers, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return PA_ERR_LAUNCH;
  }
  const hipError_t e = pa::launch_decode(p, dc.elem, head_dim, dc.kernel_algo, dc.G, (unsigned)dc.workers,
                                         pl.slots > 0, dc.lds_per_workgroup, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

extern "C" {

int32_t pa_decode_launches(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_context_len, int32_t partition_size, pa_dtype dtype, pa_algo algo,
                           int32_t fused) {
  if (!valid_dtype(dtype) || (algo != PA_ALGO_AUTO && algo != PA_ALGO_VECTOR && algo != PA_ALGO_MFMA)) return 0;
  if (!decode_shape_ok(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size)) return 0;
  if (num_kv_heads > 65535 || num_heads / num_kv_heads > pa::kMaxGroup || num_seqs == 0) return 0;
  DecodeChoice dc;
  if (choose_decode(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, partition_size, dtype, algo, &dc) !=
      PA_OK)
    return 0;
  const int planning = dc.pl.mode == pa::kModeShared ? 2 : 0;
  const int closing = !dc.in_kernel && (dc.pl.slots > 0 || fused) ? 1 : 0;
  return planning + 1 + closing;
}

pa_status pa_decode_ex(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                       int32_t max_blocks_per_seq, int32_t max_context_len, float scale, int32_t partition_size,
                       void* workspace, size_t workspace_bytes, pa_dtype dtype, pa_dtype out_dtype, pa_algo algo,
                       void* stream) {
  return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                     partition_size, workspace, workspace_bytes, dtype, out_dtype, algo, stream);
}

pa_status pa_write_decode(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                          int32_t partition_size, void* workspace, size_t workspace_bytes, pa_dtype dtype,
                          pa_dtype out_dtype, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return PA_ERR_INVALID_ARG;
  return decode_impl(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                     partition_size, workspace, workspace_bytes, dtype, out_dtype, PA_ALGO_AUTO, stream);
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                            int32_t partition_size, pa_dtype dtype, pa_dtype out_dtype, void* stream) {
  return decode_impl(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale,
                     partition_size, nullptr, 0, dtype, out_dtype, PA_ALGO_AUTO, stream, true);
}

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                    int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, pa_dtype dtype, pa_dtype out_dtype, void* stream) {
  return pa_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                      head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, partition_size,
                      workspace, workspace_bytes, dtype, out_dtype, PA_ALGO_AUTO, stream);
}

}  // extern "C"
