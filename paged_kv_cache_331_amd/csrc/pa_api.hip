// C-ABI entry points declared in include/pa.h: host-side validation, the
// single-pass / split-K choice, workspace carving, and launches on the
// caller's stream. No device memory is allocated and nothing synchronises.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "pa.h"
#include "pa_launch.h"

namespace {

constexpr int kAutoMinPartition = 256;       // partition sizes an automatic choice may use
constexpr int kAutoMaxPartition = 4096;
constexpr int kAutoBalancedPartition = 1024;  // cap when the batch alone fills the chip
constexpr int kAutoBalancedPartitionWide = 1792;  // the same cap for 2-byte rows and long tails
constexpr int kAutoBalancedPartitionFp8 = 1536;   // the same cap for FP8 rows and long tails
constexpr int kFallbackCUs = 256;             // if the device cannot be queried
constexpr int kMaxDevices = 64;

std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device, cached per device id.
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Workspace of pa_decode_append_static: one array per GPU, held by the loaded
// code object until the process ends. Host code never passes its name to a
// kernel (on the host the name is only a stand-in); it uses the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, looked up on the
// first call on that device (with it current) and kept.
int static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return PA_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int ilog2_exact(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return (1 << r) == x ? r : -1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct SplitLayout {
  size_t m_off, l_off, o_off, total;
};

// Workspace of a split call: the scheduler words (pa::kSchedBytes), then the
// running maxima, exp-sums and weighted V sums of every partial slot.
SplitLayout split_layout(int64_t num_seqs, int64_t num_q_heads, int64_t head_size, int64_t parts) {
  SplitLayout s;
  const size_t n = (size_t)(num_seqs * num_q_heads * parts);
  s.m_off = pa::kSchedBytes;
  s.l_off = s.m_off + align256(n * sizeof(float));
  s.o_off = s.l_off + align256(n * sizeof(float));
  s.total = s.o_off + align256(n * (size_t)head_size * sizeof(float));
  return s;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tag that marks a workspace's scheduler words as left by a finished call on
// this same buffer (a copy of them elsewhere, or stale bytes, does not match).
uint32_t sched_tag(const void* workspace) {
  const uint64_t x = (uint64_t)(uintptr_t)workspace;
  return (uint32_t)(x ^ (x >> 32)) ^ 0x5ca1ab1eu;
}

// Persistent scheduling of a split call's partition kernel (the counter in
// the workspace head; see decode_persistent_kernel). One counter hands out
// about 60 tickets per microsecond, so it is used only where the items are
// few and large enough to stay well below that: partitions of at least 1024
// tokens and at most 8192 items. Within that, it is used when the
// (sequence, kv head) pairs alone fill the chip (partition-major grid) and
// the kernel is bound by memory: 2-byte caches, and FP8 caches with one
// query head per kv head. The grid is 2 work-groups per compute unit for
// 2-byte caches and 3 for FP8 (whose items are half the bytes). Sweeps of
// 0 (one work-group per item) and 2..8 per compute unit over the decode
// workloads: 4-6% faster for the many-sequence 2-byte and FP8 MHA batches;
// slower for few long sequences (sequence-major grid), for FP8 GQA, where
// the dequantisation shared by the group makes the kernel VALU-heavy and the
// one-per-item grid keeps more waves resident, and for partitions of 512
// tokens or fewer (16384+ items: 10-50% slower).
#ifndef PA_PERSIST_WGS_PER_CU
#define PA_PERSIST_WGS_PER_CU 2
#endif
#ifndef PA_PERSIST_WGS_PER_CU_FP8
#define PA_PERSIST_WGS_PER_CU_FP8 3
#endif
constexpr int kPersistWgsPerCu = PA_PERSIST_WGS_PER_CU;
constexpr int kPersistWgsPerCuFp8 = PA_PERSIST_WGS_PER_CU_FP8;
constexpr int kPersistMinPartition = 1024;
constexpr int64_t kPersistMaxItems = 8192;

void set_sched(pa::DecodeParams& a, void* workspace, int cus, bool fp8_cache, int group) {
  a.sched = (unsigned long long*)workspace;
  a.sched_done = (uint32_t*)((char*)workspace + pa::kSchedDoneOffset);
  a.sched_tag = sched_tag(workspace);
  const int64_t items = (int64_t)a.num_seqs * a.num_kv_heads * a.num_parts;
  const bool persist = !a.seq_major && (!fp8_cache || group == 1) &&
                       a.part_tokens >= kPersistMinPartition && items <= kPersistMaxItems;
  a.persist_grid = persist ? (fp8_cache ? kPersistWgsPerCuFp8 : kPersistWgsPerCu) * cus : 0;
}

void clear_sched(pa::DecodeParams& a) {
  a.sched = nullptr;
  a.sched_done = nullptr;
  a.sched_tag = 0;
  a.persist_grid = 0;
}

// The automatic partition size (tokens), or -1 for a single pass. The
// largest power of two in [256, 4096] that still yields about four
// work-groups per compute unit; once the (sequence, kv head) pairs alone give
// that many, partitions only trim the tail left by the longest sequences and
// are held at 1024 tokens -- 1792 for 2-byte rows and 1536 for FP8 rows when
// that still splits the longest context (the lognormal GQA batch on the
// matrix-core item: 262-263 us at 1792 against 264-265 at 1664, 265-266 at
// 1920, 269-270 at 2048 and 267 at 2304; its FP8 form 156-157 us at 1536,
// 158 at 1792 and 2560, 161-163 at 3072). A split that would cut no more
// than a short tail off the longest sequence is not worth its combine. The
// thresholds come from sweeps of 128..4096-token partitions over the decode
// workloads.
int auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len, int cus,
                   int kv_elem_bytes) {
  const int64_t items = (int64_t)num_seqs * num_kv_heads;
  const int64_t target = 4LL * cus;
  int P = kAutoMinPartition;
  for (int c = kAutoMaxPartition; c >= kAutoMinPartition; c /= 2) {
    if (items * ceil_div(max_context_len, c) >= target) {
      P = c;
      break;
    }
  }
  if (items >= target && P > kAutoBalancedPartition) {
    const int wide = kv_elem_bytes >= 2 ? kAutoBalancedPartitionWide : kAutoBalancedPartitionFp8;
    P = 2LL * max_context_len > 3LL * wide ? wide : kAutoBalancedPartition;
  }
  if (2LL * max_context_len <= 3LL * P) return -1;
  return P;
}

bool valid_scale(float x) { return isfinite(x) && x > 0.f; }

// Host validation shared by the 2-byte and the FP8 cache writes.
int check_cache_write(const void* k, const void* v, const void* key_cache,
                      const void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                      int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                      int32_t head_size, int32_t dtype) {
  if (dtype != PA_DTYPE_FP16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_blocks < 0 || block_size < 1 || num_kv_heads < 1 || head_size < 1)
    return PA_ERR_SHAPE;
  if (num_blocks * (int64_t)block_size > INT32_MAX) return PA_ERR_SHAPE;
  if ((int64_t)num_kv_heads * head_size > INT32_MAX / 2) return PA_ERR_SHAPE;
  if (head_size % 8 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !key_cache || !value_cache || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(key_cache) || !aligned16(value_cache))
    return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// Shared body of pa_decode and pa_decode_fp8.
// The new tokens a write-then-attend call stores before attending (all
// nullptr for a plain decode).
struct Append {
  const void* k = nullptr;
  const void* v = nullptr;
  int32_t* slots = nullptr;
};

// Host checks of an append: both rows present and 16-byte aligned, slots
// representable in int32.
int check_append(const Append& ap, int64_t num_blocks, int32_t block_size) {
  if (!ap.k && !ap.v) return PA_OK;
  if (!ap.k || !ap.v) return PA_ERR_NULL;
  if (!aligned16(ap.k) || !aligned16(ap.v)) return PA_ERR_UNSUPPORTED;
  if (num_blocks * (int64_t)block_size > INT32_MAX) return PA_ERR_SHAPE;
  return PA_OK;
}

void set_append(pa::DecodeParams& a, const Append& ap, float k_scale, float v_scale) {
  a.k_new = (const uint16_t*)ap.k;
  a.v_new = (const uint16_t*)ap.v;
  a.slots_out = ap.k ? ap.slots : nullptr;
  a.k_scale_w = k_scale;
  a.v_scale_w = v_scale;
}

int decode_impl(const void* q, const void* key_cache, const void* value_cache, bool fp8_cache,
                float k_scale, float v_scale, const int32_t* block_tables,
                const int32_t* context_lens, float scale, void* out, int32_t num_seqs,
                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                int32_t partition_size, int32_t dtype, void* workspace, size_t workspace_size,
                void* stream, const Append& ap = Append()) {
  if (dtype != PA_DTYPE_FP16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_size < 1 || block_size < 1 ||
      num_blocks < 0 || max_blocks_per_seq < 1 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_SHAPE;
  if (max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  if (fp8_cache && (!valid_scale(k_scale) || !valid_scale(v_scale))) return PA_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && (partition_size % 16 != 0 || partition_size % block_size != 0))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!q || !key_cache || !value_cache || !block_tables || !context_lens || !out)
    return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(key_cache) || !aligned16(value_cache) || !aligned16(out))
    return PA_ERR_UNSUPPORTED;
  const int ast = check_append(ap, num_blocks, block_size);
  if (ast != PA_OK) return ast;

  int cus = device_cu_count();
  if (cus <= 0) cus = kFallbackCUs;
  const int P = partition_size == 0
                    ? auto_partition(num_seqs, num_kv_heads, max_context_len, cus, fp8_cache ? 1 : 2)
                    : partition_size;
  const bool split = P > 0;

  pa::DecodeParams a;
  a.q = (const uint16_t*)q;
  a.kc = key_cache;
  a.vc = value_cache;
  a.bt = block_tables;
  a.lens = context_lens;
  a.out = (uint16_t*)out;
  a.ws_m = a.ws_l = a.ws_o = nullptr;
  // log2(e): logits are kept in base 2; an FP8 cache's K scale folds in here
  a.scale_log2 = (float)((double)scale * (double)k_scale * 1.4426950408889634);
  a.v_scale = v_scale;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.log2_block_size = ilog2_exact(block_size);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.len_cap = max_context_len;
  a.tok_offset = 0;
  a.slot_base = 0;
  a.always_combine = 0;
  a.prefix_len = 0;
  a.prefix_chunks = 0;
  a.prefix_row_tiles = 0;
  if (split) {
    const int64_t parts = max_context_len > 0 ? ceil_div(max_context_len, P) : 1;
    const SplitLayout lay = split_layout(num_seqs, num_q_heads, head_size, parts);
    if (!workspace || workspace_size < lay.total) return PA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return PA_ERR_UNSUPPORTED;
    char* ws = (char*)workspace;
    a.ws_m = (float*)(ws + lay.m_off);
    a.ws_l = (float*)(ws + lay.l_off);
    a.ws_o = (float*)(ws + lay.o_off);
    a.part_tokens = P;
    a.num_parts = (int32_t)parts;
    a.part_stride = (int32_t)parts;
    // Few (sequence, kv head) pairs: order the grid sequence by sequence.
    a.seq_major = (int64_t)num_seqs * num_kv_heads < cus ? 1 : 0;
    set_sched(a, workspace, cus, fp8_cache, group);
  } else {
    a.part_tokens = max_context_len > 0 ? max_context_len : 1;
    a.num_parts = 1;
    a.part_stride = 1;
    a.seq_major = 0;
    clear_sched(a);
  }
  set_append(a, ap, k_scale, v_scale);
  const hipError_t e =
      pa::launch_decode(a, dtype, fp8_cache, head_size, group, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// Partition plan of a cascade call: the suffix positions [prefix_len,
// max_context_len) are split like an ordinary call over that range.
struct CascadePlan {
  int32_t prefix_len, suffix_max, part_tokens, num_parts, chunks, slots;
};

CascadePlan cascade_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                         int32_t max_context_len, int32_t shared_prefix_blocks,
                         int32_t partition_size, int cus) {
  CascadePlan c;
  c.prefix_len = shared_prefix_blocks * block_size;
  c.suffix_max = max_context_len > c.prefix_len ? max_context_len - c.prefix_len : 0;
  int P = partition_size;
  if (P == 0) P = auto_partition(num_seqs, num_kv_heads, c.suffix_max, cus, 2);
  if (P < 0) P = (int32_t)((c.suffix_max + 31) / 32 * 32);   // one partition
  if (P <= 0) P = 32;                                           // no suffix at all
  c.part_tokens = P;
  c.num_parts = c.suffix_max > 0 ? (int32_t)ceil_div(c.suffix_max, P) : 1;
  c.chunks = (int32_t)ceil_div(c.prefix_len, pa::kPrefixChunk);
  c.slots = c.chunks + c.num_parts;
  return c;
}

// Shared body of pa_decode_cascade and pa_decode_append.
int cascade_impl(const void* q, const void* key_cache, const void* value_cache,
                 const int32_t* block_tables, const int32_t* context_lens, float scale,
                 void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                 int32_t head_size, int32_t block_size, int64_t num_blocks,
                 int32_t max_blocks_per_seq, int32_t max_context_len,
                 int32_t shared_prefix_blocks, int32_t partition_size, int32_t dtype,
                 void* workspace, size_t workspace_size, void* stream, const Append& ap) {
  if (shared_prefix_blocks < 0 || shared_prefix_blocks > max_blocks_per_seq) return PA_ERR_SHAPE;
  if (shared_prefix_blocks == 0)
    return decode_impl(q, key_cache, value_cache, false, 1.f, 1.f, block_tables, context_lens,
                       scale, out, num_seqs, num_q_heads, num_kv_heads, head_size, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, partition_size, dtype,
                       workspace, workspace_size, stream, ap);
  // Same validation as pa_decode (run with a single pass, which enqueues nothing
  // when it fails and is not used when it passes).
  if (dtype != PA_DTYPE_FP16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_size < 1 || block_size < 1 ||
      num_blocks < 0 || max_blocks_per_seq < 1 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_SHAPE;
  if (max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
  if (partition_size > 0 && (partition_size % 16 != 0 || partition_size % block_size != 0))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  // A shared prefix lives in the pool; the matrix-core kernel also relies on
  // slot 0 existing (a masked position reads it).
  if (num_blocks < 1) return PA_ERR_SHAPE;
  if (num_blocks * (int64_t)block_size > INT32_MAX) return PA_ERR_SHAPE;   // int32 slots
  if (!q || !key_cache || !value_cache || !block_tables || !context_lens || !out)
    return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(key_cache) || !aligned16(value_cache) || !aligned16(out))
    return PA_ERR_UNSUPPORTED;
  const int ast = check_append(ap, num_blocks, block_size);
  if (ast != PA_OK) return ast;

  int cus = device_cu_count();
  if (cus <= 0) cus = kFallbackCUs;
  const CascadePlan c = cascade_plan(num_seqs, num_kv_heads, block_size, max_context_len,
                                     shared_prefix_blocks, partition_size, cus);
  const SplitLayout lay = split_layout(num_seqs, num_q_heads, head_size, c.slots);
  if (!workspace || workspace_size < lay.total) return PA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return PA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)num_seqs * group;

  pa::DecodeParams a;
  a.q = (const uint16_t*)q;
  a.kc = key_cache;
  a.vc = value_cache;
  a.bt = block_tables;
  a.lens = context_lens;
  a.out = (uint16_t*)out;
  char* ws = (char*)workspace;
  a.ws_m = (float*)(ws + lay.m_off);
  a.ws_l = (float*)(ws + lay.l_off);
  a.ws_o = (float*)(ws + lay.o_off);
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.v_scale = 1.f;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.log2_block_size = ilog2_exact(block_size);
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.len_cap = max_context_len;
  a.part_tokens = c.part_tokens;
  a.num_parts = c.num_parts;
  a.seq_major = (int64_t)num_seqs * num_kv_heads < cus ? 1 : 0;
  a.tok_offset = c.prefix_len;
  a.slot_base = c.chunks;
  a.part_stride = c.slots;
  a.always_combine = 1;     // prefix and suffix partials meet in the combine kernel
  a.prefix_len = c.prefix_len;
  a.prefix_chunks = c.chunks;
  const int rows_per_wg = pa::cascade_rows_per_wg(head_size);
  a.prefix_row_tiles = (int32_t)((rows + rows_per_wg - 1) / rows_per_wg);
  clear_sched(a);           // one work-group per item: the scheduler words stay as they are
  set_append(a, ap, 1.f, 1.f);
  const hipError_t e = pa::launch_cascade(a, dtype, head_size, group, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// Shared body of pa_prefill and pa_prefill_fp8 (fp8: the caches hold E4M3
// codes standing for their values times k_scale / v_scale).
int prefill_call(const void* q, const void* key_cache, const void* value_cache,
                 const int32_t* block_tables, const int32_t* context_lens,
                 const int32_t* query_start, float scale, void* out, int32_t num_seqs,
                 int32_t num_tokens, int32_t max_query_len, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_size, int32_t block_size, int64_t num_blocks,
                 int32_t max_blocks_per_seq, int32_t max_context_len, int32_t dtype, bool fp8,
                 float k_scale, float v_scale, void* stream) {
  if (dtype != PA_DTYPE_FP16 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || num_q_heads < 1 ||
      num_kv_heads < 1 || head_size < 1 || block_size < 1 || num_blocks < 0 ||
      max_blocks_per_seq < 1 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX) return PA_ERR_SHAPE;
  if (max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  if (fp8 && (!valid_scale(k_scale) || !valid_scale(v_scale))) return PA_ERR_SHAPE;
  const int group = num_q_heads / num_kv_heads;
  if (head_size != 64 && head_size != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
  // New tokens were written into the pool, so it has blocks; the matrix-core
  // kernel also relies on slot 0 existing (a masked position reads it).
  if (num_blocks < 1) return PA_ERR_SHAPE;
  if (num_blocks * (int64_t)block_size > INT32_MAX) return PA_ERR_SHAPE;   // int32 slots
  if (!q || !key_cache || !value_cache || !block_tables || !context_lens || !query_start ||
      !out)
    return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(key_cache) || !aligned16(value_cache) || !aligned16(out))
    return PA_ERR_UNSUPPORTED;
  pa::PrefillParams p = {};
  p.q = (const uint16_t*)q;
  p.kc = key_cache;
  p.vc = value_cache;
  p.bt = block_tables;
  p.lens = context_lens;
  p.query_start = query_start;
  p.out = (uint16_t*)out;
  // K's scale multiplies every logit: it joins the softmax scale (a positive
  // factor, so the sign the kernel folds into q is unchanged).
  p.scale_log2 = (float)((double)scale * 1.4426950408889634 * (fp8 ? (double)k_scale : 1.0));
  p.v_scale = fp8 ? v_scale : 1.f;
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.max_query_len = max_query_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.block_size = block_size;
  p.log2_block_size = ilog2_exact(block_size);
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.len_cap = max_context_len;
  p.num_blocks = num_blocks;
  const hipError_t e = pa::launch_prefill(p, dtype, head_size, group, fp8,
                                              (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "sizes are inconsistent, negative or out of range";
    case PA_ERR_DTYPE: return "unknown dtype code";
    case PA_ERR_UNSUPPORTED: return "no kernel for this head size, block size, group size, "
                                    "partition size or pointer alignment";
    case PA_ERR_WORKSPACE: return "split-K workspace missing or too small (pa_decode_append_static: "
                                  "the call needs more than PA_STATIC_SCRATCH_BYTES)";
    case PA_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case PA_ERR_NO_BLOCKS: return "the block pool has too few free blocks";
    case PA_ERR_STATE: return "the block is not allocated in the pool (or freed more often than "
                              "it is referenced)";
    default: return "unknown status";
  }
}

int pa_decode_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                           int32_t* slot_mapping, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 1) return PA_ERR_SHAPE;
  if (block_size < 1) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !context_lens || !slot_mapping) return PA_ERR_NULL;
  const hipError_t e = pa::launch_slot_mapping(block_tables, max_blocks_per_seq, context_lens,
                                               num_seqs, block_size, slot_mapping,
                                               (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_cache_write(const void* k, const void* v, void* key_cache, void* value_cache,
                   const int32_t* slot_mapping, int32_t num_tokens, int64_t num_blocks,
                   int32_t block_size, int32_t num_kv_heads, int32_t head_size, int32_t dtype,
                   void* stream) {
  const int st = check_cache_write(k, v, key_cache, value_cache, slot_mapping, num_tokens,
                                   num_blocks, block_size, num_kv_heads, head_size, dtype);
  if (st != PA_OK || num_tokens == 0) return st;
  const hipError_t e = pa::launch_cache_write(
      (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)key_cache, (uint16_t*)value_cache,
      slot_mapping, num_tokens, num_blocks * (int64_t)block_size, num_kv_heads * head_size,
      (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_cache_write_fp8(const void* k, const void* v, void* key_cache, void* value_cache,
                       const int32_t* slot_mapping, int32_t num_tokens, int64_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_size,
                       int32_t src_dtype, float k_scale, float v_scale, void* stream) {
  const int st = check_cache_write(k, v, key_cache, value_cache, slot_mapping, num_tokens,
                                   num_blocks, block_size, num_kv_heads, head_size, src_dtype);
  if (st != PA_OK) return st;
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  const hipError_t e = pa::launch_cache_write_fp8(
      (const uint16_t*)k, (const uint16_t*)v, (uint8_t*)key_cache, (uint8_t*)value_cache,
      slot_mapping, num_tokens, num_blocks * (int64_t)block_size, num_kv_heads * head_size,
      src_dtype, k_scale, v_scale, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                 int32_t max_context_len, int32_t cache_elem_bytes,
                                 int32_t num_cus) {
  if (num_seqs < 0 || num_kv_heads < 1 || max_context_len < 0) return 0;
  if (cache_elem_bytes != 1 && cache_elem_bytes != 2) return 0;
  int cus = num_cus > 0 ? num_cus : device_cu_count();
  if (cus <= 0) cus = kFallbackCUs;
  return auto_partition(num_seqs, num_kv_heads, max_context_len, cus, cache_elem_bytes);
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_size,
                                int32_t max_context_len, int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads < 0 || head_size < 0 || max_context_len < 0) return 0;
  if (partition_size < 0) return 0;
  const int64_t P = partition_size == 0 ? kAutoMinPartition : partition_size;
  const int64_t parts = max_context_len > 0 ? ceil_div(max_context_len, P) : 1;
  return split_layout(num_seqs, num_q_heads, head_size, parts).total;
}

int pa_decode(const void* q, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
              int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
              int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
              int32_t max_context_len, int32_t partition_size, int32_t dtype, void* workspace,
              size_t workspace_size, void* stream) {
  return decode_impl(q, key_cache, value_cache, false, 1.f, 1.f, block_tables, context_lens,
                     scale, out, num_seqs, num_q_heads, num_kv_heads, head_size, block_size,
                     num_blocks, max_blocks_per_seq, max_context_len, partition_size, dtype,
                     workspace, workspace_size, stream);
}

int pa_decode_fp8(const void* q, const void* key_cache, const void* value_cache,
                  const int32_t* block_tables, const int32_t* context_lens, float scale,
                  float k_scale, float v_scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_size, int32_t block_size, int64_t num_blocks,
                  int32_t max_blocks_per_seq, int32_t max_context_len, int32_t partition_size,
                  int32_t dtype, void* workspace, size_t workspace_size, void* stream) {
  return decode_impl(q, key_cache, value_cache, true, k_scale, v_scale, block_tables,
                     context_lens, scale, out, num_seqs, num_q_heads, num_kv_heads, head_size,
                     block_size, num_blocks, max_blocks_per_seq, max_context_len, partition_size,
                     dtype, workspace, workspace_size, stream);
}


size_t pa_decode_cascade_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t head_size, int32_t block_size,
                                        int32_t max_context_len, int32_t shared_prefix_blocks,
                                        int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads < 0 || head_size < 0 || block_size < 1 ||
      max_context_len < 0 || shared_prefix_blocks < 0)
    return 0;
  if (shared_prefix_blocks == 0)
    return pa_decode_workspace_size(num_seqs, num_q_heads, head_size, max_context_len,
                                    partition_size);
  const int64_t prefix_len = (int64_t)shared_prefix_blocks * block_size;
  if (prefix_len > INT32_MAX) return 0;
  const int64_t suffix_max = max_context_len > prefix_len ? max_context_len - prefix_len : 0;
  const int64_t P = partition_size > 0 ? partition_size : kAutoMinPartition;
  const int64_t parts = (partition_size < 0 || suffix_max == 0) ? 1 : ceil_div(suffix_max, P);
  const int64_t slots = ceil_div(prefix_len, pa::kPrefixChunk) + parts;
  return split_layout(num_seqs, num_q_heads, head_size, slots).total;
}

int pa_decode_cascade(const void* q, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_size, int32_t block_size, int64_t num_blocks,
                      int32_t max_blocks_per_seq, int32_t max_context_len,
                      int32_t shared_prefix_blocks, int32_t partition_size, int32_t dtype,
                      void* workspace, size_t workspace_size, void* stream) {
  return cascade_impl(q, key_cache, value_cache, block_tables, context_lens, scale, out,
                      num_seqs, num_q_heads, num_kv_heads, head_size, block_size, num_blocks,
                      max_blocks_per_seq, max_context_len, shared_prefix_blocks, partition_size,
                      dtype, workspace, workspace_size, stream, Append());
}

int pa_decode_append(const void* q, const void* k, const void* v, void* key_cache,
                     void* value_cache, const int32_t* block_tables, const int32_t* context_lens,
                     float scale, void* out, int32_t* slot_mapping, int32_t num_seqs,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                     int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                     int32_t max_context_len, int32_t shared_prefix_blocks,
                     int32_t partition_size, int32_t dtype, void* workspace,
                     size_t workspace_size, void* stream) {
  if (num_seqs > 0 && (!k || !v)) return PA_ERR_NULL;
  Append ap;
  ap.k = k;
  ap.v = v;
  ap.slots = slot_mapping;
  return cascade_impl(q, key_cache, value_cache, block_tables, context_lens, scale, out,
                      num_seqs, num_q_heads, num_kv_heads, head_size, block_size, num_blocks,
                      max_blocks_per_seq, max_context_len, shared_prefix_blocks, partition_size,
                      dtype, workspace, workspace_size, stream, ap);
}

int pa_decode_append_static(const void* q, const void* k, const void* v, void* key_cache,
                            void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, float scale, void* out,
                            int32_t* slot_mapping, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                            int64_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_context_len, int32_t shared_prefix_blocks,
                            int32_t partition_size, int32_t dtype, void* stream) {
  if (num_seqs > 0 && (!k || !v)) return PA_ERR_NULL;
  void* ws = nullptr;
  if (num_seqs > 0) {
    const int st = static_scratch(&ws);
    if (st != PA_OK) return st;
  }
  Append ap;
  ap.k = k;
  ap.v = v;
  ap.slots = slot_mapping;
  return cascade_impl(q, key_cache, value_cache, block_tables, context_lens, scale, out,
                      num_seqs, num_q_heads, num_kv_heads, head_size, block_size, num_blocks,
                      max_blocks_per_seq, max_context_len, shared_prefix_blocks, partition_size,
                      dtype, ws, PA_STATIC_SCRATCH_BYTES, stream, ap);
}

int pa_decode_append_fp8(const void* q, const void* k, const void* v, void* key_cache,
                         void* value_cache, const int32_t* block_tables,
                         const int32_t* context_lens, float scale, float k_scale, float v_scale,
                         void* out, int32_t* slot_mapping, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                         int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_context_len, int32_t partition_size, int32_t dtype,
                         void* workspace, size_t workspace_size, void* stream) {
  if (num_seqs > 0 && (!k || !v)) return PA_ERR_NULL;
  Append ap;
  ap.k = k;
  ap.v = v;
  ap.slots = slot_mapping;
  return decode_impl(q, key_cache, value_cache, true, k_scale, v_scale, block_tables,
                     context_lens, scale, out, num_seqs, num_q_heads, num_kv_heads, head_size,
                     block_size, num_blocks, max_blocks_per_seq, max_context_len, partition_size,
                     dtype, workspace, workspace_size, stream, ap);
}



int pa_prefill_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, const int32_t* query_start,
                            int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                            int32_t block_size, int32_t max_context_len, int32_t* slot_mapping,
                            void* stream) {
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || max_blocks_per_seq < 1 ||
      block_size < 1 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
  if (num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!block_tables || !context_lens || !query_start || !slot_mapping) return PA_ERR_NULL;
  pa::PrefillParams p = {};
  p.bt = block_tables;
  p.lens = context_lens;
  p.query_start = query_start;
  p.slots = slot_mapping;
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.max_query_len = max_query_len;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.len_cap = max_context_len;
  const hipError_t e = pa::launch_prefill_slots(p, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_prefill(const void* q, const void* key_cache, const void* value_cache,
               const int32_t* block_tables, const int32_t* context_lens,
               const int32_t* query_start, float scale, void* out, int32_t num_seqs,
               int32_t num_tokens, int32_t max_query_len, int32_t num_q_heads,
               int32_t num_kv_heads, int32_t head_size, int32_t block_size, int64_t num_blocks,
               int32_t max_blocks_per_seq, int32_t max_context_len, int32_t dtype, void* stream) {
  return prefill_call(q, key_cache, value_cache, block_tables, context_lens, query_start, scale,
                      out, num_seqs, num_tokens, max_query_len, num_q_heads, num_kv_heads,
                      head_size, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                      dtype, false, 1.f, 1.f, stream);
}

int pa_prefill_fp8(const void* q, const void* key_cache, const void* value_cache,
                   const int32_t* block_tables, const int32_t* context_lens,
                   const int32_t* query_start, float scale, float k_scale, float v_scale,
                   void* out, int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                   int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                   int32_t max_context_len, int32_t dtype, void* stream) {
  return prefill_call(q, key_cache, value_cache, block_tables, context_lens, query_start, scale,
                      out, num_seqs, num_tokens, max_query_len, num_q_heads, num_kv_heads,
                      head_size, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                      dtype, true, k_scale, v_scale, stream);
}


int pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* block_pairs,
                   int32_t num_pairs, int64_t num_blocks, int32_t block_size,
                   int32_t num_kv_heads, int32_t head_size, int32_t elem_bytes, void* stream) {
  if (num_pairs < 0 || num_blocks < 0 || block_size < 1 || num_kv_heads < 1 || head_size < 1)
    return PA_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2) return PA_ERR_DTYPE;
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_size * elem_bytes;
  if (block_bytes % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !block_pairs) return PA_ERR_NULL;
  if (!aligned16(key_cache) || !aligned16(value_cache)) return PA_ERR_UNSUPPORTED;
  const hipError_t e = pa::launch_copy_blocks(key_cache, value_cache, block_pairs, num_pairs,
                                              num_blocks, block_bytes, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
