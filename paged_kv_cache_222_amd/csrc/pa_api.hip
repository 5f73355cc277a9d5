// C ABI of libpa: argument checks, launch geometry, dispatch to the kernels.
// Declarations and the full contract are in include/pa.h.
#include <algorithm>
#include <atomic>
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>

#include "pa.h"
#include "pa_launch.h"

namespace {

bool dtype_ok(int32_t dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }
int elem_bytes(int32_t dt) { return dt == PA_F32 ? 4 : 2; }
bool dhead_ok(int32_t d) { return d == 64 || d == 128; }
int block_shift_of(int32_t bs) {
  switch (bs) {
    case 8: return 3;
    case 16: return 4;
    case 32: return 5;
    case 64: return 6;
    default: return -1;
  }
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// A failed launch returns PA_ERR_HIP; with PA_DEBUG set in the environment
// the runtime's own message is also printed to stderr.
int launch_status(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  if (getenv("PA_DEBUG"))
    fprintf(stderr, "libpa: launch failed: %s (%d)\n", hipGetErrorString(e), (int)e);
  return PA_ERR_HIP;
}

// Query heads per chunk: the whole group when it is at most 8, otherwise the
// smallest even split into chunks of at most 8.
void head_chunks(int32_t g, int* gc, int* nhc) {
  *nhc = (g + 7) / 8;
  *gc = (g + *nhc - 1) / *nhc;
}

// Shared checks of pa_decode and pa_decode_partitioned.
int check_attention(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, int32_t max_blocks,
                    const int32_t* context_lens, int32_t batch, int32_t n_kv_heads,
                    int32_t gqa_group, int32_t d_head, int32_t block_size,
                    int32_t n_blocks, int32_t dtype) {
  if (!q || !k_pool || !v_pool || !block_table || !context_lens) return PA_ERR_NULL;
  if (!dtype_ok(dtype) || !dhead_ok(d_head) || block_shift_of(block_size) < 0)
    return PA_ERR_UNSUPPORTED;
  if (n_kv_heads < 1 || gqa_group < 1 || max_blocks < 1 || n_blocks < 1)
    return PA_ERR_SHAPE;
  if ((int64_t)n_kv_heads * gqa_group > INT_MAX / 4) return PA_ERR_SHAPE;
  if ((int64_t)max_blocks * block_size > INT_MAX / 2) return PA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned4(block_table) ||
      !aligned4(context_lens))
    return PA_ERR_ALIGN;
  return PA_OK;
}

pa::AttnArgs attention_args(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, int32_t max_blocks,
                            const int32_t* context_lens, int32_t batch,
                            int32_t n_kv_heads, int32_t gqa_group, int32_t block_size,
                            int32_t n_blocks, float scale) {
  pa::AttnArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.max_blocks = max_blocks;
  a.batch = batch;
  a.n_kv_heads = n_kv_heads;
  a.gqa_group = gqa_group;
  a.n_queries = 1;
  int gc, nhc;
  head_chunks(gqa_group, &gc, &nhc);
  a.n_hchunks = nhc;
  a.heads_per_chunk = gc;
  a.block_shift = block_shift_of(block_size);
  a.n_blocks = n_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  return a;
}

// CUs of the current device and work groups of the matrix-core kernel that
// fit on one.  They depend only on the device and the kernel, and an
// occupancy query per call would cost more than a small decode step, so
// they are memoised per (device, dtype, d_head) for devices 0 ..
// kMemoDevices - 1 in relaxed atomics (concurrent first calls store the same
// value); other devices are queried on every call.
constexpr int kMemoDevices = 64;

struct DeviceFit {
  int cus;      // compute units
  int per_cu;   // work groups of the kernel per CU
};

DeviceFit query_fit(int dev, int32_t dtype, int32_t d_head) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  return DeviceFit{cus, std::min(pa::attention_mfma_occupancy(dtype, d_head), 255)};
}

DeviceFit device_fit(int32_t dtype, int32_t d_head) {
  static std::atomic<int> memo[kMemoDevices][2][2];   // cus << 8 | per_cu
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev >= kMemoDevices) return query_fit(dev, dtype, d_head);
  std::atomic<int>& c = memo[dev][dtype == PA_F16 ? 0 : 1][d_head == 64 ? 0 : 1];
  int v = c.load(std::memory_order_relaxed);
  if (v == 0) {
    const DeviceFit f = query_fit(dev, dtype, d_head);
    v = f.cus << 8 | f.per_cu;
    c.store(v, std::memory_order_relaxed);
  }
  return DeviceFit{v >> 8, v & 255};
}

// fp16/bf16 run on the matrix cores (query heads in chunks of 16); fp32 on
// the vector ALUs (chunks of at most 8).  For a partitioned launch with a
// batch the in-kernel plan can hold, the grid is sized to the device and
// every work group loops over the non-empty items.
hipError_t dispatch_attention(pa::AttnArgs a, int32_t dtype, int32_t d_head, int64_t rows,
                              hipStream_t s, int* status) {
  *status = PA_OK;
  if (dtype == PA_F32) {
    const int64_t grid = rows * a.n_kv_heads * a.n_hchunks;
    if (grid > INT_MAX) {
      *status = PA_ERR_SHAPE;
      return hipSuccess;
    }
    return pa::launch_attention_f32(a, d_head, a.heads_per_chunk, (unsigned)grid, s);
  }
  // columns of a KV head: (query token, head of the group) pairs
  a.n_hchunks = (a.gqa_group * a.n_queries + pa::kMfmaHeads - 1) / pa::kMfmaHeads;
  a.heads_per_chunk = pa::kMfmaHeads;
  const int64_t cols = (int64_t)a.n_kv_heads * a.n_hchunks;
  int64_t grid = rows * cols;
  a.persistent = 0;
  a.cu_deal = 0;
  a.xcd_spread = 0;
  const DeviceFit fit = device_fit(dtype, d_head);
  const int64_t slots = (int64_t)fit.cus * fit.per_cu;
  if ((a.partition_size > 0 || a.split) && a.batch <= pa::kPlanBatch && slots >= cols) {
    // a whole number of work groups per column (KV head and head chunk); a
    // split launch fills the device whatever the batch
    a.persistent = 1;
    grid = a.split ? slots - slots % cols : std::min(grid, slots - slots % cols);
  }
  // Shared-prefix items need the in-kernel plan and one query token; without
  // them every sequence reads its prefix through its own table (the same
  // attention, rounded in a different order).
  if (a.prefix_parts > 0 && a.persistent && a.n_queries == 1) {
    a.prefix_seqs = std::max(1, pa::kMfmaHeads * a.n_hchunks / a.gqa_group);
  } else {
    a.prefix_parts = 0;
    a.prefix_seqs = 0;
  }
  // Items dealt over CUs: the grid fills two work groups on every CU and a
  // CU's two work groups are in one column.  With shared items a CU's work
  // groups take pairs of rounds, and the columns stay on their XCDs (there
  // each XCD's L2 holds its column's prefix tiles).
  const bool cu_fit = a.persistent && !a.split && fit.per_cu == 2 && grid == slots &&
                      (grid / cols) % 2 == 0;
  a.cu_deal = cu_fit ? (a.prefix_parts > 0 ? 2 : 1) : 0;
  a.xcd_spread = a.cu_deal == 1 && (grid / 2) % (8 * cols) == 0;
  if (grid > INT_MAX || cols > INT_MAX) {
    *status = PA_ERR_SHAPE;
    return hipSuccess;
  }
  return dtype == PA_F16 ? pa::launch_attention_mfma_f16(a, d_head, (unsigned)grid, s)
                         : pa::launch_attention_mfma_bf16(a, d_head, (unsigned)grid, s);
}

// Shared by pa_decode_partitioned and pa_decode_multi.
int decode_partitioned(float* max_logits, float* exp_sums, float* tmp_out,
                       int32_t partition_size, int32_t max_partitions, const void* q,
                       const void* k_pool, const void* v_pool, const int32_t* block_table,
                       int32_t max_blocks, const int32_t* context_lens, int32_t batch,
                       int32_t n_queries, int32_t n_kv_heads, int32_t gqa_group,
                       int32_t d_head, int32_t block_size, int32_t n_blocks, float scale,
                       int32_t dtype, void* stream, const void* key_new = nullptr,
                       const void* value_new = nullptr, int32_t prefix_len = 0,
                       bool vector = false) {
  if (batch < 0 || n_queries < 1) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!max_logits || !exp_sums || !tmp_out) return PA_ERR_NULL;
  if ((key_new != nullptr) != (value_new != nullptr)) return PA_ERR_NULL;
  if (key_new && (!aligned16(key_new) || !aligned16(value_new))) return PA_ERR_ALIGN;
  int st = check_attention(q, k_pool, v_pool, block_table, max_blocks, context_lens, batch,
                           n_kv_heads, gqa_group, d_head, block_size, n_blocks, dtype);
  if (st != PA_OK) return st;
  if (n_queries > 1 && dtype == PA_F32) return PA_ERR_UNSUPPORTED;
  if ((int64_t)n_queries * n_kv_heads * gqa_group > INT_MAX / 4 ||
      (int64_t)batch * n_queries * n_kv_heads * gqa_group > INT_MAX / 2)
    return PA_ERR_SHAPE;
  if (partition_size <= 0 || partition_size % block_size != 0) return PA_ERR_PARTITION;
  if (max_partitions < 1) return PA_ERR_WORKSPACE;
  if (!aligned4(max_logits) || !aligned4(exp_sums) || !aligned16(tmp_out)) return PA_ERR_ALIGN;
  pa::AttnArgs a = attention_args(q, k_pool, v_pool, block_table, max_blocks, context_lens,
                                  batch, n_kv_heads, gqa_group, block_size, n_blocks, scale);
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.tmp_out = tmp_out;
  a.partition_size = partition_size;
  a.max_partitions = max_partitions;
  a.n_queries = n_queries;
  if (prefix_len < 0) return PA_ERR_SHAPE;
  a.prefix_parts = prefix_len / partition_size;
  // a folded write must not land in the shared positions (contract check)
  a.shared_len = key_new ? prefix_len : 0;
  const int64_t rows = (int64_t)max_partitions * batch;
  if (rows * n_kv_heads * (((int64_t)gqa_group * n_queries + 7) / 8) > INT_MAX)
    return PA_ERR_SHAPE;
  (void)hipGetLastError();
  if (key_new) {
    if (dtype == PA_F32) {
      // no folded write on the vector-ALU kernel: a separate append first
      pa::AppendArgs w{};
      w.key = key_new;
      w.value = value_new;
      w.k_pool = const_cast<void*>(k_pool);
      w.v_pool = const_cast<void*>(v_pool);
      w.block_table = block_table;
      w.context_lens = context_lens;
      w.batch = batch;
      w.max_blocks = max_blocks;
      w.n_kv_heads = n_kv_heads;
      w.row_bytes = d_head * elem_bytes(dtype);
      w.block_shift = block_shift_of(block_size);
      w.n_blocks = n_blocks;
      w.shared_len = prefix_len;
      const hipError_t e = pa::launch_append(w, (hipStream_t)stream);
      if (e != hipSuccess) return launch_status(e);
    } else {
      a.key_new = key_new;
      a.value_new = value_new;
    }
  }
  if (vector) {
    // the vector-ALU kernel for any dtype (one query token, no folded write)
    const unsigned grid = (unsigned)(rows * n_kv_heads * a.n_hchunks);
    const hipError_t e =
        dtype == PA_F32
            ? pa::launch_attention_f32(a, d_head, a.heads_per_chunk, grid, (hipStream_t)stream)
        : dtype == PA_F16
            ? pa::launch_attention_vector_f16(a, d_head, a.heads_per_chunk, grid,
                                              (hipStream_t)stream)
            : pa::launch_attention_vector_bf16(a, d_head, a.heads_per_chunk, grid,
                                               (hipStream_t)stream);
    return launch_status(e);
  }
  int st2 = PA_OK;
  const hipError_t e = dispatch_attention(a, dtype, d_head, rows, (hipStream_t)stream, &st2);
  return st2 != PA_OK ? st2 : launch_status(e);
}

// The fixed workspace of pa_decode_step_noalloc: one array per GPU the
// library runs on, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address comes
// from hipGetSymbolAddress, once per device (with that device current), and
// only that address is handed to kernels.  Calls that overlap on one GPU
// share the array and race.
constexpr int64_t kScratchBytes = int64_t(32) << 20;
__device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` on the current device, memoised for devices
// 0 .. kMemoDevices - 1 (concurrent first calls store the same address);
// null if the runtime cannot give it.
void* scratch_address() {
  static std::atomic<void*> memo[kMemoDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  if (dev < kMemoDevices) {
    void* p = memo[dev].load(std::memory_order_relaxed);
    if (p) return p;
  }
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
  if (dev < kMemoDevices && p) memo[dev].store(p, std::memory_order_relaxed);
  return p;
}

// Events set by pa_time_next_attention for the next attention launch of
// this thread.
thread_local hipEvent_t t_timing_start = nullptr;
thread_local hipEvent_t t_timing_stop = nullptr;

}  // namespace

bool pa::take_attention_events(hipEvent_t* start, hipEvent_t* stop) {
  if (!t_timing_start && !t_timing_stop) return false;
  *start = t_timing_start;
  *stop = t_timing_stop;
  t_timing_start = t_timing_stop = nullptr;
  return true;
}

extern "C" {

int pa_time_next_attention(void* start_event, void* stop_event) {
  t_timing_start = static_cast<hipEvent_t>(start_event);
  t_timing_stop = static_cast<hipEvent_t>(stop_event);
  return PA_OK;
}

const char* pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "a size is negative, zero where it must be positive, or too large";
    case PA_ERR_UNSUPPORTED: return "unsupported d_head, block_size or dtype";
    case PA_ERR_WORKSPACE: return "max_partitions must be at least 1";
    case PA_ERR_PARTITION: return "partition_size must be a positive multiple of block_size";
    case PA_ERR_HIP: return "the HIP runtime reported an error at kernel launch";
    case PA_ERR_ALIGN: return "an array pointer is not 16-byte aligned";
    case PA_ERR_NOSPACE: return "the block pool has too few free blocks";
    case PA_ERR_SCRATCH:
      return "the partition workspace would exceed the library's fixed 32 MiB scratch buffer";
    default: return "unknown status";
  }
}

int pa_cache_write(const void* key, const void* value, void* k_pool, void* v_pool,
                   const int32_t* slot_mapping, int32_t n_tokens, int32_t n_kv_heads,
                   int32_t d_head, int32_t block_size, int32_t n_blocks, int32_t dtype,
                   void* stream) {
  if (n_tokens < 0) return PA_ERR_SHAPE;
  if (n_tokens == 0) return PA_OK;
  if (!key || !value || !k_pool || !v_pool || !slot_mapping) return PA_ERR_NULL;
  if (!dtype_ok(dtype) || !dhead_ok(d_head) || block_shift_of(block_size) < 0)
    return PA_ERR_UNSUPPORTED;
  if (n_kv_heads < 1 || n_blocks < 1) return PA_ERR_SHAPE;
  if ((int64_t)n_kv_heads * d_head * elem_bytes(dtype) > INT_MAX / 2) return PA_ERR_SHAPE;
  if ((int64_t)n_tokens * n_kv_heads * d_head * elem_bytes(dtype) / 16 / 256 >= INT_MAX)
    return PA_ERR_SHAPE;  // launch grid
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned4(slot_mapping))
    return PA_ERR_ALIGN;
  pa::CacheWriteArgs a{};
  a.key = key;
  a.value = value;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.slot_mapping = slot_mapping;
  a.n_tokens = n_tokens;
  a.n_kv_heads = n_kv_heads;
  a.row_bytes = d_head * elem_bytes(dtype);
  a.block_shift = block_shift_of(block_size);
  a.n_blocks = n_blocks;
  (void)hipGetLastError();
  return launch_status(pa::launch_cache_write(a, (hipStream_t)stream));
}

int pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_pairs, int32_t n_pairs,
                   int32_t n_kv_heads, int32_t d_head, int32_t block_size, int32_t n_blocks,
                   int32_t dtype, void* stream) {
  if (n_pairs < 0) return PA_ERR_SHAPE;
  if (n_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !block_pairs) return PA_ERR_NULL;
  if (!dtype_ok(dtype) || !dhead_ok(d_head) || block_shift_of(block_size) < 0)
    return PA_ERR_UNSUPPORTED;
  if (n_kv_heads < 1 || n_blocks < 1) return PA_ERR_SHAPE;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned4(block_pairs)) return PA_ERR_ALIGN;
  pa::CopyBlocksArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_pairs = block_pairs;
  a.n_pairs = n_pairs;
  a.n_blocks = n_blocks;
  a.block_bytes = (int64_t)n_kv_heads * block_size * d_head * elem_bytes(dtype);
  if ((int64_t)n_pairs * 2 * ((a.block_bytes + pa::kCopyChunk - 1) / pa::kCopyChunk) > INT_MAX)
    return PA_ERR_SHAPE;  // launch grid
  (void)hipGetLastError();
  return launch_status(pa::launch_copy_blocks(a, (hipStream_t)stream));
}

int pa_read_ceiling(const void* buf, int64_t buf_bytes, const int32_t* tile_order,
                    int64_t n_tiles, int32_t tile_bytes, uint32_t* sink, void* stream) {
  if (n_tiles < 0 || buf_bytes < 0) return PA_ERR_SHAPE;
  if (n_tiles == 0) return PA_OK;
  if (!buf || !sink) return PA_ERR_NULL;
  if (tile_bytes <= 0 || tile_bytes % 16 != 0) return PA_ERR_SHAPE;
  const int64_t buf_tiles = buf_bytes / tile_bytes;
  if (n_tiles > INT_MAX || buf_tiles > INT_MAX) return PA_ERR_SHAPE;
  if (!tile_order && n_tiles > buf_tiles) return PA_ERR_SHAPE;
  if (!aligned16(buf) || !aligned4(sink) || (tile_order && !aligned4(tile_order)))
    return PA_ERR_ALIGN;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  pa::ReadCeilingArgs a{};
  a.buf = buf;
  a.tile_order = tile_order;
  a.sink = sink;
  a.n_tiles = n_tiles;
  a.buf_tiles = buf_tiles;
  a.tile_bytes = tile_bytes;
  const int64_t grid = std::min<int64_t>((int64_t)cus * 8, n_tiles);
  (void)hipGetLastError();
  return launch_status(pa::launch_read_ceiling(a, (unsigned)grid, (hipStream_t)stream));
}

int pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_table, int32_t max_blocks, const int32_t* context_lens,
              int32_t batch, int32_t n_kv_heads, int32_t gqa_group, int32_t d_head,
              int32_t block_size, int32_t n_blocks, float scale, int32_t dtype,
              void* stream) {
  if (batch < 0) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!out) return PA_ERR_NULL;
  int st = check_attention(q, k_pool, v_pool, block_table, max_blocks, context_lens, batch,
                           n_kv_heads, gqa_group, d_head, block_size, n_blocks, dtype);
  if (st != PA_OK) return st;
  if (!aligned16(out)) return PA_ERR_ALIGN;
  pa::AttnArgs a = attention_args(q, k_pool, v_pool, block_table, max_blocks, context_lens,
                                  batch, n_kv_heads, gqa_group, block_size, n_blocks, scale);
  a.out = out;
  a.partition_size = 0;
  a.max_partitions = 0;
  (void)hipGetLastError();
  int st2 = PA_OK;
  const hipError_t e = dispatch_attention(a, dtype, d_head, batch, (hipStream_t)stream, &st2);
  return st2 != PA_OK ? st2 : launch_status(e);
}


int pa_decode_partitioned(float* max_logits, float* exp_sums, float* tmp_out,
                          int32_t partition_size, int32_t max_partitions, const void* q,
                          const void* k_pool, const void* v_pool,
                          const int32_t* block_table, int32_t max_blocks,
                          const int32_t* context_lens, int32_t batch, int32_t n_kv_heads,
                          int32_t gqa_group, int32_t d_head, int32_t block_size,
                          int32_t n_blocks, float scale, int32_t dtype, void* stream) {
  return decode_partitioned(max_logits, exp_sums, tmp_out, partition_size, max_partitions, q,
                            k_pool, v_pool, block_table, max_blocks, context_lens, batch, 1,
                            n_kv_heads, gqa_group, d_head, block_size, n_blocks, scale, dtype,
                            stream);
}

int pa_decode_partitioned_vector(float* max_logits, float* exp_sums, float* tmp_out,
                                 int32_t partition_size, int32_t max_partitions, const void* q,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, int32_t max_blocks,
                                 const int32_t* context_lens, int32_t batch,
                                 int32_t n_kv_heads, int32_t gqa_group, int32_t d_head,
                                 int32_t block_size, int32_t n_blocks, float scale,
                                 int32_t dtype, void* stream) {
  return decode_partitioned(max_logits, exp_sums, tmp_out, partition_size, max_partitions, q,
                            k_pool, v_pool, block_table, max_blocks, context_lens, batch, 1,
                            n_kv_heads, gqa_group, d_head, block_size, n_blocks, scale, dtype,
                            stream, nullptr, nullptr, 0, true);
}

int pa_decode_step(float* max_logits, float* exp_sums, float* tmp_out, int32_t partition_size,
                   int32_t max_partitions, const void* key_new, const void* value_new,
                   const void* q, void* k_pool, void* v_pool, const int32_t* block_table,
                   int32_t max_blocks, const int32_t* context_lens, int32_t batch,
                   int32_t n_kv_heads, int32_t gqa_group, int32_t d_head, int32_t block_size,
                   int32_t n_blocks, float scale, int32_t dtype, void* stream) {
  if (batch > 0 && (!key_new || !value_new)) return PA_ERR_NULL;
  return decode_partitioned(max_logits, exp_sums, tmp_out, partition_size, max_partitions, q,
                            k_pool, v_pool, block_table, max_blocks, context_lens, batch, 1,
                            n_kv_heads, gqa_group, d_head, block_size, n_blocks, scale, dtype,
                            stream, key_new, value_new);
}

int pa_decode_shared_prefix(float* max_logits, float* exp_sums, float* tmp_out,
                            int32_t partition_size, int32_t max_partitions,
                            const void* key_new, const void* value_new, const void* q,
                            void* k_pool, void* v_pool, const int32_t* block_table,
                            int32_t max_blocks, const int32_t* context_lens, int32_t batch,
                            int32_t n_kv_heads, int32_t gqa_group, int32_t d_head,
                            int32_t block_size, int32_t n_blocks, int32_t prefix_len,
                            float scale, int32_t dtype, void* stream) {
  return decode_partitioned(max_logits, exp_sums, tmp_out, partition_size, max_partitions, q,
                            k_pool, v_pool, block_table, max_blocks, context_lens, batch, 1,
                            n_kv_heads, gqa_group, d_head, block_size, n_blocks, scale, dtype,
                            stream, key_new, value_new, prefix_len);
}

int pa_decode_split(float* max_logits, float* exp_sums, float* tmp_out, int32_t max_partitions,
                    const void* key_new, const void* value_new, const void* q, void* k_pool,
                    void* v_pool, const int32_t* block_table, int32_t max_blocks,
                    const int32_t* context_lens, int32_t batch, int32_t n_kv_heads,
                    int32_t gqa_group, int32_t d_head, int32_t block_size, int32_t n_blocks,
                    float scale, int32_t dtype, void* stream) {
  if (batch < 0) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!max_logits || !exp_sums || !tmp_out) return PA_ERR_NULL;
  if ((key_new != nullptr) != (value_new != nullptr)) return PA_ERR_NULL;
  if (key_new && (!aligned16(key_new) || !aligned16(value_new))) return PA_ERR_ALIGN;
  const int st = check_attention(q, k_pool, v_pool, block_table, max_blocks, context_lens, batch,
                                 n_kv_heads, gqa_group, d_head, block_size, n_blocks, dtype);
  if (st != PA_OK) return st;
  if (dtype == PA_F32) return PA_ERR_UNSUPPORTED;
  if (max_partitions < 2) return PA_ERR_WORKSPACE;
  // tile counts are summed in 32 bits
  if ((int64_t)batch * (((int64_t)max_blocks * block_size + 15) / 16) > INT_MAX / 2 ||
      (int64_t)batch * n_kv_heads * gqa_group > INT_MAX / 2)
    return PA_ERR_SHAPE;
  if (!aligned4(max_logits) || !aligned4(exp_sums) || !aligned16(tmp_out)) return PA_ERR_ALIGN;
  pa::AttnArgs a = attention_args(q, k_pool, v_pool, block_table, max_blocks, context_lens,
                                  batch, n_kv_heads, gqa_group, block_size, n_blocks, scale);
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.tmp_out = tmp_out;
  a.partition_size = 0;
  a.max_partitions = max_partitions;
  a.split = 1;
  a.key_new = key_new;
  a.value_new = value_new;
  (void)hipGetLastError();
  int st2 = PA_OK;
  const hipError_t e = dispatch_attention(a, dtype, d_head, batch, (hipStream_t)stream, &st2);
  return st2 != PA_OK ? st2 : launch_status(e);
}

int pa_decode_multi(float* max_logits, float* exp_sums, float* tmp_out, int32_t partition_size,
                    int32_t max_partitions, const void* q, const void* k_pool,
                    const void* v_pool, const int32_t* block_table, int32_t max_blocks,
                    const int32_t* context_lens, int32_t batch, int32_t n_queries,
                    int32_t n_kv_heads, int32_t gqa_group, int32_t d_head, int32_t block_size,
                    int32_t n_blocks, float scale, int32_t dtype, void* stream) {
  return decode_partitioned(max_logits, exp_sums, tmp_out, partition_size, max_partitions, q,
                            k_pool, v_pool, block_table, max_blocks, context_lens, batch,
                            n_queries, n_kv_heads, gqa_group, d_head, block_size, n_blocks,
                            scale, dtype, stream);
}

int pa_reduce(void* out, const float* max_logits, const float* exp_sums,
              const float* tmp_out, const int32_t* context_lens, int32_t batch,
              int32_t n_q_heads, int32_t d_head, int32_t partition_size,
              int32_t max_partitions, int32_t dtype, void* stream) {
  if (batch < 0) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!out || !max_logits || !exp_sums || !tmp_out || !context_lens) return PA_ERR_NULL;
  if (!dtype_ok(dtype) || !dhead_ok(d_head)) return PA_ERR_UNSUPPORTED;
  if (n_q_heads < 1) return PA_ERR_SHAPE;
  if (partition_size < 0) return PA_ERR_PARTITION;   // 0: a split workspace
  if (max_partitions < 1) return PA_ERR_WORKSPACE;
  if ((int64_t)batch * n_q_heads > INT_MAX) return PA_ERR_SHAPE;
  if (!aligned16(out) || !aligned4(max_logits) || !aligned4(exp_sums) ||
      !aligned16(tmp_out) || !aligned4(context_lens))
    return PA_ERR_ALIGN;
  pa::ReduceArgs a{};
  a.out = out;
  a.max_logits = max_logits;
  a.exp_sums = exp_sums;
  a.tmp_out = tmp_out;
  a.context_lens = context_lens;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.partition_size = partition_size;
  a.max_partitions = max_partitions;
  (void)hipGetLastError();
  return launch_status(pa::launch_reduce(a, dtype, d_head, (hipStream_t)stream));
}

int pa_decode_step_noalloc(void* out, int32_t partition_size, const void* key_new,
                           const void* value_new, const void* q, void* k_pool, void* v_pool,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* context_lens, int32_t batch, int32_t n_kv_heads,
                           int32_t gqa_group, int32_t d_head, int32_t block_size,
                           int32_t n_blocks, float scale, int32_t dtype, void* stream) {
  if (batch < 0) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!out || !key_new || !value_new) return PA_ERR_NULL;
  // every host-side check before the first HIP call
  const int st0 = check_attention(q, k_pool, v_pool, block_table, max_blocks, context_lens,
                                  batch, n_kv_heads, gqa_group, d_head, block_size, n_blocks,
                                  dtype);
  if (st0 != PA_OK) return st0;
  if (partition_size <= 0 || partition_size % block_size != 0) return PA_ERR_PARTITION;
  if (!aligned16(out) || !aligned16(key_new) || !aligned16(value_new)) return PA_ERR_ALIGN;
  // enough partitions for the longest context the table can hold
  const int64_t pmax = ((int64_t)max_blocks * block_size + partition_size - 1) / partition_size;
  const int64_t rows = (int64_t)batch * n_kv_heads * gqa_group;
  const int64_t bytes = rows * pmax * (d_head + 2) * 4;
  if (bytes > kScratchBytes) return PA_ERR_SCRATCH;
  void* base = scratch_address();
  if (!base) return PA_ERR_HIP;
  float* tmp_out = static_cast<float*>(base);       // [rows, pmax, d_head]
  float* max_logits = tmp_out + rows * pmax * d_head;  // [rows, pmax]
  float* exp_sums = max_logits + rows * pmax;           // [rows, pmax]
  // every workspace entry pa_reduce reads is written first by the attention
  // launch, so nothing needs clearing between calls
  const int st = pa_decode_step(max_logits, exp_sums, tmp_out, partition_size, (int32_t)pmax,
                                key_new, value_new, q, k_pool, v_pool, block_table, max_blocks,
                                context_lens, batch, n_kv_heads, gqa_group, d_head, block_size,
                                n_blocks, scale, dtype, stream);
  if (st != PA_OK) return st;
  return pa_reduce(out, max_logits, exp_sums, tmp_out, context_lens, batch,
                   n_kv_heads * gqa_group, d_head, partition_size, (int32_t)pmax, dtype, stream);
}

}  // extern "C"
