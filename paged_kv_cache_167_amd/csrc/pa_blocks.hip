// Block copies and the reference-counted block allocator (gfx950 host + device code).
//
// Sources (page title, section):
//  [SRC]  vLLM source walk-through (peacm.com), section 3.2 (the block manager: a free pool,
//         allocate on demand, append a token into the last block or a new one), section 3.3
//         (preemption by swapping a sequence's KV blocks out to CPU memory).
//  [DRV]  "揭开 NVIDIA 驱动栈的面纱..." (kwkd.cn), section 4: several tables may point at one
//         physical block; reference counts and copy-on-write protect the writes.
//  [SOSP] "《Efficient Memory Management for LLM Serving with PagedAttention》深度解读报告"
//         (zako-mio.github.io), section 2.4 (block-level sharing, as pages after fork) and
//         section 3.5 (CPU swap keeps the block as its unit).
//  [CON]  "PagedAttention：当 KV Cache 遇到操作系统分页" (forceinjection.github.io), section 4.3
//         (copy-on-write and block-granular offloading grow out of the block abstraction).
//
// The allocator is host code: a stack of free block ids over an initial order, one
// reference count per block.  Appending a token that starts a block takes a new block;
// appending into a partly filled block that another table also references first moves the
// writer onto a private copy (the returned pair is what pa_copy_blocks must copy).  A move
// rewrites a group of tables onto another allocator's pool (swap out / in), each distinct
// block once, so sharing survives the round trip.  Every call either completes or changes
// nothing.  One allocator must not be used from two threads at once.
//
// The copy kernel moves whole blocks (every kv head, slot and dim) of a K and a V pool, each
// pool in device memory or in pinned host memory the device can address.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

using pa_detail::fail;
using pa_detail::g_error;

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte chunks per thread, all loads before the stores

// grid: x = (pool, chunk group) with K groups first, y = pair.  A pair with an id outside
// its pool copies nothing.
__global__ __launch_bounds__(kCopyThreads) void pa_copy_blocks_kernel(
    const char* __restrict__ src_k, const char* __restrict__ src_v, char* __restrict__ dst_k,
    char* __restrict__ dst_v, const int32_t* __restrict__ pairs, int64_t src_blocks,
    int64_t dst_blocks, int64_t block_bytes, int groups_per_pool, int pair_base) {
  const int pair = pair_base + static_cast<int>(blockIdx.y);
  const int64_t s = pairs[2 * pair], d = pairs[2 * pair + 1];
  if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;
  const bool is_v = static_cast<int>(blockIdx.x) >= groups_per_pool;
  const int group = static_cast<int>(blockIdx.x) - (is_v ? groups_per_pool : 0);
  const char* src = (is_v ? src_v : src_k) + s * block_bytes;
  char* dst = (is_v ? dst_v : dst_k) + d * block_bytes;
  const int64_t chunks = block_bytes / 16;
  const int64_t c0 = static_cast<int64_t>(group) * kCopyThreads * kCopyUnroll + threadIdx.x;
  u32x4 x[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kCopyThreads;
    if (c < chunks) x[u] = *reinterpret_cast<const u32x4*>(src + c * 16);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kCopyThreads;
    if (c < chunks) *reinterpret_cast<u32x4*>(dst + c * 16) = x[u];
  }
}

// The address the current device uses for bytes [p, p + bytes): device memory of this
// device, or pinned host memory mapped for it.  Anything else (pageable host memory, another
// device's memory, a range leaving its allocation) is refused before any launch.
int device_view(const void* p, size_t bytes, const char* what, const char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
  hipPointerAttribute_t a0, a1;
  const char* last = static_cast<const char*>(p) + (bytes - 1);
  if (hipPointerGetAttributes(&a0, p) != hipSuccess || hipPointerGetAttributes(&a1, last) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", what);
  }
  if (a0.type != a1.type || (a0.type != hipMemoryTypeDevice && a0.type != hipMemoryTypeHost))
    return fail(PA_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", what);
  if (a0.type == hipMemoryTypeDevice && (a0.device != dev || a1.device != dev))
    return fail(PA_ERR_INVALID_ARG, "%s lives on device %d, not the current device %d", what, a0.device, dev);
  if (!a0.devicePointer) return fail(PA_ERR_INVALID_ARG, "%s has no device address", what);
  const char* base = static_cast<const char*>(a0.devicePointer);
  if (a0.hostPointer) base += static_cast<const char*>(p) - static_cast<const char*>(a0.hostPointer);
  *out = a0.type == hipMemoryTypeDevice ? static_cast<const char*>(p) : base;
  return PA_OK;
}

}  // namespace

// The allocator (declared opaque in pa.h): a stack of free block ids, top = next handed out,
// and one reference count per block.
struct pa_allocator {
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;
  std::vector<int32_t> refcount;

  bool valid(int32_t b) const { return b >= 0 && b < static_cast<int32_t>(refcount.size()); }
  int32_t take() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    refcount[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refcount[b] == 0) free_stack.push_back(b);
  }
};

extern "C" {

int pa_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                   const int32_t* pairs, int32_t num_pairs, int64_t src_num_blocks,
                   int64_t dst_num_blocks, int64_t block_bytes, void* stream) {
  g_error.clear();
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs %d < 0", num_pairs);
  if (src_num_blocks <= 0 || dst_num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "pools need at least one block");
  if (block_bytes <= 0 || block_bytes % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "block_bytes %lld must be a positive multiple of 16", (long long)block_bytes);
  if (block_bytes > (static_cast<int64_t>(1) << 32))
    return fail(PA_ERR_INVALID_ARG, "block_bytes above 4 GiB");
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return fail(PA_ERR_INVALID_ARG, "a pointer is NULL");
  if ((reinterpret_cast<uintptr_t>(src_k) | reinterpret_cast<uintptr_t>(src_v) |
       reinterpret_cast<uintptr_t>(dst_k) | reinterpret_cast<uintptr_t>(dst_v)) & 15)
    return fail(PA_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(pairs) & 3) return fail(PA_ERR_INVALID_ARG, "pairs must be 4-byte aligned");
  const char *sk, *sv, *dk, *dv, *pp;
  int rc;
  const size_t src_bytes = static_cast<size_t>(src_num_blocks) * static_cast<size_t>(block_bytes);
  const size_t dst_bytes = static_cast<size_t>(dst_num_blocks) * static_cast<size_t>(block_bytes);
  if ((rc = device_view(src_k, src_bytes, "src_k", &sk)) != PA_OK) return rc;
  if ((rc = device_view(src_v, src_bytes, "src_v", &sv)) != PA_OK) return rc;
  if ((rc = device_view(dst_k, dst_bytes, "dst_k", &dk)) != PA_OK) return rc;
  if ((rc = device_view(dst_v, dst_bytes, "dst_v", &dv)) != PA_OK) return rc;
  if ((rc = device_view(pairs, static_cast<size_t>(num_pairs) * 8, "pairs", &pp)) != PA_OK) return rc;
  const int64_t chunks = block_bytes / 16;
  const int64_t groups = (chunks + kCopyThreads * kCopyUnroll - 1) / (kCopyThreads * kCopyUnroll);
  if (2 * groups > 0x7FFFFFFF) return fail(PA_ERR_INVALID_ARG, "block too large");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  for (int base = 0; base < num_pairs; base += 65535) {  // grid y is at most 65535
    const int n = num_pairs - base < 65535 ? num_pairs - base : 65535;
    hipLaunchKernelGGL(pa_copy_blocks_kernel, dim3(static_cast<unsigned>(2 * groups), n), dim3(kCopyThreads),
                       0, st, sk, sv, const_cast<char*>(dk), const_cast<char*>(dv),
                       reinterpret_cast<const int32_t*>(pp), src_num_blocks, dst_num_blocks, block_bytes,
                       static_cast<int>(groups), base);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_copy_blocks_kernel launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

pa_allocator* pa_allocator_create(int32_t num_blocks, int32_t block_size, const int32_t* order) {
  g_error.clear();
  if (num_blocks <= 0 || block_size <= 0) {
    fail(PA_ERR_INVALID_ARG, "num_blocks %d and block_size %d must be > 0", num_blocks, block_size);
    return nullptr;
  }
  pa_allocator* a = new pa_allocator();
  a->block_size = block_size;
  a->refcount.assign(static_cast<size_t>(num_blocks), 0);
  a->free_stack.resize(static_cast<size_t>(num_blocks));
  std::vector<char> seen(static_cast<size_t>(num_blocks), 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = order ? order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete a;
      fail(PA_ERR_INVALID_ARG, "order is not a permutation of 0..%d", num_blocks - 1);
      return nullptr;
    }
    seen[b] = 1;
    a->free_stack[static_cast<size_t>(num_blocks - 1 - i)] = b;  // order[0] on top
  }
  return a;
}

void pa_allocator_destroy(pa_allocator* a) { delete a; }

int32_t pa_allocator_num_free(const pa_allocator* a) {
  return a ? static_cast<int32_t>(a->free_stack.size()) : -1;
}

int32_t pa_allocator_refcount(const pa_allocator* a, int32_t block) {
  return (a && a->valid(block)) ? a->refcount[block] : -1;
}

int pa_allocator_allocate(pa_allocator* a, int32_t* block) {
  g_error.clear();
  if (!a || !block) return fail(PA_ERR_INVALID_ARG, "NULL allocator or output");
  if (a->free_stack.empty()) return fail(PA_ERR_EXHAUSTED, "no free block");
  *block = a->take();
  return PA_OK;
}

int pa_allocator_share(pa_allocator* a, int32_t block) {
  g_error.clear();
  if (!a || !a->valid(block) || a->refcount[block] == 0)
    return fail(PA_ERR_INVALID_ARG, "block %d is not allocated", block);
  ++a->refcount[block];
  return PA_OK;
}

int pa_allocator_release(pa_allocator* a, int32_t block) {
  g_error.clear();
  if (!a || !a->valid(block) || a->refcount[block] == 0)
    return fail(PA_ERR_INVALID_ARG, "block %d is not allocated", block);
  a->drop(block);
  return PA_OK;
}

int pa_allocator_append_slot(pa_allocator* a, int32_t* table, int32_t capacity, int32_t* num_table_blocks,
                             int32_t ctx, int64_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  g_error.clear();
  if (!a || !table || !num_table_blocks || !slot || !cow_src || !cow_dst)
    return fail(PA_ERR_INVALID_ARG, "a pointer is NULL");
  const int32_t B = a->block_size;
  const int32_t n = *num_table_blocks;
  if (ctx < 0 || n < 0 || n > capacity) return fail(PA_ERR_INVALID_ARG, "ctx %d or table length %d invalid", ctx, n);
  const int32_t idx = ctx / B, off = ctx % B;
  *cow_src = *cow_dst = -1;
  if (off == 0) {
    if (idx != n) return fail(PA_ERR_INVALID_ARG, "position %d starts block %d but the table has %d", ctx, idx, n);
    if (n >= capacity) return fail(PA_ERR_INVALID_ARG, "table full (%d blocks)", capacity);
    if (a->free_stack.empty()) return fail(PA_ERR_EXHAUSTED, "no free block");
    table[n] = a->take();
    *num_table_blocks = n + 1;
  } else {
    if (idx != n - 1) return fail(PA_ERR_INVALID_ARG, "position %d is not in the last block of %d", ctx, n);
    const int32_t last = table[idx];
    if (!a->valid(last) || a->refcount[last] == 0)
      return fail(PA_ERR_INVALID_ARG, "table entry %d (block %d) is not allocated", idx, last);
    if (a->refcount[last] > 1) {
      if (a->free_stack.empty()) return fail(PA_ERR_EXHAUSTED, "no free block for the copy");
      const int32_t fresh = a->take();
      a->drop(last);
      table[idx] = fresh;
      *cow_src = last;
      *cow_dst = fresh;
    }
  }
  *slot = static_cast<int64_t>(table[idx]) * B + off;
  return PA_OK;
}

int pa_allocator_fork(pa_allocator* a, const int32_t* table, int32_t n, int32_t* child) {
  g_error.clear();
  if (!a || (n > 0 && (!table || !child)) || n < 0) return fail(PA_ERR_INVALID_ARG, "invalid arguments");
  for (int32_t j = 0; j < n; ++j)
    if (!a->valid(table[j]) || a->refcount[table[j]] == 0)
      return fail(PA_ERR_INVALID_ARG, "table entry %d (block %d) is not allocated", j, table[j]);
  for (int32_t j = 0; j < n; ++j) {
    ++a->refcount[table[j]];
    child[j] = table[j];
  }
  return PA_OK;
}

int pa_allocator_free_table(pa_allocator* a, const int32_t* table, int32_t n) {
  g_error.clear();
  if (!a || (n > 0 && !table) || n < 0) return fail(PA_ERR_INVALID_ARG, "invalid arguments");
  std::unordered_map<int32_t, int32_t> uses;
  for (int32_t j = 0; j < n; ++j) {
    if (!a->valid(table[j]) || a->refcount[table[j]] <= uses[table[j]])
      return fail(PA_ERR_INVALID_ARG, "table entry %d (block %d) is not allocated", j, table[j]);
    ++uses[table[j]];
  }
  for (int32_t j = 0; j < n; ++j) a->drop(table[j]);
  return PA_OK;
}

int pa_allocator_move(pa_allocator* src, pa_allocator* dst, int32_t* tables, const int32_t* lens,
                      int32_t num_tables, int32_t stride, int32_t* pairs, int32_t pairs_capacity,
                      int32_t* num_pairs) {
  g_error.clear();
  if (!src || !dst || src == dst || num_tables < 0 || stride < 0 || !num_pairs ||
      (num_tables > 0 && (!tables || !lens)))
    return fail(PA_ERR_INVALID_ARG, "invalid arguments");
  // check everything first, so that a refused move changes nothing
  std::unordered_map<int32_t, int32_t> uses;
  std::vector<int32_t> order;
  for (int32_t t = 0; t < num_tables; ++t) {
    if (lens[t] < 0 || lens[t] > stride) return fail(PA_ERR_INVALID_ARG, "table %d length %d", t, lens[t]);
    for (int32_t j = 0; j < lens[t]; ++j) {
      const int32_t b = tables[static_cast<int64_t>(t) * stride + j];
      if (!src->valid(b) || src->refcount[b] <= uses[b])
        return fail(PA_ERR_INVALID_ARG, "table %d entry %d (block %d) is not allocated", t, j, b);
      if (uses[b]++ == 0) order.push_back(b);
    }
  }
  if (order.size() > dst->free_stack.size())
    return fail(PA_ERR_EXHAUSTED, "%zu blocks to move, %zu free", order.size(), dst->free_stack.size());
  if (static_cast<int64_t>(order.size()) > pairs_capacity || (!order.empty() && !pairs))
    return fail(PA_ERR_INVALID_ARG, "room for %d pairs, %zu needed", pairs_capacity, order.size());
  std::unordered_map<int32_t, int32_t> mapping;
  int32_t np = 0;
  for (int32_t t = 0; t < num_tables; ++t) {
    for (int32_t j = 0; j < lens[t]; ++j) {
      int32_t& e = tables[static_cast<int64_t>(t) * stride + j];
      auto it = mapping.find(e);
      int32_t to;
      if (it == mapping.end()) {
        to = dst->take();
        mapping.emplace(e, to);
        pairs[2 * np] = e;
        pairs[2 * np + 1] = to;
        ++np;
      } else {
        to = it->second;
        ++dst->refcount[to];
      }
      src->drop(e);
      e = to;
    }
  }
  *num_pairs = np;
  return PA_OK;
}

}  // extern "C"
