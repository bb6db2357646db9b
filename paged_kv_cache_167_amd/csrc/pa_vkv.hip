// A virtually contiguous K/V cache over HIP virtual memory: the design the vAttention page
// sets against paging, built here as the baseline that measures what paging costs.
//
// Source (page title, section):
//  [VATT] "vAttention：无 PagedAttention 的 LLM 服务动态显存管理" (zenmind.me), sections
//         "核心机制" 1-3 (reserve a large virtually contiguous buffer per request at start-up,
//         back it with physical pages only as the KV grows, through the reserve / create /
//         map / set-access / unmap calls; a step call per iteration makes sure every active
//         request is backed before the kernels run) and "GPU / 系统数据路径" (the attention
//         kernel addresses the KV as a flat tensor; the MMU does the translation).
//
// HIP's virtual memory calls stand in for CUDA's (hipMemAddressReserve, hipMemCreate,
// hipMemMap, hipMemSetAccess, hipMemUnmap, hipMemRelease).  Layout per sequence: token-
// major [max_ctx][num_kv_heads][head_dim], so growth by a token touches one place and a page
// holds a whole number of 16-token tiles (a tile never reaches an unmapped page).  The
// device arrays of lengths and backed capacities let every kernel here refuse a position
// that no page backs: nothing reads or writes unmapped memory, whatever the caller passes.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <numeric>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

using pa_detail::fail;
using pa_detail::g_error;

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// one thread per 16-byte chunk of one (token, kv head) row; rows of positions no page backs
// are skipped
__global__ __launch_bounds__(256) void pa_vkv_write_kernel(
    const char* __restrict__ k, const char* __restrict__ v, const int32_t* __restrict__ seq_ids,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ cap, char* __restrict__ k_base,
    char* __restrict__ v_base, int64_t num_chunks, int chunks_per_row, int num_kv_heads, int max_seqs,
    int64_t seq_bytes, int64_t token_bytes) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= num_chunks) return;
  const int c = static_cast<int>(i % chunks_per_row);
  const int64_t row = i / chunks_per_row;  // = t * Hkv + h
  const int h = static_cast<int>(row % num_kv_heads);
  const int64_t t = row / num_kv_heads;
  const int64_t src = row * chunks_per_row * 16 + c * 16;
  const u32x4 kx = *reinterpret_cast<const u32x4*>(k + src);
  const u32x4 vx = *reinterpret_cast<const u32x4*>(v + src);
  const int s = seq_ids[t];
  if (s < 0 || s >= max_seqs) return;
  const int p = positions[t];
  if (p < 0 || p >= cap[s]) return;  // no page behind it
  const int64_t dst = s * seq_bytes + p * token_bytes + static_cast<int64_t>(h) * chunks_per_row * 16 + c * 16;
  *reinterpret_cast<u32x4*>(k_base + dst) = kx;
  *reinterpret_cast<u32x4*>(v_base + dst) = vx;
}

hipMemAllocationProp page_prop(int dev) {
  hipMemAllocationProp prop{};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = dev;
  return prop;
}

// Map one page of physical memory at addr (read/write for this device).
int map_page(pa_vkv* kv, char* addr, hipMemGenericAllocationHandle_t* h) {
  const hipMemAllocationProp prop = page_prop(kv->device);
  if (hipMemCreate(h, static_cast<size_t>(kv->page_bytes), &prop, 0) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_EXHAUSTED, "hipMemCreate of a %lld-byte page failed", (long long)kv->page_bytes);
  }
  if (hipMemMap(addr, static_cast<size_t>(kv->page_bytes), 0, *h, 0) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipMemRelease(*h);
    return fail(PA_ERR_HIP, "hipMemMap failed");
  }
  hipMemAccessDesc desc{};
  desc.location = prop.location;
  desc.flags = hipMemAccessFlagsProtReadWrite;
  if (hipMemSetAccess(addr, static_cast<size_t>(kv->page_bytes), &desc, 1) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipMemUnmap(addr, static_cast<size_t>(kv->page_bytes));
    (void)hipMemRelease(*h);
    return fail(PA_ERR_HIP, "hipMemSetAccess failed");
  }
  kv->mapped_bytes += kv->page_bytes;
  return PA_OK;
}

void unmap_page(pa_vkv* kv, char* addr, hipMemGenericAllocationHandle_t h) {
  (void)hipMemUnmap(addr, static_cast<size_t>(kv->page_bytes));
  (void)hipMemRelease(h);
  kv->mapped_bytes -= kv->page_bytes;
}

char* page_addr(const pa_vkv* kv, bool is_v, int32_t s, size_t page) {
  return (is_v ? kv->v_base() : kv->k_base()) + s * kv->seq_bytes + static_cast<int64_t>(page) * kv->page_bytes;
}

// Drop pages of sequence s beyond the first `keep`.
void shrink(pa_vkv* kv, int32_t s, size_t keep) {
  while (kv->k_pages[s].size() > keep) {
    const size_t pg = kv->k_pages[s].size() - 1;
    unmap_page(kv, page_addr(kv, false, s, pg), kv->k_pages[s][pg]);
    unmap_page(kv, page_addr(kv, true, s, pg), kv->v_pages[s][pg]);
    kv->k_pages[s].pop_back();
    kv->v_pages[s].pop_back();
  }
  kv->cap[s] = static_cast<int32_t>(std::min<int64_t>(kv->max_ctx, static_cast<int64_t>(kv->k_pages[s].size()) * kv->tokens_per_page));
}

void destroy(pa_vkv* kv) {
  if (!kv) return;
  (void)hipDeviceSynchronize();
  for (int32_t s = 0; s < static_cast<int32_t>(kv->k_pages.size()); ++s) shrink(kv, s, 0);
  if (kv->guard_mapped) {
    unmap_page(kv, kv->k_reserve, kv->guard_k);
    unmap_page(kv, kv->v_reserve, kv->guard_v);
  }
  if (kv->k_reserve) (void)hipMemAddressFree(kv->k_reserve, kv->reserve_bytes);
  if (kv->v_reserve) (void)hipMemAddressFree(kv->v_reserve, kv->reserve_bytes);
  if (kv->d_ctx) (void)hipFree(kv->d_ctx);
  if (kv->d_cap) (void)hipFree(kv->d_cap);
  (void)hipGetLastError();
  delete kv;
}

}  // namespace

extern "C" {

pa_vkv* pa_vkv_create(int32_t max_seqs, int32_t max_context_len, int32_t num_kv_heads, int32_t head_dim,
                      int32_t dtype, int64_t page_bytes) {
  g_error.clear();
  if (max_seqs <= 0 || max_context_len <= 0 || num_kv_heads <= 0) {
    fail(PA_ERR_INVALID_ARG, "max_seqs, max_context_len and num_kv_heads must be > 0");
    return nullptr;
  }
  if (dtype != PA_F16 || (head_dim != 64 && head_dim != 128)) {
    fail(PA_ERR_UNSUPPORTED, "the contiguous cache is built for PA_F16 and head_dim 64 or 128");
    return nullptr;
  }
  pa_vkv* kv = new pa_vkv();
  if (hipGetDevice(&kv->device) != hipSuccess) {
    (void)hipGetLastError();
    delete kv;
    fail(PA_ERR_HIP, "no device");
    return nullptr;
  }
  kv->max_seqs = max_seqs;
  kv->max_ctx = max_context_len;
  kv->num_kv_heads = num_kv_heads;
  kv->head_dim = head_dim;
  kv->dtype = dtype;
  kv->token_bytes = static_cast<int64_t>(num_kv_heads) * head_dim * 2;
  const hipMemAllocationProp prop = page_prop(kv->device);
  size_t gran = 0;
  if (hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum) != hipSuccess || gran == 0) {
    (void)hipGetLastError();
    delete kv;
    fail(PA_ERR_HIP, "hipMemGetAllocationGranularity failed");
    return nullptr;
  }
  // a page holds whole 16-token tiles and is a multiple of the granularity; by default the
  // smallest such page of at least 2 MB (measured: 32 KB pages made the decode 2.2x slower
  // than the paged pool, and the number of mappable pages runs out near ten thousand)
  const int64_t tile = 16 * kv->token_bytes;
  const int64_t unit = std::lcm(static_cast<int64_t>(gran), tile);
  constexpr int64_t kDefaultPage = static_cast<int64_t>(2) << 20;
  kv->page_bytes = page_bytes > 0 ? page_bytes : ((kDefaultPage + unit - 1) / unit) * unit;
  if (kv->page_bytes % unit != 0) {
    const int64_t want = page_bytes;
    delete kv;
    fail(PA_ERR_INVALID_ARG, "page_bytes %lld is not a multiple of %lld (granularity and 16 tokens)",
         (long long)want, (long long)unit);
    return nullptr;
  }
  kv->tokens_per_page = kv->page_bytes / kv->token_bytes;
  const int64_t pages_per_seq = (static_cast<int64_t>(max_context_len) + kv->tokens_per_page - 1) / kv->tokens_per_page;
  kv->seq_bytes = pages_per_seq * kv->page_bytes;
  kv->reserve_bytes = static_cast<size_t>(kv->page_bytes + static_cast<int64_t>(max_seqs) * kv->seq_bytes);
  kv->k_pages.resize(max_seqs);
  kv->v_pages.resize(max_seqs);
  kv->cap.assign(max_seqs, 0);
  void* kr = nullptr;
  void* vr = nullptr;
  if (hipMemAddressReserve(&kr, kv->reserve_bytes, static_cast<size_t>(kv->page_bytes), nullptr, 0) != hipSuccess ||
      hipMemAddressReserve(&vr, kv->reserve_bytes, static_cast<size_t>(kv->page_bytes), nullptr, 0) != hipSuccess) {
    (void)hipGetLastError();
    kv->k_reserve = static_cast<char*>(kr);
    destroy(kv);
    fail(PA_ERR_HIP, "hipMemAddressReserve of %zu bytes failed", kv->reserve_bytes);
    return nullptr;
  }
  kv->k_reserve = static_cast<char*>(kr);
  kv->v_reserve = static_cast<char*>(vr);
  if (map_page(kv, kv->k_reserve, &kv->guard_k) != PA_OK) {
    const std::string why = g_error;
    destroy(kv);
    fail(PA_ERR_HIP, "guard page: %s", why.c_str());
    return nullptr;
  }
  if (map_page(kv, kv->v_reserve, &kv->guard_v) != PA_OK) {
    const std::string why = g_error;
    unmap_page(kv, kv->k_reserve, kv->guard_k);
    destroy(kv);
    fail(PA_ERR_HIP, "guard page: %s", why.c_str());
    return nullptr;
  }
  kv->guard_mapped = true;
  if (hipMalloc(&kv->d_ctx, sizeof(int32_t) * max_seqs) != hipSuccess ||
      hipMalloc(&kv->d_cap, sizeof(int32_t) * max_seqs) != hipSuccess ||
      hipMemset(kv->d_ctx, 0, sizeof(int32_t) * max_seqs) != hipSuccess ||
      hipMemset(kv->d_cap, 0, sizeof(int32_t) * max_seqs) != hipSuccess) {
    (void)hipGetLastError();
    destroy(kv);
    fail(PA_ERR_HIP, "device arrays");
    return nullptr;
  }
  return kv;
}

void pa_vkv_destroy(pa_vkv* kv) { destroy(kv); }

int pa_vkv_step(pa_vkv* kv, const int32_t* context_lens, int32_t num_seqs, void* stream) {
  g_error.clear();
  if (!kv || (num_seqs > 0 && !context_lens)) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  if (num_seqs < 0 || num_seqs > kv->max_seqs)
    return fail(PA_ERR_INVALID_ARG, "num_seqs %d outside [0, %d]", num_seqs, kv->max_seqs);
  for (int32_t s = 0; s < num_seqs; ++s)
    if (context_lens[s] < 0 || context_lens[s] > kv->max_ctx)
      return fail(PA_ERR_INVALID_ARG, "context_lens[%d] = %d outside [0, %d]", s, context_lens[s], kv->max_ctx);
  // map what is missing; on failure undo this call's pages, so nothing changes
  std::vector<size_t> before(num_seqs);
  for (int32_t s = 0; s < num_seqs; ++s) before[s] = kv->k_pages[s].size();
  for (int32_t s = 0; s < num_seqs; ++s) {
    const size_t need = static_cast<size_t>((context_lens[s] + kv->tokens_per_page - 1) / kv->tokens_per_page);
    while (kv->k_pages[s].size() < need) {
      const size_t pg = kv->k_pages[s].size();
      hipMemGenericAllocationHandle_t hk{}, hv{};
      int rc = map_page(kv, page_addr(kv, false, s, pg), &hk);
      if (rc == PA_OK) {
        rc = map_page(kv, page_addr(kv, true, s, pg), &hv);
        if (rc != PA_OK) unmap_page(kv, page_addr(kv, false, s, pg), hk);
      }
      if (rc != PA_OK) {
        const std::string why = g_error;
        for (int32_t r = 0; r <= s; ++r) shrink(kv, r, before[r]);
        return fail(rc, "sequence %d, page %zu: %s", s, pg, why.c_str());
      }
      kv->k_pages[s].push_back(hk);
      kv->v_pages[s].push_back(hv);
    }
    kv->cap[s] = static_cast<int32_t>(std::min<int64_t>(kv->max_ctx, static_cast<int64_t>(kv->k_pages[s].size()) * kv->tokens_per_page));
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (num_seqs > 0 &&
      (hipMemcpyAsync(kv->d_ctx, context_lens, sizeof(int32_t) * num_seqs, hipMemcpyHostToDevice, st) != hipSuccess ||
       hipMemcpyAsync(kv->d_cap, kv->cap.data(), sizeof(int32_t) * kv->max_seqs, hipMemcpyHostToDevice, st) != hipSuccess ||
       hipStreamSynchronize(st) != hipSuccess)) {
    (void)hipGetLastError();
    return fail(PA_ERR_HIP, "copying the lengths to the device failed");
  }
  kv->num_seqs = num_seqs;
  return PA_OK;
}

int pa_vkv_free_seq(pa_vkv* kv, int32_t seq) {
  g_error.clear();
  if (!kv || seq < 0 || seq >= kv->max_seqs) return fail(PA_ERR_INVALID_ARG, "bad sequence");
  if (hipDeviceSynchronize() != hipSuccess) {  // no kernel may still read the pages
    (void)hipGetLastError();
    return fail(PA_ERR_HIP, "device synchronisation failed");
  }
  shrink(kv, seq, 0);
  const int32_t zero = 0;
  if (hipMemcpy(kv->d_cap + seq, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(kv->d_ctx + seq, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_HIP, "device arrays");
  }
  return PA_OK;
}

void* pa_vkv_k(const pa_vkv* kv) { return kv ? kv->k_base() : nullptr; }
void* pa_vkv_v(const pa_vkv* kv) { return kv ? kv->v_base() : nullptr; }
int64_t pa_vkv_seq_bytes(const pa_vkv* kv) { return kv ? kv->seq_bytes : -1; }
int64_t pa_vkv_page_bytes(const pa_vkv* kv) { return kv ? kv->page_bytes : -1; }
int64_t pa_vkv_mapped_bytes(const pa_vkv* kv) { return kv ? kv->mapped_bytes : -1; }
int32_t pa_vkv_capacity(const pa_vkv* kv, int32_t seq) {
  return (kv && seq >= 0 && seq < kv->max_seqs) ? kv->cap[seq] : -1;
}

int pa_vkv_write(pa_vkv* kv, const void* k, const void* v, const int32_t* seq_ids, const int32_t* positions,
                 int32_t num_tokens, void* stream) {
  g_error.clear();
  if (!kv) return fail(PA_ERR_INVALID_ARG, "NULL cache");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !seq_ids || !positions) return fail(PA_ERR_INVALID_ARG, "a pointer is NULL");
  if ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)
    return fail(PA_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(seq_ids) | reinterpret_cast<uintptr_t>(positions)) & 3)
    return fail(PA_ERR_INVALID_ARG, "seq_ids and positions must be 4-byte aligned");
  const int chunks_per_row = kv->head_dim * 2 / 16;
  const int64_t chunks = static_cast<int64_t>(num_tokens) * kv->num_kv_heads * chunks_per_row;
  hipLaunchKernelGGL(pa_vkv_write_kernel, dim3(static_cast<unsigned>((chunks + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(k), static_cast<const char*>(v),
                     seq_ids, positions, kv->d_cap, kv->k_base(), kv->v_base(), chunks, chunks_per_row,
                     kv->num_kv_heads, kv->max_seqs, kv->seq_bytes, kv->token_bytes);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_vkv_write_kernel launch: %s", hipGetErrorString(e));
  return PA_OK;
}

}  // extern "C"
