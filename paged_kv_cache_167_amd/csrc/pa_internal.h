// Internal to libpa.so: the per-thread error text that every C entry point sets, shared
// by the library's source files.
#ifndef PA_INTERNAL_H
#define PA_INTERNAL_H

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

namespace pa_detail {

inline thread_local std::string g_error;

// Record a formatted error and return its code.
inline int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

}  // namespace pa_detail

// A virtually contiguous K/V cache (one layer): one address range reserved for K and one
// for V, each a guard page followed by max_seqs regions of seq_bytes, sequence s's token p
// of kv head h at base + s * seq_bytes + p * token_bytes + h * head_dim * element size.
// Physical pages are mapped into a region only as far as its sequence has grown.
struct pa_vkv {
  int device = 0;
  int32_t max_seqs = 0, max_ctx = 0, num_kv_heads = 0, head_dim = 0, dtype = 0;
  int64_t token_bytes = 0, page_bytes = 0, seq_bytes = 0, tokens_per_page = 0;
  char* k_reserve = nullptr;  // guard page, then the sequence regions
  char* v_reserve = nullptr;
  size_t reserve_bytes = 0;
  hipMemGenericAllocationHandle_t guard_k{}, guard_v{};
  bool guard_mapped = false;
  std::vector<std::vector<hipMemGenericAllocationHandle_t>> k_pages, v_pages;  // per sequence
  std::vector<int32_t> cap;  // tokens of each sequence backed by mapped pages
  int32_t* d_ctx = nullptr;  // device [max_seqs]: lengths given to the last step
  int32_t* d_cap = nullptr;  // device [max_seqs]: cap
  int32_t num_seqs = 0;      // sequences of the last step
  int64_t mapped_bytes = 0;  // K and V pages mapped, guard pages included

  char* k_base() const { return k_reserve + page_bytes; }
  char* v_base() const { return v_reserve + page_bytes; }
};

#endif  // PA_INTERNAL_H
